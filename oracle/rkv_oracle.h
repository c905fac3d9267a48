/* CPU oracle for the fused RoPE + KV-cache write -- TEST INFRASTRUCTURE.
 *
 * Plain, slow, single-threaded C.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header or
 * constant with the HIP library and the HIP library never calls it.
 *
 * All arrays are host memory in dense row-major order.  fp16 values are
 * passed as uint16_t IEEE binary16 bit patterns; tables are fp32.
 * Every function returns RKV_REF_OK (0) or a nonzero RKV_REF_ERR_* code and
 * writes nothing when it returns an error.
 */
#ifndef RKV_ORACLE_H
#define RKV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  RKV_REF_OK = 0,
  RKV_REF_ERR_ARG = 1,      /* null pointer, negative size, bad style, inconsistent shape */
  RKV_REF_ERR_CAPACITY = 2  /* positions do not fit the cache or the cos/sin table */
};

enum { RKV_REF_NEOX = 0, RKV_REF_GPTJ = 1 };

#define RKV_REF_TOKENS_PER_PAGE 64

/* exact binary16 -> binary64 */
double rkv_ref_half_to_double(uint16_t h);
/* binary64 -> binary16, round to nearest, ties to even, with subnormals */
uint16_t rkv_ref_double_to_half(double x);

/* exact E4M3 -> binary64 (OCP 8-bit float, e4m3fn: no infinities, 0x7f/0xff NaN) */
double rkv_ref_e4m3_to_double(uint8_t b);
/* binary64 -> E4M3, round to nearest even, saturating to +-448, NaN kept */
uint8_t rkv_ref_double_to_e4m3(double x);

/* The rotation of one head row in binary64, before any rounding to fp16;
 * w[d] = x[d] for d >= R. */
void rkv_ref_rotate_row_wide(const uint16_t* x, double* w, const float* cos_sin_row,
                             int32_t head_dim, int32_t rotary_dim, int32_t style);

/* Mean of the squares of an fp16 head row, computed exactly, rounded once. */
double rkv_ref_mean_square(const uint16_t* x, int32_t head_dim);
/* RMS normalisation: n_d = x_d * r * w_d, r = 1 / sqrt(mean_square + eps). */
void rkv_ref_rms_normalize(const uint16_t* x, double* n, const float* weight, int32_t head_dim,
                           double eps);

/* Rotate one head row x[0:D] with one table row [cos(R/2) | sin(R/2)];
 * y may equal x.  Dims d >= R are copied bit for bit. */
void rkv_ref_rotate_row(const uint16_t* x, uint16_t* y, const float* cos_sin_row,
                        int32_t head_dim, int32_t rotary_dim, int32_t style);

/* Call 1: empty-cache prefill on packed QKV, in place. */
int rkv_ref_packed_qkv(const float* cos_sin, int32_t table_batch, int32_t table_len,
                       int32_t rotary_dim, uint16_t* qkv, int32_t batch, int32_t seq_len,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       uint16_t* kv_cache, int32_t capacity, int32_t style);

/* Call 2: continuous write ending at end_lens[b]; rotated Q goes to q_out. */
int rkv_ref_continuous(const float* cos_sin, int32_t table_batch, int32_t table_len,
                       int32_t rotary_dim, const int32_t* end_lens, const uint16_t* qkv,
                       int32_t batch, int32_t seq_len, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, uint16_t* kv_cache,
                       int32_t capacity, uint16_t* q_out, int32_t style);

/* Call 3: tree-decoding write; slot from end_lens, rotary position from pos_ids. */
int rkv_ref_tree(const float* cos_sin, int32_t table_batch, int32_t table_len,
                 int32_t rotary_dim, const int32_t* end_lens, const int32_t* pos_ids,
                 const uint16_t* qkv, int32_t batch, int32_t seq_len, int32_t num_q_heads,
                 int32_t num_kv_heads, int32_t head_dim, uint16_t* kv_cache,
                 int32_t capacity, uint16_t* q_out, int32_t style);

/* Call 4: paged delta update through a page table. */
int rkv_ref_paged_delta(const uint16_t* k_delta, const uint16_t* v_delta, uint16_t* pool,
                        const float* token_cos_sin, const int32_t* delta_positions,
                        const int32_t* delta_to_seq, const int32_t* page_table,
                        int32_t num_delta, int32_t batch, int32_t num_kv_heads,
                        int32_t head_dim, int32_t rotary_dim, int32_t num_pages,
                        int32_t max_pages_per_seq, int32_t style);

/* Gather of the delta rows' cos/sin rows from a rope table
 * [rope_states, rope_rows, R]: out[i] = table[state(seq_i)][pos_i] for rows that
 * have one; other rows are set to NaN. */
int rkv_ref_gather_delta_rope(const float* rope, int32_t rope_states, int32_t rope_rows,
                              const int32_t* state_indices, const int32_t* delta_positions,
                              const int32_t* delta_to_seq, int32_t num_delta, int32_t batch,
                              int32_t rotary_dim, float* out);

/* Call 4 with the gather fused in: K of row i is rotated with the rope table
 * row of (state(seq_i), pos_i) and written only when that row exists. */
int rkv_ref_paged_delta_gather(const uint16_t* k_delta, const uint16_t* v_delta, uint16_t* pool,
                               const float* rope, int32_t rope_states, int32_t rope_rows,
                               const int32_t* state_indices, const int32_t* delta_positions,
                               const int32_t* delta_to_seq, const int32_t* page_table,
                               int32_t num_delta, int32_t batch, int32_t num_kv_heads,
                               int32_t head_dim, int32_t rotary_dim, int32_t num_pages,
                               int32_t max_pages_per_seq, int32_t style);

/* fp8 (E4M3) cache variants of the calls above: the same arguments with the
 * cache (pool) as bytes plus the per-tensor scales; each cache value is the
 * fp16 variant's unrounded K / V times 1/scale, rounded to E4M3. */
int rkv_ref_packed_qkv_fp8(const float* cos_sin, int32_t table_batch, int32_t table_len,
                           int32_t rotary_dim, uint16_t* qkv, int32_t batch, int32_t seq_len,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           uint8_t* kv_cache, int32_t capacity, float k_scale, float v_scale,
                           int32_t style);
int rkv_ref_continuous_fp8(const float* cos_sin, int32_t table_batch, int32_t table_len,
                           int32_t rotary_dim, const int32_t* end_lens, const uint16_t* qkv,
                           int32_t batch, int32_t seq_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, uint8_t* kv_cache,
                           int32_t capacity, uint16_t* q_out, float k_scale, float v_scale,
                           int32_t style);
int rkv_ref_tree_fp8(const float* cos_sin, int32_t table_batch, int32_t table_len,
                     int32_t rotary_dim, const int32_t* end_lens, const int32_t* pos_ids,
                     const uint16_t* qkv, int32_t batch, int32_t seq_len, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, uint8_t* kv_cache,
                     int32_t capacity, uint16_t* q_out, float k_scale, float v_scale,
                     int32_t style);
int rkv_ref_paged_delta_fp8(const uint16_t* k_delta, const uint16_t* v_delta, uint8_t* pool,
                            const float* token_cos_sin, const int32_t* delta_positions,
                            const int32_t* delta_to_seq, const int32_t* page_table,
                            int32_t num_delta, int32_t batch, int32_t num_kv_heads,
                            int32_t head_dim, int32_t rotary_dim, int32_t num_pages,
                            int32_t max_pages_per_seq, float k_scale, float v_scale,
                            int32_t style);
int rkv_ref_paged_delta_gather_fp8(const uint16_t* k_delta, const uint16_t* v_delta,
                                   uint8_t* pool, const float* rope, int32_t rope_states,
                                   int32_t rope_rows, const int32_t* state_indices,
                                   const int32_t* delta_positions, const int32_t* delta_to_seq,
                                   const int32_t* page_table, int32_t num_delta, int32_t batch,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t rotary_dim,
                                   int32_t num_pages, int32_t max_pages_per_seq, float k_scale,
                                   float v_scale, int32_t style);

/* Calls 1-3 with Q and K heads RMS-normalised before the rotation: q_weight /
 * k_weight [D] (either may be NULL), eps finite and >= 0; exactly one of
 * cache (fp16) and cache8 (E4M3 with k_scale / v_scale) is non-NULL. */
int rkv_ref_packed_qkv_qknorm(const float* cos_sin, int32_t table_batch, int32_t table_len,
                              int32_t rotary_dim, uint16_t* qkv, int32_t batch, int32_t seq_len,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              uint16_t* cache, uint8_t* cache8, int32_t capacity,
                              const float* q_weight, const float* k_weight, double eps,
                              float k_scale, float v_scale, int32_t style);
int rkv_ref_continuous_qknorm(const float* cos_sin, int32_t table_batch, int32_t table_len,
                              int32_t rotary_dim, const int32_t* end_lens, const uint16_t* qkv,
                              int32_t batch, int32_t seq_len, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, uint16_t* cache,
                              uint8_t* cache8, int32_t capacity, uint16_t* q_out,
                              const float* q_weight, const float* k_weight, double eps,
                              float k_scale, float v_scale, int32_t style);
int rkv_ref_tree_qknorm(const float* cos_sin, int32_t table_batch, int32_t table_len,
                        int32_t rotary_dim, const int32_t* end_lens, const int32_t* pos_ids,
                        const uint16_t* qkv, int32_t batch, int32_t seq_len, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, uint16_t* cache, uint8_t* cache8,
                        int32_t capacity, uint16_t* q_out, const float* q_weight,
                        const float* k_weight, double eps, float k_scale, float v_scale,
                        int32_t style);

/* Delta metadata: row b*delta_width + j -> (old_lengths[b] + j, b) for
 * j < min(delta_lengths[b], delta_width), else (-1, -1). */
int rkv_ref_prepare_delta_metadata(const int32_t* old_lengths, const int32_t* delta_lengths,
                                   int32_t delta_width, int32_t* delta_positions,
                                   int32_t* delta_to_seq, int32_t batch);

/* Linear tree: parent i-1 (-1 for the root), depth i, for every sequence. */
int rkv_ref_linear_tree_metadata(int32_t* parent_ids, int32_t* depths, int32_t batch,
                                 int32_t verify_size);

/* Capacity check: RKV_REF_ERR_CAPACITY iff cos_sin_len > kv_capacity. */
int rkv_ref_check_rope_capacity(int32_t cos_sin_len, int32_t kv_capacity);

#ifdef __cplusplus
}
#endif
#endif
