/* CPU oracle for the fused RoPE + KV-cache write -- TEST INFRASTRUCTURE.
 *
 * Only tests/, __graft_entry__.smoke() and the CPU-baseline leg of bench.py
 * may load this library.  It is the definition written out as plain loops:
 * no tiling, no fusion, no reordering, one (token, head) row at a time, and
 * it shares nothing with the HIP library.
 *
 * Arithmetic: inputs are fp16 (Q, K, V) and fp32 (cos/sin).  Every rotated
 * element is evaluated in binary64 as x_u*c - x_v*s (or x_v*c + x_u*s).  Both
 * products of an 11-bit by a 24-bit significand are exact in binary64, so the
 * only roundings are the one binary64 subtraction/addition and the final
 * round-to-nearest-even to binary16.  Build with -ffp-contract=off.
 * The fp8 variants take the same binary64 rotation, multiply it by the
 * reciprocal scale in binary64 and round the product once to E4M3.
 *
 * Sources (cited by page title and section):
 *  [P1] TensorRT-Edge-LLM 0.4.0 C++ API, "Apply Rope Write KV":
 *       launchApplyRopeWriteKVPackedQKV, launchApplyRopeWriteKVContinuousQAndKVCache,
 *       launchApplyRopeWriteKVTreeDecoding (shapes, dtypes, in-place and
 *       end-position semantics).
 *  [P2] sglang kernels/ops/kvcache/rope_cache.py: _get_neox_rotated_x,
 *       _get_gptj_rotated_x, _unit_rope, _load_cos_sin (pairing, sign,
 *       [cos | sin] row layout), and the slot < 0 skip of the cache write.
 *  [P3] TensorRT-Edge-LLM C++ API, "Dflash Runtime Kernels":
 *       launchDFlashTargetKVCacheUpdate (paged pool, page table, skip rules),
 *       checkDFlashRopeCapacity.
 *  [P4] libmir-cuda execution.rs, Dynamic::new: the newest token of a cache
 *       of length L sits at position L - 1.
 *  [P5] libmir-cuda execution.rs, DecodeAttentionBf16: the qkv_postprocess
 *       step (query / key norm weights, rms_norm_epsilon) ahead of the KV
 *       store.
 *
 * Readings where the pages are silent (same numbering as the design notes):
 *  R1  a table row holds cos in [0, R/2) and sin in [R/2, R).
 *  R3  with R < D, pairs are formed inside the first R dims; dims >= R are
 *      copied bit for bit.
 *  R4  table batch 1 broadcasts over the batch; table batch B is per batch.
 *  R5  kvCacheEndLens is the length after the write: the S new tokens take
 *      slots end-S .. end-1.
 *  R6  tree call: slot = end-S+s, rotary position = tokenPosIds[b,s].
 *  R7  call 1 rotates Q and K in place in the packed tensor; V is unchanged.
 *  R10 calls 2/3: a token whose slot or position is out of range writes
 *      nothing (neither qOut nor cache).
 *  R11 call 4: a row is padding if either index array is negative.
 *  R12 call 4: a row whose sequence index is >= batchSize is skipped.
 *  R13 call 4: K writes iff its id is in [0, numPages); V writes iff its id
 *      is in [numPages, 2*numPages).
 *  R14 call 4: the rotation layout is an explicit argument.
 *  R17 the capacity check rejects exactly cosSinSeqLen > kvCapacity.
 *  R23 fused gather: sequence q reads rope-table state stateIndices[q] (q
 *      itself without state indices; 0 for a single-state table); a row
 *      whose state or position has no table row writes no K (V as usual).
 *  R24 fp8 cache ([P2] HAVE_K_SCALE / HAVE_V_SCALE): the cache value is the
 *      rotated K (before any fp16 rounding; dims >= R unrotated) or the V
 *      value, times the fp32 reciprocal of the per-tensor scale, rounded to
 *      nearest-even E4M3; magnitudes past 448 saturate to 448, NaN stays NaN.
 *      Q, and the in-place K of call 1, stay fp16 as in the fp16 variant.
 *  R25 fp8 cache: a missing scale means 1; the reciprocal is 1/scale rounded
 *      once to fp32; the product is formed in binary64 and rounded to E4M3.
 *  R26 Q/K RMS norm ([P5] qkv_postprocess with query / key norm weights and
 *      rms_norm_epsilon): each Q (K) head row x becomes
 *      n_d = x_d * w_d / sqrt(mean_d(x_d^2) + eps) before the rotation, with
 *      one fp32 weight vector [D] for all Q heads and one for all K heads;
 *      dims >= R carry n_d; V is not normalised; one rounding at the end.
 *  R28 delta metadata (signature only on [P3]): rows are b*deltaWidth + j;
 *      valid for j < min(deltaLengths[b], deltaWidth) at position
 *      oldDraftCacheLengths[b] + j, owner b; padding rows are -1 / -1.
 *  Parity unpinned against the original system for R6, R7, R26 and R28: no page
 *  fixes them; they are the plainest reading consistent with the rest.
 */
#include "rkv_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- fp16 -- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exponent field 0 encodes zero and subnormals (fraction * 2^-24),
 * field 31 encodes infinity (fraction 0) and NaN. */
double rkv_ref_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

/* Round |x| to a multiple of the binary16 quantum of its binade, ties to
 * even; the subnormal range shares the quantum 2^-24 of the smallest normal
 * binade.  A result of 2^16 or more (i.e. |x| >= 65520) is infinity. */
uint16_t rkv_ref_double_to_half(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return (uint16_t)(sign | 0x7e00);
  double a = fabs(x);
  if (isinf(a)) return (uint16_t)(sign | 0x7c00);
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);              /* a = m * 2^e2, 0.5 <= m < 1 */
  int ue = e2 - 1;            /* 2^ue <= a < 2^(ue+1) */
  if (ue < -14) ue = -14;
  if (ue > 15) return (uint16_t)(sign | 0x7c00);
  double n = ldexp(a, 10 - ue);   /* a / quantum, exact */
  double fl = floor(n);
  double rem = n - fl;
  long long k = (long long)fl;
  if (rem > 0.5 || (rem == 0.5 && (k & 1))) k += 1;
  if (k >= 2048) {            /* carried into the next binade */
    k >>= 1;
    ue += 1;
  }
  if (k < 1024) return (uint16_t)(sign | (uint16_t)k);        /* subnormal */
  if (ue + 15 >= 31) return (uint16_t)(sign | 0x7c00);        /* overflow */
  return (uint16_t)(sign | (uint16_t)((ue + 15) << 10) | (uint16_t)(k - 1024));
}

/* -------------------------------------------------------------- rotate -- */

/* One head row.  [P2] _unit_rope: y = x*cos + rotate(x)*sin, where rotate
 * negates the first member of each pair and swaps it with the second
 * (_get_neox_rotated_x: partner at +R/2; _get_gptj_rotated_x: adjacent
 * partner).  Frequency i drives pair i; cos_i = row[i], sin_i = row[R/2+i]
 * ([P2] _load_cos_sin with the half-width table; R1).  Written per pair:
 *   y_u = x_u*cos_i - x_v*sin_i,  y_v = x_v*cos_i + x_u*sin_i,
 * in binary64: each product and the sum rounded once (for fp16 inputs the
 * products are exact, so only the sum rounds).  Dims >= R keep x (R3). */
static void rotate_values(const double* in, double* w, const float* row, int32_t head_dim,
                          int32_t rotary_dim, int32_t style) {
  int half = rotary_dim / 2;
  for (int d = 0; d < head_dim; ++d) w[d] = in[d];
  for (int i = 0; i < half; ++i) {
    int u, v;
    if (style == RKV_REF_NEOX) {
      u = i;
      v = i + half;
    } else {
      u = 2 * i;
      v = 2 * i + 1;
    }
    double c = (double)row[i];
    double s = (double)row[half + i];
    double xu = in[u];
    double xv = in[v];
    double pu_c = xu * c, pv_s = xv * s;
    double pv_c = xv * c, pu_s = xu * s;
    w[u] = pu_c - pv_s;
    w[v] = pv_c + pu_s;
  }
}

static void widen_row(const uint16_t* x, double* w, int32_t D) {
  for (int32_t d = 0; d < D; ++d) w[d] = rkv_ref_half_to_double(x[d]);
}

/* --------------------------------------------------------------- norm -- */

/* The mean of the squares of a head row of fp16 values, computed exactly and
 * rounded once to binary64.  Every fp16 value is an integer multiple of
 * 2^-24 below 2^16, so its square is an integer multiple of 2^-48 below 2^32:
 * the squares are summed exactly as 128-bit integer counts of 2^-48.  A row
 * holding NaN gives NaN, one holding an infinity (and no NaN) infinity. */
double rkv_ref_mean_square(const uint16_t* x, int32_t head_dim) {
  unsigned __int128 acc = 0;
  int has_nan = 0, has_inf = 0;
  for (int32_t d = 0; d < head_dim; ++d) {
    double a = fabs(rkv_ref_half_to_double(x[d]));
    if (isnan(a)) has_nan = 1;
    else if (isinf(a)) has_inf = 1;
    else {
      unsigned long long k = (unsigned long long)(a * 16777216.0);   /* a * 2^24, exact */
      acc += (unsigned __int128)k * k;
    }
  }
  if (has_nan) return NAN;
  if (has_inf) return INFINITY;
  return ldexp((double)acc, -48) / (double)head_dim;   /* one rounding; the rest is exact */
}

/* RMS normalisation of one head row (libmir-cuda execution.rs,
 * DecodeAttentionBf16: the qkv_postprocess step takes query and key norm
 * weights and the model's rms_norm_epsilon before it produces the rotated
 * Q and K; R26): n_d = x_d * r * w_d with r = 1 / sqrt(mean(x^2) + eps), in
 * binary64 (sqrt, the division and the two products rounded once each). */
void rkv_ref_rms_normalize(const uint16_t* x, double* n, const float* weight, int32_t head_dim,
                           double eps) {
  double r = 1.0 / sqrt(rkv_ref_mean_square(x, head_dim) + eps);
  for (int32_t d = 0; d < head_dim; ++d)
    n[d] = (rkv_ref_half_to_double(x[d]) * r) * (double)weight[d];
}

/* The unrounded output of one Q or K head row: RMS-normalised first when a
 * weight is given (R26), then rotated. */
static void head_row_wide(const uint16_t* x, double* w, const float* row, int32_t D, int32_t R,
                          int32_t style, const float* norm_w, double eps) {
  double in[4096];
  if (norm_w)
    rkv_ref_rms_normalize(x, in, norm_w, D, eps);
  else
    widen_row(x, in, D);
  rotate_values(in, w, row, D, R, style);
}

/* The same rounded once to binary16.  A row that is not normalised keeps
 * the input bits of dims >= R (NaN payloads included).  y may equal x. */
static void head_row16(const uint16_t* x, uint16_t* y, const float* row, int32_t D, int32_t R,
                       int32_t style, const float* norm_w, double eps) {
  double w[4096];
  uint16_t tmp[4096];
  head_row_wide(x, w, row, D, R, style, norm_w, eps);
  for (int d = 0; d < D; ++d) tmp[d] = (d < R || norm_w) ? rkv_ref_double_to_half(w[d]) : x[d];
  for (int d = 0; d < D; ++d) y[d] = tmp[d];
}

void rkv_ref_rotate_row_wide(const uint16_t* x, double* w, const float* row, int32_t head_dim,
                             int32_t rotary_dim, int32_t style) {
  head_row_wide(x, w, row, head_dim, rotary_dim, style, NULL, 0.0);
}

void rkv_ref_rotate_row(const uint16_t* x, uint16_t* y, const float* row, int32_t head_dim,
                        int32_t rotary_dim, int32_t style) {
  head_row16(x, y, row, head_dim, rotary_dim, style, NULL, 0.0);
}

/* ----------------------------------------------------------------- fp8 -- */

/* OCP 8-bit E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3
 * mantissa bits; exponent field 0 encodes zero and subnormals (m * 2^-9);
 * no infinities; S.1111.111 is NaN, so the largest finite value is 448. */
double rkv_ref_e4m3_to_double(uint8_t b) {
  int sign = (b >> 7) & 1;
  int e = (b >> 3) & 0xf;
  int m = b & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10);
  return sign ? -v : v;
}

/* binary64 -> E4M3, round to nearest even, saturating: magnitudes that round
 * beyond 448 (and infinities) become 448 (R24); NaN stays NaN. */
uint8_t rkv_ref_double_to_e4m3(double x) {
  uint8_t sign = signbit(x) ? 0x80 : 0;
  if (isnan(x)) return (uint8_t)(sign | 0x7f);
  double a = fabs(x);
  if (a >= 448.0) return (uint8_t)(sign | 0x7e);
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);
  int ue = e2 - 1;             /* 2^ue <= a < 2^(ue+1) */
  if (ue < -6) ue = -6;        /* subnormals share the quantum of the lowest binade */
  double n = ldexp(a, 3 - ue); /* a / quantum, exact */
  double fl = floor(n);
  double rem = n - fl;
  long long k = (long long)fl;
  if (rem > 0.5 || (rem == 0.5 && (k & 1))) k += 1;
  if (k >= 16) {
    k >>= 1;
    ue += 1;
  }
  if (k < 8) return (uint8_t)(sign | (uint8_t)k);                 /* subnormal */
  if (ue + 7 > 15 || (ue + 7 == 15 && k - 8 == 7)) return (uint8_t)(sign | 0x7e);
  return (uint8_t)(sign | (uint8_t)((ue + 7) << 3) | (uint8_t)(k - 8));
}

/* The scale step of the fp8 cache write ([P2] HAVE_K_SCALE / HAVE_V_SCALE):
 * the reciprocal of the per-tensor scale, as an fp32 value. */
static float reciprocal_of(float scale) { return (float)(1.0 / (double)scale); }

/* One fp8 cache row: each value times the reciprocal scale, rounded once to
 * E4M3. */
static void store_row8(uint8_t* dst, const double* w, int32_t D, float rcp) {
  for (int32_t d = 0; d < D; ++d) dst[d] = rkv_ref_double_to_e4m3(w[d] * (double)rcp);
}

/* ------------------------------------------------------------ helpers -- */

static int bad_common(const float* cos_sin, int32_t table_batch, int32_t table_len,
                      int32_t rotary_dim, const uint16_t* qkv, int32_t batch, int32_t seq_len,
                      int32_t hq, int32_t hkv, int32_t head_dim, const void* cache,
                      int32_t capacity, int32_t style) {
  if (!cos_sin || !qkv || !cache) return 1;
  if (batch < 0 || seq_len < 0 || hq < 0 || hkv < 0 || capacity < 0 || table_len < 0) return 1;
  if (head_dim <= 0 || head_dim > 4096) return 1;
  if (rotary_dim < 0 || rotary_dim > head_dim || (rotary_dim & 1)) return 1;
  if (table_batch != 1 && table_batch != batch) return 1;   /* R4 */
  if (style != RKV_REF_NEOX && style != RKV_REF_GPTJ) return 1;
  return 0;
}

static const float* table_row(const float* cos_sin, int32_t table_batch, int32_t table_len,
                              int32_t rotary_dim, int32_t b, int32_t pos) {
  int32_t tb = (table_batch == 1) ? 0 : b;   /* R4 */
  return cos_sin + ((size_t)tb * table_len + pos) * rotary_dim;
}

/* packed [B, S, Hq+Hkv+Hkv, D]: head row (b, s, h) */
static size_t qkv_row(int32_t b, int32_t s, int32_t h, int32_t S, int32_t H, int32_t D) {
  return (((size_t)b * S + s) * H + h) * (size_t)D;
}

/* contiguous cache [B, 2, Hkv, cap, D]: plane 0 holds K, plane 1 holds V */
static size_t cache_row(int32_t b, int32_t plane, int32_t h, int32_t slot, int32_t Hkv,
                        int32_t cap, int32_t D) {
  return ((((size_t)b * 2 + plane) * Hkv + h) * cap + slot) * (size_t)D;
}

/* One token of calls 2 and 3: rotate its Q rows into q_out, its K rows into
 * cache plane 0 at `slot`, copy its V rows into plane 1 at `slot`.  With an
 * fp8 cache (cache8 != NULL) the cache rows are the rotated K / the V values
 * times the reciprocal scales, rounded once to E4M3 (R24).  Q and K rows are
 * RMS-normalised before the rotation when their weight is given (R26). */
static void write_token(const float* row, const uint16_t* qkv, int32_t b, int32_t s,
                        int32_t slot, int32_t S, int32_t hq, int32_t hkv, int32_t D,
                        int32_t R, uint16_t* cache, uint8_t* cache8, float k_rcp, float v_rcp,
                        int32_t cap, uint16_t* q_out, const float* q_w, const float* k_w,
                        double eps, int32_t style) {
  int32_t H = hq + 2 * hkv;
  double w[4096];
  for (int32_t h = 0; h < hq; ++h)
    head_row16(qkv + qkv_row(b, s, h, S, H, D), q_out + (((size_t)b * S + s) * hq + h) * (size_t)D,
               row, D, R, style, q_w, eps);
  for (int32_t h = 0; h < hkv; ++h) {
    const uint16_t* k = qkv + qkv_row(b, s, hq + h, S, H, D);
    if (cache8) {
      head_row_wide(k, w, row, D, R, style, k_w, eps);
      store_row8(cache8 + cache_row(b, 0, h, slot, hkv, cap, D), w, D, k_rcp);
    } else {
      head_row16(k, cache + cache_row(b, 0, h, slot, hkv, cap, D), row, D, R, style, k_w, eps);
    }
  }
  for (int32_t h = 0; h < hkv; ++h) {
    const uint16_t* v = qkv + qkv_row(b, s, hq + hkv + h, S, H, D);
    if (cache8) {
      widen_row(v, w, D);
      store_row8(cache8 + cache_row(b, 1, h, slot, hkv, cap, D), w, D, v_rcp);
    } else {
      memcpy(cache + cache_row(b, 1, h, slot, hkv, cap, D), v, (size_t)D * sizeof(uint16_t));
    }
  }
}

/* ------------------------------------------------------------- call 1 -- */

/* [P1] launchApplyRopeWriteKVPackedQKV: the cache is empty, so token s of
 * every sequence takes position s and cache slot s.  Q and K heads of the
 * packed tensor are rotated in place (R7); K also goes to cache plane 0 and
 * V, unrotated, to plane 1.  Slots >= S are not touched. */
static int packed_core(const float* cos_sin, int32_t table_batch, int32_t table_len,
                       int32_t rotary_dim, uint16_t* qkv, int32_t batch, int32_t seq_len,
                       int32_t hq, int32_t hkv, int32_t head_dim, uint16_t* cache,
                       uint8_t* cache8, float k_rcp, float v_rcp, int32_t capacity,
                       const float* q_w, const float* k_w, double eps, int32_t style) {
  if (bad_common(cos_sin, table_batch, table_len, rotary_dim, qkv, batch, seq_len, hq, hkv,
                 head_dim, cache ? (const void*)cache : (const void*)cache8, capacity, style))
    return RKV_REF_ERR_ARG;
  if (seq_len > capacity || seq_len > table_len) return RKV_REF_ERR_CAPACITY;
  int32_t H = hq + 2 * hkv, D = head_dim, R = rotary_dim;
  double w[4096];
  for (int32_t b = 0; b < batch; ++b) {
    for (int32_t s = 0; s < seq_len; ++s) {
      int32_t pos = s;
      const float* row = table_row(cos_sin, table_batch, table_len, R, b, pos);
      for (int32_t h = 0; h < hq; ++h) {
        uint16_t* x = qkv + qkv_row(b, s, h, seq_len, H, D);
        head_row16(x, x, row, D, R, style, q_w, eps);
      }
      for (int32_t h = 0; h < hkv; ++h) {
        uint16_t* x = qkv + qkv_row(b, s, hq + h, seq_len, H, D);
        if (cache8) {   /* the cache gets the unrounded rotation, scaled (R24) */
          head_row_wide(x, w, row, D, R, style, k_w, eps);
          store_row8(cache8 + cache_row(b, 0, h, pos, hkv, capacity, D), w, D, k_rcp);
        }
        head_row16(x, x, row, D, R, style, k_w, eps);
        if (!cache8)
          memcpy(cache + cache_row(b, 0, h, pos, hkv, capacity, D), x,
                 (size_t)D * sizeof(uint16_t));
      }
      for (int32_t h = 0; h < hkv; ++h) {
        const uint16_t* v = qkv + qkv_row(b, s, hq + hkv + h, seq_len, H, D);
        if (cache8) {
          widen_row(v, w, D);
          store_row8(cache8 + cache_row(b, 1, h, pos, hkv, capacity, D), w, D, v_rcp);
        } else {
          memcpy(cache + cache_row(b, 1, h, pos, hkv, capacity, D), v,
                 (size_t)D * sizeof(uint16_t));
        }
      }
    }
  }
  return RKV_REF_OK;
}

int rkv_ref_packed_qkv(const float* cos_sin, int32_t table_batch, int32_t table_len,
                       int32_t rotary_dim, uint16_t* qkv, int32_t batch, int32_t seq_len,
                       int32_t hq, int32_t hkv, int32_t head_dim, uint16_t* cache,
                       int32_t capacity, int32_t style) {
  if (!cache) return RKV_REF_ERR_ARG;
  return packed_core(cos_sin, table_batch, table_len, rotary_dim, qkv, batch, seq_len, hq, hkv,
                     head_dim, cache, NULL, 1.0f, 1.0f, capacity, NULL, NULL, 0.0, style);
}

int rkv_ref_packed_qkv_fp8(const float* cos_sin, int32_t table_batch, int32_t table_len,
                           int32_t rotary_dim, uint16_t* qkv, int32_t batch, int32_t seq_len,
                           int32_t hq, int32_t hkv, int32_t head_dim, uint8_t* cache8,
                           int32_t capacity, float k_scale, float v_scale, int32_t style) {
  if (!cache8) return RKV_REF_ERR_ARG;
  return packed_core(cos_sin, table_batch, table_len, rotary_dim, qkv, batch, seq_len, hq, hkv,
                     head_dim, NULL, cache8, reciprocal_of(k_scale), reciprocal_of(v_scale),
                     capacity, NULL, NULL, 0.0, style);
}

/* ------------------------------------------------------------- call 2 -- */

/* [P1] launchApplyRopeWriteKVContinuousQAndKVCache: end_lens[b] is the cache
 * length after the write (R5, and [P4]: the newest token sits at length-1),
 * so token s takes position and slot end-S+s.  Rotated Q goes to q_out, the
 * packed tensor is only read.  Out-of-range tokens write nothing (R10). */
static int continuous_core(const float* cos_sin, int32_t table_batch, int32_t table_len,
                           int32_t rotary_dim, const int32_t* end_lens, const uint16_t* qkv,
                           int32_t batch, int32_t seq_len, int32_t hq, int32_t hkv,
                           int32_t head_dim, uint16_t* cache, uint8_t* cache8, float k_rcp,
                           float v_rcp, int32_t capacity, uint16_t* q_out, const float* q_w,
                           const float* k_w, double eps, int32_t style) {
  if (bad_common(cos_sin, table_batch, table_len, rotary_dim, qkv, batch, seq_len, hq, hkv,
                 head_dim, cache ? (const void*)cache : (const void*)cache8, capacity, style) ||
      !end_lens || !q_out)
    return RKV_REF_ERR_ARG;
  for (int32_t b = 0; b < batch; ++b) {
    for (int32_t s = 0; s < seq_len; ++s) {
      int64_t slot = (int64_t)end_lens[b] - seq_len + s;
      int64_t pos = slot;
      if (slot < 0 || slot >= capacity || pos >= table_len) continue;
      const float* row = table_row(cos_sin, table_batch, table_len, rotary_dim, b, (int32_t)pos);
      write_token(row, qkv, b, s, (int32_t)slot, seq_len, hq, hkv, head_dim, rotary_dim, cache,
                  cache8, k_rcp, v_rcp, capacity, q_out, q_w, k_w, eps, style);
    }
  }
  return RKV_REF_OK;
}

int rkv_ref_continuous(const float* cos_sin, int32_t table_batch, int32_t table_len,
                       int32_t rotary_dim, const int32_t* end_lens, const uint16_t* qkv,
                       int32_t batch, int32_t seq_len, int32_t hq, int32_t hkv,
                       int32_t head_dim, uint16_t* cache, int32_t capacity, uint16_t* q_out,
                       int32_t style) {
  if (!cache) return RKV_REF_ERR_ARG;
  return continuous_core(cos_sin, table_batch, table_len, rotary_dim, end_lens, qkv, batch,
                         seq_len, hq, hkv, head_dim, cache, NULL, 1.0f, 1.0f, capacity, q_out,
                         NULL, NULL, 0.0, style);
}

int rkv_ref_continuous_fp8(const float* cos_sin, int32_t table_batch, int32_t table_len,
                           int32_t rotary_dim, const int32_t* end_lens, const uint16_t* qkv,
                           int32_t batch, int32_t seq_len, int32_t hq, int32_t hkv,
                           int32_t head_dim, uint8_t* cache8, int32_t capacity,
                           uint16_t* q_out, float k_scale, float v_scale, int32_t style) {
  if (!cache8) return RKV_REF_ERR_ARG;
  return continuous_core(cos_sin, table_batch, table_len, rotary_dim, end_lens, qkv, batch,
                         seq_len, hq, hkv, head_dim, NULL, cache8, reciprocal_of(k_scale),
                         reciprocal_of(v_scale), capacity, q_out, NULL, NULL, 0.0, style);
}

/* ------------------------------------------------------------- call 3 -- */

/* [P1] launchApplyRopeWriteKVTreeDecoding: as call 2, but the rotary
 * position of token s is tokenPosIds[b, s]; the cache slot stays end-S+s,
 * since tree siblings share a position (R6). */
static int tree_core(const float* cos_sin, int32_t table_batch, int32_t table_len,
                     int32_t rotary_dim, const int32_t* end_lens, const int32_t* pos_ids,
                     const uint16_t* qkv, int32_t batch, int32_t seq_len, int32_t hq,
                     int32_t hkv, int32_t head_dim, uint16_t* cache, uint8_t* cache8,
                     float k_rcp, float v_rcp, int32_t capacity, uint16_t* q_out,
                     const float* q_w, const float* k_w, double eps, int32_t style) {
  if (bad_common(cos_sin, table_batch, table_len, rotary_dim, qkv, batch, seq_len, hq, hkv,
                 head_dim, cache ? (const void*)cache : (const void*)cache8, capacity, style) ||
      !end_lens || !pos_ids || !q_out)
    return RKV_REF_ERR_ARG;
  for (int32_t b = 0; b < batch; ++b) {
    for (int32_t s = 0; s < seq_len; ++s) {
      int64_t slot = (int64_t)end_lens[b] - seq_len + s;
      int64_t pos = pos_ids[(size_t)b * seq_len + s];
      if (slot < 0 || slot >= capacity || pos < 0 || pos >= table_len) continue;
      const float* row = table_row(cos_sin, table_batch, table_len, rotary_dim, b, (int32_t)pos);
      write_token(row, qkv, b, s, (int32_t)slot, seq_len, hq, hkv, head_dim, rotary_dim, cache,
                  cache8, k_rcp, v_rcp, capacity, q_out, q_w, k_w, eps, style);
    }
  }
  return RKV_REF_OK;
}

int rkv_ref_tree(const float* cos_sin, int32_t table_batch, int32_t table_len,
                 int32_t rotary_dim, const int32_t* end_lens, const int32_t* pos_ids,
                 const uint16_t* qkv, int32_t batch, int32_t seq_len, int32_t hq, int32_t hkv,
                 int32_t head_dim, uint16_t* cache, int32_t capacity, uint16_t* q_out,
                 int32_t style) {
  if (!cache) return RKV_REF_ERR_ARG;
  return tree_core(cos_sin, table_batch, table_len, rotary_dim, end_lens, pos_ids, qkv, batch,
                   seq_len, hq, hkv, head_dim, cache, NULL, 1.0f, 1.0f, capacity, q_out, NULL,
                   NULL, 0.0, style);
}

int rkv_ref_tree_fp8(const float* cos_sin, int32_t table_batch, int32_t table_len,
                     int32_t rotary_dim, const int32_t* end_lens, const int32_t* pos_ids,
                     const uint16_t* qkv, int32_t batch, int32_t seq_len, int32_t hq,
                     int32_t hkv, int32_t head_dim, uint8_t* cache8, int32_t capacity,
                     uint16_t* q_out, float k_scale, float v_scale, int32_t style) {
  if (!cache8) return RKV_REF_ERR_ARG;
  return tree_core(cos_sin, table_batch, table_len, rotary_dim, end_lens, pos_ids, qkv, batch,
                   seq_len, hq, hkv, head_dim, NULL, cache8, reciprocal_of(k_scale),
                   reciprocal_of(v_scale), capacity, q_out, NULL, NULL, 0.0, style);
}

/* ------------------------------------------ calls 1-3 with Q/K RMS norm -- */

/* Calls 1-3 with Q and K heads RMS-normalised before the rotation (R26):
 * q_w / k_w are the per-dimension weights [D] of the Q and K heads, either
 * may be NULL (those heads are not normalised); eps must be finite and
 * >= 0.  Exactly one of cache (fp16) and cache8 (E4M3, with the scales) is
 * given. */
static int norm_args_bad(const uint16_t* cache, const uint8_t* cache8, double eps) {
  return (!cache == !cache8) || !isfinite(eps) || eps < 0.0;
}

int rkv_ref_packed_qkv_qknorm(const float* cos_sin, int32_t table_batch, int32_t table_len,
                              int32_t rotary_dim, uint16_t* qkv, int32_t batch, int32_t seq_len,
                              int32_t hq, int32_t hkv, int32_t head_dim, uint16_t* cache,
                              uint8_t* cache8, int32_t capacity, const float* q_weight,
                              const float* k_weight, double eps, float k_scale, float v_scale,
                              int32_t style) {
  if (norm_args_bad(cache, cache8, eps)) return RKV_REF_ERR_ARG;
  return packed_core(cos_sin, table_batch, table_len, rotary_dim, qkv, batch, seq_len, hq, hkv,
                     head_dim, cache, cache8, reciprocal_of(k_scale), reciprocal_of(v_scale),
                     capacity, q_weight, k_weight, eps, style);
}

int rkv_ref_continuous_qknorm(const float* cos_sin, int32_t table_batch, int32_t table_len,
                              int32_t rotary_dim, const int32_t* end_lens, const uint16_t* qkv,
                              int32_t batch, int32_t seq_len, int32_t hq, int32_t hkv,
                              int32_t head_dim, uint16_t* cache, uint8_t* cache8,
                              int32_t capacity, uint16_t* q_out, const float* q_weight,
                              const float* k_weight, double eps, float k_scale, float v_scale,
                              int32_t style) {
  if (norm_args_bad(cache, cache8, eps)) return RKV_REF_ERR_ARG;
  return continuous_core(cos_sin, table_batch, table_len, rotary_dim, end_lens, qkv, batch,
                         seq_len, hq, hkv, head_dim, cache, cache8, reciprocal_of(k_scale),
                         reciprocal_of(v_scale), capacity, q_out, q_weight, k_weight, eps, style);
}

int rkv_ref_tree_qknorm(const float* cos_sin, int32_t table_batch, int32_t table_len,
                        int32_t rotary_dim, const int32_t* end_lens, const int32_t* pos_ids,
                        const uint16_t* qkv, int32_t batch, int32_t seq_len, int32_t hq,
                        int32_t hkv, int32_t head_dim, uint16_t* cache, uint8_t* cache8,
                        int32_t capacity, uint16_t* q_out, const float* q_weight,
                        const float* k_weight, double eps, float k_scale, float v_scale,
                        int32_t style) {
  if (norm_args_bad(cache, cache8, eps)) return RKV_REF_ERR_ARG;
  return tree_core(cos_sin, table_batch, table_len, rotary_dim, end_lens, pos_ids, qkv, batch,
                   seq_len, hq, hkv, head_dim, cache, cache8, reciprocal_of(k_scale),
                   reciprocal_of(v_scale), capacity, q_out, q_weight, k_weight, eps, style);
}

/* ------------------------------------------------------------- call 4 -- */

/* [P3] launchDFlashTargetKVCacheUpdate.  Delta row i belongs to sequence
 * delta_to_seq[i] at absolute position delta_positions[i]; either negative
 * marks padding (R11), a sequence >= batch is inactive (R12), and a position
 * beyond max_pages_per_seq pages is skipped.  The position's logical page
 * p/64 is looked up per plane in page_table[seq, plane, :]; the ids are
 * canonical, so the pool reads as [2*numPages][64][Hkv][D] and the K (V)
 * plane writes only ids in its own range (R13).  K is rotated with the
 * row's cos/sin row; V is copied bit for bit.
 *
 * The cos/sin row of delta row i is either row i of token_cos_sin (the
 * page's tokenAlignedCosSin) or, when token_cos_sin is NULL, the rope-table
 * row of rope_row_of (the fused gather below); a row without one writes no
 * K. */
static const float* rope_row_of(const float* rope, int32_t rope_states, int32_t rope_rows,
                                const int32_t* state_indices, int64_t p, int64_t q,
                                int32_t batch, int32_t rotary_dim);

static int paged_update(const uint16_t* k_delta, const uint16_t* v_delta, uint16_t* pool,
                        uint8_t* pool8, float k_rcp, float v_rcp, const float* token_cos_sin, const float* rope, int32_t rope_states,
                        int32_t rope_rows, const int32_t* state_indices,
                        const int32_t* delta_positions, const int32_t* delta_to_seq,
                        const int32_t* page_table, int32_t num_delta, int32_t batch, int32_t hkv,
                        int32_t head_dim, int32_t rotary_dim, int32_t num_pages,
                        int32_t max_pages_per_seq, int32_t style) {
  if (!k_delta || !v_delta || (!pool && !pool8) || (!token_cos_sin && !rope) || !delta_positions ||
      !delta_to_seq || !page_table)
    return RKV_REF_ERR_ARG;
  if (num_delta < 0 || batch < 0 || hkv < 0 || num_pages < 0 || max_pages_per_seq < 0 ||
      rope_states < 0 || rope_rows < 0)
    return RKV_REF_ERR_ARG;
  if (head_dim <= 0 || head_dim > 4096 || rotary_dim < 0 || rotary_dim > head_dim ||
      (rotary_dim & 1))
    return RKV_REF_ERR_ARG;
  if (style != RKV_REF_NEOX && style != RKV_REF_GPTJ) return RKV_REF_ERR_ARG;
  const int64_t TPP = RKV_REF_TOKENS_PER_PAGE;
  int32_t D = head_dim;
  double w[4096];
  for (int32_t i = 0; i < num_delta; ++i) {
    int64_t p = delta_positions[i];
    int64_t q = delta_to_seq[i];
    if (p < 0 || q < 0) continue;                       /* padding */
    if (q >= batch) continue;                           /* inactive sequence */
    if (p >= (int64_t)max_pages_per_seq * TPP) continue; /* beyond capacity */
    int64_t lp = p / TPP, off = p % TPP;
    int64_t kid = page_table[((size_t)q * 2 + 0) * max_pages_per_seq + lp];
    int64_t vid = page_table[((size_t)q * 2 + 1) * max_pages_per_seq + lp];
    const float* row = token_cos_sin ? token_cos_sin + (size_t)i * rotary_dim
                                     : rope_row_of(rope, rope_states, rope_rows, state_indices,
                                                   p, q, batch, rotary_dim);
    if (row && kid >= 0 && kid < num_pages) {
      for (int32_t h = 0; h < hkv; ++h) {
        const uint16_t* k = k_delta + ((size_t)i * hkv + h) * D;
        size_t dst = (((size_t)kid * TPP + off) * hkv + h) * D;
        if (pool8) {
          rkv_ref_rotate_row_wide(k, w, row, D, rotary_dim, style);
          store_row8(pool8 + dst, w, D, k_rcp);
        } else {
          rkv_ref_rotate_row(k, pool + dst, row, D, rotary_dim, style);
        }
      }
    }
    if (vid >= num_pages && vid < 2 * (int64_t)num_pages) {
      for (int32_t h = 0; h < hkv; ++h) {
        const uint16_t* v = v_delta + ((size_t)i * hkv + h) * D;
        size_t dst = (((size_t)vid * TPP + off) * hkv + h) * D;
        if (pool8) {
          widen_row(v, w, D);
          store_row8(pool8 + dst, w, D, v_rcp);
        } else {
          memcpy(pool + dst, v, (size_t)D * sizeof(uint16_t));
        }
      }
    }
  }
  return RKV_REF_OK;
}

int rkv_ref_paged_delta(const uint16_t* k_delta, const uint16_t* v_delta, uint16_t* pool,
                        const float* token_cos_sin, const int32_t* delta_positions,
                        const int32_t* delta_to_seq, const int32_t* page_table,
                        int32_t num_delta, int32_t batch, int32_t hkv, int32_t head_dim,
                        int32_t rotary_dim, int32_t num_pages, int32_t max_pages_per_seq,
                        int32_t style) {
  if (!token_cos_sin || !pool) return RKV_REF_ERR_ARG;
  return paged_update(k_delta, v_delta, pool, NULL, 1.0f, 1.0f, token_cos_sin, NULL, 0, 0, NULL,
                      delta_positions, delta_to_seq, page_table, num_delta, batch, hkv,
                      head_dim, rotary_dim, num_pages, max_pages_per_seq, style);
}

int rkv_ref_paged_delta_fp8(const uint16_t* k_delta, const uint16_t* v_delta, uint8_t* pool8,
                            const float* token_cos_sin, const int32_t* delta_positions,
                            const int32_t* delta_to_seq, const int32_t* page_table,
                            int32_t num_delta, int32_t batch, int32_t hkv, int32_t head_dim,
                            int32_t rotary_dim, int32_t num_pages, int32_t max_pages_per_seq,
                            float k_scale, float v_scale, int32_t style) {
  if (!token_cos_sin || !pool8) return RKV_REF_ERR_ARG;
  return paged_update(k_delta, v_delta, NULL, pool8, reciprocal_of(k_scale),
                      reciprocal_of(v_scale), token_cos_sin, NULL, 0, 0, NULL, delta_positions,
                      delta_to_seq, page_table, num_delta, batch, hkv, head_dim, rotary_dim,
                      num_pages, max_pages_per_seq, style);
}

/* ------------------------------------------------- call 4, gather fused -- */

/* [P3] launchDFlashGatherDeltaRope builds tokenAlignedCosSin from a rope
 * table (the page gives its parameters only).  Reading: the table is
 * [rope_states, rope_rows, R]; sequence q uses state state_indices[q], or q
 * itself when no state indices are given (state 0 when the table has a
 * single state).  Row i gets table[state(q_i)][p_i] when p_i and q_i are
 * not padding, q_i < batch, the state exists and p_i < rope_rows;
 * otherwise it gets NaN (no row). */
static const float* rope_row_of(const float* rope, int32_t rope_states, int32_t rope_rows,
                                const int32_t* state_indices, int64_t p, int64_t q,
                                int32_t batch, int32_t rotary_dim) {
  if (p < 0 || q < 0 || q >= batch) return NULL;
  int64_t st = state_indices ? state_indices[q] : (rope_states == 1 ? 0 : q);
  if (st < 0 || st >= rope_states || p >= rope_rows) return NULL;
  return rope + ((size_t)st * rope_rows + p) * rotary_dim;
}

int rkv_ref_gather_delta_rope(const float* rope, int32_t rope_states, int32_t rope_rows,
                              const int32_t* state_indices, const int32_t* delta_positions,
                              const int32_t* delta_to_seq, int32_t num_delta, int32_t batch,
                              int32_t rotary_dim, float* out) {
  if (!rope || !delta_positions || !delta_to_seq || !out) return RKV_REF_ERR_ARG;
  if (rope_states < 0 || rope_rows < 0 || num_delta < 0 || batch < 0 || rotary_dim < 0)
    return RKV_REF_ERR_ARG;
  for (int32_t i = 0; i < num_delta; ++i) {
    const float* row = rope_row_of(rope, rope_states, rope_rows, state_indices,
                                   delta_positions[i], delta_to_seq[i], batch, rotary_dim);
    for (int32_t d = 0; d < rotary_dim; ++d)
      out[(size_t)i * rotary_dim + d] = row ? row[d] : NAN;
  }
  return RKV_REF_OK;
}

/* The update of call 4 with each row's cos/sin row taken from the rope
 * table as the gather above would; a row without one writes no K. */
int rkv_ref_paged_delta_gather(const uint16_t* k_delta, const uint16_t* v_delta, uint16_t* pool,
                               const float* rope, int32_t rope_states, int32_t rope_rows,
                               const int32_t* state_indices, const int32_t* delta_positions,
                               const int32_t* delta_to_seq, const int32_t* page_table,
                               int32_t num_delta, int32_t batch, int32_t hkv, int32_t head_dim,
                               int32_t rotary_dim, int32_t num_pages, int32_t max_pages_per_seq,
                               int32_t style) {
  if (!rope || !pool) return RKV_REF_ERR_ARG;
  return paged_update(k_delta, v_delta, pool, NULL, 1.0f, 1.0f, NULL, rope, rope_states,
                      rope_rows, state_indices, delta_positions, delta_to_seq, page_table,
                      num_delta, batch, hkv, head_dim, rotary_dim, num_pages, max_pages_per_seq,
                      style);
}

int rkv_ref_paged_delta_gather_fp8(const uint16_t* k_delta, const uint16_t* v_delta,
                                   uint8_t* pool8, const float* rope, int32_t rope_states,
                                   int32_t rope_rows, const int32_t* state_indices,
                                   const int32_t* delta_positions, const int32_t* delta_to_seq,
                                   const int32_t* page_table, int32_t num_delta, int32_t batch,
                                   int32_t hkv, int32_t head_dim, int32_t rotary_dim,
                                   int32_t num_pages, int32_t max_pages_per_seq, float k_scale,
                                   float v_scale, int32_t style) {
  if (!rope || !pool8) return RKV_REF_ERR_ARG;
  return paged_update(k_delta, v_delta, NULL, pool8, reciprocal_of(k_scale),
                      reciprocal_of(v_scale), NULL, rope, rope_states, rope_rows, state_indices,
                      delta_positions, delta_to_seq, page_table, num_delta, batch, hkv,
                      head_dim, rotary_dim, num_pages, max_pages_per_seq, style);
}

/* --------------------------------------------------- metadata builders -- */

/* [P3] launchDFlashPrepareDeltaMetadata (signature only; R28): the delta
 * rows are token-major, deltaWidth rows per sequence.  Row b*width + j is
 * token j of sequence b's delta when j < min(deltaLengths[b], width): its
 * position continues the old draft cache, oldDraftCacheLengths[b] + j (the
 * page's proposal-input kernel puts the delta right after the old length),
 * its owner is b.  Every other row is padding: -1 in both arrays.  A
 * position beyond the int32 range is written as padding too. */
int rkv_ref_prepare_delta_metadata(const int32_t* old_lengths, const int32_t* delta_lengths,
                                   int32_t delta_width, int32_t* delta_positions,
                                   int32_t* delta_to_seq, int32_t batch) {
  if (!old_lengths || !delta_lengths || !delta_positions || !delta_to_seq) return RKV_REF_ERR_ARG;
  if (batch < 0 || delta_width < 0) return RKV_REF_ERR_ARG;
  for (int32_t b = 0; b < batch; ++b) {
    int64_t len = delta_lengths[b];
    for (int32_t j = 0; j < delta_width; ++j) {
      size_t i = (size_t)b * delta_width + j;
      int64_t pos = (int64_t)old_lengths[b] + j;
      if (j < len && pos <= INT32_MAX) {
        delta_positions[i] = (int32_t)pos;
        delta_to_seq[i] = b;
      } else {
        delta_positions[i] = -1;
        delta_to_seq[i] = -1;
      }
    }
  }
  return RKV_REF_OK;
}

/* [P3] launchDFlashBuildLinearTreeMetadata: a linear verification path of
 * verifySize nodes per sequence; node 0 is the root (parent -1, depth 0),
 * node i > 0 has parent i - 1 and depth i. */
int rkv_ref_linear_tree_metadata(int32_t* parent_ids, int32_t* depths, int32_t batch,
                                 int32_t verify_size) {
  if (!parent_ids || !depths || batch < 0 || verify_size < 0) return RKV_REF_ERR_ARG;
  for (int32_t b = 0; b < batch; ++b)
    for (int32_t i = 0; i < verify_size; ++i) {
      parent_ids[(size_t)b * verify_size + i] = i - 1;
      depths[(size_t)b * verify_size + i] = i;
    }
  return RKV_REF_OK;
}

/* [P3] checkDFlashRopeCapacity: the table may be shorter than the padded
 * capacity; only a table longer than the capacity is rejected (R17). */
int rkv_ref_check_rope_capacity(int32_t cos_sin_len, int32_t kv_capacity) {
  return cos_sin_len > kv_capacity ? RKV_REF_ERR_CAPACITY : RKV_REF_OK;
}
