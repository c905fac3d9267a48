// Internal interface between the C ABI (rkv_abi.hip) and the kernels
// (rkv_kernels.hip): validated parameter blocks and launch entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkv {

enum Call : int { kCallPacked = 0, kCallContinuous = 1, kCallTree = 2 };

constexpr int kTokensPerPage = 64;

// Workgroup shape of the rope kernels: 256 threads, 4 waves of 64 lanes.
constexpr int kBlockThreads = 256;
constexpr int kWaveLanes = 64;
// A dispatch covers at most 2^32 - 1 work-items, which bounds the waves of
// one launch.
constexpr long long kMaxWavesPerLaunch =
    (0xFFFFFFFFLL / kBlockThreads) * (kBlockThreads / kWaveLanes);

// Division by a launch constant d >= 1 for numerators n < 2^31, by
// multiply-high and shift (Granlund & Montgomery, "Division by invariant
// integers using multiplication", PLDI 1994, round-up method):
// l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(m, n) + n) >> l.
struct FastDiv {
  uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, l};
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv& f) {
  return (__umulhi(f.m, n) + n) >> f.l;
}

struct ContigParams {
  const float* cos_sin;     // [table_batch, table_len, R]
  uint16_t* qkv;            // [B, S, Hq + 2*Hkv, D]; written only by call 1
  uint16_t* cache;          // [B, 2, Hkv, cap, D] fp16 cache, or
  uint8_t* cache8;          // [B, 2, Hkv, cap, D] E4M3 cache (fp8 kernels)
  const float* k_scale;     // fp8: per-tensor scales (one fp32 each) or null for 1
  const float* v_scale;
  const float* q_norm_w;    // Q/K norm: per-dimension weights [D] of Q and K heads,
  const float* k_norm_w;    //   or null (those heads are not normalised)
  float eps;                // Q/K norm: added to the mean square
  uint16_t* q_out;          // [B, S, Hq, D]; calls 2 and 3
  const int32_t* end_lens;  // [B]; calls 2 and 3
  const int32_t* pos_ids;   // [B, S]; call 3
  int32_t B, S, Hq, Hkv, cap;
  int32_t table_batch, table_len, R;
  uint32_t cache_b_bytes;   // bytes of one batch's cache slice (2 * Hkv * cap * D
                            //   elements), or 0 when it reaches 2^32
  int32_t xcd_chunk_log2;   // workgroup numbering: 0 contiguous eighths per XCD,
                            //   else chunks of 2^xcd_chunk_log2 taken in turn
  int32_t groups_per_wave;  // G: row groups of 512/D rows handled by one wave (1, 2 or 4)
  int32_t waves_per_token;  // ceil(row groups per token / G)
  int32_t total_waves;      // B * S * waves_per_token
  FastDiv div_waves;        // by waves_per_token
  FastDiv div_seq;          // by S
};

struct PagedParams {
  const uint16_t* k_delta;  // [N, Hkv, D]
  const uint16_t* v_delta;  // [N, Hkv, D]
  uint16_t* pool;           // [2 * num_pages, 64, Hkv, D] fp16 pool, or
  uint8_t* pool8;           // [2 * num_pages, 64, Hkv, D] E4M3 pool (fp8 kernels)
  const float* k_scale;     // fp8: per-tensor scales (one fp32 each) or null for 1
  const float* v_scale;
  const float* cos_sin;     // [N, R]
  const int32_t* positions; // [N]
  const int32_t* seq;       // [N]
  const int32_t* page_table;// [batch, 2, max_pages]
  const float* rope;        // fused gather: [rope_states, rope_rows, R]; else unused
  const int32_t* state_idx; // fused gather: [batch] state of each sequence, or null
  int32_t rope_states, rope_rows;
  int32_t N, batch, Hkv, R, num_pages, max_pages;
  int32_t groups_per_wave;  // G: row groups of 512/D rows handled by one wave (1, 2 or 4)
  int32_t waves_per_row;    // ceil(row groups per delta row / G)
  int32_t total_waves;      // N * waves_per_row
  FastDiv div_waves;        // by waves_per_row
};

hipError_t launch_contig(const ContigParams& p, int call, int D, int style, bool exact,
                         hipStream_t stream);
// late_loads: a delta row is loaded once its page ids are known, and only if
// it is written; otherwise every row is requested with the index loads.
hipError_t launch_paged(const PagedParams& p, int D, int style, bool exact, bool gather,
                        bool late_loads, hipStream_t stream);
hipError_t launch_contig_fp8(const ContigParams& p, int call, int D, int style, bool exact,
                             hipStream_t stream);
hipError_t launch_contig_norm(const ContigParams& p, int call, int D, int style, bool exact,
                              hipStream_t stream);
hipError_t launch_contig_norm_fp8(const ContigParams& p, int call, int D, int style, bool exact,
                                  hipStream_t stream);
hipError_t launch_paged_fp8(const PagedParams& p, int D, int style, bool exact, bool gather,
                            bool late_loads, hipStream_t stream);

// Index builders (rkv_meta.hip): rows = batch * width > 0, nodes = batch *
// verify > 0, all pointers valid device arrays of that many int32.
hipError_t launch_delta_metadata(const int32_t* old_lengths, const int32_t* delta_lengths,
                                 int32_t width, int32_t* positions, int32_t* owners,
                                 int32_t rows, hipStream_t stream);
hipError_t launch_linear_tree(int32_t* parents, int32_t* depths, int32_t verify, int32_t nodes,
                              hipStream_t stream);

}  // namespace rkv
