// Internal interface between the C ABI (rkv_abi.hip) and the kernels
// (rkv_kernels.hip): validated parameter blocks and launch entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkv {

enum Call : int { kCallPacked = 0, kCallContinuous = 1, kCallTree = 2 };

constexpr int kTokensPerPage = 64;
// Row sets a wave keeps in flight at once (two 16-byte loads per lane each).
constexpr int kContigUnroll = 4;
constexpr int kPagedUnroll = 2;

struct ContigParams {
  const float* cos_sin;     // [table_batch, table_len, R]
  uint16_t* qkv;            // [B, S, Hq + 2*Hkv, D]; written only by call 1
  uint16_t* cache;          // [B, 2, Hkv, cap, D]
  uint16_t* q_out;          // [B, S, Hq, D]; calls 2 and 3
  const int32_t* end_lens;  // [B]; calls 2 and 3
  const int32_t* pos_ids;   // [B, S]; call 3
  int32_t B, S, Hq, Hkv, cap;
  int32_t table_batch, table_len, R;
  int32_t row_sets;         // ceil((Hq + 2*Hkv) / rows per set)
  int32_t waves_per_token;  // waves sharing one token's row sets
  int32_t total_waves;      // B * S * waves_per_token
};

struct PagedParams {
  const uint16_t* k_delta;  // [N, Hkv, D]
  const uint16_t* v_delta;  // [N, Hkv, D]
  uint16_t* pool;           // [2 * num_pages, 64, Hkv, D]
  const float* cos_sin;     // [N, R]
  const int32_t* positions; // [N]
  const int32_t* seq;       // [N]
  const int32_t* page_table;// [batch, 2, max_pages]
  int32_t N, batch, Hkv, R, num_pages, max_pages;
  int32_t row_sets;         // ceil(2*Hkv / rows per set)
  int32_t waves_per_row;    // waves sharing one delta row
  int32_t total_waves;      // N * waves_per_row
};

hipError_t launch_contig(const ContigParams& p, int call, int D, int style, hipStream_t stream);
hipError_t launch_paged(const PagedParams& p, int D, int style, hipStream_t stream);

}  // namespace rkv
