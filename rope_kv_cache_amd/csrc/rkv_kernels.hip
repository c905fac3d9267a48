// HIP kernels for gfx950: fused RoPE + KV-cache write.
//
// Work decomposition.  The unit is a (token, head) row of D fp16 values.  A
// wavefront (64 lanes) owns one token -- or, for small problems, a slice of
// a token's rows -- and sweeps its rows in "row sets": D/16 lanes per row,
// 16 bytes per lane per access, so one row set is 64/(D/16) rows and every
// load or store instruction of the wave moves whole 128-byte lines.  Each
// lane owns two 16-byte chunks of its row, the second R/2 elements after the
// first, so NeoX partners meet in one lane and GPT-J partners in one dword:
// no cross-lane exchange is needed.  The token's cos/sin values are fetched
// once per wave into registers and reused for every Q and K row it sweeps.
// There is no contraction anywhere: the path is bandwidth-bound, so there is
// no MFMA and no LDS staging.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rkv_launch.hpp"
#include "rkv_rotate.hpp"

namespace rkv {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ void st16(uint16_t* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

__device__ __forceinline__ int wave_id_uniform() {
  return __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)));
}

// ------------------------------------------------------------ calls 1-3 --
//
// Call 1 (packed prefill): position = slot = s; Q and K rotated in place in
//   qkv, K also to cache plane 0, V copied to plane 1.
// Call 2 (continuous): position = slot = endLens[b] - S + s; Q to qOut.
// Call 3 (tree): slot = endLens[b] - S + s, position = tokenPosIds[b, s].
// Calls 2 and 3 skip a token whose slot or position is out of range.
// (TensorRT-Edge-LLM C++ API, "Apply Rope Write KV".)
template <int D, int kCall, int kStyle, bool kExact, int kUnroll>
__global__ __launch_bounds__(kBlock) void contig_kernel(ContigParams p) {
  constexpr int kLanesPerRow = D / 16;
  constexpr int kRowsPerSet = kWave / kLanesPerRow;

  const int wave = wave_id_uniform();
  if (wave >= p.total_waves) return;
  const int token = wave / p.waves_per_token;
  const int part = wave - token * p.waves_per_token;
  const int b = token / p.S;
  const int s = token - b * p.S;

  int slot, pos;
  if constexpr (kCall == kCallPacked) {
    slot = s;
    pos = s;
  } else {
    const long long slot64 = (long long)p.end_lens[b] - p.S + s;
    const long long pos64 = (kCall == kCallTree) ? (long long)p.pos_ids[token] : slot64;
    if (slot64 < 0 || slot64 >= p.cap || pos64 < 0 || pos64 >= p.table_len) return;
    slot = (int)slot64;
    pos = (int)pos64;
  }

  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane / kLanesPerRow;
  const int j = lane - g * kLanesPerRow;
  const LaneChunks lc = lane_chunks<D>(j, p.R);

  float cs[8], sn[8];
  if (lc.rotary) {
    const int tb = (p.table_batch == 1) ? 0 : b;
    const float* row = p.cos_sin + ((size_t)tb * p.table_len + pos) * p.R;
    load_cos_sin<kStyle>(row, j, p.R, cs, sn);
  }

  const int H = p.Hq + 2 * p.Hkv;
  const int rs_begin = (int)(((long long)part * p.row_sets) / p.waves_per_token);
  const int rs_end = (int)(((long long)(part + 1) * p.row_sets) / p.waves_per_token);
  uint16_t* const tok_base = p.qkv + (size_t)token * H * D;

  for (int rs0 = rs_begin; rs0 < rs_end; rs0 += kUnroll) {
    uint4 A[kUnroll], B[kUnroll];
    int r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      r[u] = (rs0 + u) * kRowsPerSet + g;
      if (rs0 + u < rs_end && r[u] < H) {
        const uint16_t* src = tok_base + (size_t)r[u] * D;
        A[u] = ld16(src + lc.off_a);
        B[u] = ld16(src + lc.off_b);
      } else {
        r[u] = H;   // inactive
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int rr = r[u];
      if (rr >= H) continue;
      if (rr < p.Hq + p.Hkv && lc.rotary) rotate_chunks<kStyle, kExact>(A[u], B[u], cs, sn);
      if (rr < p.Hq) {
        uint16_t* dst = (kCall == kCallPacked) ? tok_base + (size_t)rr * D
                                               : p.q_out + ((size_t)token * p.Hq + rr) * D;
        st16(dst + lc.off_a, A[u]);
        st16(dst + lc.off_b, B[u]);
      } else {
        const bool is_k = rr < p.Hq + p.Hkv;
        const int h = is_k ? rr - p.Hq : rr - p.Hq - p.Hkv;
        const int plane = is_k ? 0 : 1;
        uint16_t* dst =
            p.cache + ((((size_t)b * 2 + plane) * p.Hkv + h) * (size_t)p.cap + slot) * D;
        st16(dst + lc.off_a, A[u]);
        st16(dst + lc.off_b, B[u]);
        if (kCall == kCallPacked && is_k) {
          uint16_t* src = tok_base + (size_t)rr * D;
          st16(src + lc.off_a, A[u]);
          st16(src + lc.off_b, B[u]);
        }
      }
    }
  }
}

// --------------------------------------------------------------- call 4 --
//
// Paged delta update (TensorRT-Edge-LLM C++ API, "Dflash Runtime Kernels",
// launchDFlashTargetKVCacheUpdate).  A wave owns one delta row i (or a
// slice of its 2*Hkv head rows: K heads first, then V heads).  The pool is
// addressed as [2*numPages][64][Hkv][D] by canonical page id, in 64-bit.
template <int D, int kStyle, bool kExact, int kUnroll>
__global__ __launch_bounds__(kBlock) void paged_kernel(PagedParams p) {
  constexpr int kLanesPerRow = D / 16;
  constexpr int kRowsPerSet = kWave / kLanesPerRow;
  constexpr int kTpp = kTokensPerPage;

  const int wave = wave_id_uniform();
  if (wave >= p.total_waves) return;
  const int i = wave / p.waves_per_row;
  const int part = wave - i * p.waves_per_row;

  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane / kLanesPerRow;
  const int j = lane - g * kLanesPerRow;
  const LaneChunks lc = lane_chunks<D>(j, p.R);
  const int rows = 2 * p.Hkv;
  const int rs_begin = (int)(((long long)part * p.row_sets) / p.waves_per_row);
  const int rs_end = (int)(((long long)(part + 1) * p.row_sets) / p.waves_per_row);

  // Index metadata first; the data loads below do not depend on it.
  const int pos = p.positions[i];
  const int seq = p.seq[i];

  const size_t delta_row = (size_t)i * p.Hkv;
  for (int rs0 = rs_begin; rs0 < rs_end; rs0 += kUnroll) {
    uint4 A[kUnroll], B[kUnroll];
    int r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      r[u] = (rs0 + u) * kRowsPerSet + g;
      if (rs0 + u < rs_end && r[u] < rows) {
        const bool is_k = r[u] < p.Hkv;
        const uint16_t* src =
            (is_k ? p.k_delta + (delta_row + r[u]) * D : p.v_delta + (delta_row + r[u] - p.Hkv) * D);
        A[u] = ld16(src + lc.off_a);
        B[u] = ld16(src + lc.off_b);
      } else {
        r[u] = rows;
      }
    }

    if (pos < 0 || seq < 0 || seq >= p.batch ||
        (long long)pos >= (long long)p.max_pages * kTpp)
      return;
    const int lp = pos / kTpp;
    const int off = pos - lp * kTpp;
    const int* pt = p.page_table + (size_t)seq * 2 * p.max_pages;
    const int kid = pt[lp];
    const int vid = pt[p.max_pages + lp];
    const bool k_ok = kid >= 0 && kid < p.num_pages;
    const bool v_ok = vid >= p.num_pages && (long long)vid < 2LL * p.num_pages;

    float cs[8], sn[8];
    if (k_ok && lc.rotary) load_cos_sin<kStyle>(p.cos_sin + (size_t)i * p.R, j, p.R, cs, sn);

#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int rr = r[u];
      if (rr >= rows) continue;
      const bool is_k = rr < p.Hkv;
      if (is_k ? !k_ok : !v_ok) continue;
      const int h = is_k ? rr : rr - p.Hkv;
      const size_t page = (size_t)(is_k ? kid : vid);
      if (is_k && lc.rotary) rotate_chunks<kStyle, kExact>(A[u], B[u], cs, sn);
      uint16_t* dst = p.pool + ((page * kTpp + off) * p.Hkv + h) * D;
      st16(dst + lc.off_a, A[u]);
      st16(dst + lc.off_b, B[u]);
    }
  }
}

// ------------------------------------------------------------- launches --

namespace {

template <int D, int kCall, int kStyle>
hipError_t launch_contig_d(const ContigParams& p, hipStream_t stream) {
  const unsigned blocks = (unsigned)((p.total_waves + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL((contig_kernel<D, kCall, kStyle, true, kContigUnroll>), dim3(blocks),
                     dim3(kBlock), 0, stream, p);
  return hipGetLastError();
}

template <int kCall, int kStyle>
hipError_t launch_contig_s(const ContigParams& p, int D, hipStream_t stream) {
  switch (D) {
    case 64: return launch_contig_d<64, kCall, kStyle>(p, stream);
    case 128: return launch_contig_d<128, kCall, kStyle>(p, stream);
    case 256: return launch_contig_d<256, kCall, kStyle>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int kCall>
hipError_t launch_contig_c(const ContigParams& p, int D, int style, hipStream_t stream) {
  return style == kNeox ? launch_contig_s<kCall, kNeox>(p, D, stream)
                        : launch_contig_s<kCall, kGptj>(p, D, stream);
}

template <int D, int kStyle>
hipError_t launch_paged_d(const PagedParams& p, hipStream_t stream) {
  const unsigned blocks = (unsigned)((p.total_waves + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL((paged_kernel<D, kStyle, true, kPagedUnroll>), dim3(blocks), dim3(kBlock), 0,
                     stream, p);
  return hipGetLastError();
}

template <int kStyle>
hipError_t launch_paged_s(const PagedParams& p, int D, hipStream_t stream) {
  switch (D) {
    case 64: return launch_paged_d<64, kStyle>(p, stream);
    case 128: return launch_paged_d<128, kStyle>(p, stream);
    case 256: return launch_paged_d<256, kStyle>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_contig(const ContigParams& p, int call, int D, int style, hipStream_t stream) {
  switch (call) {
    case kCallPacked: return launch_contig_c<kCallPacked>(p, D, style, stream);
    case kCallContinuous: return launch_contig_c<kCallContinuous>(p, D, style, stream);
    case kCallTree: return launch_contig_c<kCallTree>(p, D, style, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_paged(const PagedParams& p, int D, int style, hipStream_t stream) {
  return style == kNeox ? launch_paged_s<kNeox>(p, D, stream) : launch_paged_s<kGptj>(p, D, stream);
}

}  // namespace rkv
