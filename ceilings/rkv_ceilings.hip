// Measurement kernels that bound the library's kernels on the same chip.
//
// They are not part of the library (librkv.so never contains them): bench.py
// times them beside the library's kernels so that every ceiling, floor and
// design alternative the performance figures are held against is reproduced
// from committed code.  They use the library's own access primitives (buffer
// resources, non-temporal loads, nt sc1 stores, XCD workgroup order) and its
// rotate unit, from rkv_kernels.hpp, so a ceiling differs from the kernel it
// bounds only in what it leaves out.
//
//  * streams: copy, narrowing (16 bytes read, 8 written per lane) and
//    in-place passes over a buffer, one 16-byte chunk read per lane, with
//    the library's load and store policy or with plain accesses;
//  * the in-place stream in persistent form: a fixed grid whose workgroups
//    loop over the buffer, U chunks per step, optionally loading the next
//    step before storing the current one (the alternative to one short-lived
//    workgroup per chunk, the library's choice);
//  * an empty kernel of a given grid (the fixed cost of a launch);
//  * exhaustive checks of the library's fp32 reciprocal of a scale and of
//    its packed fp16 conversion;
//  * a paged-update floor: the paged update's decomposition, cos/sin fetch,
//    NeoX rotation and stores for the same row shapes, with every address
//    computed from the row number (no position, sequence or page-table
//    loads), into contiguous rows or scattered over pool pages;
//  * the packed prefill (call 1, fp16 cache, default arithmetic) with one
//    workgroup per token, its cos/sin row staged in LDS once and reused by
//    all its waves (the alternative to each wave fetching the values its
//    lanes need, the library's choice), or fetched per wave with the NeoX
//    partners exchanged by DPP instead of ds_bpermute.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../rope_kv_cache_amd/csrc/rkv_kernels.hpp"

using namespace rkv;

namespace {

constexpr int kD = 128;                     // head dim of the floors and the LDS prefill
constexpr int kLanesPerRow = kD / 8;        // 16
constexpr int kRowsPerGroup = kWave / kLanesPerRow;   // 4
constexpr uint32_t kChunkBytes = 4096;      // one workgroup of the streams: 256 lanes x 16 B

// ------------------------------------------------------------- streams --

template <bool kLibPolicy>
__global__ __launch_bounds__(256) void copy_kernel(const uint8_t* src, uint8_t* dst,
                                                   int chunk_log2) {
  const size_t base = (size_t)block_id_xcd(chunk_log2, (int)gridDim.x) * kChunkBytes;
  const uint32_t off = threadIdx.x * 16u;
  if constexpr (kLibPolicy) {
    const BufRes s = buffer_of(src + base, kChunkBytes);
    const BufRes d = buffer_of(dst + base, kChunkBytes);
    st16_buf(d, off, ld16_buf(s, off));
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(src + base + off);
    *reinterpret_cast<uint4*>(dst + base + off) = v;
  }
}

// Read 16 bytes, write 8 (the xor of each pair of dwords): the 2:1 read to
// write mix of an update that narrows fp16 rows to one-byte cache entries.
template <bool kLibPolicy>
__global__ __launch_bounds__(256) void narrow_kernel(const uint8_t* src, uint8_t* dst,
                                                     int chunk_log2) {
  const int blk = block_id_xcd(chunk_log2, (int)gridDim.x);
  const size_t base = (size_t)blk * kChunkBytes;
  const uint32_t off = threadIdx.x * 16u;
  if constexpr (kLibPolicy) {
    const BufRes s = buffer_of(src + base, kChunkBytes);
    const BufRes d = buffer_of(dst + base / 2, kChunkBytes / 2);
    const uint4 v = ld16_buf(s, off);
    st8_buf(d, off / 2, make_uint2(v.x ^ v.y, v.z ^ v.w));
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(src + base + off);
    *reinterpret_cast<uint2*>(dst + base / 2 + off / 2) = make_uint2(v.x ^ v.y, v.z ^ v.w);
  }
}

// Read, modify (xor with `key`), write back.
template <bool kLibPolicy>
__global__ __launch_bounds__(256) void inplace_kernel(uint8_t* buf, uint32_t key,
                                                      int chunk_log2) {
  const size_t base = (size_t)block_id_xcd(chunk_log2, (int)gridDim.x) * kChunkBytes;
  const uint32_t off = threadIdx.x * 16u;
  if constexpr (kLibPolicy) {
    const BufRes r = buffer_of(buf + base, kChunkBytes);
    uint4 v = ld16_buf(r, off);
    v.x ^= key; v.y ^= key; v.z ^= key; v.w ^= key;
    st16_buf(r, off, v);
  } else {
    uint4 v = *reinterpret_cast<const uint4*>(buf + base + off);
    v.x ^= key; v.y ^= key; v.z ^= key; v.w ^= key;
    *reinterpret_cast<uint4*>(buf + base + off) = v;
  }
}

// Persistent in-place stream: every workgroup loops over the buffer, U
// consecutive 4 KB chunks per step.  kXcd: workgroup b (on XCD b mod 8)
// walks its XCD's own contiguous regions of 128 chunks, as the 128-workgroup
// chunk order does; otherwise step i of workgroup b takes chunks
// (i * grid + b) * U ...  kPipe: the next step's loads are issued before the
// current step's stores.  The host checks that the chunk count is a
// multiple of 8 * 128 and the grid a multiple of 8, so every chunk is
// visited exactly once.
template <int U, bool kPipe, bool kXcd>
__global__ __launch_bounds__(256) void persistent_inplace_kernel(uint8_t* buf, uint32_t bytes,
                                                                 uint32_t key) {
  const BufRes r = buffer_of(buf, bytes);
  const uint32_t nchunks = bytes / kChunkBytes;
  constexpr uint32_t kGroups = 128 / U;          // U-chunk steps per XCD region
  const uint32_t xcd = blockIdx.x & 7u, per_xcd = gridDim.x >> 3;
  const uint32_t lane_off = threadIdx.x * 16u;
  auto first_chunk = [&](uint32_t j) {
    if constexpr (kXcd) return (xcd * kGroups + (j % kGroups) + (j / kGroups) * 8u * kGroups) * U;
    else return j * U;
  };
  uint32_t j = kXcd ? blockIdx.x >> 3 : blockIdx.x;
  const uint32_t j_step = kXcd ? per_xcd : gridDim.x;
  uint32_t c0 = first_chunk(j);
  uint4 cur[U];
  if constexpr (kPipe) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      cur[u] = c0 < nchunks ? ld16_buf(r, (c0 + u) * kChunkBytes + lane_off) : make_uint4(0, 0, 0, 0);
  }
  while (c0 < nchunks) {
    j += j_step;
    const uint32_t c1 = first_chunk(j);
    uint4 nxt[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (kPipe)
        nxt[u] = c1 < nchunks ? ld16_buf(r, (c1 + u) * kChunkBytes + lane_off) : make_uint4(0, 0, 0, 0);
      else
        cur[u] = ld16_buf(r, (c0 + u) * kChunkBytes + lane_off);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      cur[u].x ^= key; cur[u].y ^= key; cur[u].z ^= key; cur[u].w ^= key;
      st16_buf(r, (c0 + u) * kChunkBytes + lane_off, cur[u]);
    }
    if constexpr (kPipe) {
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    }
    c0 = c1;
  }
}

// Exhaustive check of the library's reciprocal() (rkv_rotate.hpp): for
// every fp32 pattern b, reciprocal(b) against the binary64 quotient 1/b
// rounded to binary32 (any NaN equals any NaN).  Thread t covers patterns
// [t * per_thread, (t + 1) * per_thread); counts[2t] is its number of
// mismatches, counts[2t + 1] its first mismatching pattern (or all ones).
__global__ __launch_bounds__(256) void reciprocal_check_kernel(uint32_t* counts,
                                                               uint32_t per_thread) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t n = 0, first = 0xffffffffu;
  for (uint32_t j = 0; j < per_thread; ++j) {
    const uint32_t u = tid * per_thread + j;
    const float b = __builtin_bit_cast(float, u);
    const float got = reciprocal(b);
    const float want = (float)(1.0 / (double)b);
    const bool same = __builtin_bit_cast(uint32_t, got) == __builtin_bit_cast(uint32_t, want) ||
                      (got != got && want != want);
    if (!same) {
      if (n == 0) first = u;
      ++n;
    }
  }
  counts[2 * tid] = n;
  counts[2 * tid + 1] = first;
}

// Exhaustive check of the library's packed fp16 conversion (f2h_pair in
// rkv_rotate.hpp) against two scalar conversions (f2h_bits): every fp32
// pattern u in the low half, with an unrelated pattern in the high half.
// Same output layout as reciprocal_check_kernel.
__global__ __launch_bounds__(256) void f16_pair_check_kernel(uint32_t* counts,
                                                             uint32_t per_thread) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t n = 0, first = 0xffffffffu;
  for (uint32_t j = 0; j < per_thread; ++j) {
    const uint32_t u = tid * per_thread + j;
    const uint32_t u2 = u * 2654435761u + 12345u;
    const float lo = __builtin_bit_cast(float, u), hi = __builtin_bit_cast(float, u2);
    if (f2h_pair(lo, hi) != (f2h_bits(lo) | (f2h_bits(hi) << 16))) {
      if (n == 0) first = u;
      ++n;
    }
  }
  counts[2 * tid] = n;
  counts[2 * tid + 1] = first;
}

__global__ __launch_bounds__(256) void empty_kernel() {}

// ------------------------------------------------------ paged floor --

struct FloorParams {
  uint16_t* pool;            // [2 * num_pages, 64, Hkv, 128]
  const float* cos_sin;      // [N, R]
  int32_t N, num_pages;
  int32_t scatter;           // 0: contiguous destination rows, 1: scattered over pool pages
};

// Row i = (sequence q, row j of q).  Contiguous: K row i goes to the K
// plane's row i, V to the V plane's row i.  Scattered: the row sits at
// position ((37 q) mod 64) + j of sequence q, and logical page lp of q maps
// to K page (1021 (4q + lp)) mod num_pages and V page num_pages + (2053 (4q
// + lp)) mod num_pages: odd multipliers modulo a power of two are one to
// one, so no two rows share a slot (the host checks 4 * sequences <=
// num_pages).  Writes come in runs of up to 64 slots per page, as a
// sequence's consecutive positions do in the paged workload.
// Like the library's paged kernel, the values a wave needs first are leading
// scalar arguments, preloaded into SGPRs (rows_per_seq_log2: delta rows of
// one sequence are 2^rows_per_seq_log2; the first live_per_seq of them are
// written).
template <int G, bool kStream>
__global__ __launch_bounds__(256) void paged_floor_kernel(
    int32_t total_waves, uint32_t waves_div_m, uint32_t waves_div_l, int32_t waves_per_row,
    int32_t Hkv, int32_t R, int32_t rows_per_seq_log2, int32_t live_per_seq,
    const uint16_t* __restrict__ k_delta, const uint16_t* __restrict__ v_delta, FloorParams p) {
  const int wave = wave_id_uniform(0, total_waves);
  if (wave >= total_waves) return;
  const FastDiv div_waves{(uint32_t)waves_per_row, waves_div_m, waves_div_l};
  const int i = (int)fast_div((uint32_t)wave, div_waves);
  const int part = wave - i * waves_per_row;
  const int q = i >> rows_per_seq_log2;
  const int j = i & ((1 << rows_per_seq_log2) - 1);
  if (j >= live_per_seq) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane % kLanesPerRow;
  const int row_in_group = lane / kLanesPerRow;
  const ChunkRole role = chunk_role<kNeox>(c, R);
  const int rows = 2 * Hkv;
  const size_t delta_row = (size_t)i * Hkv;

  int row[G];
  uint4 x[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int r = (part * G + g) * kRowsPerGroup + row_in_group;
    row[g] = r;
    x[g] = make_uint4(0, 0, 0, 0);
    if (r < Hkv) {
      const uint16_t* src = k_delta + (delta_row + r) * kD + 8 * c;
      x[g] = kStream ? ld16_stream(src) : ld16(src);
    } else if (r < rows) {
      const uint16_t* src = v_delta + (delta_row + (r - Hkv)) * kD + 8 * c;
      x[g] = kStream ? ld16_stream(src) : ld16(src);
    }
  }
  float cs[8] = {}, sn[8] = {};
  const bool has_k = part * G * kRowsPerGroup < Hkv;   // wave-uniform
  if (has_k && role.rotary)
    load_cos_sin_direct<kNeox>(p.cos_sin + (size_t)i * R, role.freq0, R, cs, sn);

  size_t k_slot, v_slot;   // first element of the row's K and V slot rows
  const size_t plane = (size_t)p.num_pages * kTokensPerPage * Hkv * kD;
  if (p.scatter) {
    const int pos = ((q * 37) & 63) + j;
    const int lp = pos >> 6, off = pos & 63;
    const int page_key = 4 * q + lp;
    const int kid = (page_key * 1021) & (p.num_pages - 1);
    const int vid = p.num_pages + ((page_key * 2053) & (p.num_pages - 1));
    k_slot = ((size_t)kid * kTokensPerPage + off) * Hkv * kD;
    v_slot = ((size_t)vid * kTokensPerPage + off) * Hkv * kD;
  } else {
    k_slot = (size_t)i * Hkv * kD;
    v_slot = plane + (size_t)i * Hkv * kD;
  }
  constexpr uint32_t kNowhere = 0x80000000u;
  const uint32_t row_bytes = (uint32_t)Hkv * kD * 2;
  const BufRes kp = buffer_of(p.pool + k_slot, row_bytes);
  const BufRes vp = buffer_of(p.pool + v_slot, row_bytes);

#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int r = row[g];
    const bool is_k = r < Hkv;
    const uint4 y = rotate_chunk<kNeox, false>(x[g], lane, role, is_k, cs, sn);
    if (r >= rows) continue;
    const int h = is_k ? r : r - Hkv;
    if constexpr (kStream) {
      const int g0 = (part * G + g) * kRowsPerGroup;
      const uint32_t el_k = is_k ? (uint32_t)(h * kD + 8 * c) * 2 : kNowhere;
      const uint32_t el_v = !is_k ? (uint32_t)(h * kD + 8 * c) * 2 : kNowhere;
      if (g0 < Hkv) st16_buf(kp, el_k, y);
      if (g0 + kRowsPerGroup > Hkv) st16_buf(vp, el_v, y);
    } else {
      st16(p.pool + (is_k ? k_slot : v_slot) + (size_t)h * kD + 8 * c, y);
    }
  }
}

// ------------------------------------------------ LDS-staged prefill --

struct LdsParams {
  const float* cos_sin;      // [table_batch, table_len, R]
  uint16_t* qkv;             // [B, S, Hq + 2 Hkv, 128], rotated in place
  uint16_t* cache;           // [B, 2, Hkv, cap, 128]
  int32_t B, S, Hq, Hkv, cap, table_batch, table_len, R;
  uint32_t cache_b_bytes;    // one batch's cache slice (the host keeps it below 2^32)
  int32_t chunk_log2;        // workgroup (token) order over the XCDs
  FastDiv div_seq;           // by S
};

// NeoX partner chunk of a lane (the lane R/16 away in its row): the
// library's ds_bpermute, or, for R = D = 128 only, a DPP rotation by 8 inside
// each row of 16 lanes (the partner of lane l is then l ^ 8).
template <bool kDpp>
__device__ __forceinline__ uint4 neox_partner(uint4 x, int lane, const ChunkRole& role) {
  if constexpr (kDpp) {
    constexpr int kRowRor8 = 0x128;
    return make_uint4(__builtin_amdgcn_mov_dpp((int)x.x, kRowRor8, 0xf, 0xf, false),
                      __builtin_amdgcn_mov_dpp((int)x.y, kRowRor8, 0xf, 0xf, false),
                      __builtin_amdgcn_mov_dpp((int)x.z, kRowRor8, 0xf, 0xf, false),
                      __builtin_amdgcn_mov_dpp((int)x.w, kRowRor8, 0xf, 0xf, false));
  } else {
    return lane_fetch(x, lane + role.partner);
  }
}

// One workgroup per token, blockDim = 64 * ceil(row groups / G): the token's
// table row (R floats) is loaded once into LDS by the first R/4 threads,
// every wave waits at one barrier and reads its lanes' cos/sin values from
// LDS (kLds); or every wave fetches the values its lanes need, as the
// library does (the lower half of the wave the cosines, the upper half the
// sines, joined by v_permlane32_swap).  kDpp (NeoX, R = D = 128) exchanges
// NeoX partners by DPP instead of ds_bpermute.  Row loads, rotation and
// stores are the library's call-1 kernel's.
template <int kStyle, int G, bool kLds, bool kDpp>
__global__ __launch_bounds__(1024) void prefill_lds_kernel(LdsParams p) {
  __shared__ float4 table_row[kD / 4];
  const int token = block_id_xcd(p.chunk_log2, (int)gridDim.x);
  const int b = (int)fast_div((uint32_t)token, p.div_seq);
  const int s = token - b * p.S;
  const int part = threadIdx.x >> 6;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane % kLanesPerRow;
  const int row_in_group = lane / kLanesPerRow;
  const ChunkRole role = chunk_role<kStyle>(c, p.R);

  const int H = p.Hq + 2 * p.Hkv;
  uint16_t* const tok_base = p.qkv + (size_t)token * H * kD;
  const BufRes tok_buf = buffer_of(tok_base, (uint32_t)H * kD * 2);
  uint4 x[G];
  int row[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    row[g] = (part * G + g) * kRowsPerGroup + row_in_group;
    x[g] = ld16_buf(tok_buf, (uint32_t)(row[g] * kD + 8 * c) * 2);
  }
  const int tb = (p.table_batch == 1) ? 0 : b;
  const float* trow = p.cos_sin + ((size_t)tb * p.table_len + s) * p.R;
  float cs[8] = {}, sn[8] = {};
  if constexpr (kLds) {
    if ((int)threadIdx.x < (p.R >> 2))
      table_row[threadIdx.x] = reinterpret_cast<const float4*>(trow)[threadIdx.x];
    __syncthreads();
    if (role.rotary) {
      const float* t = reinterpret_cast<const float*>(table_row);
      const int half = p.R >> 1;
      const int nf = kStyle == kNeox ? 8 : 4;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (k < nf) {
          cs[k] = t[role.freq0 + k];
          sn[k] = t[half + role.freq0 + k];
        }
      }
    }
  } else {
    spread_cos_sin<kStyle>(load_cos_sin<kStyle>(trow, role.freq0, p.R, lane), cs, sn);
  }
  const size_t cache_b = (size_t)b * 2 * p.Hkv * p.cap * kD;
  const BufRes cache_buf = buffer_of(p.cache + cache_b, p.cache_b_bytes);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int r = row[g];
    const bool is_q = r < p.Hq;
    const bool is_k = !is_q && r < p.Hq + p.Hkv;
    uint4 y;
    if constexpr (kStyle == kNeox) {
      const uint4 q = neox_partner<kDpp>(x[g], lane, role);
      y = ((is_q || is_k) && role.rotary)
              ? rotate_neox<false>(x[g], q, cs, sn, role.first, role.neg_zero)
              : x[g];
    } else {
      y = rotate_chunk<kStyle, false>(x[g], lane, role, is_q || is_k, cs, sn);
    }
    if (r >= H) continue;
    const uint32_t row_off = (uint32_t)(r * kD + 8 * c) * 2;
    if (is_q) {
      st16_buf(tok_buf, row_off, y);
    } else {
      const int h = is_k ? r - p.Hq : r - p.Hq - p.Hkv;
      const size_t cache_el =
          (((size_t)(is_k ? 0 : 1) * p.Hkv + h) * (size_t)p.cap + s) * kD + 8 * c;
      st16_buf(cache_buf, (uint32_t)cache_el * 2, y);
      if (is_k) st16_buf(tok_buf, row_off, y);
    }
  }
}

int err(hipError_t e) { return (int)e; }

}  // namespace

extern "C" {

// All functions launch on `stream` and return a hipError_t value (0 = success);
// invalid arguments return hipErrorInvalidValue without launching.

// dst[0:bytes) = src[0:bytes); bytes a positive multiple of 4096 below 2^43.
// policy 1: the library's buffer loads (nt) and stores (nt sc1); 0: plain.
int rkvc_stream_copy(const void* src, void* dst, long long bytes, int policy, int chunk_log2,
                     hipStream_t stream) {
  if (!src || !dst || bytes <= 0 || bytes % kChunkBytes || bytes / kChunkBytes > INT32_MAX ||
      chunk_log2 < 0 || chunk_log2 > 16)
    return err(hipErrorInvalidValue);
  const dim3 grid((unsigned)(bytes / kChunkBytes));
  if (policy)
    hipLaunchKernelGGL(copy_kernel<true>, grid, dim3(256), 0, stream, (const uint8_t*)src,
                       (uint8_t*)dst, chunk_log2);
  else
    hipLaunchKernelGGL(copy_kernel<false>, grid, dim3(256), 0, stream, (const uint8_t*)src,
                       (uint8_t*)dst, chunk_log2);
  return err(hipGetLastError());
}

// dst[0:bytes/2) as 32-bit words: word i = src word 2i ^ src word 2i+1.
int rkvc_stream_narrow(const void* src, void* dst, long long bytes, int policy, int chunk_log2,
                       hipStream_t stream) {
  if (!src || !dst || bytes <= 0 || bytes % kChunkBytes || bytes / kChunkBytes > INT32_MAX ||
      chunk_log2 < 0 || chunk_log2 > 16)
    return err(hipErrorInvalidValue);
  const dim3 grid((unsigned)(bytes / kChunkBytes));
  if (policy)
    hipLaunchKernelGGL(narrow_kernel<true>, grid, dim3(256), 0, stream, (const uint8_t*)src,
                       (uint8_t*)dst, chunk_log2);
  else
    hipLaunchKernelGGL(narrow_kernel<false>, grid, dim3(256), 0, stream, (const uint8_t*)src,
                       (uint8_t*)dst, chunk_log2);
  return err(hipGetLastError());
}

// buf[0:bytes) ^= key (per 32-bit word), read and written in place.
int rkvc_stream_inplace(void* buf, long long bytes, unsigned key, int policy, int chunk_log2,
                        hipStream_t stream) {
  if (!buf || bytes <= 0 || bytes % kChunkBytes || bytes / kChunkBytes > INT32_MAX ||
      chunk_log2 < 0 || chunk_log2 > 16)
    return err(hipErrorInvalidValue);
  const dim3 grid((unsigned)(bytes / kChunkBytes));
  if (policy)
    hipLaunchKernelGGL(inplace_kernel<true>, grid, dim3(256), 0, stream, (uint8_t*)buf, key,
                       chunk_log2);
  else
    hipLaunchKernelGGL(inplace_kernel<false>, grid, dim3(256), 0, stream, (uint8_t*)buf, key,
                       chunk_log2);
  return err(hipGetLastError());
}

// buf[0:bytes) ^= key by persistent_inplace_kernel<unroll, pipe, xcd> on
// `workgroups` workgroups of 256 threads.
int rkvc_stream_persistent(void* buf, long long bytes, unsigned key, int unroll, int pipe,
                           int xcd, int workgroups, hipStream_t stream) {
  if (!buf || bytes <= 0 || bytes % (kChunkBytes * 8LL * 128) || bytes >= (1LL << 31) ||
      workgroups <= 0 || workgroups % 8 || (unroll != 1 && unroll != 2 && unroll != 4))
    return err(hipErrorInvalidValue);
  const dim3 grid((unsigned)workgroups);
  const uint32_t n = (uint32_t)bytes;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, (uint8_t*)buf, n, key);
  };
#define RKVC_PERSISTENT(U)                                                             \
  if (unroll == U) {                                                                  \
    if (pipe && xcd) go(persistent_inplace_kernel<U, true, true>);                    \
    else if (pipe) go(persistent_inplace_kernel<U, true, false>);                     \
    else if (xcd) go(persistent_inplace_kernel<U, false, true>);                      \
    else go(persistent_inplace_kernel<U, false, false>);                              \
  }
  RKVC_PERSISTENT(1) RKVC_PERSISTENT(2) RKVC_PERSISTENT(4)
#undef RKVC_PERSISTENT
  return err(hipGetLastError());
}

// reciprocal_check_kernel over all 2^32 fp32 patterns on `threads` threads
// (a power of two from 256 to 2^24); counts holds 2 * threads words.
int rkvc_check_reciprocal(uint32_t* counts, int threads, hipStream_t stream) {
  if (!counts || threads < 256 || threads > (1 << 24) || (threads & (threads - 1)))
    return err(hipErrorInvalidValue);
  const uint32_t per = (uint32_t)((1ULL << 32) / (unsigned long long)threads);
  hipLaunchKernelGGL(reciprocal_check_kernel, dim3((unsigned)threads / 256), dim3(256), 0, stream,
                     counts, per);
  return err(hipGetLastError());
}

// f16_pair_check_kernel over all 2^32 patterns, as rkvc_check_reciprocal.
int rkvc_check_f16_pair(uint32_t* counts, int threads, hipStream_t stream) {
  if (!counts || threads < 256 || threads > (1 << 24) || (threads & (threads - 1)))
    return err(hipErrorInvalidValue);
  const uint32_t per = (uint32_t)((1ULL << 32) / (unsigned long long)threads);
  hipLaunchKernelGGL(f16_pair_check_kernel, dim3((unsigned)threads / 256), dim3(256), 0, stream,
                     counts, per);
  return err(hipGetLastError());
}

// A kernel that does nothing, `workgroups` workgroups of 256 threads.
int rkvc_empty(int workgroups, hipStream_t stream) {
  if (workgroups <= 0) return err(hipErrorInvalidValue);
  hipLaunchKernelGGL(empty_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream);
  return err(hipGetLastError());
}

// The paged-update floor on D = 128, NeoX: N delta rows of Hkv K and Hkv V
// heads, sequences of 2^rows_per_seq_log2 rows of which the first
// live_per_seq are written; pool of 2 * num_pages pages (num_pages a power
// of two >= 4 * sequences when scatter = 1, >= N / 64 rows otherwise).
// stream_plan 1: non-temporal loads and nt sc1 buffer stores; 0: ordinary.
int rkvc_paged_floor(const uint16_t* k_delta, const uint16_t* v_delta, uint16_t* pool,
                     const float* cos_sin, int N, int Hkv, int R, int num_pages,
                     int rows_per_seq_log2, int live_per_seq, int scatter, int G,
                     int stream_plan, hipStream_t stream) {
  if (!k_delta || !v_delta || !pool || !cos_sin || N <= 0 || Hkv <= 0 || Hkv > 64 ||
      R <= 0 || R > kD || R % 16 || num_pages <= 0 || (num_pages & (num_pages - 1)) ||
      rows_per_seq_log2 < 0 || rows_per_seq_log2 > 20 || live_per_seq < 0 ||
      (G != 1 && G != 2 && G != 4))
    return err(hipErrorInvalidValue);
  const long long seqs = ((long long)N + (1LL << rows_per_seq_log2) - 1) >> rows_per_seq_log2;
  if (scatter ? (4 * seqs > num_pages || (1LL << rows_per_seq_log2) > 128)
              : ((long long)N > (long long)num_pages * kTokensPerPage))
    return err(hipErrorInvalidValue);
  FloorParams p{};
  p.pool = pool;
  p.cos_sin = cos_sin;
  p.N = N;
  p.num_pages = num_pages;
  p.scatter = scatter;
  const int groups = (2 * Hkv + kRowsPerGroup - 1) / kRowsPerGroup;
  const int waves_per_row = (groups + G - 1) / G;
  const long long waves = (long long)N * waves_per_row;
  if (waves > INT32_MAX - 4) return err(hipErrorInvalidValue);
  const FastDiv dw = make_fastdiv((uint32_t)waves_per_row);
  const dim3 grid((unsigned)((waves + 3) / 4));
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, (int32_t)waves, dw.m, dw.l,
                       waves_per_row, Hkv, R, rows_per_seq_log2, live_per_seq, k_delta, v_delta,
                       p);
    return err(hipGetLastError());
  };
  if (stream_plan) {
    if (G == 1) return go(paged_floor_kernel<1, true>);
    if (G == 2) return go(paged_floor_kernel<2, true>);
    return go(paged_floor_kernel<4, true>);
  }
  if (G == 1) return go(paged_floor_kernel<1, false>);
  if (G == 2) return go(paged_floor_kernel<2, false>);
  return go(paged_floor_kernel<4, false>);
}

// Call 1 (packed prefill, fp16 cache, default arithmetic) on D = 128, one
// workgroup per token; style 0 NeoX, 1 GPT-J; G = 2 or 4 row groups per
// wave; chunk_log2: tokens are taken by the XCDs in chunks of 2^chunk_log2
// (0: contiguous eighths); lds: the cos/sin row staged in LDS (else fetched
// per wave); dpp: NeoX partners by DPP (NeoX, R = 128, per-wave fetch only).
// Shapes as for rkv_apply_rope_write_kv_packed_qkv; the host checks only
// what this kernel's addressing needs.
int rkvc_prefill_lds(const float* cos_sin, int table_batch, int table_len, uint16_t* qkv,
                     uint16_t* cache, int B, int S, int Hq, int Hkv, int cap, int R, int style,
                     int G, int chunk_log2, int lds, int dpp, hipStream_t stream) {
  if (!cos_sin || !qkv || !cache || B <= 0 || S <= 0 || Hq < 0 || Hkv <= 0 || S > cap ||
      S > table_len || (table_batch != 1 && table_batch != B) || R <= 0 || R > kD || R % 16 ||
      (G != 2 && G != 4) || (style != kNeox && style != kGptj) || chunk_log2 < 0 ||
      chunk_log2 > 16 || (dpp && (style != kNeox || R != kD || lds)))
    return err(hipErrorInvalidValue);
  const long long H = Hq + 2LL * Hkv;
  const long long groups = (H + kRowsPerGroup - 1) / kRowsPerGroup;
  const long long waves = (groups + G - 1) / G;
  const unsigned long long slice = 2ull * Hkv * (unsigned long long)cap * kD * 2;
  if (waves > 16 || (long long)B * S > INT32_MAX || slice > 0xFFFFFFFFull ||
      (H + 64) * kD * 2 >= (1LL << 31))
    return err(hipErrorInvalidValue);
  LdsParams p{};
  p.cos_sin = cos_sin;
  p.qkv = qkv;
  p.cache = cache;
  p.B = B;
  p.S = S;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.cap = cap;
  p.table_batch = table_batch;
  p.table_len = table_len;
  p.R = R;
  p.cache_b_bytes = (uint32_t)slice;
  p.chunk_log2 = chunk_log2;
  p.div_seq = make_fastdiv((uint32_t)S);
  const dim3 grid((unsigned)(B * S)), block((unsigned)(64 * waves));
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, p);
    return err(hipGetLastError());
  };
  if (dpp) return G == 2 ? go(prefill_lds_kernel<kNeox, 2, false, true>)
                        : go(prefill_lds_kernel<kNeox, 4, false, true>);
  if (style == kNeox) {
    if (lds) return G == 2 ? go(prefill_lds_kernel<kNeox, 2, true, false>)
                           : go(prefill_lds_kernel<kNeox, 4, true, false>);
    return G == 2 ? go(prefill_lds_kernel<kNeox, 2, false, false>)
                  : go(prefill_lds_kernel<kNeox, 4, false, false>);
  }
  if (lds) return G == 2 ? go(prefill_lds_kernel<kGptj, 2, true, false>)
                         : go(prefill_lds_kernel<kGptj, 4, true, false>);
  return G == 2 ? go(prefill_lds_kernel<kGptj, 2, false, false>)
                : go(prefill_lds_kernel<kGptj, 4, false, false>);
}

}  // extern "C"
