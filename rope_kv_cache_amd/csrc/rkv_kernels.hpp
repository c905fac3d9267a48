// HIP kernels for gfx950: fused RoPE + KV-cache write.
//
// Work decomposition.  The unit is a (token, head) row of D fp16 values.  A
// wave instruction moves 1 KB: lane l holds 16-byte chunk l % (D/8) of row
// l / (D/8) of a "row group" of 512/D consecutive head rows of one token
// (one delta row for the paged call).  A wave owns G consecutive row groups
// of one token: it issues their G loads first, then resolves the token's
// cache slot and rotary position, fetches the cos/sin values its lanes
// need, rotates Q and K rows (NeoX partners come from a neighbouring lane
// by ds_bpermute; GPT-J pairs stay in the lane) and stores.  Waves are laid
// out token-major, so the chip sweeps the packed tensor in address order
// with G (1, 2 or 4, chosen by the host per kernel flavour and launch size)
// loads per lane in flight per wave.  Measured on MI355X, this
// fine-grained, address-ordered sweep moves the call's mixed read/write
// traffic faster than per-lane batches of many loads.  There is no
// contraction anywhere: the path is bandwidth-bound, so there is no MFMA.
//
// fp8 cache (kFp8).  Same decomposition; a lane keeps its chunk's rotation
// unrounded, writes Q (and call 1's in-place K) as fp16 and the cache row
// chunk as 8 E4M3 bytes of value * (1/scale), the per-tensor scales read
// from device memory (sglang rope_cache.py, HAVE_K_SCALE / HAVE_V_SCALE).
//
// Q/K RMS norm (kNorm, calls 1-3).  Same decomposition; each Q or K row
// with a weight vector is normalised before its rotation: the lanes of a row
// reduce its sum of squares and each lane scales its own 8 values by 1/rms
// and the per-dimension weights (loaded once per wave); a NeoX rotary lane
// takes its partner's normalised values from the partner lane.
//
// This header holds the kernel templates; rkv_kernels.hip instantiates the
// fp16-cache kernels, rkv_kernels_fp8.hip the fp8-cache ones and
// rkv_kernels_norm*.hip the Q/K-norm ones.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rkv_launch.hpp"
#include "rkv_rotate.hpp"

namespace rkv {

constexpr int kWave = kWaveLanes;
constexpr int kBlock = kBlockThreads;
constexpr int kWavesPerBlock = kBlock / kWave;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ void st16(uint16_t* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// Streaming (non-temporal) 16-byte accesses for data touched exactly once.
// On the large packed prefill they lift the kernel from ~250 us to ~228 us
// (measured on MI355X); the reused cos/sin rows keep ordinary loads.
__device__ __forceinline__ uint4 ld16_stream(const uint16_t* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

__device__ __forceinline__ void st16_stream(uint16_t* p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// 8-byte stores of E4M3 cache chunks.
__device__ __forceinline__ void st8(uint8_t* p, uint2 v) { *reinterpret_cast<uint2*>(p) = v; }

__device__ __forceinline__ void st8_stream(uint8_t* p, uint2 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x2, v), reinterpret_cast<u32x2*>(p));
}

// Buffer accesses: a resource (base address and size, wave-uniform, in
// SGPRs) and a 32-bit byte offset per lane.  A load at or past the size
// reads zeros without touching memory; a store there is dropped.  Their
// cache-policy bits reach what the generic non-temporal builtins do not:
// row stores are non-temporal at device scope (nt sc1).  Measured on MI355X
// against non-temporal global stores, written buffers rotated so that no
// launch rewrites lines the previous one left: the large GPT-J prefill
// 228.8-229.1 -> 225.2-226.3 us, NeoX 237.6-238.3 -> 232.6-233.1 us;
// without nt the stores are 8% slower.
constexpr int kBufLoadStream = 2;        // nt
constexpr int kBufStoreStream = 2 | 16;  // nt sc1
constexpr int kBufDescWord3 = 0x00020000;  // raw buffer, 32-bit data format

typedef __amdgpu_buffer_rsrc_t BufRes;

__device__ __forceinline__ BufRes buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes,
                                           kBufDescWord3);
}

__device__ __forceinline__ uint4 ld16_buf(BufRes r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufLoadStream));
}

__device__ __forceinline__ void st16_buf(BufRes r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kBufStoreStream);
}

__device__ __forceinline__ void st8_buf(BufRes r, uint32_t off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, kBufStoreStream);
}

// v held by the lower 32 lanes, and v held by the upper 32, in every lane:
// v_permlane32_swap swaps the upper half of its first operand with the lower
// half of its second; given the same register twice it returns both halves.
__device__ __forceinline__ void halves(uint32_t v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// The cos/sin values a rotary lane needs from one table row [cos | sin] of R
// floats: NeoX 8 frequencies from freq0, GPT-J 4 (c[0..3]).  Lanes l and
// l + 32 hold the same chunk (D/8 divides 32), so the lower half of the wave
// loads the cosines and the upper half the sines, and `halves` gives every
// lane both: one 16-byte load per lane for GPT-J (two for NeoX) instead of
// two (four).  Measured on MI355X, the table fetch cost the large GPT-J
// prefill 2.7% (constant cos/sin, timing only: 227 -> 221 us) although the
// table is 1.2% of its bytes.  All 64 lanes must call it together; the row is
// read through a buffer of R floats, so a lane that rotates nothing reads
// past it (zeros) or values it does not use.  The fetch is split in two:
// `load_cos_sin` issues the loads, `spread_cos_sin` swaps the halves.  The
// swap waits for the loads, and vector loads complete in order, so the
// kernels swap only once every other load of the wave has been issued.
struct CosSinRaw {
  u32x4 a, b;   // this lane's 4 (NeoX: 8) cosines or sines
};

template <int kStyle>
__device__ __forceinline__ CosSinRaw load_cos_sin(const float* row, int freq0, int R, int lane) {
  const BufRes t = buffer_of(row, (uint32_t)R * 4);
  const uint32_t off = (uint32_t)((lane < 32 ? 0 : (R >> 1)) + freq0) * 4;
  CosSinRaw raw;
  raw.a = __builtin_amdgcn_raw_buffer_load_b128(t, off, 0, 0);
  if constexpr (kStyle == kNeox) raw.b = __builtin_amdgcn_raw_buffer_load_b128(t, off + 16, 0, 0);
  else raw.b = u32x4{0, 0, 0, 0};
  return raw;
}

// The paged kernel fetches directly (each lane both halves, 2 or 4 loads):
// there the swap's wait measured 1-2% slower on the small updates.
template <int kStyle>
__device__ __forceinline__ void load_cos_sin_direct(const float* row, int freq0, int R,
                                                    float (&c)[8], float (&s)[8]) {
  const int half = R >> 1;
  const float4 c0 = *reinterpret_cast<const float4*>(row + freq0);
  const float4 s0 = *reinterpret_cast<const float4*>(row + half + freq0);
  c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
  s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
  if constexpr (kStyle == kNeox) {
    const float4 c1 = *reinterpret_cast<const float4*>(row + freq0 + 4);
    const float4 s1 = *reinterpret_cast<const float4*>(row + half + freq0 + 4);
    c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
    s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
  } else {
#pragma unroll
    for (int k = 4; k < 8; ++k) { c[k] = 0.f; s[k] = 0.f; }
  }
}

template <int kStyle>
__device__ __forceinline__ void spread_cos_sin(const CosSinRaw& raw, float (&c)[8],
                                               float (&s)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) halves(raw.a[k], c[k], s[k]);
  if constexpr (kStyle == kNeox) {
#pragma unroll
    for (int k = 0; k < 4; ++k) halves(raw.b[k], c[4 + k], s[4 + k]);
  } else {
#pragma unroll
    for (int k = 4; k < 8; ++k) { c[k] = 0.f; s[k] = 0.f; }
  }
}

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2: workgroup bid runs on XCD bid % 8.  Renumbering them sets which work
// items share an L2 and how the XCDs move through memory together.
//  chunk_log2 == 0: XCD x works through one contiguous eighth of the items.
//  chunk_log2 > 0: the XCDs take chunks of 2^chunk_log2 workgroups in turn
//   (XCD x gets chunks x, x + 8, ...), so all eight sweep the tensors side by
//   side; the blocks past the last whole round of 8 chunks are numbered as
//   for 0.  Both numberings are permutations of [0, gridDim.x).
// Measured on MI355X with the written buffers rotated, chunks of 128
// workgroups against contiguous eighths: the 16 x 1024-token NeoX continuous
// write 72.7-72.9 -> 66.4-66.5 us, the large prefill with Q/K norm
// 231.3-232.8 -> 224.9-225.2 us, NeoX 229.9-230.1 -> 223.6-224.4 us, GPT-J
// 225.9-227.2 -> 224.4-225.0 us; the paged update was 2-4% slower with them
// and small launches (all waves resident at once) 1-2%: those keep
// contiguous eighths.  chunk_log2 is wave-uniform (a launch parameter).
__device__ __forceinline__ int xcd_contiguous(int bid, int n) {
  const int x = bid & 7, q = n >> 3, r = n & 7;
  return x * q + (x < r ? x : r) + (bid >> 3);
}

// n: the grid's workgroup count (passed in: reading gridDim would cost a
// kernel-argument load before the first row load).
__device__ __forceinline__ int block_id_xcd(int chunk_log2, int n) {
  const int bid = (int)blockIdx.x;
  if (chunk_log2 == 0) return xcd_contiguous(bid, n);
  // blocks in whole rounds of 8 chunks (a power of two: no division, which
  // would put some 30 instructions before every wave's first load)
  const int full = n & ~((8 << chunk_log2) - 1);
  if (bid < full) {
    const int k = bid >> 3, mask = (1 << chunk_log2) - 1;
    return ((((k >> chunk_log2) << 3) + (bid & 7)) << chunk_log2) + (k & mask);
  }
  return full + xcd_contiguous(bid - full, n - full);
}

// The wave's work item among `waves` (the grid has ceil(waves / 4)
// workgroups of four waves).
__device__ __forceinline__ int wave_id_uniform(int chunk_log2, int waves) {
  const int n = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  return __builtin_amdgcn_readfirstlane(block_id_xcd(chunk_log2, n) * kWavesPerBlock +
                                        (int)(threadIdx.x >> 6));
}

// Kernel arguments.  The values a wave needs before its first loads are
// separate scalar arguments ahead of the parameter block: the library is
// built with kernel-argument preloading (-amdgpu-kernarg-preload-count), so
// the hardware writes them into SGPRs when the wave starts, instead of every
// wave fetching them from the kernel-argument segment before it can compute
// its first addresses (the compiler issued two or three dependent fetches of
// parameter-block fields ahead of the first row load).  At most 14 dwords
// are preloaded.  The rest of the block is fetched once the row loads are in
// flight.  Measured on MI355X (paged workload, launches back to back over
// full copies of its tensors): 9.7 -> 9.2 us; a 65,536-row update unchanged.

// ------------------------------------------------------------ calls 1-3 --
//
// Call 1 (packed prefill): position = slot = s; Q and K rotated in place in
//   qkv, K also to cache plane 0, V copied to plane 1.
// Call 2 (continuous): position = slot = endLens[b] - S + s; Q to qOut.
// Call 3 (tree): slot = endLens[b] - S + s, position = tokenPosIds[b, s].
// Calls 2 and 3 skip a token whose slot or position is out of range.
// (TensorRT-Edge-LLM C++ API, "Apply Rope Write KV".)
//
// Preloaded arguments (see "Kernel arguments" above): the launch's wave
// count, the multipliers of the divisions by waves per token and by S, the
// three shifts packed in one dword (bits 0-7 waves per token, 8-15 S, 16-23
// the XCD chunk order), H = Hq + 2 Hkv, and the qkv, end-length and
// position-id pointers (the last two null for call 1, the last for call 2).
template <int D, int kCall, int kStyle, bool kExact, int G, bool kFp8, bool kNorm>
__global__ __launch_bounds__(kBlock) void contig_kernel(
    int32_t total_waves, uint32_t waves_div_m, int32_t waves_per_token, uint32_t seq_div_m,
    int32_t S, int32_t H, uint32_t shifts, uint16_t* qkv, const int32_t* __restrict__ end_lens,
    const int32_t* __restrict__ pos_ids, ContigParams p) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerGroup = kWave / kLanesPerRow;

  // Call 1 (the prefill, a streaming launch) issues its row loads at the
  // highest wave priority and drops back once they are issued: instruction
  // issue is otherwise oldest wave first, so a newly launched wave's loads
  // waited behind older waves' arithmetic and stores.  Measured on MI355X,
  // launches back to back over copies of their tensors: the large prefill
  // 217.7 -> 214.8 us, NeoX 219.4 -> 214.5, into E4M3 203.4 -> 201.4, with
  // Q/K norm 219.4 -> 215.9, its TP=8 shard 29.70 -> 29.27.  Calls 2 and 3
  // do without: the 16 x 1024-token continuous write gained 0.4%, while the
  // small (one-generation) launches were 1-1.5% slower with the priority,
  // and as slow with a run-time test that raised it for large launches only
  // (the test sits before every wave's first load); the paged update was
  // 4% slower with it.
  if constexpr (kCall == kCallPacked) __builtin_amdgcn_s_setprio(3);
  const int wave = wave_id_uniform((int)((shifts >> 16) & 0xffu), total_waves);
  if (wave >= total_waves) return;
  const FastDiv div_waves{(uint32_t)waves_per_token, waves_div_m, shifts & 0xffu};
  const FastDiv div_seq{(uint32_t)S, seq_div_m, (shifts >> 8) & 0xffu};
  const int token = (int)fast_div((uint32_t)wave, div_waves);
  const int part = wave - token * waves_per_token;
  const int b = (int)fast_div((uint32_t)token, div_seq);
  const int s = token - b * S;

  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane % kLanesPerRow;
  const int row_in_group = lane / kLanesPerRow;

  uint16_t* const tok_base = qkv + (size_t)token * H * D;

  // Calls 2 and 3: the token's end length (and position id) are requested
  // first, as scalar loads, so that their wait does not include the row
  // loads (vector loads complete in order).
  int end_len = 0, pos_id = 0;
  if constexpr (kCall != kCallPacked) {
    end_len = end_lens[b];
    if constexpr (kCall == kCallTree) pos_id = pos_ids[token];
  }

  // Row loads next: they do not depend on the slot or the position.  They go
  // through a buffer over the token's H rows: lanes past its last row (only
  // in its last group) read zeros without touching memory and store
  // nothing.  No branch surrounds the load: one made the compiler wait for
  // every row load before the cos/sin loads of calls 2 and 3 could be
  // issued.  For those calls the empty asm keeps it from sinking the loads
  // below the range check of the slot (it waits for nothing: no register of
  // the loads is named).  The host keeps H * D * 2 below 2^32.
  const BufRes tok_buf = buffer_of(tok_base, (uint32_t)H * D * 2);
  uint4 x[G];
  int row[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    row[g] = (part * G + g) * kRowsPerGroup + row_in_group;
    x[g] = ld16_buf(tok_buf, (uint32_t)(row[g] * D + 8 * c) * 2);
  }
  if constexpr (kCall != kCallPacked) asm volatile("" ::: "memory");
  if constexpr (kCall == kCallPacked) __builtin_amdgcn_s_setprio(0);

  int slot = s, pos = s;
  if constexpr (kCall != kCallPacked) {
    const long long slot64 = (long long)end_len - S + s;
    const long long pos64 = (kCall == kCallTree) ? (long long)pos_id : slot64;
    if (slot64 < 0 || slot64 >= p.cap || pos64 < 0 || pos64 >= p.table_len) return;
    slot = (int)slot64;
    pos = (int)pos64;
  }

  const ChunkRole role = chunk_role<kStyle>(c, p.R);
  const int tb = (p.table_batch == 1) ? 0 : b;
  const CosSinRaw csr =
      load_cos_sin<kStyle>(p.cos_sin + ((size_t)tb * p.table_len + pos) * p.R, role.freq0, p.R, lane);
  // norm: the weights of the lane's chunk for the Q rows and for the K rows
  // among this wave's rows (the chunk index is the same in every row group),
  // requested once per wave with the cos/sin loads
  float qws[8] = {}, qwp[8] = {}, kws[8] = {}, kwp[8] = {};
  bool normed[G] = {};
  if constexpr (kNorm) {
    const int r_lo = part * G * kRowsPerGroup, r_end = r_lo + G * kRowsPerGroup;
    if (p.q_norm_w && r_lo < p.Hq)
      load_norm_weights<kStyle, kExact>(p.q_norm_w, c, role, qws, qwp);
    if (p.k_norm_w && r_lo < p.Hq + p.Hkv && r_end > p.Hq)
      load_norm_weights<kStyle, kExact>(p.k_norm_w, c, role, kws, kwp);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int r = row[g];
      const float* wsrc = r < p.Hq ? p.q_norm_w : (r < p.Hq + p.Hkv ? p.k_norm_w : nullptr);
      normed[g] = wsrc != nullptr && r < H;
    }
  }
  // fp8: the scales, read while the row and cos/sin loads are in flight
  float k_rcp = 1.f, v_rcp = 1.f;
  if constexpr (kFp8) load_reciprocal_scales(p.k_scale, p.v_scale, k_rcp, v_rcp);

  // Stores: Q rows (in place for call 1, to qOut for calls 2 and 3) and call
  // 1's in-place K rows through buffers over the token's rows; cache rows
  // through a buffer over batch b's two planes, or, when those reach 4 GB
  // (cache_b_bytes == 0), by non-temporal global stores.
  const BufRes q_buf = (kCall == kCallPacked)
                           ? tok_buf
                           : buffer_of(p.q_out + (size_t)token * p.Hq * D, (uint32_t)p.Hq * D * 2);
  const size_t cache_b = (size_t)b * 2 * p.Hkv * p.cap * D;   // first element of batch b
  const bool cache_buffered = p.cache_b_bytes != 0;
  const BufRes cache_buf = kFp8 ? buffer_of(p.cache8 + cache_b, p.cache_b_bytes)
                                : buffer_of(p.cache + cache_b, p.cache_b_bytes);

  float cs[8], sn[8];
  spread_cos_sin<kStyle>(csr, cs, sn);

  // A row group whose rows are all Q, all K or all V heads (every group when
  // Hq and Hkv are multiples of 512/D) stores through offsets made of a
  // wave-uniform base plus the lane's offset inside the group, computed
  // once, and a V group is copied without the rotation's lane exchange; a
  // group straddling two of them (or past the token's last row) takes
  // per-lane offsets.  kind: 0 mixed, 1 Q, 2 K, 3 V.  Measured on MI355X,
  // launches back to back over full copies of their tensors: the continuous
  // workload 5.43 -> 5.26 us, tree 5.38 -> 5.26, into E4M3 5.85 -> 5.57, with
  // Q/K norm 6.52 -> 6.25; the large prefill unchanged (the VALU work between
  // a small launch's loads and stores is on its critical path).
  const size_t lane_cache_el = (size_t)row_in_group * p.cap * D + 8 * c;
  auto group = [&](const int g, auto kind_c) {
    constexpr int kind = decltype(kind_c)::value;
    const int r = row[g];
    const int g0 = (part * G + g) * kRowsPerGroup;
    const bool is_q = kind == 1 || (kind == 0 && r < p.Hq);
    const bool is_k = kind == 2 || (kind == 0 && !is_q && r < p.Hq + p.Hkv);
    // element offset of the lane's chunk within batch b's cache, and byte
    // offset of the row's chunk within the token's rows (Q and in-place K)
    size_t cache_el = 0;
    if constexpr (kind == 2 || kind == 3) {
      const int h0 = kind == 2 ? g0 - p.Hq : g0 - p.Hq - p.Hkv;
      cache_el = (((size_t)(kind == 2 ? 0 : 1) * p.Hkv + h0) * (size_t)p.cap + slot) * D +
                 lane_cache_el;
    } else if constexpr (kind == 0) {
      const int h = is_k ? r - p.Hq : r - p.Hq - p.Hkv;
      cache_el = (((size_t)(is_k ? 0 : 1) * p.Hkv + h) * (size_t)p.cap + slot) * D + 8 * c;
    }
    const uint32_t row_off = (uint32_t)(r * D + 8 * c) * 2;
    if constexpr (kind == 3) {
      // V rows: the cache takes the row's own values
      if constexpr (kFp8) {
        WideT<kExact> w[8];
        if constexpr (kExact) {
          const uint32_t xa[4] = {x[g].x, x[g].y, x[g].z, x[g].w};
#pragma unroll
          for (int k = 0; k < 8; ++k)
            w[k] = widen<kExact>(k & 1 ? hi16(xa[k >> 1]) : lo16(xa[k >> 1]));
        }
        const uint2 e = to_e4m3<kExact>(w, x[g], false, v_rcp, role.neg_zero);
        if (cache_buffered) st8_buf(cache_buf, (uint32_t)cache_el, e);
        else st8_stream(p.cache8 + cache_b + cache_el, e);
      } else {
        if (cache_buffered) st16_buf(cache_buf, (uint32_t)cache_el * 2, x[g]);
        else st16_stream(p.cache + cache_b + cache_el, x[g]);
      }
    } else if constexpr (kFp8 || kNorm) {
      // the unrounded row values, then fp16 and / or E4M3 from them
      WideT<kExact> w[8];
      bool comp;
      if constexpr (kNorm) {
        // normalised rows: wave-uniform in a group of Q heads or of K heads,
        // so that the norm is one branch per chunk, not a select per element
        // (the continuous workload with Q/K norm 6.29 -> 6.00 us)
        const bool nrm = kind == 1   ? p.q_norm_w != nullptr
                         : kind == 2 ? p.k_norm_w != nullptr
                                     : normed[g];
        const WideT<kExact> rr = row_rms_reciprocal<D, kExact>(x[g], p.eps);
        comp = rotate_chunk_norm<kStyle, kExact>(x[g], lane, role, is_q || is_k, nrm, rr,
                                                 is_q ? qws : kws, is_q ? qwp : kwp, cs, sn, w);
      } else {
        comp = rotate_chunk_wide<kStyle, kExact>(x[g], lane, role, is_q || is_k, cs, sn, w);
      }
      if (kind == 0 && r >= H) return;
      if (is_q) {
        st16_buf(q_buf, row_off, narrow_chunk<kExact>(w, x[g], comp));
      } else if constexpr (kFp8) {
        const uint2 e = to_e4m3<kExact>(w, x[g], comp, is_k ? k_rcp : v_rcp, role.neg_zero);
        if (cache_buffered) st8_buf(cache_buf, (uint32_t)cache_el, e);
        else st8_stream(p.cache8 + cache_b + cache_el, e);
        if (kCall == kCallPacked && is_k)
          st16_buf(tok_buf, row_off, narrow_chunk<kExact>(w, x[g], comp));
      } else {
        const uint4 y = narrow_chunk<kExact>(w, x[g], comp);
        if (cache_buffered) st16_buf(cache_buf, (uint32_t)cache_el * 2, y);
        else st16_stream(p.cache + cache_b + cache_el, y);
        if (kCall == kCallPacked && is_k) st16_buf(tok_buf, row_off, y);
      }
    } else {
      const uint4 y = rotate_chunk<kStyle, kExact>(x[g], lane, role, is_q || is_k, cs, sn);
      if (kind == 0 && r >= H) return;
      if (is_q) {
        st16_buf(q_buf, row_off, y);
      } else {
        if (cache_buffered) st16_buf(cache_buf, (uint32_t)cache_el * 2, y);
        else st16_stream(p.cache + cache_b + cache_el, y);
        if (kCall == kCallPacked && is_k) st16_buf(tok_buf, row_off, y);
      }
    }
  };
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int g0 = (part * G + g) * kRowsPerGroup;   // wave-uniform
    const int q_end = p.Hq, k_end = p.Hq + p.Hkv;
    // the plain packed prefill keeps per-lane offsets everywhere: with the
    // uniform groups it measured 0.3% slower (217.7 -> 218.3 us, six paired
    // series), its VALU work not being on its critical path
    if constexpr (kCall == kCallPacked && !kFp8 && !kNorm)
      group(g, std::integral_constant<int, 0>{});
    else if (g0 + kRowsPerGroup <= q_end)
      group(g, std::integral_constant<int, 1>{});
    else if (g0 >= q_end && g0 + kRowsPerGroup <= k_end)
      group(g, std::integral_constant<int, 2>{});
    else if (g0 >= k_end && g0 + kRowsPerGroup <= H) group(g, std::integral_constant<int, 3>{});
    else group(g, std::integral_constant<int, 0>{});
  }
}

// --------------------------------------------------------------- call 4 --
//
// Paged delta update (TensorRT-Edge-LLM C++ API, "Dflash Runtime Kernels",
// launchDFlashTargetKVCacheUpdate).  Delta row i has 2*Hkv head rows: K
// heads first, then V heads; a wave owns G row groups of one delta row.
// The pool is addressed as [2*numPages][64][Hkv][D] by canonical page id,
// in 64-bit.  The row's position and sequence are requested first; the page
// ids depend on them.  Two load plans, chosen by the host as kLateLoads:
//  - small launches (all waves resident at once, so the two dependent index
//    round trips are the kernel's critical path): every delta row of the
//    wave is requested at once, with the index loads, so that the reads
//    overlap both round trips; rows that turn out to be padding or to have
//    no page are read and dropped (about 9% more reads on the paged
//    workload);
//  - large launches and E4M3 pools: a delta row is loaded once its position,
//    sequence and page ids are known, and only if it will be written.
// Both read non-temporally and store through buffers over the slot's K and
// V page rows with nt sc1.  Measured on MI355X, launches back to back over
// full copies of the paged workload's tensors (every byte from and back to
// HBM): the 4096-row fp16 update 6.5 us with early loads against 6.9 us
// with late ones (the fused gather 6.5 against 8.0), the same rows into an
// E4M3 pool 6.8 against 6.6, a 65,536-row fp16 update 83.4 against 76.0.
// Requesting the rows once the position and sequence are known (before the
// page ids) took the 4096-row update to 6.8 us: the round trip ahead of the
// reads costs more than the padding rows' reads it saves.
//
// kGather fuses the page's cos/sin gather (launchDFlashGatherDeltaRope)
// into the update: the row's cos/sin values come from the rope table row of
// (state of its sequence, its position), read once the position and
// sequence are known (in parallel with the page-table lookup); a row with
// no such table row writes no K.
//
// Preloaded arguments (see "Kernel arguments" above): the launch's wave
// count, the division by waves per row (multiplier and shift), waves per
// row, Hkv, R, and the K-delta, V-delta, position and sequence pointers.
template <int D, int kStyle, bool kExact, int G, bool kGather, bool kFp8, bool kLateLoads>
__global__ __launch_bounds__(kBlock) void paged_kernel(
    int32_t total_waves, uint32_t waves_div_m, uint32_t waves_div_l, int32_t waves_per_row,
    int32_t Hkv, int32_t R, const uint16_t* __restrict__ k_delta,
    const uint16_t* __restrict__ v_delta, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ seqs, PagedParams p) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerGroup = kWave / kLanesPerRow;
  constexpr int kTpp = kTokensPerPage;

  const int wave = wave_id_uniform(0, total_waves);
  if (wave >= total_waves) return;
  const FastDiv div_waves{(uint32_t)waves_per_row, waves_div_m, waves_div_l};
  const int i = (int)fast_div((uint32_t)wave, div_waves);
  const int part = wave - i * waves_per_row;
  const int pos = positions[i];
  const int seq = seqs[i];

  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane % kLanesPerRow;
  const int row_in_group = lane / kLanesPerRow;
  const ChunkRole role = chunk_role<kStyle>(c, R);
  const int rows = 2 * Hkv;
  const size_t delta_row = (size_t)i * Hkv;
  // A row group whose rows are all K heads or all V heads (every group when
  // Hkv is a multiple of 512/D) addresses its loads and stores as a
  // wave-uniform base plus the lane's offset inside the group, computed
  // once; a group straddling the K/V boundary or past the last V head takes
  // per-lane addresses.  Measured on MI355X, launches back to back over full
  // copies of their tensors: the 4096-row E4M3 update 6.80 -> 6.62 us, the
  // 65,536-row fp16 update 76.8 -> 76.0 us (fewer VALU instructions per
  // wave on the path between the loads and the stores).
  const uint32_t lane_el = (uint32_t)(row_in_group * D + 8 * c);

  int row[G];
  uint4 x[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int g0 = (part * G + g) * kRowsPerGroup;   // the group's first row (wave-uniform)
    const int r = g0 + row_in_group;
    row[g] = r;
    x[g] = make_uint4(0, 0, 0, 0);
    // small launches: request every row now, with the index loads
    if constexpr (!kLateLoads) {
      if (g0 + kRowsPerGroup <= Hkv)
        x[g] = ld16_stream(k_delta + (delta_row + g0) * D + lane_el);
      else if (g0 >= Hkv && g0 + kRowsPerGroup <= rows)
        x[g] = ld16_stream(v_delta + (delta_row + (g0 - Hkv)) * D + lane_el);
      else if (r < Hkv)
        x[g] = ld16_stream(k_delta + (delta_row + r) * D + 8 * c);
      else if (r < rows)
        x[g] = ld16_stream(v_delta + (delta_row + (r - Hkv)) * D + 8 * c);
    }
  }
  float cs[8], sn[8];
  const bool has_k = part * G * kRowsPerGroup < Hkv;   // wave-uniform
  if constexpr (!kGather) {
    if (has_k && role.rotary)
      load_cos_sin_direct<kStyle>(p.cos_sin + (size_t)i * R, role.freq0, R, cs, sn);
  }

  if (pos < 0 || seq < 0 || seq >= p.batch || (long long)pos >= (long long)p.max_pages * kTpp)
    return;
  const int lp = pos / kTpp;
  const int off = pos - lp * kTpp;
  const int* pt = p.page_table + (size_t)seq * 2 * p.max_pages;
  const int kid = pt[lp];
  const int vid = pt[p.max_pages + lp];
  bool k_ok = kid >= 0 && kid < p.num_pages;
  const bool v_ok = vid >= p.num_pages && (long long)vid < 2LL * p.num_pages;
  if constexpr (kGather) {
    if (has_k) {
      const int st = p.state_idx ? p.state_idx[seq] : (p.rope_states == 1 ? 0 : seq);
      const bool rope_ok = st >= 0 && st < p.rope_states && pos < p.rope_rows;
      k_ok = k_ok && rope_ok;
      if (rope_ok && role.rotary)
        load_cos_sin_direct<kStyle>(p.rope + ((size_t)st * p.rope_rows + pos) * R, role.freq0,
                                    R, cs, sn);
    }
  }
  // Large launches: load only the rows that will be written.  (Loads from
  // buffers over the row's K and V heads, each lane issuing both with the
  // wrong one out of range, measured 4% slower on a 65,536-row update than
  // these branches.)
  if constexpr (kLateLoads) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int g0 = (part * G + g) * kRowsPerGroup;
      const int r = row[g];
      if (g0 + kRowsPerGroup <= Hkv) {
        if (k_ok) x[g] = ld16_stream(k_delta + (delta_row + g0) * D + lane_el);
      } else if (g0 >= Hkv && g0 + kRowsPerGroup <= rows) {
        if (v_ok) x[g] = ld16_stream(v_delta + (delta_row + (g0 - Hkv)) * D + lane_el);
      } else if (r < Hkv ? k_ok : (r < rows && v_ok)) {
        const uint16_t* src =
            r < Hkv ? k_delta + (delta_row + r) * D : v_delta + (delta_row + (r - Hkv)) * D;
        x[g] = ld16_stream(src + 8 * c);
      }
    }
  }
  // fp8: the scales, read while the row and cos/sin loads are in flight
  float k_rcp = 1.f, v_rcp = 1.f;
  if constexpr (kFp8) load_reciprocal_scales(p.k_scale, p.v_scale, k_rcp, v_rcp);

  // Stores go through buffers over the K page row and the V page row of the
  // delta row's slot (empty when unmapped), non-temporally at device scope;
  // a group's store into a plane is skipped when none of its rows belongs to
  // that plane (a wave-uniform test), and a lane's offset in the other plane
  // is kNowhere, past the end of every buffer, as is that of a lane past the
  // row's last head.  The host keeps 4 * Hkv * D below 2^31.  Measured on
  // MI355X, a 65,536-row fp16 update with the pool rotated among four
  // buffers: 79.6-84.9 -> 77.9-78.2 us against non-temporal global stores.
  constexpr uint32_t kNowhere = 0x80000000u;
  const uint32_t row_bytes = (uint32_t)Hkv * D * (kFp8 ? 1 : 2);   // one plane's page row
  const size_t k_slot = ((size_t)(k_ok ? kid : 0) * kTpp + off) * Hkv * D;
  const size_t v_slot = ((size_t)(v_ok ? vid : 0) * kTpp + off) * Hkv * D;
  const BufRes kp = kFp8 ? buffer_of(p.pool8 + k_slot, k_ok ? row_bytes : 0u)
                         : buffer_of(p.pool + k_slot, k_ok ? row_bytes : 0u);
  const BufRes vp = kFp8 ? buffer_of(p.pool8 + v_slot, v_ok ? row_bytes : 0u)
                         : buffer_of(p.pool + v_slot, v_ok ? row_bytes : 0u);

#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int r = row[g];
    const int g0 = (part * G + g) * kRowsPerGroup;   // the group's first row (wave-uniform)
    if (g0 + kRowsPerGroup <= Hkv) {                  // K heads only
      const uint32_t el = lane_el + (uint32_t)(g0 * D);
      if constexpr (kFp8) {
        WideT<kExact> w[8];
        const bool comp =
            rotate_chunk_wide<kStyle, kExact>(x[g], lane, role, k_ok, cs, sn, w);
        st8_buf(kp, el, to_e4m3<kExact>(w, x[g], comp, k_rcp, role.neg_zero));
      } else {
        st16_buf(kp, el * 2, rotate_chunk<kStyle, kExact>(x[g], lane, role, k_ok, cs, sn));
      }
      continue;
    }
    if (g0 >= Hkv && g0 + kRowsPerGroup <= rows) {    // V heads only: no rotation
      const uint32_t el = lane_el + (uint32_t)((g0 - Hkv) * D);
      if constexpr (kFp8) {
        WideT<kExact> w[8];
        if constexpr (kExact) {
          const uint32_t xa[4] = {x[g].x, x[g].y, x[g].z, x[g].w};
#pragma unroll
          for (int k = 0; k < 8; ++k)
            w[k] = widen<kExact>(k & 1 ? hi16(xa[k >> 1]) : lo16(xa[k >> 1]));
        }
        st8_buf(vp, el, to_e4m3<kExact>(w, x[g], false, v_rcp, role.neg_zero));
      } else {
        st16_buf(vp, el * 2, x[g]);
      }
      continue;
    }
    const bool is_k = r < Hkv;
    const uint32_t el_k = r < Hkv ? (uint32_t)(r * D + 8 * c) : kNowhere;
    const uint32_t el_v = r >= Hkv && r < rows ? (uint32_t)((r - Hkv) * D + 8 * c) : kNowhere;
    if constexpr (kFp8) {
      WideT<kExact> w[8];
      const bool comp =
          rotate_chunk_wide<kStyle, kExact>(x[g], lane, role, is_k && k_ok, cs, sn, w);
      const uint2 b = to_e4m3<kExact>(w, x[g], comp, is_k ? k_rcp : v_rcp, role.neg_zero);
      if (g0 < Hkv) st8_buf(kp, el_k, b);
      if (g0 + kRowsPerGroup > Hkv) st8_buf(vp, el_v, b);
    } else {
      const uint4 y = rotate_chunk<kStyle, kExact>(x[g], lane, role, is_k && k_ok, cs, sn);
      if (g0 < Hkv) st16_buf(kp, el_k == kNowhere ? kNowhere : el_k * 2, y);
      if (g0 + kRowsPerGroup > Hkv) st16_buf(vp, el_v == kNowhere ? kNowhere : el_v * 2, y);
    }
  }
}

// ------------------------------------------------------------- launches --

namespace detail {

template <int V>
using Int = std::integral_constant<int, V>;

// Turn runtime launch choices into template arguments.
template <typename F>
hipError_t with_d(int D, F&& f) {
  switch (D) {
    case 64: return f(Int<64>{});
    case 128: return f(Int<128>{});
    case 256: return f(Int<256>{});
    default: return hipErrorInvalidValue;
  }
}

template <typename F>
hipError_t with_style_exact(int style, bool exact, F&& f) {
  if (style == kNeox) return exact ? f(Int<kNeox>{}, Int<1>{}) : f(Int<kNeox>{}, Int<0>{});
  return exact ? f(Int<kGptj>{}, Int<1>{}) : f(Int<kGptj>{}, Int<0>{});
}

template <typename F>
hipError_t with_groups(int g, F&& f) {
  switch (g) {
    case 1: return f(Int<1>{});
    case 2: return f(Int<2>{});
    case 4: return f(Int<4>{});
    default: return hipErrorInvalidValue;
  }
}

inline unsigned blocks_for(int32_t waves) {
  return (unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
}

template <int kCall, bool kFp8, bool kNorm>
hipError_t launch_contig_call(const ContigParams& p, int D, int style, bool exact,
                              hipStream_t stream) {
  const uint32_t shifts = p.div_waves.l | (p.div_seq.l << 8) | ((uint32_t)p.xcd_chunk_log2 << 16);
  const int32_t H = p.Hq + 2 * p.Hkv;
  return with_d(D, [&](auto d) {
    return with_style_exact(style, exact, [&](auto st, auto ex) {
      return with_groups(p.groups_per_wave, [&](auto g) {
        hipLaunchKernelGGL(
            (contig_kernel<decltype(d)::value, kCall, decltype(st)::value, decltype(ex)::value != 0,
                           decltype(g)::value, kFp8, kNorm>),
            dim3(blocks_for(p.total_waves)), dim3(kBlock), 0, stream, p.total_waves,
            p.div_waves.m, p.waves_per_token, p.div_seq.m, p.S, H, shifts, p.qkv, p.end_lens,
            p.pos_ids, p);
        return hipGetLastError();
      });
    });
  });
}

template <bool kFp8, bool kNorm>
hipError_t launch_contig_t(const ContigParams& p, int call, int D, int style, bool exact,
                           hipStream_t stream) {
  switch (call) {
    case kCallPacked:
      return launch_contig_call<kCallPacked, kFp8, kNorm>(p, D, style, exact, stream);
    case kCallContinuous:
      return launch_contig_call<kCallContinuous, kFp8, kNorm>(p, D, style, exact, stream);
    case kCallTree: return launch_contig_call<kCallTree, kFp8, kNorm>(p, D, style, exact, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool kGather, bool kFp8, bool kLateLoads>
hipError_t launch_paged_g(const PagedParams& p, int D, int style, bool exact,
                          hipStream_t stream) {
  return with_d(D, [&](auto d) {
    return with_style_exact(style, exact, [&](auto st, auto ex) {
      return with_groups(p.groups_per_wave, [&](auto g) {
        hipLaunchKernelGGL((paged_kernel<decltype(d)::value, decltype(st)::value,
                                         decltype(ex)::value != 0, decltype(g)::value, kGather,
                                         kFp8, kLateLoads>),
                           dim3(blocks_for(p.total_waves)), dim3(kBlock), 0, stream,
                           p.total_waves, p.div_waves.m, p.div_waves.l, p.waves_per_row, p.Hkv,
                           p.R, p.k_delta, p.v_delta, p.positions, p.seq, p);
        return hipGetLastError();
      });
    });
  });
}

template <bool kFp8>
hipError_t launch_paged_t(const PagedParams& p, int D, int style, bool exact, bool gather,
                          bool late_loads, hipStream_t stream) {
  if (late_loads)
    return gather ? launch_paged_g<true, kFp8, true>(p, D, style, exact, stream)
                  : launch_paged_g<false, kFp8, true>(p, D, style, exact, stream);
  return gather ? launch_paged_g<true, kFp8, false>(p, D, style, exact, stream)
                : launch_paged_g<false, kFp8, false>(p, D, style, exact, stream);
}

}  // namespace detail

}  // namespace rkv
