// Device-side rotate unit for gfx950: fp16 pair rotation on 16-byte chunks.
//
// Rotation (sglang rope_cache.py, _unit_rope with _get_neox_rotated_x /
// _get_gptj_rotated_x; cos/sin halves as in _load_cos_sin):
//   y_u = x_u*c - x_v*s,   y_v = x_v*c + x_u*s
// NeoX pairs element i with i + R/2, GPT-J pairs 2i with 2i+1; frequency i
// drives pair i.
//
// Lane layout.  A head row of D fp16 values is D/8 chunks of 16 bytes.  In a
// wave instruction, lane l holds chunk c = l % (D/8) of row l / (D/8), so
// one instruction covers 512/D whole rows, i.e. 1 KB of contiguous memory
// when the rows are adjacent.  Chunks c < R/8 are rotary, the others pass
// through.
//   GPT-J: chunk c holds the pairs (8c+2k, 8c+2k+1), k < 4, at frequency
//          4c + k: no data leaves the lane.
//   NeoX:  chunk c < R/16 holds the first members u = 8c + k of the pairs
//          (u, u + R/2), whose second members sit in chunk c + R/16, i.e.
//          lane l + R/16; a lane with R/16 <= c < R/8 holds second members
//          and finds its partners in lane l - R/16.  The partner chunk is
//          fetched with ds_bpermute, one dword at a time, by every lane of
//          the wave at once.  Frequency of element k: 8*(c mod R/16) + k.
//
// Exactness.  An fp16 significand has 11 bits and an fp32 one 24, so each
// product is exact in binary64; fma(x_u, c, -(x_v*s)) therefore rounds the
// exact value x_u*c - x_v*s once to binary64.  The narrowing to binary16 goes
// through binary32 with round-to-odd (truncate, then force the last bit to 1
// when inexact), which makes the final round-to-nearest-even binary32 ->
// binary16 conversion equal to a direct binary64 -> binary16 rounding,
// because binary32 carries more than two extra bits (Boldo & Melquiond,
// "Emulation of FMA and correctly rounded sums: proved algorithms using
// rounding to odd", IEEE Trans. Computers 2008).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkv {

enum Style : int { kNeox = 0, kGptj = 1 };

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ uint32_t f2h_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// binary64 -> binary16, round to nearest even, via round-to-odd binary32.
__device__ __forceinline__ uint32_t narrow_exact(double y) {
  float f = (float)y;                      // round to nearest even
  double back = (double)f;                 // exact
  uint32_t bits = __builtin_bit_cast(uint32_t, f);
  if (back != y) {                         // inexact (NaN stays NaN)
    if (__builtin_fabs(back) > __builtin_fabs(y)) bits -= 1u;   // toward zero
    bits |= 1u;                            // odd
  }
  return f2h_bits(__builtin_bit_cast(float, bits));
}

// x*c + sign*(p*s), with sign = -1 (first pair member) or +1 (second).
//
// kExact: binary64 products and sum (exact up to the one binary64 rounding),
// narrowed with round-to-odd -- bit-identical to a correctly rounded result.
// Otherwise binary32, compensated: ps = RN(p*s) and its exact rounding error
// e = fma(p, s, -ps) are formed first, then y = RN(RN(x*c - ps) - e) (the
// first by one fma).  The two remaining roundings put y within about 2^-23
// relative of the exact value, with no loss under cancellation, so the fp16
// result is the correctly rounded one or its neighbour.
template <bool kExact>
__device__ __forceinline__ uint32_t rot1(uint32_t x_bits, uint32_t p_bits, float c, float s,
                                         bool first) {
  if constexpr (kExact) {
    double x = (double)h2f(x_bits), pv = (double)h2f(p_bits);
    double ps = pv * (double)s;               // exact
    return narrow_exact(__builtin_fma(x, (double)c, first ? -ps : ps));
  } else {
    const float x = h2f(x_bits), pv = h2f(p_bits);
    const float sv = first ? -s : s;
    const float ps = pv * sv;
    const float e = __builtin_fmaf(pv, sv, -ps);   // exact: pv*sv - ps
    return f2h_bits(__builtin_fmaf(x, c, ps) + e);
  }
}

__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }
__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// NeoX: the lane's 8 elements x with the partner chunk p; c[k], s[k] are
// the cos/sin of element k's frequency; `first` for chunks c < R/16.
template <bool kExact>
__device__ __forceinline__ uint4 rotate_neox(uint4 x, uint4 p, const float (&c)[8],
                                             const float (&s)[8], bool first) {
  uint32_t xa[4] = {x.x, x.y, x.z, x.w};
  uint32_t pa[4] = {p.x, p.y, p.z, p.w};
  uint32_t y[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t y0 = rot1<kExact>(lo16(xa[w]), lo16(pa[w]), c[2 * w], s[2 * w], first);
    uint32_t y1 = rot1<kExact>(hi16(xa[w]), hi16(pa[w]), c[2 * w + 1], s[2 * w + 1], first);
    y[w] = pack2(y0, y1);
  }
  return make_uint4(y[0], y[1], y[2], y[3]);
}

// GPT-J: dword w of the chunk holds the pair (lo, hi) at frequency w.
template <bool kExact>
__device__ __forceinline__ uint4 rotate_gptj(uint4 x, const float (&c)[8], const float (&s)[8]) {
  uint32_t xa[4] = {x.x, x.y, x.z, x.w};
  uint32_t y[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t y0 = rot1<kExact>(lo16(xa[w]), hi16(xa[w]), c[w], s[w], true);
    uint32_t y1 = rot1<kExact>(hi16(xa[w]), lo16(xa[w]), c[w], s[w], false);
    y[w] = pack2(y0, y1);
  }
  return make_uint4(y[0], y[1], y[2], y[3]);
}

// Fetch lane `src_lane`'s chunk (all lanes of the wave must execute this).
__device__ __forceinline__ uint4 lane_fetch(uint4 v, int src_lane) {
  const int addr = src_lane << 2;
  return make_uint4((uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v.x),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v.y),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v.z),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v.w));
}

// Role of a lane's chunk index c in a row of D elements with rotary dim R.
struct ChunkRole {
  bool rotary;     // c < R/8
  bool first;      // NeoX: holds first pair members (c < R/16)
  int partner;     // NeoX: lane offset of the partner chunk (+R/16 or -R/16), else 0
  int freq0;       // index of the first frequency this lane uses
};

template <int kStyle>
__device__ __forceinline__ ChunkRole chunk_role(int c, int R) {
  ChunkRole r;
  const int half_chunks = R >> 4;   // R/16
  r.rotary = c < 2 * half_chunks;
  r.first = c < half_chunks;
  if constexpr (kStyle == kNeox) {
    r.partner = r.rotary ? (r.first ? half_chunks : -half_chunks) : 0;
    r.freq0 = 8 * (r.first ? c : c - half_chunks);
  } else {
    r.partner = 0;
    r.freq0 = 4 * c;
  }
  return r;
}

// The cos/sin values a rotary lane needs from one table row [cos | sin]:
// NeoX: 8 frequencies from freq0; GPT-J: 4 frequencies from freq0 (c[0..3]).
template <int kStyle>
__device__ __forceinline__ void load_cos_sin(const float* row, int freq0, int R, float (&c)[8],
                                             float (&s)[8]) {
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

// Rotate (or pass through) one chunk.  Must be called by every lane of the
// wave with the same control flow (the NeoX partner fetch is a wave-wide
// permute); lanes whose row is not rotated simply keep their value.
template <int kStyle, bool kExact>
__device__ __forceinline__ uint4 rotate_chunk(uint4 x, int lane, const ChunkRole& role,
                                              bool rotate_row, const float (&c)[8],
                                              const float (&s)[8]) {
  if constexpr (kStyle == kNeox) {
    const uint4 p = lane_fetch(x, lane + role.partner);
    if (rotate_row && role.rotary) return rotate_neox<kExact>(x, p, c, s, role.first);
    return x;
  } else {
    if (rotate_row && role.rotary) return rotate_gptj<kExact>(x, c, s);
    return x;
  }
}

}  // namespace rkv
