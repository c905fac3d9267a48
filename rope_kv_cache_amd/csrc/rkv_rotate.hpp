// Device-side rotate unit for gfx950: fp16 pair rotation on 16-byte chunks.
//
// Rotation (sglang rope_cache.py, _unit_rope with _get_neox_rotated_x /
// _get_gptj_rotated_x; cos/sin halves as in _load_cos_sin):
//   y_u = x_u*c - x_v*s,   y_v = x_v*c + x_u*s
// NeoX pairs element i with i + R/2, GPT-J pairs 2i with 2i+1; frequency i
// drives pair i.
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

// One pair: (a, b) -> (a*c - b*s, b*c + a*s), fp16 bits in and out.
template <bool kExact>
__device__ __forceinline__ void rotate_pair(uint32_t a_bits, uint32_t b_bits, float c, float s,
                                            uint32_t& ya, uint32_t& yb) {
  if constexpr (kExact) {
    double a = (double)h2f(a_bits), b = (double)h2f(b_bits);
    double cd = (double)c, sd = (double)s;
    ya = narrow_exact(__builtin_fma(a, cd, -(b * sd)));
    yb = narrow_exact(__builtin_fma(b, cd, a * sd));
  } else {
    float a = h2f(a_bits), b = h2f(b_bits);
    ya = f2h_bits(__builtin_fmaf(a, c, -(b * s)));
    yb = f2h_bits(__builtin_fmaf(b, c, a * s));
  }
}

__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }
__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// Rotate the pairs held by one lane.
//
// A lane owns two 8-element chunks of a head row: A at element offset o and
// B at o + R/2, with o = 8j for rotary lane j.
//   NeoX: element k of A pairs with element k of B, frequency 8j + k;
//         c[k], s[k] hold that frequency's cos and sin.
//   GPT-J: elements (2k, 2k+1) of A pair with each other at frequency
//         4j + k (c[k], s[k]), and those of B at frequency 4j + R/4 + k
//         (c[4+k], s[4+k]).
template <int kStyle, bool kExact>
__device__ __forceinline__ void rotate_chunks(uint4& A, uint4& B, const float (&c)[8],
                                              const float (&s)[8]) {
  uint32_t a[4] = {A.x, A.y, A.z, A.w};
  uint32_t b[4] = {B.x, B.y, B.z, B.w};
  if constexpr (kStyle == kNeox) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t ya0, yb0, ya1, yb1;
      rotate_pair<kExact>(lo16(a[w]), lo16(b[w]), c[2 * w], s[2 * w], ya0, yb0);
      rotate_pair<kExact>(hi16(a[w]), hi16(b[w]), c[2 * w + 1], s[2 * w + 1], ya1, yb1);
      a[w] = pack2(ya0, ya1);
      b[w] = pack2(yb0, yb1);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t y0, y1;
      rotate_pair<kExact>(lo16(a[w]), hi16(a[w]), c[w], s[w], y0, y1);
      a[w] = pack2(y0, y1);
      rotate_pair<kExact>(lo16(b[w]), hi16(b[w]), c[4 + w], s[4 + w], y0, y1);
      b[w] = pack2(y0, y1);
    }
  }
  A = make_uint4(a[0], a[1], a[2], a[3]);
  B = make_uint4(b[0], b[1], b[2], b[3]);
}

// Chunk placement of lane j (0 <= j < D/16) inside a head row of D elements,
// and whether it rotates.  Rotary lanes j < R/16 own chunks 8j and 8j + R/2;
// the remaining lanes own the passthrough dims [R, D), split the same way.
struct LaneChunks {
  int off_a;
  int off_b;
  bool rotary;
};

template <int D>
__device__ __forceinline__ LaneChunks lane_chunks(int j, int R) {
  LaneChunks lc;
  int rot_lanes = R >> 4;
  if (j < rot_lanes) {
    lc.rotary = true;
    lc.off_a = 8 * j;
    lc.off_b = 8 * j + (R >> 1);
  } else {
    int p = j - rot_lanes;
    lc.rotary = false;
    lc.off_a = R + 8 * p;
    lc.off_b = R + 8 * p + ((D - R) >> 1);
  }
  return lc;
}

// The cos/sin values a rotary lane needs from one table row [cos | sin].
template <int kStyle>
__device__ __forceinline__ void load_cos_sin(const float* row, int j, int R, float (&c)[8],
                                             float (&s)[8]) {
  const int half = R >> 1;
  float4 c0, c1, s0, s1;
  if constexpr (kStyle == kNeox) {
    c0 = *reinterpret_cast<const float4*>(row + 8 * j);
    c1 = *reinterpret_cast<const float4*>(row + 8 * j + 4);
    s0 = *reinterpret_cast<const float4*>(row + half + 8 * j);
    s1 = *reinterpret_cast<const float4*>(row + half + 8 * j + 4);
  } else {
    c0 = *reinterpret_cast<const float4*>(row + 4 * j);
    c1 = *reinterpret_cast<const float4*>(row + 4 * j + (R >> 2));
    s0 = *reinterpret_cast<const float4*>(row + half + 4 * j);
    s1 = *reinterpret_cast<const float4*>(row + half + 4 * j + (R >> 2));
  }
  c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
  c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
  s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
  s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
}

}  // namespace rkv
