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
//
// Q/K RMS norm.  A normalised row is n_d = x_d * r * w_d with
// r = 1/sqrt(mean(x^2) + eps); the rotation then acts on n.  The row's sum
// of squares is reduced over its D/8 lanes by a butterfly of lane moves.
// Exact mode: every fp16 square is a multiple of 2^-48 below 2^32; split
// into a multiple of 2^-13 and a remainder, both partial sums are exact in
// binary64 in any order, so their sum is the correctly rounded
// sum of squares (what the definition rounds once); sqrt and the division
// are correctly rounded binary64 operations.  The rotation of normalised
// values, no longer exact products, rounds each product and the sum
// separately (no contraction).  Default mode: binary32 sum, v_rsq_f32, and
// the compensated rotation on the binary32 normalised values.  The row
// reduction uses DPP lane moves inside 16-lane rows.
//
// fp8 cache.  The E4M3 cache value is the unrounded rotation (binary32 in
// the default mode, binary64 exact) times the reciprocal scale, clamped to
// +-448 and converted by the hardware (v_cvt_pk_fp8_f32, OCP E4M3 on gfx950,
// round to nearest even).  In the exact mode the binary64 product is first
// narrowed to binary32 with round-to-odd, which again makes the final
// rounding a correct one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rkv {

enum Style : int { kNeox = 0, kGptj = 1 };

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ uint32_t f2h_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// binary64 -> binary32 rounded to odd: truncate toward zero, then set the
// last bit when the result is inexact (NaN stays NaN).
__device__ __forceinline__ float narrow_odd(double y) {
  float f = (float)y;                      // round to nearest even
  double back = (double)f;                 // exact
  uint32_t bits = __builtin_bit_cast(uint32_t, f);
  if (back != y) {
    if (__builtin_fabs(back) > __builtin_fabs(y)) bits -= 1u;   // toward zero
    bits |= 1u;                            // odd
  }
  return __builtin_bit_cast(float, bits);
}

// The unrounded rotated value: binary64 in the exact mode, else binary32.
template <bool kExact>
using WideT = typename std::conditional<kExact, double, float>::type;

template <bool kExact>
__device__ __forceinline__ WideT<kExact> widen(uint32_t bits16) {
  return (WideT<kExact>)h2f(bits16);       // exact either way
}

// Two binary32 values rounded to fp16 (nearest even) and packed, `lo` in
// the low half: one v_cvt_pk_f16_f32, where two conversions and a pack took
// two instructions; bit for bit the two scalar conversions (an exhaustive
// comparison over all 2^32 patterns, ceilings/ f16_pair_check_kernel).
__device__ __forceinline__ uint32_t f2h_pair(float lo, float hi) {
  typedef float F2 __attribute__((ext_vector_type(2)));
  typedef _Float16 H2 __attribute__((ext_vector_type(2)));
  const F2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, H2));
}

// Two unrounded values rounded to fp16 and packed: binary64 values are
// narrowed to binary32 with round-to-odd first, so the rounding to fp16 is
// again the direct one (correctly rounded in the exact mode).
template <bool kExact>
__device__ __forceinline__ uint32_t narrow_pair(WideT<kExact> lo, WideT<kExact> hi) {
  if constexpr (kExact) return f2h_pair(narrow_odd(lo), narrow_odd(hi));
  else return f2h_pair(lo, hi);
}

// -0.0, hidden from the optimiser: fma(a, b, -0) equals RN(a*b) for every
// a, b (signed zeros included), and with `a` widened from fp16 the compiler
// emits it as one v_fma_mix_f32, which reads the fp16 operand directly,
// where a product would take a conversion and a multiply.
__device__ __forceinline__ float opaque_neg_zero() {
  float z = -0.0f;
  asm("" : "+v"(z));
  return z;
}

// x*c + sign*(p*s), with sign = -1 (first pair member) or +1 (second),
// before the rounding to fp16.
//
// kExact: binary64 products and sum (exact up to the one binary64 rounding).
// Otherwise binary32, compensated: ps = RN(p*s) and its exact rounding error
// e = fma(p, s, -ps) are formed first, then y = RN(RN(x*c - ps) - e) (the
// first by one fma).  The two remaining roundings put y within about 2^-23
// relative of the exact value, with no loss under cancellation, so the fp16
// result is the correctly rounded one or its neighbour.
template <bool kExact>
__device__ __forceinline__ WideT<kExact> rot1_wide(uint32_t x_bits, uint32_t p_bits, float c,
                                                   float s, bool first, float nz) {
  if constexpr (kExact) {
    double x = (double)h2f(x_bits), pv = (double)h2f(p_bits);
    double ps = pv * (double)s;               // exact
    return __builtin_fma(x, (double)c, first ? -ps : ps);
  } else {
    const float x = h2f(x_bits), pv = h2f(p_bits);
    const float sv = first ? -s : s;
    const float ps = __builtin_fmaf(pv, sv, nz);   // RN(pv*sv), nz = -0
    const float e = __builtin_fmaf(pv, sv, -ps);   // exact: pv*sv - ps
    return __builtin_fmaf(x, c, ps) + e;
  }
}

__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }

// NeoX: the lane's 8 elements x with the partner chunk p; c[k], s[k] are
// the cos/sin of element k's frequency; `first` for chunks c < R/16.  Each
// rotated element is rounded to fp16: correctly rounded with kExact, else
// the correctly rounded value or its neighbour.
template <bool kExact>
__device__ __forceinline__ uint4 rotate_neox(uint4 x, uint4 p, const float (&c)[8],
                                             const float (&s)[8], bool first, float nz) {
  uint32_t xa[4] = {x.x, x.y, x.z, x.w};
  uint32_t pa[4] = {p.x, p.y, p.z, p.w};
  uint32_t y[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    y[w] = narrow_pair<kExact>(
        rot1_wide<kExact>(lo16(xa[w]), lo16(pa[w]), c[2 * w], s[2 * w], first, nz),
        rot1_wide<kExact>(hi16(xa[w]), hi16(pa[w]), c[2 * w + 1], s[2 * w + 1], first, nz));
  }
  return make_uint4(y[0], y[1], y[2], y[3]);
}

// GPT-J: dword w of the chunk holds the pair (lo, hi) at frequency w.
template <bool kExact>
__device__ __forceinline__ uint4 rotate_gptj(uint4 x, const float (&c)[8], const float (&s)[8],
                                             float nz) {
  uint32_t xa[4] = {x.x, x.y, x.z, x.w};
  uint32_t y[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    y[w] = narrow_pair<kExact>(rot1_wide<kExact>(lo16(xa[w]), hi16(xa[w]), c[w], s[w], true, nz),
                               rot1_wide<kExact>(hi16(xa[w]), lo16(xa[w]), c[w], s[w], false, nz));
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
  float neg_zero;  // -0.0, opaque to the optimiser (opaque_neg_zero), made once per wave
};

template <int kStyle>
__device__ __forceinline__ ChunkRole chunk_role(int c, int R) {
  ChunkRole r;
  const int half_chunks = R >> 4;   // R/16
  r.rotary = c < 2 * half_chunks;
  r.first = c < half_chunks;
  r.neg_zero = opaque_neg_zero();
  if constexpr (kStyle == kNeox) {
    r.partner = r.rotary ? (r.first ? half_chunks : -half_chunks) : 0;
    r.freq0 = 8 * (r.first ? c : c - half_chunks);
  } else {
    r.partner = 0;
    r.freq0 = 4 * c;
  }
  return r;
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
    if (rotate_row && role.rotary)
      return rotate_neox<kExact>(x, p, c, s, role.first, role.neg_zero);
    return x;
  } else {
    if (rotate_row && role.rotary) return rotate_gptj<kExact>(x, c, s, role.neg_zero);
    return x;
  }
}

// The same rotation as rotate_chunk, kept unrounded: w[k] is element k of
// the chunk before the rounding to fp16 (its fp16 value widened when the
// chunk is not rotated).  Returns whether the chunk was rotated.  Must be
// called by every lane of the wave with the same control flow.
template <int kStyle, bool kExact>
__device__ __forceinline__ bool rotate_chunk_wide(uint4 x, int lane, const ChunkRole& role,
                                                  bool rotate_row, const float (&c)[8],
                                                  const float (&s)[8], WideT<kExact> (&w)[8]) {
  const uint32_t xa[4] = {x.x, x.y, x.z, x.w};
  const bool rot = rotate_row && role.rotary;
  if constexpr (kStyle == kNeox) {
    const uint4 p = lane_fetch(x, lane + role.partner);
    const uint32_t pa[4] = {p.x, p.y, p.z, p.w};
    if (rot) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        w[2 * k] = rot1_wide<kExact>(lo16(xa[k]), lo16(pa[k]), c[2 * k], s[2 * k], role.first,
                                     role.neg_zero);
        w[2 * k + 1] = rot1_wide<kExact>(hi16(xa[k]), hi16(pa[k]), c[2 * k + 1], s[2 * k + 1],
                                         role.first, role.neg_zero);
      }
      return true;
    }
  } else {
    if (rot) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        w[2 * k] = rot1_wide<kExact>(lo16(xa[k]), hi16(xa[k]), c[k], s[k], true, role.neg_zero);
        w[2 * k + 1] =
            rot1_wide<kExact>(hi16(xa[k]), lo16(xa[k]), c[k], s[k], false, role.neg_zero);
      }
      return true;
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    w[2 * k] = widen<kExact>(lo16(xa[k]));
    w[2 * k + 1] = widen<kExact>(hi16(xa[k]));
  }
  return false;
}

// fp16 chunk from unrounded values; an unrotated chunk keeps its bits.
template <bool kExact>
__device__ __forceinline__ uint4 narrow_chunk(const WideT<kExact> (&w)[8], uint4 x, bool rot) {
  if (!rot) return x;
  return make_uint4(narrow_pair<kExact>(w[0], w[1]), narrow_pair<kExact>(w[2], w[3]),
                    narrow_pair<kExact>(w[4], w[5]), narrow_pair<kExact>(w[6], w[7]));
}

// Magnitudes beyond the largest E4M3 value (infinities included) saturate
// to it; NaN stays NaN.  IEEE 754-2019 maximum and minimum propagate NaN
// (v_maximum3_f32 / v_minimum3_f32 on gfx950): two instructions where
// comparisons and selects took four.  Checked on MI355X over all 2^32 fp32
// inputs: the E4M3 bytes equal those of the compare-and-select form.
__device__ __forceinline__ float saturate_e4m3(float v) {
  return __builtin_elementwise_minimum(__builtin_elementwise_maximum(v, -448.f), 448.f);
}

// Eight E4M3 bytes (element k in byte k) of the chunk's values times rcp:
// the unrounded values w when `comp`, else the chunk's own fp16 values x
// (which w then holds widened; the default mode reads x directly, so the
// product is one v_fma_mix_f32 with the -0 addend nz).
template <bool kExact>
__device__ __forceinline__ uint2 to_e4m3(const WideT<kExact> (&w)[8], uint4 x, bool comp,
                                         float rcp, float nz) {
  float v[8];
  if constexpr (kExact) {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = saturate_e4m3(narrow_odd(w[k] * (double)rcp));
  } else {
    const uint32_t xa[4] = {x.x, x.y, x.z, x.w};
    if (comp) {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = __builtin_fmaf(w[k], rcp, nz);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        v[k] = __builtin_fmaf(h2f(k & 1 ? hi16(xa[k >> 1]) : lo16(xa[k >> 1])), rcp, nz);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = saturate_e4m3(v[k]);
  }
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// A per-tensor scale that is not given is 1: the kernels then read this
// constant instead, so the scale load needs no branch and both scale loads
// are in flight together.
static __device__ float kUnitScale = 1.0f;   // global memory, never written

// The scale is read through the constant address space: no kernel writes
// it, and a wave-uniform load from there is a scalar load, whose wait does
// not include the row loads issued before it (vector loads complete in
// order; as a vector load the scale, and with it the reciprocal, waited for
// every row of the wave).
typedef __attribute__((address_space(4))) const float ConstFloat;

__device__ __forceinline__ float load_scale(const float* scale) {
  return *(ConstFloat*)(scale ? scale : &kUnitScale);
}

// The fp32 reciprocal of a scale, correctly rounded: the binary64 quotient
// rounded to binary32 (binary64 has more than 2*24+2 bits, so the double
// rounding is innocuous).  For 2^-120 <= |scale| < 2^121 the same value
// comes from binary32 arithmetic: the hardware estimate y (v_rcp_f32), the
// residual e = 1 - scale*y by one fused multiply-add (exact for an estimate
// this close), and y + e*y by another -- one Newton step, equal to the
// rounded binary64 quotient for every such input (an exhaustive comparison,
// ceilings/ reciprocal_check_kernel).  Zeros, subnormals, huge values,
// infinities and NaN take the division.  The scale is wave-uniform, so the
// branch is too.  With the scalar scale loads above, measured on MI355X
// (launches back to back over full copies of their tensors): the continuous
// call into an E4M3 cache 5.58 -> 5.49 us, the large prefill into an E4M3
// cache 205.2 -> 203.6 us, the paged updates unchanged; bytes identical.
// (The compiler turns the binary64 quotient into a correctly rounded
// binary32 division, about ten instructions.)
__device__ __forceinline__ float reciprocal(float scale) {
  const uint32_t biased = (__builtin_bit_cast(uint32_t, scale) >> 23) & 0xffu;
  if (biased >= 127u - 120u && biased <= 127u + 120u) {
    const float y = __builtin_amdgcn_rcpf(scale);
    return __builtin_fmaf(__builtin_fmaf(-scale, y, 1.0f), y, y);
  }
  return (float)(1.0 / (double)scale);
}

// Both reciprocal scales, computed where this is called.  The first empty
// volatile asm takes both raw scales, so the two scalar loads are issued
// together and share one wait; the second keeps the compiler from sinking
// the loads and that wait into the branch that first uses the reciprocals.
// Callers place this after their vector loads are issued, so the wait
// overlaps those loads' latency.
__device__ __forceinline__ void load_reciprocal_scales(const float* k_scale, const float* v_scale,
                                                       float& k_rcp, float& v_rcp) {
  const float ks = load_scale(k_scale), vs = load_scale(v_scale);
  asm volatile("" ::"s"(ks), "s"(vs));
  k_rcp = reciprocal(ks);
  v_rcp = reciprocal(vs);
  asm volatile("" : "+v"(k_rcp), "+v"(v_rcp));
}

// ---------------------------------------------------------------- norm --

// The value of lane l ^ kXor (within each 32 lanes), by ds_swizzle in
// bit-mask mode.
template <int kXor>
__device__ __forceinline__ float swizzle_xor(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x1F | (kXor << 10)));
}

template <int kXor>
__device__ __forceinline__ double swizzle_xor(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)b, 0x1F | (kXor << 10));
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)(b >> 32), 0x1F | (kXor << 10));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// DPP lane moves inside a row of 16 lanes (GFX9 encodings): quad_perm
// [1,0,3,2] and [2,3,0,1], row_half_mirror (lane i <- 7-i within each 8),
// row_mirror (lane i <- 15-i).
constexpr int kDppQuadSwap1 = 0xB1;
constexpr int kDppQuadSwap2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int kCtrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

template <int kCtrl>
__device__ __forceinline__ double dpp_move(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, kCtrl, 0xF, 0xF,
                                                            false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), kCtrl,
                                                            0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over groups of kLanes lanes by DPP moves inside 16-lane rows (no LDS
// round trip): each step adds the value of a lane in the other half of the
// current group, so after log2(kLanes) steps every lane holds the group's
// total, the same value in every lane (each step adds the same two operands
// in both lanes, and addition is commutative).  Groups of 32 take a last
// ds_swizzle step across the two 16-lane rows.  It measured 2% faster than
// a butterfly of ds_swizzle steps.
template <int kLanes, typename T>
__device__ __forceinline__ T row_sum_dpp(T v) {
  if constexpr (kLanes > 1) v += dpp_move<kDppQuadSwap1>(v);
  if constexpr (kLanes > 2) v += dpp_move<kDppQuadSwap2>(v);
  if constexpr (kLanes > 4) v += dpp_move<kDppHalfMirror>(v);
  if constexpr (kLanes > 8) v += dpp_move<kDppMirror>(v);
  if constexpr (kLanes > 16) v += swizzle_xor<16>(v);
  return v;
}

// Sum over the kLanes consecutive, aligned lanes of one row (a power of two
// <= 32); every lane of the row gets the same total.  Called by every lane.
template <int kLanes, typename T>
__device__ __forceinline__ T row_sum(T v) {
  return row_sum_dpp<kLanes>(v);
}

// 1 / sqrt(mean of squares + eps) of the row whose chunk this lane holds.
// Called by every lane (the reduction exchanges data across lanes).
template <int D, bool kExact>
__device__ __forceinline__ WideT<kExact> row_rms_reciprocal(uint4 x, float eps) {
  const uint32_t xa[4] = {x.x, x.y, x.z, x.w};
  if constexpr (kExact) {
    double hi = 0.0, lo = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const double v = (double)h2f(k & 1 ? hi16(xa[k >> 1]) : lo16(xa[k >> 1]));
      const double q = v * v;                                      // exact
      const double h = __builtin_trunc(q * 8192.0) * (1.0 / 8192.0);   // exact
      hi += h;
      lo += (h == q) ? 0.0 : q - h;                                // exact; keeps inf / NaN
    }
    hi = row_sum<D / 8>(hi);
    lo = row_sum<D / 8>(lo);
    const double ms = (hi + lo) * (1.0 / D);                       // one rounding
    return 1.0 / __builtin_sqrt(ms + (double)eps);
  } else {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float v = h2f(k & 1 ? hi16(xa[k >> 1]) : lo16(xa[k >> 1]));
      ss = __builtin_fmaf(v, v, ss);
    }
    ss = row_sum<D / 8>(ss);
    return __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
  }
}

// x*c + sign*(p*s) for values that are not fp16 (normalised rows).  Exact
// mode: each product and the sum rounded once in binary64, no contraction.
// Default mode: one fused multiply-add over the rounded product p*s.  The
// normalised inputs already carry two binary32 roundings each, so the
// compensation term of rot1_wide (exact for fp16 inputs) would not tighten
// the result; without it the large prefill with Q/K norm runs about 3%
// faster (measured on MI355X: 248 -> 240 us median).  Where |result| >=
// 2^-6 the error stays far below half an fp16 ulp, so the fp16 result is
// the correctly rounded one or its neighbour.
template <bool kExact>
__device__ __forceinline__ WideT<kExact> rot1_general(WideT<kExact> x, WideT<kExact> p, float c,
                                                      float s, bool first) {
  if constexpr (kExact) {
#pragma clang fp contract(off)
    const double a = x * (double)c;
    const double b = p * (double)s;
    return first ? a - b : a + b;
  } else {
    return __builtin_fmaf(x, c, p * (first ? -s : s));
  }
}

// The weights a lane needs: its own 8 dims and, for a NeoX rotary lane in
// exact mode, its partner chunk's 8 dims (the default mode fetches the
// partner's normalised values from the partner lane instead).
template <int kStyle, bool kExact>
__device__ __forceinline__ void load_norm_weights(const float* w, int c, const ChunkRole& role,
                                                  float (&ws)[8], float (&wp)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(w + 8 * c);
  const float4 b = *reinterpret_cast<const float4*>(w + 8 * c + 4);
  ws[0] = a.x; ws[1] = a.y; ws[2] = a.z; ws[3] = a.w;
  ws[4] = b.x; ws[5] = b.y; ws[6] = b.z; ws[7] = b.w;
  if constexpr (kStyle == kNeox && kExact) {
    if (role.rotary) {
      const int pc = c + role.partner;
      const float4 e = *reinterpret_cast<const float4*>(w + 8 * pc);
      const float4 f = *reinterpret_cast<const float4*>(w + 8 * pc + 4);
      wp[0] = e.x; wp[1] = e.y; wp[2] = e.z; wp[3] = e.w;
      wp[4] = f.x; wp[5] = f.y; wp[6] = f.z; wp[7] = f.w;
    }
  }
}

// The chunk's unrounded output when its row may be normalised: n = x*r*w
// (normed rows; else n = x), rotated when rotate_row and the chunk is
// rotary.  Returns whether the output must be rounded from w (rotated or
// normalised) rather than copied from x.  Called by every lane.
//
// NeoX partners: in the default mode the partner lane's own n values are
// fetched (8 binary32 values by ds_bpermute).  Every lane of a row holds
// the same 1/rms and the partner lane applies the same formula with its own
// weights, so these are bit for bit the values this lane would compute, and
// no partner weights are needed.  Exact mode fetches the partner's fp16 bits
// and normalises them here with the partner's weights (wp).
template <int kStyle, bool kExact>
__device__ __forceinline__ bool rotate_chunk_norm(uint4 x, int lane, const ChunkRole& role,
                                                  bool rotate_row, bool normed, WideT<kExact> r,
                                                  const float (&ws)[8], const float (&wp)[8],
                                                  const float (&c)[8], const float (&s)[8],
                                                  WideT<kExact> (&w)[8]) {
  using T = WideT<kExact>;
  const uint32_t xa[4] = {x.x, x.y, x.z, x.w};
  const bool rot = rotate_row && role.rotary;
  T n[8];
  if (normed) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const T v = widen<kExact>(k & 1 ? hi16(xa[k >> 1]) : lo16(xa[k >> 1]));
      n[k] = (v * r) * (T)ws[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) n[k] = widen<kExact>(k & 1 ? hi16(xa[k >> 1]) : lo16(xa[k >> 1]));
  }
  if constexpr (kStyle == kNeox) {
    T np[8];
    if constexpr (kExact) {
      const uint4 pch = lane_fetch(x, lane + role.partner);
      const uint32_t pa[4] = {pch.x, pch.y, pch.z, pch.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const T v = widen<kExact>(k & 1 ? hi16(pa[k >> 1]) : lo16(pa[k >> 1]));
        np[k] = normed ? (v * r) * (T)wp[k] : v;
      }
    } else {
      const uint4 lo = lane_fetch(make_uint4(__builtin_bit_cast(uint32_t, n[0]),
                                             __builtin_bit_cast(uint32_t, n[1]),
                                             __builtin_bit_cast(uint32_t, n[2]),
                                             __builtin_bit_cast(uint32_t, n[3])),
                                  lane + role.partner);
      const uint4 hi = lane_fetch(make_uint4(__builtin_bit_cast(uint32_t, n[4]),
                                             __builtin_bit_cast(uint32_t, n[5]),
                                             __builtin_bit_cast(uint32_t, n[6]),
                                             __builtin_bit_cast(uint32_t, n[7])),
                                  lane + role.partner);
      const uint32_t pa[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) np[k] = __builtin_bit_cast(float, pa[k]);
    }
    if (rot) {
#pragma unroll
      for (int k = 0; k < 8; ++k) w[k] = rot1_general<kExact>(n[k], np[k], c[k], s[k], role.first);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) w[k] = n[k];
    }
  } else {
    if (rot) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        w[2 * k] = rot1_general<kExact>(n[2 * k], n[2 * k + 1], c[k], s[k], true);
        w[2 * k + 1] = rot1_general<kExact>(n[2 * k + 1], n[2 * k], c[k], s[k], false);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) w[k] = n[k];
    }
  }
  return rot || normed;
}

}  // namespace rkv
