// C ABI of the fused RoPE + KV-cache write library (include/rope_kv_cache.h).
//
// Host side only: argument validation, launch-shape selection and the
// launch itself.  Nothing here reads device memory or synchronises.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/rope_kv_cache.h"
#include "rkv_launch.hpp"

namespace {

thread_local char g_err[512] = "";
thread_local int32_t g_last_groups = 0;   // row groups per wave of this thread's last launch
thread_local int32_t g_last_loads = 0;    // paged load plan of the last launch (1 early, 2 late)
thread_local int32_t g_force_groups = 0;  // rkv_set_launch_overrides: 0 or 1, 2, 4
thread_local int32_t g_force_loads = 0;   // rkv_set_launch_overrides: 0, 1 early, 2 late

rkv_status fail(rkv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() {
  g_err[0] = '\0';
  g_last_groups = 0;
  g_last_loads = 0;
}

// Launch shape.  A wave handles G row groups (512/D rows each) of one work
// item (a token of calls 1-3, a delta row of call 4); its loads for all G
// groups are in flight together and it fetches its cos/sin values (and norm
// weights) once for all of them.  The choices below come from sweeps of
// every forced G (rkv_set_launch_overrides) on MI355X, three interleaved
// rounds each, large launches back to back over four copies of the written
// tensors, small ones back to back over full copies of all their tensors
// (medians, us):
//  - large prefill (1.43 GB, call 1): two row groups per wave for every
//    flavour (GPT-J 217.3, one 222.1, four 236.2; E4M3 203.7 against 212.0 /
//    223.5; Q/K norm 218.7 against 225.7 / 234.0; exact NeoX 223.5 against
//    234.3 at four, exact E4M3 206.1 against 214.9); large launches of calls
//    2 and 3 in the exact mode of the NeoX layout or of the E4M3 cache, whose
//    binary64 arithmetic per byte is highest, take four (they do not raise
//    their wave priority; call 1 took four too before it did);
//  - small launches are latency-bound: every wave is resident at once
//    (256 CUs x 4 SIMDs x 8 waves), so a small launch doubles G while its
//    waves would not all fit; the continuous and tree calls run alike at two
//    and four (5.3-5.4), the Q/K-norm kernel starts from four (5.9 against
//    6.0 at two);
//  - the paged update's small fp16 launches take four, one wave per delta
//    row, which then resolves its index chain once (NeoX 6.5 against 8.2 at
//    two, GPT-J 7.2 against 7.8, exact 7.3 against 8.3, fused gather 6.5
//    against 7.5); small E4M3 ones take two with late loads (6.6, against 7.3
//    at four); large ones take two in every flavour (65,536 rows, NeoX: 75.7
//    against 83.9 at one and 84.8 at four; GPT-J 78.9 against 83.6 / 82.9;
//    E4M3 pools 60.4 against 63.1 at four, GPT-J 62.5 against 63.7).
constexpr long long kResidentWaves = 8192;
constexpr long long kStreamingGroups = 65536;

int elem_size(int32_t dtype) {
  return dtype == RKV_F8E4M3 ? 1 : dtype == RKV_F16 ? 2 : 4;
}

struct Span {
  const char* name;
  uintptr_t lo, hi;
};

bool overlaps(const Span& a, const Span& b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

// Checked product of non-negative extents.
bool mul_ok(long long a, long long b, long long* out) {
  return !__builtin_mul_overflow(a, b, out);
}

rkv_status check_tensor(const rkv_tensor* t, const char* name, int32_t dtype, int32_t ndim,
                        Span* span) {
  if (!t) return fail(RKV_ERR_NULL, "%s: null descriptor", name);
  if (t->dtype != dtype)
    return fail(RKV_ERR_DTYPE, "%s: dtype %d, expected %d", name, t->dtype, dtype);
  if (t->ndim != ndim)
    return fail(RKV_ERR_SHAPE, "%s: rank %d, expected %d", name, t->ndim, ndim);
  long long n = 1;
  for (int d = 0; d < ndim; ++d) {
    if (t->shape[d] < 0 || t->shape[d] > INT32_MAX)
      return fail(RKV_ERR_SHAPE, "%s: extent %d is %lld", name, d, (long long)t->shape[d]);
    if (!mul_ok(n, t->shape[d], &n)) return fail(RKV_ERR_SHAPE, "%s: size overflows", name);
  }
  long long bytes;
  if (!mul_ok(n, elem_size(dtype), &bytes)) return fail(RKV_ERR_SHAPE, "%s: size overflows", name);
  if (n > 0 && !t->data) return fail(RKV_ERR_NULL, "%s: null data pointer", name);
  if (((uintptr_t)t->data & 15u) != 0)
    return fail(RKV_ERR_ALIGNMENT, "%s: data pointer is not 16-byte aligned", name);
  span->name = name;
  span->lo = (uintptr_t)t->data;
  span->hi = (uintptr_t)t->data + (uintptr_t)bytes;
  return RKV_OK;
}

rkv_status check_no_alias(const Span* outs, int n_out, const Span* ins, int n_in) {
  for (int a = 0; a < n_out; ++a) {
    for (int b = a + 1; b < n_out; ++b)
      if (overlaps(outs[a], outs[b]))
        return fail(RKV_ERR_ALIAS, "%s overlaps %s", outs[a].name, outs[b].name);
    for (int b = 0; b < n_in; ++b)
      if (overlaps(outs[a], ins[b]))
        return fail(RKV_ERR_ALIAS, "%s overlaps %s", outs[a].name, ins[b].name);
  }
  return RKV_OK;
}

rkv_status check_style(int32_t style) {
  const int32_t layout = style & ~RKV_ROUND_EXACT;
  if (layout != RKV_ROPE_NEOX && layout != RKV_ROPE_GPTJ)
    return fail(RKV_ERR_SHAPE,
                "ropeStyle %d: layout must be NeoX (0) or GPT-J (1), optionally | RKV_ROUND_EXACT",
                style);
  return RKV_OK;
}

int32_t layout_of(int32_t style) { return style & ~RKV_ROUND_EXACT; }
bool exact_of(int32_t style) { return (style & RKV_ROUND_EXACT) != 0; }

rkv_status check_dims(int32_t D, int32_t R) {
  if (R < 0 || R > D || (R & 1))
    return fail(RKV_ERR_SHAPE, "rotaryDim %d must be even and within [0, headDim=%d]", R, D);
  if (D != 64 && D != 128 && D != 256)
    return fail(RKV_ERR_UNSUPPORTED, "headDim %d: supported values are 64, 128, 256", D);
  if (R % 16)
    return fail(RKV_ERR_UNSUPPORTED, "rotaryDim %d: must be a multiple of 16", R);
  return RKV_OK;
}

struct Split {
  int32_t groups_per_wave;
  int32_t waves_per_item;
};

// Returns G = 0 when even four row groups per wave leave more waves than one
// dispatch can hold (2^32 - 1 work-items).  g_large / g_small: the row
// groups per wave a kernel starts from in large and small launches (capped
// by the row groups a work item has).
// A row-group override (rkv_set_launch_overrides) replaces the starting
// choice and skips the small-launch doubling.
Split pick_split(long long items, long long groups_per_item, int g_large, int g_small) {
  auto waves = [&](int g) { return items * ((groups_per_item + g - 1) / g); };
  const bool small = items * groups_per_item <= kStreamingGroups;
  const int start = g_force_groups ? g_force_groups : (small ? g_small : g_large);
  int g = 1;
  while (g < start && 2 * g <= groups_per_item) g *= 2;
  if (small && !g_force_groups) {
    while (g < 4 && waves(g) > kResidentWaves) g *= 2;
  }
  while (g < 4 && waves(g) > rkv::kMaxWavesPerLaunch) g *= 2;
  if (waves(g) > rkv::kMaxWavesPerLaunch) return Split{0, 0};
  return Split{g, (int32_t)((groups_per_item + g - 1) / g)};
}

rkv_status launched(hipError_t e) {
  if (e != hipSuccess) {
    g_last_groups = 0;
    g_last_loads = 0;
    return fail(RKV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  }
  return RKV_OK;
}

// The per-tensor fp8 scales: each null (scale 1) or one fp32 value.
rkv_status check_scales(const float* k_scale, const float* v_scale, Span* spans) {
  if (((uintptr_t)k_scale & 3u) || ((uintptr_t)v_scale & 3u))
    return fail(RKV_ERR_ALIGNMENT, "kScale / vScale must be 4-byte aligned");
  spans[0] = Span{"kScale", (uintptr_t)k_scale, (uintptr_t)k_scale + (k_scale ? 4u : 0u)};
  spans[1] = Span{"vScale", (uintptr_t)v_scale, (uintptr_t)v_scale + (v_scale ? 4u : 0u)};
  return RKV_OK;
}

// Q/K norm arguments of calls 1-3 (a null `norm` means no normalisation).
struct NormArgs {
  const float* q_w = nullptr;
  const float* k_w = nullptr;
  float eps = 0.f;
};

// Shared validation of calls 1-3.  `call` selects which descriptors exist;
// `fp8` selects the E4M3 cache (with its scales) over the fp16 one; `norm`
// (non-null) selects the Q/K-norm kernels.
rkv_status contig(int call, const rkv_tensor* cos_sin, const rkv_tensor* end_lens,
                  const rkv_tensor* pos_ids, const rkv_tensor* qkv, rkv_tensor* cache,
                  rkv_tensor* q_out, bool fp8, const float* k_scale, const float* v_scale,
                  const NormArgs* norm, int32_t style, hipStream_t stream) {
  clear_error();
  rkv_status st;
  Span s_cs, s_qkv, s_cache, s_qo = {}, s_end = {}, s_pos = {}, s_sc[2] = {}, s_nw[2] = {};
  if ((st = check_tensor(cos_sin, "cosSinCache", RKV_F32, 3, &s_cs))) return st;
  if ((st = check_tensor(qkv, "qkv", RKV_F16, 4, &s_qkv))) return st;
  if ((st = check_tensor(cache, "kvCache", fp8 ? RKV_F8E4M3 : RKV_F16, 5, &s_cache))) return st;
  if ((st = check_style(style))) return st;
  if (fp8 && (st = check_scales(k_scale, v_scale, s_sc))) return st;
  if (norm) {
    if (!(norm->eps >= 0.f) || norm->eps > 3.4e38f)
      return fail(RKV_ERR_SHAPE, "epsilon %g must be finite and >= 0", (double)norm->eps);
    const long long wbytes = qkv->shape[3] * 4;
    const float* ws[2] = {norm->q_w, norm->k_w};
    const char* names[2] = {"qNormWeight", "kNormWeight"};
    for (int k = 0; k < 2; ++k) {
      if ((uintptr_t)ws[k] & 15u)
        return fail(RKV_ERR_ALIGNMENT, "%s is not 16-byte aligned", names[k]);
      s_nw[k] = Span{names[k], (uintptr_t)ws[k], (uintptr_t)ws[k] + (ws[k] ? wbytes : 0)};
    }
  }

  const long long B = qkv->shape[0], S = qkv->shape[1], H = qkv->shape[2], D = qkv->shape[3];
  const long long Hkv = cache->shape[2], cap = cache->shape[3];
  const long long TB = cos_sin->shape[0], TL = cos_sin->shape[1], R = cos_sin->shape[2];
  if (cache->shape[0] != B || cache->shape[1] != 2 || cache->shape[4] != D)
    return fail(RKV_ERR_SHAPE, "kvCache must be [B=%lld, 2, Hkv, cap, D=%lld]", B, D);
  if (TB != 1 && TB != B)
    return fail(RKV_ERR_SHAPE, "cosSinCache batch %lld must be 1 or B=%lld", TB, B);
  long long Hq;
  if (call == rkv::kCallPacked) {
    Hq = H - 2 * Hkv;
    if (Hq < 0)
      return fail(RKV_ERR_SHAPE, "qkv heads %lld < 2 * Hkv (%lld)", H, Hkv);
  } else {
    if ((st = check_tensor(q_out, "qOut", RKV_F16, 4, &s_qo))) return st;
    if ((st = check_tensor(end_lens, "kvCacheEndLens", RKV_I32, 1, &s_end))) return st;
    Hq = q_out->shape[2];
    if (q_out->shape[0] != B || q_out->shape[1] != S || q_out->shape[3] != D)
      return fail(RKV_ERR_SHAPE, "qOut must be [B, S, Hq, D]");
    if (H != Hq + 2 * Hkv)
      return fail(RKV_ERR_SHAPE, "qkv heads %lld != Hq + 2*Hkv = %lld", H, Hq + 2 * Hkv);
    if (end_lens->shape[0] != B) return fail(RKV_ERR_SHAPE, "kvCacheEndLens must be [B]");
    if (call == rkv::kCallTree) {
      if ((st = check_tensor(pos_ids, "tokenPosIds", RKV_I32, 2, &s_pos))) return st;
      if (pos_ids->shape[0] != B || pos_ids->shape[1] != S)
        return fail(RKV_ERR_SHAPE, "tokenPosIds must be [B, S]");
    }
  }
  if ((st = check_dims((int32_t)D, (int32_t)R))) return st;
  if (call == rkv::kCallPacked && (S > cap || S > TL))
    return fail(RKV_ERR_CAPACITY, "S=%lld exceeds capacity %lld or cos/sin length %lld", S, cap,
                TL);
  {
    Span outs[3], ins[8];
    int no = 0, ni = 0;
    outs[no++] = s_cache;
    if (call == rkv::kCallPacked) {
      outs[no++] = s_qkv;
    } else {
      outs[no++] = s_qo;
      ins[ni++] = s_qkv;
      ins[ni++] = s_end;
      if (call == rkv::kCallTree) ins[ni++] = s_pos;
    }
    ins[ni++] = s_cs;
    if (fp8) {
      ins[ni++] = s_sc[0];
      ins[ni++] = s_sc[1];
    }
    if (norm) {
      ins[ni++] = s_nw[0];
      ins[ni++] = s_nw[1];
    }
    if ((st = check_no_alias(outs, no, ins, ni))) return st;
  }
  const long long tokens = B * S;
  if (tokens > INT32_MAX) return fail(RKV_ERR_UNSUPPORTED, "B*S=%lld exceeds 2^31-1", tokens);
  // a token's head rows (and the padding rows of its last wave) are
  // addressed by 32-bit byte offsets from the token's first row
  if ((H + 64) * D >= (1LL << 31))
    return fail(RKV_ERR_UNSUPPORTED, "%lld heads of %lld values per token is too many", H, D);
  if (tokens == 0 || H == 0) return RKV_OK;

  rkv::ContigParams p{};
  p.cos_sin = (const float*)cos_sin->data;
  p.qkv = (uint16_t*)qkv->data;
  p.cache = fp8 ? nullptr : (uint16_t*)cache->data;
  p.cache8 = fp8 ? (uint8_t*)cache->data : nullptr;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  if (norm) {
    p.q_norm_w = norm->q_w;
    p.k_norm_w = norm->k_w;
    p.eps = norm->eps;
  }
  p.q_out = q_out ? (uint16_t*)q_out->data : nullptr;
  p.end_lens = end_lens ? (const int32_t*)end_lens->data : nullptr;
  p.pos_ids = pos_ids ? (const int32_t*)pos_ids->data : nullptr;
  p.B = (int32_t)B;
  p.S = (int32_t)S;
  p.Hq = (int32_t)Hq;
  p.Hkv = (int32_t)Hkv;
  p.cap = (int32_t)cap;
  // one batch's cache slice; stored through a buffer resource when its byte
  // count fits the resource's 32-bit size
  const unsigned long long slice = 2ull * (unsigned long long)Hkv * (unsigned long long)cap *
                                   (unsigned long long)D * (fp8 ? 1u : 2u);
  p.cache_b_bytes = slice <= 0xFFFFFFFFull ? (uint32_t)slice : 0u;
  p.table_batch = (int32_t)TB;
  p.table_len = (int32_t)TL;
  p.R = (int32_t)R;
  const long long rows_per_group = 512 / D;
  const bool heavy = exact_of(style) || fp8 || norm != nullptr;
  const bool neox = layout_of(style) == RKV_ROPE_NEOX;
  const bool exact = exact_of(style);
  // (call 1, which raises its wave priority while issuing its row loads,
  // runs its exact modes fastest at two as well; calls 2 and 3 keep four)
  const int g_large = (exact && (neox || fp8) && call != rkv::kCallPacked) ? 4 : 2;
  const Split sp = pick_split(tokens, (H + rows_per_group - 1) / rows_per_group, g_large,
                              norm ? 4 : (heavy ? 2 : 1));
  if (!sp.groups_per_wave) return fail(RKV_ERR_UNSUPPORTED, "too many rows for one launch");
  p.groups_per_wave = sp.groups_per_wave;
  p.waves_per_token = sp.waves_per_item;
  // large launches: the XCDs take chunks of 128 workgroups in turn
  const long long groups = tokens * ((H + rows_per_group - 1) / rows_per_group);
  p.xcd_chunk_log2 = groups > kStreamingGroups ? 7 : 0;
  p.total_waves = (int32_t)(tokens * p.waves_per_token);
  p.div_waves = rkv::make_fastdiv((uint32_t)p.waves_per_token);
  p.div_seq = rkv::make_fastdiv((uint32_t)S);
  const int lay = layout_of(style);
  const bool ex = exact_of(style);
  g_last_groups = p.groups_per_wave;
  if (norm)
    return launched(fp8 ? rkv::launch_contig_norm_fp8(p, call, (int)D, lay, ex, stream)
                        : rkv::launch_contig_norm(p, call, (int)D, lay, ex, stream));
  return launched(fp8 ? rkv::launch_contig_fp8(p, call, (int)D, lay, ex, stream)
                      : rkv::launch_contig(p, call, (int)D, lay, ex, stream));
}

// Shared validation and launch of call 4, with the cos/sin rows given per
// delta row (tokenAlignedCosSin) or gathered from a rope table, into an
// fp16 pool or (fp8) an E4M3 pool with its scales.
rkv_status paged(const uint16_t* kDelta, const uint16_t* vDelta, void* kvCache, bool fp8,
                 const float* k_scale, const float* v_scale,
                 const float* tokenAlignedCosSin, const float* rope, int32_t ropeStates,
                 int32_t ropeRows, const int32_t* stateIndices, const int32_t* deltaPositions,
                 const int32_t* deltaTokenToSequence, const int32_t* pageTable,
                 int32_t numDeltaTokens, int32_t batchSize, int32_t numKVHeads, int32_t headDim,
                 int32_t rotaryDim, int32_t numPages, int32_t maxPagesPerSeq, int32_t ropeStyle,
                 bool gather, hipStream_t stream) {
  clear_error();
  rkv_status st;
  if (numDeltaTokens < 0 || batchSize < 0 || numKVHeads < 0 || numPages < 0 ||
      maxPagesPerSeq < 0 || ropeStates < 0 || ropeRows < 0)
    return fail(RKV_ERR_SHAPE, "negative size argument");
  if ((st = check_style(ropeStyle))) return st;
  if ((st = check_dims(headDim, rotaryDim))) return st;
  Span s_sc[2] = {};
  if (fp8 && (st = check_scales(k_scale, v_scale, s_sc))) return st;
  const long long N = numDeltaTokens, Hkv = numKVHeads, D = headDim, R = rotaryDim;
  long long delta_elems, pool_elems, pt_elems, cs_elems;
  if (!mul_ok(N * Hkv, D, &delta_elems) ||
      !mul_ok(2LL * numPages * rkv::kTokensPerPage, Hkv * D, &pool_elems) ||
      !mul_ok((long long)batchSize * 2, maxPagesPerSeq, &pt_elems) ||
      !mul_ok(gather ? (long long)ropeStates * ropeRows : N, R, &cs_elems) ||
      pool_elems > (INT64_MAX / 2))
    return fail(RKV_ERR_SHAPE, "sizes overflow");
  // a delta row's 2*Hkv head rows (and the padding rows of its last wave)
  // are addressed by 32-bit byte offsets below 2^31
  if ((2 * Hkv + 64) * D * 2 >= (1LL << 31))
    return fail(RKV_ERR_UNSUPPORTED, "numKVHeads %lld too large", Hkv);
  if (N == 0 || Hkv == 0) return RKV_OK;
  const float* cs = gather ? rope : tokenAlignedCosSin;
  const char* cs_name = gather ? "ropeCosSin" : "tokenAlignedCosSin";
  // An array with no elements (e.g. the cos/sin rows when rotaryDim = 0) may be null.
  if ((delta_elems > 0 && (!kDelta || !vDelta)) || (cs_elems > 0 && !cs) || !deltaPositions ||
      !deltaTokenToSequence)
    return fail(RKV_ERR_NULL, "null delta-row or cos/sin pointer");
  if ((pool_elems > 0 && !kvCache) || (pt_elems > 0 && !pageTable))
    return fail(RKV_ERR_NULL, "null kvCache or pageTable");
  const void* ptrs[] = {kDelta, vDelta, kvCache, cs, deltaPositions, deltaTokenToSequence,
                        pageTable, stateIndices};
  const char* names[] = {"kDelta", "vDelta", "kvCache", cs_name, "deltaPositions",
                         "deltaTokenToSequence", "pageTable", "stateIndices"};
  for (int k = 0; k < 8; ++k)
    if (((uintptr_t)ptrs[k] & 15u) != 0)
      return fail(RKV_ERR_ALIGNMENT, "%s is not 16-byte aligned", names[k]);
  auto span = [](const char* n, const void* p, long long bytes) {
    return Span{n, (uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes};
  };
  Span out = span("kvCache", kvCache, pool_elems * (fp8 ? 1 : 2));
  Span ins[] = {span("kDelta", kDelta, delta_elems * 2), span("vDelta", vDelta, delta_elems * 2),
                span(cs_name, cs, cs_elems * 4), span("deltaPositions", deltaPositions, N * 4),
                span("deltaTokenToSequence", deltaTokenToSequence, N * 4),
                span("pageTable", pageTable, pt_elems * 4),
                span("stateIndices", stateIndices, stateIndices ? batchSize * 4LL : 0),
                s_sc[0], s_sc[1]};
  if ((st = check_no_alias(&out, 1, ins, 9))) return st;
  if (pool_elems == 0 || pt_elems == 0) return RKV_OK;   // nothing can be written

  rkv::PagedParams p{};
  p.k_delta = kDelta;
  p.v_delta = vDelta;
  p.pool = fp8 ? nullptr : (uint16_t*)kvCache;
  p.pool8 = fp8 ? (uint8_t*)kvCache : nullptr;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.cos_sin = tokenAlignedCosSin;
  p.rope = rope;
  p.state_idx = stateIndices;
  p.rope_states = ropeStates;
  p.rope_rows = ropeRows;
  p.positions = deltaPositions;
  p.seq = deltaTokenToSequence;
  p.page_table = pageTable;
  p.N = numDeltaTokens;
  p.batch = batchSize;
  p.Hkv = numKVHeads;
  p.R = rotaryDim;
  p.num_pages = numPages;
  p.max_pages = maxPagesPerSeq;
  const long long rows_per_group = 512 / D;
  const long long groups_per_row = (2 * Hkv + rows_per_group - 1) / rows_per_group;
  // row groups per wave (see "Launch shape" above)
  const int g_small = fp8 ? 2 : 4;
  const int g_large = 2;
  const Split sp = pick_split(N, groups_per_row, g_large, g_small);
  // large launches and E4M3 pools load a delta row once its page ids are
  // known (only rows that are written move bytes); small fp16 ones request
  // every row with the index loads, so that the reads overlap the two
  // dependent index round trips
  const bool late_loads =
      g_force_loads ? g_force_loads == 2 : (fp8 || N * groups_per_row > kStreamingGroups);
  if (!sp.groups_per_wave) return fail(RKV_ERR_UNSUPPORTED, "too many rows for one launch");
  p.groups_per_wave = sp.groups_per_wave;
  p.waves_per_row = sp.waves_per_item;
  p.total_waves = (int32_t)(N * p.waves_per_row);
  p.div_waves = rkv::make_fastdiv((uint32_t)p.waves_per_row);
  g_last_groups = p.groups_per_wave;
  g_last_loads = late_loads ? 2 : 1;
  return launched(fp8 ? rkv::launch_paged_fp8(p, headDim, layout_of(ropeStyle),
                                              exact_of(ropeStyle), gather, late_loads, stream)
                      : rkv::launch_paged(p, headDim, layout_of(ropeStyle), exact_of(ropeStyle),
                                          gather, late_loads, stream));
}

}  // namespace

extern "C" {

rkv_status rkv_apply_rope_write_kv_packed_qkv(const rkv_tensor* cosSinCache, rkv_tensor* qkv,
                                              rkv_tensor* kvCache, int32_t ropeStyle,
                                              hipStream_t stream) {
  return contig(rkv::kCallPacked, cosSinCache, nullptr, nullptr, qkv, kvCache, nullptr, false,
                nullptr, nullptr, nullptr, ropeStyle, stream);
}

rkv_status rkv_apply_rope_write_kv_continuous(const rkv_tensor* cosSinCache,
                                              const rkv_tensor* kvCacheEndLens,
                                              const rkv_tensor* qkv, rkv_tensor* kvCache,
                                              rkv_tensor* qOut, int32_t ropeStyle,
                                              hipStream_t stream) {
  return contig(rkv::kCallContinuous, cosSinCache, kvCacheEndLens, nullptr, qkv, kvCache, qOut,
                false, nullptr, nullptr, nullptr, ropeStyle, stream);
}

rkv_status rkv_apply_rope_write_kv_tree(const rkv_tensor* cosSinCache,
                                        const rkv_tensor* kvCacheEndLens,
                                        const rkv_tensor* tokenPosIds, const rkv_tensor* qkv,
                                        rkv_tensor* kvCache, rkv_tensor* qOut,
                                        int32_t ropeStyle, hipStream_t stream) {
  return contig(rkv::kCallTree, cosSinCache, kvCacheEndLens, tokenPosIds, qkv, kvCache, qOut,
                false, nullptr, nullptr, nullptr, ropeStyle, stream);
}

rkv_status rkv_dflash_target_kv_cache_update(
    const uint16_t* kDelta, const uint16_t* vDelta, uint16_t* kvCache,
    const float* tokenAlignedCosSin, const int32_t* deltaPositions,
    const int32_t* deltaTokenToSequence, const int32_t* pageTable, int32_t numDeltaTokens,
    int32_t batchSize, int32_t numKVHeads, int32_t headDim, int32_t rotaryDim, int32_t numPages,
    int32_t maxPagesPerSeq, int32_t ropeStyle, hipStream_t stream) {
  return paged(kDelta, vDelta, kvCache, false, nullptr, nullptr, tokenAlignedCosSin, nullptr, 0,
               0, nullptr, deltaPositions, deltaTokenToSequence, pageTable, numDeltaTokens, batchSize,
               numKVHeads, headDim, rotaryDim, numPages, maxPagesPerSeq, ropeStyle, false, stream);
}

rkv_status rkv_dflash_target_kv_cache_update_gather_rope(
    const uint16_t* kDelta, const uint16_t* vDelta, uint16_t* kvCache, const float* ropeCosSin,
    int32_t ropeStates, int32_t ropeRows, const int32_t* stateIndices,
    const int32_t* deltaPositions, const int32_t* deltaTokenToSequence, const int32_t* pageTable,
    int32_t numDeltaTokens, int32_t batchSize, int32_t numKVHeads, int32_t headDim,
    int32_t rotaryDim, int32_t numPages, int32_t maxPagesPerSeq, int32_t ropeStyle,
    hipStream_t stream) {
  return paged(kDelta, vDelta, kvCache, false, nullptr, nullptr, nullptr, ropeCosSin, ropeStates,
               ropeRows, stateIndices, deltaPositions, deltaTokenToSequence, pageTable, numDeltaTokens, batchSize,
               numKVHeads, headDim, rotaryDim, numPages, maxPagesPerSeq, ropeStyle, true, stream);
}

rkv_status rkv_apply_rope_write_kv_packed_qkv_fp8(const rkv_tensor* cosSinCache, rkv_tensor* qkv,
                                                  rkv_tensor* kvCache, const float* kScale,
                                                  const float* vScale, int32_t ropeStyle,
                                                  hipStream_t stream) {
  return contig(rkv::kCallPacked, cosSinCache, nullptr, nullptr, qkv, kvCache, nullptr, true,
                kScale, vScale, nullptr, ropeStyle, stream);
}

rkv_status rkv_apply_rope_write_kv_continuous_fp8(const rkv_tensor* cosSinCache,
                                                  const rkv_tensor* kvCacheEndLens,
                                                  const rkv_tensor* qkv, rkv_tensor* kvCache,
                                                  rkv_tensor* qOut, const float* kScale,
                                                  const float* vScale, int32_t ropeStyle,
                                                  hipStream_t stream) {
  return contig(rkv::kCallContinuous, cosSinCache, kvCacheEndLens, nullptr, qkv, kvCache, qOut,
                true, kScale, vScale, nullptr, ropeStyle, stream);
}

rkv_status rkv_apply_rope_write_kv_tree_fp8(const rkv_tensor* cosSinCache,
                                            const rkv_tensor* kvCacheEndLens,
                                            const rkv_tensor* tokenPosIds, const rkv_tensor* qkv,
                                            rkv_tensor* kvCache, rkv_tensor* qOut,
                                            const float* kScale, const float* vScale,
                                            int32_t ropeStyle, hipStream_t stream) {
  return contig(rkv::kCallTree, cosSinCache, kvCacheEndLens, tokenPosIds, qkv, kvCache, qOut,
                true, kScale, vScale, nullptr, ropeStyle, stream);
}

rkv_status rkv_dflash_target_kv_cache_update_fp8(
    const uint16_t* kDelta, const uint16_t* vDelta, uint8_t* kvCache, const float* kScale,
    const float* vScale, const float* tokenAlignedCosSin, const int32_t* deltaPositions,
    const int32_t* deltaTokenToSequence, const int32_t* pageTable, int32_t numDeltaTokens,
    int32_t batchSize, int32_t numKVHeads, int32_t headDim, int32_t rotaryDim, int32_t numPages,
    int32_t maxPagesPerSeq, int32_t ropeStyle, hipStream_t stream) {
  return paged(kDelta, vDelta, kvCache, true, kScale, vScale, tokenAlignedCosSin, nullptr, 0, 0,
               nullptr, deltaPositions, deltaTokenToSequence, pageTable, numDeltaTokens,
               batchSize, numKVHeads, headDim, rotaryDim, numPages, maxPagesPerSeq, ropeStyle,
               false, stream);
}

rkv_status rkv_dflash_target_kv_cache_update_gather_rope_fp8(
    const uint16_t* kDelta, const uint16_t* vDelta, uint8_t* kvCache, const float* kScale,
    const float* vScale, const float* ropeCosSin, int32_t ropeStates, int32_t ropeRows,
    const int32_t* stateIndices, const int32_t* deltaPositions,
    const int32_t* deltaTokenToSequence, const int32_t* pageTable, int32_t numDeltaTokens,
    int32_t batchSize, int32_t numKVHeads, int32_t headDim, int32_t rotaryDim, int32_t numPages,
    int32_t maxPagesPerSeq, int32_t ropeStyle, hipStream_t stream) {
  return paged(kDelta, vDelta, kvCache, true, kScale, vScale, nullptr, ropeCosSin, ropeStates,
               ropeRows, stateIndices, deltaPositions, deltaTokenToSequence, pageTable,
               numDeltaTokens, batchSize, numKVHeads, headDim, rotaryDim, numPages,
               maxPagesPerSeq, ropeStyle, true, stream);
}

}  // extern "C"

namespace {

// The fp8 flag of a Q/K-norm call follows the cache descriptor's dtype;
// scales come with an E4M3 cache only.
rkv_status norm_call(int call, const rkv_tensor* cos_sin, const rkv_tensor* end_lens,
                     const rkv_tensor* pos_ids, const rkv_tensor* qkv, rkv_tensor* cache,
                     rkv_tensor* q_out, const float* qNormWeight, const float* kNormWeight,
                     float epsilon, const float* kScale, const float* vScale, int32_t style,
                     hipStream_t stream) {
  clear_error();
  if (!cache) return fail(RKV_ERR_NULL, "kvCache: null descriptor");
  const bool fp8 = cache->dtype == RKV_F8E4M3;
  if (!fp8 && (kScale || vScale))
    return fail(RKV_ERR_DTYPE, "kScale / vScale apply to an E4M3 cache only");
  NormArgs n;
  n.q_w = qNormWeight;
  n.k_w = kNormWeight;
  n.eps = epsilon;
  return contig(call, cos_sin, end_lens, pos_ids, qkv, cache, q_out, fp8, kScale, vScale, &n,
                style, stream);
}

}  // namespace

extern "C" {

rkv_status rkv_apply_rope_write_kv_packed_qkv_qknorm(const rkv_tensor* cosSinCache,
                                                     rkv_tensor* qkv, rkv_tensor* kvCache,
                                                     const float* qNormWeight,
                                                     const float* kNormWeight, float epsilon,
                                                     const float* kScale, const float* vScale,
                                                     int32_t ropeStyle, hipStream_t stream) {
  return norm_call(rkv::kCallPacked, cosSinCache, nullptr, nullptr, qkv, kvCache, nullptr,
                   qNormWeight, kNormWeight, epsilon, kScale, vScale, ropeStyle, stream);
}

rkv_status rkv_apply_rope_write_kv_continuous_qknorm(
    const rkv_tensor* cosSinCache, const rkv_tensor* kvCacheEndLens, const rkv_tensor* qkv,
    rkv_tensor* kvCache, rkv_tensor* qOut, const float* qNormWeight, const float* kNormWeight,
    float epsilon, const float* kScale, const float* vScale, int32_t ropeStyle,
    hipStream_t stream) {
  return norm_call(rkv::kCallContinuous, cosSinCache, kvCacheEndLens, nullptr, qkv, kvCache, qOut,
                   qNormWeight, kNormWeight, epsilon, kScale, vScale, ropeStyle, stream);
}

rkv_status rkv_apply_rope_write_kv_tree_qknorm(
    const rkv_tensor* cosSinCache, const rkv_tensor* kvCacheEndLens,
    const rkv_tensor* tokenPosIds, const rkv_tensor* qkv, rkv_tensor* kvCache, rkv_tensor* qOut,
    const float* qNormWeight, const float* kNormWeight, float epsilon, const float* kScale,
    const float* vScale, int32_t ropeStyle, hipStream_t stream) {
  return norm_call(rkv::kCallTree, cosSinCache, kvCacheEndLens, tokenPosIds, qkv, kvCache, qOut,
                   qNormWeight, kNormWeight, epsilon, kScale, vScale, ropeStyle, stream);
}

rkv_status rkv_dflash_prepare_delta_metadata(const int32_t* oldDraftCacheLengths,
                                             const int32_t* deltaLengths, int32_t deltaWidth,
                                             int32_t* deltaPositions,
                                             int32_t* deltaTokenToSequence, int32_t batchSize,
                                             hipStream_t stream) {
  clear_error();
  if (batchSize < 0 || deltaWidth < 0) return fail(RKV_ERR_SHAPE, "negative size argument");
  const long long rows = (long long)batchSize * deltaWidth;
  if (rows > INT32_MAX) return fail(RKV_ERR_UNSUPPORTED, "batchSize*deltaWidth exceeds 2^31-1");
  if (rows == 0) return RKV_OK;
  if (!oldDraftCacheLengths || !deltaLengths || !deltaPositions || !deltaTokenToSequence)
    return fail(RKV_ERR_NULL, "null metadata pointer");
  const void* ptrs[] = {oldDraftCacheLengths, deltaLengths, deltaPositions, deltaTokenToSequence};
  for (const void* q : ptrs)
    if ((uintptr_t)q & 3u) return fail(RKV_ERR_ALIGNMENT, "metadata arrays must be 4-byte aligned");
  auto span = [](const char* n, const void* q, long long bytes) {
    return Span{n, (uintptr_t)q, (uintptr_t)q + (uintptr_t)bytes};
  };
  Span outs[] = {span("deltaPositions", deltaPositions, rows * 4),
                 span("deltaTokenToSequence", deltaTokenToSequence, rows * 4)};
  Span ins[] = {span("oldDraftCacheLengths", oldDraftCacheLengths, batchSize * 4LL),
                span("deltaLengths", deltaLengths, batchSize * 4LL)};
  rkv_status st;
  if ((st = check_no_alias(outs, 2, ins, 2))) return st;
  return launched(rkv::launch_delta_metadata(oldDraftCacheLengths, deltaLengths, deltaWidth,
                                             deltaPositions, deltaTokenToSequence, (int32_t)rows,
                                             stream));
}

rkv_status rkv_dflash_build_linear_tree_metadata(int32_t* treeParentIds, int32_t* treeDepths,
                                                 int32_t batchSize, int32_t verifySize,
                                                 hipStream_t stream) {
  clear_error();
  if (batchSize < 0 || verifySize < 0) return fail(RKV_ERR_SHAPE, "negative size argument");
  const long long nodes = (long long)batchSize * verifySize;
  if (nodes > INT32_MAX) return fail(RKV_ERR_UNSUPPORTED, "batchSize*verifySize exceeds 2^31-1");
  if (nodes == 0) return RKV_OK;
  if (!treeParentIds || !treeDepths) return fail(RKV_ERR_NULL, "null tree metadata pointer");
  if (((uintptr_t)treeParentIds & 3u) || ((uintptr_t)treeDepths & 3u))
    return fail(RKV_ERR_ALIGNMENT, "tree metadata arrays must be 4-byte aligned");
  Span outs[] = {Span{"treeParentIds", (uintptr_t)treeParentIds,
                      (uintptr_t)treeParentIds + (uintptr_t)(nodes * 4)},
                 Span{"treeDepths", (uintptr_t)treeDepths,
                      (uintptr_t)treeDepths + (uintptr_t)(nodes * 4)}};
  rkv_status st;
  if ((st = check_no_alias(outs, 2, nullptr, 0))) return st;
  return launched(rkv::launch_linear_tree(treeParentIds, treeDepths, verifySize, (int32_t)nodes,
                                          stream));
}

rkv_status rkv_check_rope_capacity(int32_t cosSinSeqLen, int32_t kvCapacity) {
  clear_error();
  if (cosSinSeqLen > kvCapacity)
    return fail(RKV_ERR_CAPACITY, "cos/sin cache length %d exceeds KV capacity %d", cosSinSeqLen,
                kvCapacity);
  return RKV_OK;
}

int32_t rkv_tokens_per_page(void) { return rkv::kTokensPerPage; }

int32_t rkv_last_launch_groups_per_wave(void) { return g_last_groups; }

rkv_status rkv_set_launch_overrides(int32_t groupsPerWave, int32_t pagedLoads) {
  g_err[0] = '\0';
  if (groupsPerWave != 0 && groupsPerWave != 1 && groupsPerWave != 2 && groupsPerWave != 4)
    return fail(RKV_ERR_SHAPE, "groupsPerWave %d: must be 0, 1, 2 or 4", groupsPerWave);
  if (pagedLoads < 0 || pagedLoads > 2)
    return fail(RKV_ERR_SHAPE, "pagedLoads %d: must be 0, 1 or 2", pagedLoads);
  g_force_groups = groupsPerWave;
  g_force_loads = pagedLoads;
  return RKV_OK;
}

int32_t rkv_last_launch_paged_loads(void) { return g_last_loads; }

const char* rkv_last_error(void) { return g_err; }

const char* rkv_status_string(int32_t status) {
  switch (status) {
    case RKV_OK: return "RKV_OK";
    case RKV_ERR_NULL: return "RKV_ERR_NULL";
    case RKV_ERR_DTYPE: return "RKV_ERR_DTYPE";
    case RKV_ERR_SHAPE: return "RKV_ERR_SHAPE";
    case RKV_ERR_UNSUPPORTED: return "RKV_ERR_UNSUPPORTED";
    case RKV_ERR_CAPACITY: return "RKV_ERR_CAPACITY";
    case RKV_ERR_ALIGNMENT: return "RKV_ERR_ALIGNMENT";
    case RKV_ERR_ALIAS: return "RKV_ERR_ALIAS";
    case RKV_ERR_HIP: return "RKV_ERR_HIP";
    default: return "unknown status";
  }
}

}  // extern "C"
