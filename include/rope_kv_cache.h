/* rope_kv_cache.h -- fused rotary position embedding + KV-cache write for
 * AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Four device calls follow the
 * problem statement of TensorRT-Edge-LLM's "Apply Rope Write KV" (calls 1-3)
 * and "Dflash Runtime Kernels" (call 4) pages; a fifth, host-only call is
 * that page's capacity check.
 *
 * Common conventions
 * ------------------
 * Ownership.  Every tensor pointer is a DEVICE pointer owned by the caller.
 *   The library allocates no device memory, keeps no pointer after a call
 *   returns and holds no state besides a thread-local error message.
 * Asynchrony.  A call validates its arguments on the host, enqueues one
 *   kernel on `stream` and returns without synchronising.  Buffers must stay
 *   alive until the stream has executed the kernel.  A null stream is the
 *   default stream.
 * Layout.  Tensors are dense, row-major, with the shapes stated per call, and
 *   every data pointer is 16-byte aligned.  fp16 is IEEE binary16.
 * Aliasing.  Only call 1 updates a tensor in place (`qkv`).  Otherwise no
 *   output may overlap an input or another output; overlapping buffers are
 *   rejected with RKV_ERR_ALIAS where the host can see it.
 * Errors.  Each call returns RKV_OK or an error status and, on error,
 *   enqueues nothing.  rkv_last_error() describes the last error raised on
 *   the calling thread.  Index values that live in device memory (end
 *   lengths, position ids, delta metadata, page ids) are not read by the
 *   host; the kernels skip rows whose indices fall out of range instead (the
 *   rules are given per call).
 * Supported shapes.  headDim in {64, 128, 256}; rotaryDim a multiple of 16
 *   with 0 <= rotaryDim <= headDim.  Other values return
 *   RKV_ERR_UNSUPPORTED, as do token or delta-row counts beyond 2^31 - 1 and
 *   launches that would need more waves than one dispatch holds (2^32 - 1
 *   work-items, 2^26 waves).  A wave handles up to four 1 KB row groups of
 *   one token or delta row (512/headDim head rows each), so the limit is
 *   about 2^28 row groups, and lower when tokens have few heads.  A token's
 *   head rows, and a delta row's K and V head rows, are addressed by 32-bit
 *   byte offsets: (heads + 64) * headDim must stay below 2^31 (calls 1-3,
 *   heads = Hq + 2*Hkv) and (2*numKVHeads + 64) * headDim below 2^30
 *   (paged calls); beyond that the calls return RKV_ERR_UNSUPPORTED.
 * Rotation.  For frequency i < rotaryDim/2 with c = row[i] and
 *   s = row[rotaryDim/2 + i] of the token's cos/sin row, the pair (u, v)
 *   becomes (x_u*c - x_v*s, x_v*c + x_u*s), rounded to fp16 to nearest-even.
 *   NeoX pairs (i, i + rotaryDim/2); GPT-J pairs (2i, 2i+1).  Dims
 *   >= rotaryDim are copied bit for bit.  (sglang rope_cache.py,
 *   _get_neox_rotated_x, _get_gptj_rotated_x, _unit_rope, _load_cos_sin.)
 * Arithmetic.  By default each rotated element is computed in binary32,
 *   compensated so that the value before the final rounding is within about
 *   2^-23 relative of the exact x_u*c - x_v*s (also under cancellation); the
 *   fp16 result is then the correctly rounded value or, rarely, its
 *   neighbour (at most 1 fp16 ulp away).  With RKV_ROUND_EXACT OR-ed into
 *   ropeStyle, the products and the sum are evaluated exactly in binary64
 *   and rounded once to binary16: the correctly rounded result, bit for bit,
 *   at some extra arithmetic cost.
 */
#ifndef ROPE_KV_CACHE_H
#define ROPE_KV_CACHE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A HIP stream.  This is the same type as HIP's hipStream_t, declared here
 * under its own name so that C callers need no HIP header and may include
 * hip_runtime_api.h before or after this one (C99 forbids a second typedef
 * of the same name). */
struct ihipStream_t;
typedef struct ihipStream_t* rkv_stream_t;

typedef enum {
  RKV_OK = 0,
  RKV_ERR_NULL = 1,         /* a required pointer is null */
  RKV_ERR_DTYPE = 2,        /* a descriptor has the wrong element type */
  RKV_ERR_SHAPE = 3,        /* ranks or dimensions are inconsistent */
  RKV_ERR_UNSUPPORTED = 4,  /* valid but outside the supported shape set */
  RKV_ERR_CAPACITY = 5,     /* positions cannot fit the cache or the cos/sin table */
  RKV_ERR_ALIGNMENT = 6,    /* a data pointer is not 16-byte aligned */
  RKV_ERR_ALIAS = 7,        /* an output overlaps an input or another output */
  RKV_ERR_HIP = 8           /* the HIP runtime reported an error at launch */
} rkv_status;

/* ropeStyle: the pair layout, optionally OR-ed with RKV_ROUND_EXACT. */
typedef enum {
  RKV_ROPE_NEOX = 0,      /* pairs (i, i + R/2) */
  RKV_ROPE_GPTJ = 1,      /* pairs (2i, 2i + 1) */
  RKV_ROUND_EXACT = 0x100 /* correctly rounded results (see Rotation above) */
} rkv_rope_style;

typedef enum {
  RKV_F16 = 0,
  RKV_F32 = 1,
  RKV_I32 = 2,
  RKV_F8E4M3 = 3   /* OCP 8-bit float E4M3 ("e4m3fn"), one byte per element */
} rkv_dtype;

/* A dense row-major device tensor: element type, rank (<= 5) and extents.
 * The descriptor itself is host memory and is read only during the call. */
typedef struct {
  void* data;
  int32_t dtype;
  int32_t ndim;
  int64_t shape[5];
} rkv_tensor;

/* Call 1 -- empty-cache prefill on packed QKV, in place.
 * (TensorRT-Edge-LLM C++ API, "Apply Rope Write KV",
 *  launchApplyRopeWriteKVPackedQKV.)
 *   cosSinCache  [in]     f32 [T, L, R]: T = 1 (shared by all sequences) or B
 *                         (one table per sequence); row p = [cos | sin] of
 *                         position p; R = rotaryDim.
 *   qkv          [in,out] f16 [B, S, Hq + Hkv + Hkv, D]: heads in Q, K, V
 *                         order.  Q and K heads are rotated in place (token s
 *                         at position s); V heads are left unchanged.
 *   kvCache      [out]    f16 [B, 2, Hkv, cap, D]: plane 0 = K, plane 1 = V.
 *                         Slot s of each head receives token s's rotated K and
 *                         its V; slots >= S are not written.
 * Errors: RKV_ERR_CAPACITY if S > cap or S > L.  Hq = qkv dim 2 - 2*Hkv must
 * be >= 0.  B = 0 or S = 0 is a valid call that enqueues nothing. */
rkv_status rkv_apply_rope_write_kv_packed_qkv(const rkv_tensor* cosSinCache, rkv_tensor* qkv,
                                              rkv_tensor* kvCache, int32_t ropeStyle,
                                              rkv_stream_t stream);

/* Call 2 -- write into a non-empty cache, rotated Q to a separate tensor.
 * (TensorRT-Edge-LLM C++ API, "Apply Rope Write KV",
 *  launchApplyRopeWriteKVContinuousQAndKVCache.)
 *   cosSinCache     [in]  f32 [T, L, R], T in {1, B}.
 *   kvCacheEndLens  [in]  i32 [B]: cache length of sequence b after the
 *                         write; token s takes position and slot
 *                         endLens[b] - S + s.
 *   qkv             [in]  f16 [B, S, Hq + 2*Hkv, D]; never written.
 *   kvCache         [out] f16 [B, 2, Hkv, cap, D]: rotated K and raw V at the
 *                         token's slot; other slots are not written.
 *   qOut            [out] f16 [B, S, Hq, D]: rotated Q.
 * A token whose slot is outside [0, cap) or whose position is outside
 * [0, L) writes nothing, neither qOut nor the cache. */
rkv_status rkv_apply_rope_write_kv_continuous(const rkv_tensor* cosSinCache,
                                              const rkv_tensor* kvCacheEndLens,
                                              const rkv_tensor* qkv, rkv_tensor* kvCache,
                                              rkv_tensor* qOut, int32_t ropeStyle,
                                              rkv_stream_t stream);

/* Call 3 -- tree-decoding write for speculative decoding.
 * (TensorRT-Edge-LLM C++ API, "Apply Rope Write KV",
 *  launchApplyRopeWriteKVTreeDecoding.)
 * As call 2, except that the rotary position of token s is
 * tokenPosIds[b, s] (i32 [B, S]) while its cache slot stays endLens[b]-S+s,
 * so that tree siblings at one depth keep distinct slots.  A token whose
 * slot is outside [0, cap) or whose position is outside [0, L) writes
 * nothing. */
rkv_status rkv_apply_rope_write_kv_tree(const rkv_tensor* cosSinCache,
                                        const rkv_tensor* kvCacheEndLens,
                                        const rkv_tensor* tokenPosIds, const rkv_tensor* qkv,
                                        rkv_tensor* kvCache, rkv_tensor* qOut,
                                        int32_t ropeStyle, rkv_stream_t stream);

/* Call 4 -- paged delta update.
 * (TensorRT-Edge-LLM C++ API, "Dflash Runtime Kernels",
 *  launchDFlashTargetKVCacheUpdate.)
 *   kDelta, vDelta        [in]     f16 [N, Hkv, D], token-major rows.
 *   kvCache               [in,out] f16 [2, numPages, 64, Hkv, D] paged pool;
 *                                  canonical page id p addresses
 *                                  pool[p / numPages][p % numPages].
 *   tokenAlignedCosSin    [in]     f32 [N, R]: the cos/sin row of delta row i.
 *   deltaPositions        [in]     i32 [N]: absolute position of row i.
 *   deltaTokenToSequence  [in]     i32 [N]: owning sequence of row i.
 *   pageTable             [in]     i32 [batchSize, 2, maxPagesPerSeq]:
 *                                  canonical ids, K entries in [0, numPages),
 *                                  V entries in [numPages, 2*numPages).
 *   N = numDeltaTokens (physical rows), batchSize = active sequences.
 * Row i is skipped if its position or sequence is negative (padding), if its
 * sequence is >= batchSize, or if its position is >= maxPagesPerSeq*64.
 * Otherwise, with lp = pos / 64 and off = pos % 64, K (rotated) is written
 * to page pageTable[seq, 0, lp] at token off if that id is in [0, numPages),
 * and V (copied) to page pageTable[seq, 1, lp] if that id is in
 * [numPages, 2*numPages); an unmapped or out-of-plane id skips that plane.
 * Rows must not map to the same (page, token): such writes race.
 * The rotation layout is given by ropeStyle.  The pool may exceed 2 GiB. */
rkv_status rkv_dflash_target_kv_cache_update(
    const uint16_t* kDelta, const uint16_t* vDelta, uint16_t* kvCache,
    const float* tokenAlignedCosSin, const int32_t* deltaPositions,
    const int32_t* deltaTokenToSequence, const int32_t* pageTable, int32_t numDeltaTokens,
    int32_t batchSize, int32_t numKVHeads, int32_t headDim, int32_t rotaryDim,
    int32_t numPages, int32_t maxPagesPerSeq, int32_t ropeStyle, rkv_stream_t stream);

/* Call 4 with the cos/sin gather fused in (the page's
 * launchDFlashGatherDeltaRope builds tokenAlignedCosSin from a rope table;
 * only its parameter list is given, so its meaning here is a reading).
 *   ropeCosSin    [in] f32 [ropeStates, ropeRows, R]: rope table(s), rows
 *                      [cos | sin] by position.
 *   stateIndices  [in] i32 [batchSize] or NULL: sequence q uses table
 *                      stateIndices[q]; NULL means table q (table 0 when
 *                      ropeStates == 1).
 * Everything else is as in rkv_dflash_target_kv_cache_update.  The K row of
 * delta row i is rotated with ropeCosSin[state(q_i), p_i] and written only
 * if that state exists and p_i < ropeRows; V follows the page table alone.
 * Saves the separate gather launch and its N*R*4-byte buffer. */
rkv_status rkv_dflash_target_kv_cache_update_gather_rope(
    const uint16_t* kDelta, const uint16_t* vDelta, uint16_t* kvCache, const float* ropeCosSin,
    int32_t ropeStates, int32_t ropeRows, const int32_t* stateIndices,
    const int32_t* deltaPositions, const int32_t* deltaTokenToSequence, const int32_t* pageTable,
    int32_t numDeltaTokens, int32_t batchSize, int32_t numKVHeads, int32_t headDim,
    int32_t rotaryDim, int32_t numPages, int32_t maxPagesPerSeq, int32_t ropeStyle,
    rkv_stream_t stream);

/* fp8 (E4M3) KV cache
 * ---------------------
 * The five calls below are the calls above with the cache (or pool) stored
 * as E4M3 bytes and two per-tensor scales; everything else -- shapes,
 * positions, slots, skip rules, qkv / qOut outputs, errors -- is unchanged.
 * (sglang rope_cache.py, fused_qk_rope_reshape_and_cache with HAVE_K_SCALE /
 * HAVE_V_SCALE: K and V are multiplied by the reciprocal of their scale
 * before the cast to the cache type.)
 *   kScale, vScale  [in] DEVICE pointers to one fp32 value each, or NULL for
 *                   a scale of 1; read by the kernel when it runs, so they
 *                   may be updated on the stream between calls.  4-byte
 *                   aligned, not overlapping any output.
 * Cache value.  A K element is the unrounded rotation (dims >= rotaryDim:
 *   the fp16 input), a V element the fp16 input, times rcp = 1/scale
 *   correctly rounded to fp32; that product is rounded to the nearest E4M3
 *   value, ties to even, magnitudes beyond 448 (and infinities) saturate to
 *   +-448, NaN stays NaN.  Q and call 1's in-place K are fp16 exactly as in
 *   the fp16 calls.
 * Arithmetic.  By default the rotation and the product are formed in
 *   binary32 and converted by the hardware: the code is the correctly
 *   rounded one or, rarely, its neighbour.  With RKV_ROUND_EXACT the
 *   rotation and the product are formed in binary64 and the code is the
 *   correctly rounded one, bit for bit.
 * The cache descriptor (calls 1-3) has dtype RKV_F8E4M3 and the same shape
 * as the fp16 cache; the paged pool (call 4) is [2, numPages, 64, Hkv, D]
 * bytes.  Cache traffic halves: D bytes per head row instead of 2*D. */
rkv_status rkv_apply_rope_write_kv_packed_qkv_fp8(const rkv_tensor* cosSinCache, rkv_tensor* qkv,
                                                  rkv_tensor* kvCache, const float* kScale,
                                                  const float* vScale, int32_t ropeStyle,
                                                  rkv_stream_t stream);

rkv_status rkv_apply_rope_write_kv_continuous_fp8(const rkv_tensor* cosSinCache,
                                                  const rkv_tensor* kvCacheEndLens,
                                                  const rkv_tensor* qkv, rkv_tensor* kvCache,
                                                  rkv_tensor* qOut, const float* kScale,
                                                  const float* vScale, int32_t ropeStyle,
                                                  rkv_stream_t stream);

rkv_status rkv_apply_rope_write_kv_tree_fp8(const rkv_tensor* cosSinCache,
                                            const rkv_tensor* kvCacheEndLens,
                                            const rkv_tensor* tokenPosIds, const rkv_tensor* qkv,
                                            rkv_tensor* kvCache, rkv_tensor* qOut,
                                            const float* kScale, const float* vScale,
                                            int32_t ropeStyle, rkv_stream_t stream);

rkv_status rkv_dflash_target_kv_cache_update_fp8(
    const uint16_t* kDelta, const uint16_t* vDelta, uint8_t* kvCache, const float* kScale,
    const float* vScale, const float* tokenAlignedCosSin, const int32_t* deltaPositions,
    const int32_t* deltaTokenToSequence, const int32_t* pageTable, int32_t numDeltaTokens,
    int32_t batchSize, int32_t numKVHeads, int32_t headDim, int32_t rotaryDim, int32_t numPages,
    int32_t maxPagesPerSeq, int32_t ropeStyle, rkv_stream_t stream);

rkv_status rkv_dflash_target_kv_cache_update_gather_rope_fp8(
    const uint16_t* kDelta, const uint16_t* vDelta, uint8_t* kvCache, const float* kScale,
    const float* vScale, const float* ropeCosSin, int32_t ropeStates, int32_t ropeRows,
    const int32_t* stateIndices, const int32_t* deltaPositions,
    const int32_t* deltaTokenToSequence, const int32_t* pageTable, int32_t numDeltaTokens,
    int32_t batchSize, int32_t numKVHeads, int32_t headDim, int32_t rotaryDim, int32_t numPages,
    int32_t maxPagesPerSeq, int32_t ropeStyle, rkv_stream_t stream);

/* Q/K RMS norm fused before the rotation
 * ---------------------------------------
 * Calls 1-3 with each Q and K head row normalised before it is rotated: the
 * postprocess step of the libmir-cuda decode path (execution.rs,
 * DecodeAttentionBf16: qkv_postprocess with query / key norm weights and the
 * model's rms_norm_epsilon, ahead of the KV store).  That page gives the
 * parameters only; the reading taken here:
 *   n_d = x_d * w_d / sqrt(mean_d(x_d^2) + epsilon)
 * over the whole head row (all headDim dims), with one weight vector for all
 * Q heads and one for all K heads; the rotation then acts on n, dims >=
 * rotaryDim carry n_d, and the result is rounded once (to fp16, or scaled to
 * E4M3).  V is not normalised.
 *   qNormWeight, kNormWeight  [in] DEVICE fp32 [headDim] each, 16-byte
 *                             aligned, or NULL: those heads are not
 *                             normalised (both NULL is the plain call).
 *   epsilon                   [in] finite, >= 0 (else RKV_ERR_SHAPE).
 *   kvCache                   f16 (RKV_F16) or E4M3 (RKV_F8E4M3) descriptor:
 *                             its dtype selects the cache format;
 *   kScale, vScale            the E4M3 cache's scales as in the _fp8 calls;
 *                             must be NULL with an fp16 cache (else
 *                             RKV_ERR_DTYPE).
 * Everything else is as in calls 1-3.  Arithmetic: by default binary32 (the
 * sum of squares reduced across the row's lanes, v_rsq_f32, the compensated
 * rotation), within the tolerance the tests state; with RKV_ROUND_EXACT the
 * mean square is exact and rounded once, sqrt, the division, each product
 * and each sum are binary64 operations in a fixed order, and the result is
 * bit-identical to the reference evaluation. */
rkv_status rkv_apply_rope_write_kv_packed_qkv_qknorm(const rkv_tensor* cosSinCache,
                                                     rkv_tensor* qkv, rkv_tensor* kvCache,
                                                     const float* qNormWeight,
                                                     const float* kNormWeight, float epsilon,
                                                     const float* kScale, const float* vScale,
                                                     int32_t ropeStyle, rkv_stream_t stream);

rkv_status rkv_apply_rope_write_kv_continuous_qknorm(
    const rkv_tensor* cosSinCache, const rkv_tensor* kvCacheEndLens, const rkv_tensor* qkv,
    rkv_tensor* kvCache, rkv_tensor* qOut, const float* qNormWeight, const float* kNormWeight,
    float epsilon, const float* kScale, const float* vScale, int32_t ropeStyle,
    rkv_stream_t stream);

rkv_status rkv_apply_rope_write_kv_tree_qknorm(
    const rkv_tensor* cosSinCache, const rkv_tensor* kvCacheEndLens,
    const rkv_tensor* tokenPosIds, const rkv_tensor* qkv, rkv_tensor* kvCache, rkv_tensor* qOut,
    const float* qNormWeight, const float* kNormWeight, float epsilon, const float* kScale,
    const float* vScale, int32_t ropeStyle, rkv_stream_t stream);

/* Device metadata builders
 * ------------------------
 * Delta metadata for call 4 (TensorRT-Edge-LLM C++ API, "Dflash Runtime
 * Kernels", launchDFlashPrepareDeltaMetadata; the page gives the signature
 * only, the reading here follows its proposal-input kernel, which places a
 * sequence's delta right after its old draft cache length).
 *   oldDraftCacheLengths  [in]  i32 [batchSize] draft cache length before the delta
 *   deltaLengths          [in]  i32 [batchSize] delta tokens of each sequence
 *   deltaWidth            rows reserved per sequence (token-major layout)
 *   deltaPositions        [out] i32 [batchSize * deltaWidth]
 *   deltaTokenToSequence  [out] i32 [batchSize * deltaWidth]
 * Row b*deltaWidth + j is token j of sequence b's delta when
 * j < min(deltaLengths[b], deltaWidth): position oldDraftCacheLengths[b] + j,
 * owner b.  Every other row (and a position beyond the int32 range) is
 * padding: -1 in both arrays, which call 4 skips.  Device pointers,
 * 4-byte aligned; outputs may not overlap inputs or each other.  Nothing is
 * enqueued when batchSize*deltaWidth is 0. */
rkv_status rkv_dflash_prepare_delta_metadata(const int32_t* oldDraftCacheLengths,
                                             const int32_t* deltaLengths, int32_t deltaWidth,
                                             int32_t* deltaPositions,
                                             int32_t* deltaTokenToSequence, int32_t batchSize,
                                             rkv_stream_t stream);

/* Tree metadata of a linear verification path (same page,
 * launchDFlashBuildLinearTreeMetadata): for every sequence, node 0 is the
 * root (parent -1, depth 0) and node i > 0 has parent i - 1 and depth i.
 *   treeParentIds, treeDepths  [out] i32 [batchSize, verifySize], device,
 *                              4-byte aligned, not overlapping.
 * With these depths, call 3 at tokenPosIds = endLens[b] - S + depth writes
 * exactly what call 2 writes. */
rkv_status rkv_dflash_build_linear_tree_metadata(int32_t* treeParentIds, int32_t* treeDepths,
                                                 int32_t batchSize, int32_t verifySize,
                                                 rkv_stream_t stream);

/* Host-only capacity check.
 * (TensorRT-Edge-LLM C++ API, "Dflash Runtime Kernels",
 *  checkDFlashRopeCapacity.)
 * Returns RKV_ERR_CAPACITY exactly when cosSinSeqLen > kvCapacity (a table
 * shorter than the padded capacity is accepted), else RKV_OK.  Where the
 * original API throws, this returns the status and sets rkv_last_error(). */
rkv_status rkv_check_rope_capacity(int32_t cosSinSeqLen, int32_t kvCapacity);

/* Tokens per page of the paged pool: 64. */
int32_t rkv_tokens_per_page(void);

/* Row groups per wave (1, 2 or 4) of the kernel that this thread's most
 * recent rope / KV-cache call (calls 1-4 and their fp8 and Q/K-norm forms)
 * launched; 0 when that call launched nothing (an error, or an input with
 * no rows).  The metadata builders and the capacity check reset it to 0;
 * the other query functions leave it.  A row group is the 1 KB of
 * 512/headDim consecutive head rows that one wave instruction moves.  The
 * choice depends on the sizes and the kernel flavour only, never on data;
 * it is reported for tests and tuning and has no effect on results. */
int32_t rkv_last_launch_groups_per_wave(void);

/* Launch-shape overrides, for tuning and tests (no page defines such a
 * call).  They hold for this thread's later rope / KV-cache calls until they
 * are set again; results are the same bit for bit under every setting, only
 * the time differs.
 *   groupsPerWave: 0 lets the library choose; 1, 2 or 4 asks for that many
 *     row groups per wave (fewer when a work item -- a token of calls 1-3, a
 *     delta row of call 4 -- has fewer; more when one dispatch could not
 *     hold the waves).
 *   pagedLoads: 0 lets the library choose; 1 makes call 4 request every
 *     delta row together with its index loads ("early"); 2 loads a delta
 *     row once its page ids are known, and only if it is written ("late").
 * Returns RKV_ERR_SHAPE and changes nothing for any other value. */
rkv_status rkv_set_launch_overrides(int32_t groupsPerWave, int32_t pagedLoads);

/* Load plan of this thread's most recent call: 1 early, 2 late (see
 * rkv_set_launch_overrides); 0 when that call was not a paged update or
 * launched nothing. */
int32_t rkv_last_launch_paged_loads(void);

/* Message for the last error raised on this thread ("" if none).  The
 * pointer stays valid until the next call on the same thread. */
const char* rkv_last_error(void);

/* Static name of a status code. */
const char* rkv_status_string(int32_t status);

#ifdef __cplusplus
}
#endif
#endif /* ROPE_KV_CACHE_H */
