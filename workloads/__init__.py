"""Seeded synthetic inputs for the fused RoPE + KV-cache write.

This module only makes inputs: random fp16 activations, cos/sin tables,
end lengths, speculative trees, page tables and delta metadata.  It holds
none of the rotate or scatter arithmetic, and imports neither the CPU oracle
nor the HIP library; the tests, ``bench.py`` and ``__graft_entry__.smoke()``
hand the same arrays to both.

fp16 tensors are numpy ``uint16`` arrays holding IEEE binary16 bit patterns,
so that NaN sentinels and signed zeros survive every comparison.

Shapes follow the pages:
  * packed QKV ``[B, S, Hq+Hk+Hv, D]``, cos/sin ``[tableBatch, tableLen, R]``,
    contiguous cache ``[B, 2, Hkv, cap, D]``, ``qOut [B, S, Hq, D]``
    (TensorRT-Edge-LLM C++ API, "Apply Rope Write KV", parameter lists);
  * K/V deltas ``[N, Hkv, D]``, ``tokenAlignedCosSin [N, R]``, paged pool
    ``[2, numPages, 64, Hkv, D]``, ``pageTable [B, 2, maxPagesPerSeq]``
    (TensorRT-Edge-LLM, "Dflash Runtime Kernels",
    launchDFlashTargetKVCacheUpdate).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

NEOX = 0
GPTJ = 1
TOKENS_PER_PAGE = 64
# A quiet NaN with a payload: never produced by arithmetic, so a slot that
# still holds it after a call was not written.
SENTINEL = 0x7E5A
# The E4M3 NaN code: finite inputs never produce it, so an fp8 cache byte
# that still holds it was not written.
SENTINEL8 = 0x7F
# Per-tensor fp8 scales of the synthetic workloads: N(0,1) activations of
# magnitude up to about 5 land near the top of the E4M3 range (448), and the
# rare tails beyond 5.5 sigma saturate.
K_SCALE = 0.0123
V_SCALE = 0.0109


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def normal_f16(r: np.random.Generator, shape) -> np.ndarray:
    """fp16 N(0,1) samples as uint16 bit patterns (round-to-nearest-even)."""
    n = int(np.prod(shape, dtype=np.int64))
    x = r.standard_normal(n, dtype=np.float32).astype(np.float16)
    return x.view(np.uint16).reshape(shape)


def sentinel_f16(shape, value: int = SENTINEL) -> np.ndarray:
    return np.full(shape, value, dtype=np.uint16)


def rope_table(batch: int, length: int, rotary_dim: int, theta: float,
               offsets=None) -> np.ndarray:
    """cos/sin table, fp32 ``[batch, length, rotary_dim]``.

    Row ``t`` of batch ``b`` is ``[cos(a_0..a_{R/2-1}) | sin(a_0..a_{R/2-1})]``
    with ``a_i = (offsets[b] + t) * theta**(-2i/R)``, evaluated in float64 and
    rounded once to fp32.  This is the caller-side table the calls read; the
    calls never compute it.
    """
    if offsets is None:
        offsets = np.zeros(batch, dtype=np.int64)
    half = rotary_dim // 2
    out = np.empty((batch, length, rotary_dim), dtype=np.float32)
    if half == 0:
        return out
    inv_freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / rotary_dim)
    for b in range(batch):
        pos = (int(offsets[b]) + np.arange(length, dtype=np.float64))[:, None]
        ang = pos * inv_freq[None, :]
        out[b, :, :half] = np.cos(ang)
        out[b, :, half:] = np.sin(ang)
    return out


def rope_rows(positions, rotary_dim: int, theta: float) -> np.ndarray:
    """Table rows gathered at arbitrary positions, fp32 ``[len(positions), R]``.

    Negative positions (padding) get NaN rows.
    """
    positions = np.asarray(positions, dtype=np.int64)
    half = rotary_dim // 2
    out = np.full((positions.size, rotary_dim), np.nan, dtype=np.float32)
    ok = positions >= 0
    if half:
        inv_freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / rotary_dim)
        ang = positions[ok].astype(np.float64)[:, None] * inv_freq[None, :]
        rows = np.concatenate([np.cos(ang), np.sin(ang)], axis=1)
        out[ok] = rows.astype(np.float32)
    return out


def random_tree_depths(r: np.random.Generator, n: int, max_depth: int = 8) -> np.ndarray:
    """Depths of a random tree on ``n`` nodes.

    Node 0 is the root (depth 0); node ``i`` picks its parent uniformly among
    earlier nodes of depth < ``max_depth``, so every depth is <= ``max_depth``.
    """
    depth = np.zeros(n, dtype=np.int32)
    for i in range(1, n):
        cand = np.nonzero(depth[:i] < max_depth)[0]
        parent = cand[r.integers(0, cand.size)]
        depth[i] = depth[parent] + 1
    return depth


# --------------------------------------------------------------------------
# The five workloads.  Seeds 1001..1005.
# --------------------------------------------------------------------------

@dataclass
class Contig:
    """Inputs of calls 1-3 (contiguous cache)."""
    call: str                 # "packed" | "continuous" | "tree"
    style: int
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    R: int
    cap: int
    cos_sin: np.ndarray       # f32 [tb, tlen, R]
    qkv: np.ndarray           # u16 [B, S, Hq+2Hkv, D]
    cache: np.ndarray         # u16 [B, 2, Hkv, cap, D]
    q_out: np.ndarray | None = None      # u16 [B, S, Hq, D] (calls 2, 3)
    end_lens: np.ndarray | None = None   # i32 [B]
    pos_ids: np.ndarray | None = None    # i32 [B, S]
    name: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def tokens(self) -> int:
        return self.B * self.S


@dataclass
class Paged:
    """Inputs of call 4 (paged delta update)."""
    style: int
    N: int
    batch: int
    Hkv: int
    D: int
    R: int
    num_pages: int
    max_pages: int
    k_delta: np.ndarray       # u16 [N, Hkv, D]
    v_delta: np.ndarray       # u16 [N, Hkv, D]
    pool: np.ndarray          # u16 [2, numPages, 64, Hkv, D]
    cos_sin: np.ndarray       # f32 [N, R]
    positions: np.ndarray     # i32 [N]
    seq: np.ndarray           # i32 [N]
    page_table: np.ndarray    # i32 [batch, 2, maxPages]
    name: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def tokens(self) -> int:
        return self.N


def packed(B, S, Hq, Hkv, D, R, cap, style, seed, table_batch=1, table_len=None,
           theta=10000.0, offsets=None, cache_fill="sentinel", name="") -> Contig:
    r = rng(seed)
    tlen = cap if table_len is None else table_len
    qkv = normal_f16(r, (B, S, Hq + 2 * Hkv, D))
    cos_sin = rope_table(table_batch, tlen, R, theta, offsets)
    cache = _fill(r, (B, 2, Hkv, cap, D), cache_fill)
    return Contig("packed", style, B, S, Hq, Hkv, D, R, cap, cos_sin, qkv, cache, name=name)


def continuous(B, S, Hq, Hkv, D, R, cap, style, seed, end_lo, end_hi, theta=10000.0,
               table_len=None, cache_fill="normal", table_batch=1, name="") -> Contig:
    """Call-2 inputs.  ``table_batch`` B gives each sequence its own table
    (sequence b's positions offset by 5*b), 1 a shared one."""
    r = rng(seed)
    tlen = cap if table_len is None else table_len
    qkv = normal_f16(r, (B, S, Hq + 2 * Hkv, D))
    end = r.integers(end_lo, end_hi + 1, size=B).astype(np.int32)
    cos_sin = rope_table(table_batch, tlen, R, theta, offsets=5 * np.arange(table_batch))
    cache = _fill(r, (B, 2, Hkv, cap, D), cache_fill)
    q_out = sentinel_f16((B, S, Hq, D))
    return Contig("continuous", style, B, S, Hq, Hkv, D, R, cap, cos_sin, qkv, cache,
                  q_out=q_out, end_lens=end, name=name)


def tree(B, S, Hq, Hkv, D, R, cap, style, seed, end_lo, end_hi, theta=10000.0,
         max_depth=8, cache_fill="normal", table_batch=1, name="") -> Contig:
    """Call-3 inputs: one seeded random tree per sequence, positions
    end - S + depth; ``table_batch`` as for ``continuous``."""
    r = rng(seed)
    qkv = normal_f16(r, (B, S, Hq + 2 * Hkv, D))
    end = r.integers(end_lo, end_hi + 1, size=B).astype(np.int32)
    pos = np.empty((B, S), dtype=np.int32)
    for b in range(B):
        pos[b] = end[b] - S + random_tree_depths(r, S, max_depth)
    cos_sin = rope_table(table_batch, cap, R, theta, offsets=5 * np.arange(table_batch))
    cache = _fill(r, (B, 2, Hkv, cap, D), cache_fill)
    q_out = sentinel_f16((B, S, Hq, D))
    return Contig("tree", style, B, S, Hq, Hkv, D, R, cap, cos_sin, qkv, cache,
                  q_out=q_out, end_lens=end, pos_ids=pos, name=name)


def paged(N, batch, Hkv, D, R, num_pages, max_pages, style, seed, theta=10000.0,
          width=None, pad_frac=0.10, bad_frac=0.05, pool_fill="normal", name="") -> Paged:
    """Paged-delta inputs.

    Rows are grouped ``width`` per sequence (row i -> sequence i // width,
    slot j = i % width).  Sequence b has ``deltaLen_b`` valid rows; the rest
    are padding with both index arrays -1, about ``pad_frac`` of all rows.
    Valid rows sit at ``pos = old_b + j``.  The page table maps the K plane to
    a random permutation of [0, numPages) and the V plane to numPages + a
    second permutation; ``bad_frac`` of its entries are replaced, in equal
    thirds, by -1, the other plane's id, or an id >= 2*numPages.
    """
    r = rng(seed)
    if width is None:
        width = max(1, N // max(batch, 1))
    cap_tokens = max_pages * TOKENS_PER_PAGE
    seq = np.full(N, -1, dtype=np.int32)
    pos = np.full(N, -1, dtype=np.int32)
    n_seq_rows = min(batch, (N + width - 1) // width)
    max_pad = int(round(2 * pad_frac * width))
    for b in range(n_seq_rows):
        lo, hi = b * width, min(N, (b + 1) * width)
        dlen = (hi - lo) - int(r.integers(0, max_pad + 1))
        dlen = max(dlen, 0)
        old = int(r.integers(0, max(cap_tokens - width, 0) + 1))
        seq[lo:lo + dlen] = b
        pos[lo:lo + dlen] = old + np.arange(dlen, dtype=np.int32)
    n_entries = batch * max_pages
    k_ids = r.permutation(num_pages)[:n_entries] if n_entries <= num_pages else \
        r.integers(0, num_pages, n_entries)
    v_ids = num_pages + (r.permutation(num_pages)[:n_entries] if n_entries <= num_pages else
                         r.integers(0, num_pages, n_entries))
    pt = np.empty((batch, 2, max_pages), dtype=np.int64)
    pt[:, 0, :] = k_ids.reshape(batch, max_pages)
    pt[:, 1, :] = v_ids.reshape(batch, max_pages)
    flat = pt.reshape(-1)
    n_bad = int(round(bad_frac * flat.size))
    bad = r.choice(flat.size, size=n_bad, replace=False)
    for t, idx in enumerate(bad):
        plane = (idx // max_pages) % 2
        kind = t % 3
        if kind == 0:
            flat[idx] = -1
        elif kind == 1:   # a page id from the other plane
            flat[idx] = (num_pages + int(r.integers(0, num_pages))) if plane == 0 else \
                int(r.integers(0, num_pages))
        else:             # beyond both planes
            flat[idx] = 2 * num_pages + int(r.integers(0, 1 << 20))
    page_table = pt.astype(np.int32)
    k_delta = normal_f16(r, (N, Hkv, D))
    v_delta = normal_f16(r, (N, Hkv, D))
    cos_sin = rope_rows(pos, R, theta)
    pool = _fill(r, (2, num_pages, TOKENS_PER_PAGE, Hkv, D), pool_fill)
    return Paged(style, N, batch, Hkv, D, R, num_pages, max_pages, k_delta, v_delta, pool,
                 cos_sin, pos, seq, page_table, name=name)


_TILE = 1 << 24


def with_fp8_cache(w, seed: int, k_scale=K_SCALE, v_scale=V_SCALE, fill="bits"):
    """The same workload with an E4M3 cache (pool): ``uint8`` bytes, filled
    with seeded random bytes (``"bits"``) or the NaN sentinel, and fp32
    per-tensor scales in ``extra["fp8"]`` (None means no scale)."""
    r = rng(seed)
    shape = w.pool.shape if hasattr(w, "pool") else w.cache.shape
    if fill == "sentinel":
        buf = np.full(shape, SENTINEL8, dtype=np.uint8)
    elif fill == "bits":
        n = int(np.prod(shape, dtype=np.int64))
        if n <= _TILE:
            buf = r.integers(0, 256, size=n, dtype=np.uint8).reshape(shape)
        else:
            block = r.integers(0, 256, size=_TILE, dtype=np.uint8)
            buf = np.resize(block, n).reshape(shape)
    else:
        raise ValueError(fill)
    if hasattr(w, "pool"):
        w.pool = buf
    else:
        w.cache = buf
    w.extra["fp8"] = {"k_scale": None if k_scale is None else np.float32(k_scale),
                      "v_scale": None if v_scale is None else np.float32(v_scale)}
    w.name = (w.name + "_fp8") if w.name else "fp8"
    return w


def paged_gather(N, batch, Hkv, D, R, num_pages, max_pages, style, seed, rope_states=1,
                 rope_rows=None, theta=10000.0, state_indices=True, width=None, pad_frac=0.10,
                 bad_frac=0.05, pool_fill="normal", name="") -> Paged:
    """Inputs of the paged update with the cos/sin gather fused in: the paged
    workload plus a rope table [rope_states, rope_rows, R] (state k holds
    positions offset by 7*k) and, optionally, per-sequence state indices
    (a seeded draw in [0, rope_states))."""
    w = paged(N, batch, Hkv, D, R, num_pages, max_pages, style, seed, theta=theta, width=width,
              pad_frac=pad_frac, bad_frac=bad_frac, pool_fill=pool_fill, name=name)
    r = rng(seed + 7)
    rows = max_pages * TOKENS_PER_PAGE if rope_rows is None else rope_rows
    w.extra["gather"] = True
    w.extra["rope"] = rope_table(rope_states, rows, R, theta,
                                 offsets=7 * np.arange(rope_states))
    w.extra["state_indices"] = (r.integers(0, rope_states, size=batch).astype(np.int32)
                                if state_indices else None)
    return w


def with_qk_norm(w, seed: int, eps: float = 1e-6, q_weight=True, k_weight=True, scale=1.0):
    """The same workload (calls 1-3) with Q/K RMS norm before the rotation:
    fp32 per-dimension weights [D] drawn seeded around 1 (0.5 + U[0, 1)), or
    None for a side that is not normalised; ``scale`` multiplies the packed
    activations (held in fp16) so that the norm has something to undo."""
    r = rng(seed)
    qw = (0.5 + r.random(w.D)).astype(np.float32) if q_weight else None
    kw = (0.5 + r.random(w.D)).astype(np.float32) if k_weight else None
    if scale != 1.0:
        x = w.qkv.view(np.float16).astype(np.float32) * np.float32(scale)
        w.qkv = x.astype(np.float16).view(np.uint16)
    w.extra["qknorm"] = {"q_weight": qw, "k_weight": kw, "eps": float(np.float32(eps))}
    w.name = (w.name + "_qknorm") if w.name else "qknorm"
    return w


def _fill(r, shape, how):
    if how == "none":   # no cache / pool: for callers that need only the index arrays
        return np.empty((0,), dtype=np.uint16)
    if how == "sentinel":
        return sentinel_f16(shape)
    if how == "normal":
        # Large caches and pools repeat a seeded 2^24-element block: every
        # slot still holds an ordinary N(0,1) value that a stray write would
        # change, and the fill stays cheap at gigabyte sizes.
        n = int(np.prod(shape, dtype=np.int64))
        if n <= _TILE:
            return normal_f16(r, shape)
        block = normal_f16(r, (_TILE,))
        return np.resize(block, n).reshape(shape)
    if how == "bits":   # arbitrary bit patterns, NaNs included
        n = int(np.prod(shape, dtype=np.int64))
        return r.integers(0, 1 << 16, size=n, dtype=np.uint16).reshape(shape)
    raise ValueError(how)


def config(idx: int, style: int | None = None):
    """The five workloads, 1-based.  Workload 2 takes ``style`` (NeoX default)."""
    if idx == 1:   # empty-cache prefill, tiny
        return packed(1, 16, 4, 2, 64, 64, 32, NEOX, 1001, table_len=32,
                      name="prefill_tiny_b1_s16_d64")
    if idx == 2:   # continuous write into a non-empty cache
        st = NEOX if style is None else style
        return continuous(8, 128, 32, 8, 128, 128, 4096, st, 1002, 128, 4096,
                          theta=500000.0,
                          name=f"continuous_b8_s128_d128_{'neox' if st == NEOX else 'gptj'}")
    if idx == 3:   # tree decoding, partial rotary
        return tree(16, 64, 32, 8, 128, 64, 8192, NEOX, 1003, 512, 8192,
                    name="tree_b16_s64_d128_r64")
    if idx == 4:   # paged delta update
        return paged(4096, 32, 8, 128, 128, 8192, 128, NEOX, 1004,
                     name="paged_delta_n4096_p8192")
    if idx == 41:  # paged delta update with the cos/sin gather fused in
        return paged_gather(4096, 32, 8, 128, 128, 8192, 128, NEOX, 1004, rope_states=1,
                            state_indices=False, name="paged_delta_gather_n4096_p8192")
    if idx == 5:   # large prefill
        r = rng(10050)
        offs = np.concatenate([[0], r.integers(1, 8193, size=3)])
        return packed(4, 8192, 64, 8, 128, 128, 16384, GPTJ, 1005, table_batch=4,
                      table_len=8192, offsets=offs, name="prefill_b4_s8192_h64_d128")
    raise ValueError(idx)


def prefill_tp_shard(tp: int):
    """One GPU's share of the large prefill under tensor parallelism of degree
    ``tp``: the same sequences, positions and tables, Hq/tp query heads and
    Hkv/tp KV heads (the cache is head-sharded the same way)."""
    assert 64 % tp == 0 and 8 % tp == 0, tp
    r = rng(10050)
    offs = np.concatenate([[0], r.integers(1, 8193, size=3)])
    return packed(4, 8192, 64 // tp, 8 // tp, 128, 128, 16384, GPTJ, 1005 + 10 * tp,
                  table_batch=4, table_len=8192, offsets=offs,
                  name=f"prefill_tp{tp}_shard_b4_s8192_h{64 // tp}_kv{8 // tp}_d128")
