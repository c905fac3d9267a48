"""Run a seeded workload through the HIP library and compare with the oracle.

Used by the GPU parity tests, ``__graft_entry__.smoke()`` and ``bench.py``.
Moving arrays to and from the device and calling the binding is all it does;
every step of the computation runs in the library's kernels.

Comparison rules:
* every element that is not a rotated Q/K output inside the call's write set
  (V copies, passthrough dims >= R, every cache slot, pool row and qOut row
  the call does not write, derived from its end lengths, position ids and
  page ids by the skip rules: ``computed_at``) must match the oracle bit for
  bit;
* rotated Q/K elements must satisfy |gpu - ref| <= 2^-10*|ref| + 1e-3
  (non-finite values must match in kind);
* ``compare`` also counts rotated elements whose bits differ and their
  largest distance in fp16 ulps, so that a test can require bit equality
  (the library's RKV_ROUND_EXACT mode) or at most one ulp (its default
  binary32 arithmetic);
* an fp8 (E4M3) cache or pool: bytes outside the write set must match the
  oracle bit for bit; written bytes must be within one code step of the
  oracle's (both NaN counts as equal), and the count and largest step are
  reported so that a test can require bit equality.
"""
from __future__ import annotations

import numpy as np
import torch

import workloads as W

TOKENS_PER_PAGE = W.TOKENS_PER_PAGE
TOL_REL = 2.0 ** -10
TOL_ABS = 1e-3


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


def host8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint8)


def _scale_tensor(v, device):
    return None if v is None else torch.tensor([float(v)], dtype=torch.float32, device=device)


def is_fp8(w) -> bool:
    return bool(w.extra.get("fp8"))


def upload(w, device="cuda") -> dict:
    if isinstance(w, W.Paged):
        t = {"k_delta": dev(w.k_delta, device), "v_delta": dev(w.v_delta, device),
             "pool": dev(w.pool, device), "cos_sin": dev(w.cos_sin, device),
             "positions": dev(w.positions, device), "seq": dev(w.seq, device),
             "page_table": dev(w.page_table, device)}
        if w.extra.get("gather"):
            t["rope"] = dev(w.extra["rope"], device)
            si = w.extra["state_indices"]
            t["state_indices"] = None if si is None else dev(si, device)
        _upload_scales(w, t, device)
        return t
    t = {"cos_sin": dev(w.cos_sin, device), "qkv": dev(w.qkv, device),
         "cache": dev(w.cache, device)}
    _upload_scales(w, t, device)
    if w.call != "packed":
        t["q_out"] = dev(w.q_out, device)
        t["end_lens"] = dev(w.end_lens, device)
    if w.call == "tree":
        t["pos_ids"] = dev(w.pos_ids, device)
    return t


def _upload_scales(w, t, device):
    if is_fp8(w):
        t["k_scale"] = _scale_tensor(w.extra["fp8"]["k_scale"], device)
        t["v_scale"] = _scale_tensor(w.extra["fp8"]["v_scale"], device)
    norm = w.extra.get("qknorm")
    if norm:
        for key in ("q_weight", "k_weight"):
            t[key] = None if norm[key] is None else dev(norm[key], device)


def launch(w, t: dict, exact: bool = False) -> None:
    """One call of the library on the uploaded workload; ``exact`` ORs
    ROUND_EXACT into the rope style (binary64, correctly rounded)."""
    import rope_kv_cache_amd as rkv
    style = w.style | (rkv.ROUND_EXACT if exact else 0)
    if w.extra.get("qknorm"):
        _launch_qknorm(rkv, w, t, style)
        return
    if is_fp8(w):
        _launch_fp8(rkv, w, t, style)
        return
    if isinstance(w, W.Paged) and w.extra.get("gather"):
        rkv.dflash_target_kv_cache_update_gather_rope(t["k_delta"], t["v_delta"], t["pool"],
                                                      t["rope"], t["state_indices"],
                                                      t["positions"], t["seq"], t["page_table"],
                                                      w.batch, style)
    elif isinstance(w, W.Paged):
        rkv.dflash_target_kv_cache_update(t["k_delta"], t["v_delta"], t["pool"], t["cos_sin"],
                                          t["positions"], t["seq"], t["page_table"], w.batch,
                                          style)
    elif w.call == "packed":
        rkv.apply_rope_write_kv_packed_qkv(t["cos_sin"], t["qkv"], t["cache"], style)
    elif w.call == "continuous":
        rkv.apply_rope_write_kv_continuous(t["cos_sin"], t["end_lens"], t["qkv"], t["cache"],
                                           t["q_out"], style)
    else:
        rkv.apply_rope_write_kv_tree(t["cos_sin"], t["end_lens"], t["pos_ids"], t["qkv"],
                                     t["cache"], t["q_out"], style)


def _launch_fp8(rkv, w, t, style):
    ks, vs = t["k_scale"], t["v_scale"]
    if isinstance(w, W.Paged) and w.extra.get("gather"):
        rkv.dflash_target_kv_cache_update_gather_rope_fp8(
            t["k_delta"], t["v_delta"], t["pool"], ks, vs, t["rope"], t["state_indices"],
            t["positions"], t["seq"], t["page_table"], w.batch, style)
    elif isinstance(w, W.Paged):
        rkv.dflash_target_kv_cache_update_fp8(t["k_delta"], t["v_delta"], t["pool"], ks, vs,
                                              t["cos_sin"], t["positions"], t["seq"],
                                              t["page_table"], w.batch, style)
    elif w.call == "packed":
        rkv.apply_rope_write_kv_packed_qkv_fp8(t["cos_sin"], t["qkv"], t["cache"], ks, vs, style)
    elif w.call == "continuous":
        rkv.apply_rope_write_kv_continuous_fp8(t["cos_sin"], t["end_lens"], t["qkv"], t["cache"],
                                               t["q_out"], ks, vs, style)
    else:
        rkv.apply_rope_write_kv_tree_fp8(t["cos_sin"], t["end_lens"], t["pos_ids"], t["qkv"],
                                         t["cache"], t["q_out"], ks, vs, style)


def _launch_qknorm(rkv, w, t, style):
    eps = w.extra["qknorm"]["eps"]
    ks, vs = (t["k_scale"], t["v_scale"]) if is_fp8(w) else (None, None)
    qw, kw = t["q_weight"], t["k_weight"]
    if w.call == "packed":
        rkv.apply_rope_write_kv_packed_qkv_qknorm(t["cos_sin"], t["qkv"], t["cache"], qw, kw, eps,
                                                  style, ks, vs)
    elif w.call == "continuous":
        rkv.apply_rope_write_kv_continuous_qknorm(t["cos_sin"], t["end_lens"], t["qkv"],
                                                  t["cache"], t["q_out"], qw, kw, eps, style, ks,
                                                  vs)
    else:
        rkv.apply_rope_write_kv_tree_qknorm(t["cos_sin"], t["end_lens"], t["pos_ids"], t["qkv"],
                                            t["cache"], t["q_out"], qw, kw, eps, style, ks, vs)


def download(w, t: dict) -> dict:
    torch.cuda.synchronize()
    cache_host = host8 if is_fp8(w) else host16
    if isinstance(w, W.Paged):
        return {"pool": cache_host(t["pool"])}
    out = {"cache": cache_host(t["cache"])}
    if w.call == "packed":
        out["qkv"] = host16(t["qkv"])
    else:
        out["q_out"] = host16(t["q_out"])
        out["qkv"] = host16(t["qkv"])      # must be unchanged
    return out


def run_gpu(w, device="cuda", exact: bool = False) -> dict:
    t = upload(w, device)
    launch(w, t, exact)
    return download(w, t)


def expected(w, L=None) -> dict:
    import oracle
    want = oracle.run(w, L=L)
    if not isinstance(w, W.Paged) and w.call != "packed":
        want["qkv"] = w.qkv          # calls 2 and 3 never write qkv
    return want


def written_tokens(w):
    """Calls 1-3: ([B, S] bool, [B, S] int64) -- which tokens the call
    writes and the cache slot of each.  Call 1 writes every token at slot s;
    calls 2 and 3 place token s at end - S + s and skip it when that slot is
    outside [0, cap) or its position outside the table (the skip rules of
    the pages' statement, as the oracle and the kernels apply them)."""
    tlen = w.cos_sin.shape[1]
    if w.call == "packed":
        slot = np.broadcast_to(np.arange(w.S, dtype=np.int64), (w.B, w.S))
        return np.ones((w.B, w.S), dtype=bool), slot
    slot = w.end_lens.astype(np.int64)[:, None] - w.S + np.arange(w.S, dtype=np.int64)[None, :]
    pos = slot if w.call == "continuous" else w.pos_ids.astype(np.int64)
    ok = (slot >= 0) & (slot < w.cap) & (pos >= 0) & (pos < tlen)
    return ok, slot


def written_slots(w) -> np.ndarray:
    """Calls 1-3: [B, cap] bool, the cache slots (both planes) the call writes."""
    ok, slot = written_tokens(w)
    t = np.zeros((w.B, w.cap), dtype=bool)
    b = np.broadcast_to(np.arange(w.B)[:, None], ok.shape)
    t[b[ok], slot[ok]] = True
    return t


def written_pool_rows(w):
    """Call 4: ([numPages, 64] bool, [numPages, 64] bool) -- the K-plane and
    V-plane page slots the call writes: rows that are not padding, whose
    sequence is active and position inside the page table, through page ids
    inside their own plane (and, with the cos/sin gather fused in, with a
    rope-table row for K)."""
    P = w.num_pages
    p = w.positions.astype(np.int64)
    q = w.seq.astype(np.int64)
    live = (p >= 0) & (q >= 0) & (q < w.batch) & (p < w.max_pages * TOKENS_PER_PAGE)
    lp = np.where(live, p // TOKENS_PER_PAGE, 0)
    qq = np.where(live, q, 0)
    off = np.where(live, p % TOKENS_PER_PAGE, 0)
    kid = w.page_table[qq, 0, lp].astype(np.int64)
    vid = w.page_table[qq, 1, lp].astype(np.int64)
    k_ok = live & (kid >= 0) & (kid < P)
    v_ok = live & (vid >= P) & (vid < 2 * P)
    if w.extra.get("gather"):
        rope = w.extra["rope"]
        si = w.extra["state_indices"]
        st = si[qq].astype(np.int64) if si is not None else \
            (np.zeros_like(qq) if rope.shape[0] == 1 else qq)
        k_ok &= (st >= 0) & (st < rope.shape[0]) & (p < rope.shape[1])
    tk = np.zeros((P, TOKENS_PER_PAGE), dtype=bool)
    tv = np.zeros((P, TOKENS_PER_PAGE), dtype=bool)
    tk[kid[k_ok], off[k_ok]] = True
    tv[vid[v_ok] - P, off[v_ok]] = True
    return tk, tv


def _dims(w):
    """(dims of a Q row, dims of a K row) that hold computed values: the
    rotary dims, or all D of a head normalised by the Q/K norm."""
    norm = w.extra.get("qknorm") or {}
    rq = w.D if norm.get("q_weight") is not None else w.R
    rk = w.D if norm.get("k_weight") is not None else w.R
    return rq, rk


def computed_at(w, key, where) -> np.ndarray:
    """For the elements of output `key` at index arrays `where` (as returned
    by np.nonzero), whether each holds a value the call computes rather
    than copies: rotated (or normalised) Q and K elements inside the write
    set, and with an E4M3 cache every cache element the call writes (V too
    is scaled and rounded there).  Everything else -- V copies, passthrough
    dims, slots, rows and pages the call does not write -- must match the
    oracle bit for bit."""
    rq, rk = _dims(w)
    fp8 = is_fp8(w)
    if key == "pool":
        plane, page, off, _, d = where
        tk, tv = written_pool_rows(w)
        k_row = (plane == 0) & tk[page, off]
        if fp8:
            return k_row | ((plane == 1) & tv[page, off])
        return k_row & (d < rk)
    if key == "cache":
        b, plane, _, slot, d = where
        rows = written_slots(w)[b, slot]
        if fp8:
            return rows
        return rows & (plane == 0) & (d < rk)
    if key == "q_out":
        b, s_, _, d = where
        ok, _ = written_tokens(w)
        return ok[b, s_] & (d < rq)
    if key == "qkv":
        if w.call != "packed":
            return np.zeros(where[0].shape, dtype=bool)
        _, _, h, d = where
        return ((h < w.Hq) & (d < rq)) | ((h >= w.Hq) & (h < w.Hq + w.Hkv) & (d < rk))
    raise KeyError(key)


def _within_tol(g: np.ndarray, r: np.ndarray) -> np.ndarray:
    gv = g.view(np.float16).astype(np.float64)
    rv = r.view(np.float16).astype(np.float64)
    fin = np.isfinite(rv) & np.isfinite(gv)
    ok = np.zeros(g.shape, dtype=bool)
    ok[fin] = np.abs(gv[fin] - rv[fin]) <= TOL_REL * np.abs(rv[fin]) + TOL_ABS
    both_nan = np.isnan(gv) & np.isnan(rv)
    same_inf = np.isinf(gv) & np.isinf(rv) & (gv == rv)
    return ok | both_nan | same_inf


def _is_nan16(x: np.ndarray) -> np.ndarray:
    return ((x & 0x7C00) == 0x7C00) & ((x & 0x3FF) != 0)


INFO_SUFFIXES = ("_max_ulp", "_max_ulp_ge_2m6", "_max_code_step", "_nan_bits_differ",
                 "_nan_sign_differs")


def exact_diffs(rep: dict) -> dict:
    """Counts of elements that differ from the oracle (informational keys
    such as ulp maxima and NaN sign differences left out)."""
    return {k: v for k, v in rep.items() if not k.endswith(INFO_SUFFIXES) and v}


def _ulps(g: np.ndarray, r: np.ndarray) -> np.ndarray:
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(ordered(g) - ordered(r))


def _e4m3_steps(g: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Distance in E4M3 code steps (+0 and -0 are 0 steps apart)."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x80, -(x & 0x7F), x)
    return np.abs(ordered(g) - ordered(r))


def _is_nan8(x: np.ndarray) -> np.ndarray:
    return (x & 0x7F) == 0x7F


def _compare_fp8(w, key, g, ref, report):
    diff = g != ref
    if not diff.any():
        report[key] = 0
        return
    where = np.nonzero(diff)
    written = computed_at(w, key, where)
    if not written.all():
        k = int(np.argmin(written))
        idx = tuple(int(a[k]) for a in where)
        raise AssertionError(f"{w.name}: {key}{list(idx)} differs outside the bytes the call "
                             f"writes: gpu {g[idx]:#04x} oracle {ref[idx]:#04x} "
                             f"({int((~written).sum())} such bytes)")
    gd, rd = g[where], ref[where]
    both_nan = _is_nan8(gd) & _is_nan8(rd)
    steps = np.where(both_nan, 0, _e4m3_steps(gd, rd))
    steps = np.where(_is_nan8(gd) ^ _is_nan8(rd), 999, steps)
    if steps.max() > 1:
        k = int(np.argmax(steps))
        idx = tuple(int(a[k]) for a in where)
        raise AssertionError(f"{w.name}: {key}{list(idx)} more than one E4M3 step from the "
                             f"oracle: gpu {gd[k]:#04x} oracle {rd[k]:#04x} "
                             f"({int((steps > 1).sum())} such bytes)")
    report[key] = int((steps > 0).sum())
    report[key + "_max_code_step"] = int(steps.max())
    report[key + "_nan_sign_differs"] = int(both_nan.sum())


def compare(w, got: dict, want: dict) -> dict:
    """Assert the parity rules; return {key: n_rotated_bit_differences}."""
    report = {}
    for key, ref in want.items():
        g = got[key]
        assert g.shape == ref.shape, (key, g.shape, ref.shape)
        if ref.dtype == np.uint8:
            _compare_fp8(w, key, g, ref, report)
            continue
        diff = g != ref
        if not diff.any():
            report[key] = 0
            continue
        where = np.nonzero(diff)
        rot = computed_at(w, key, where)
        if not rot.all():
            k = int(np.argmin(rot))
            idx = tuple(int(a[k]) for a in where)
            raise AssertionError(
                f"{w.name}: {key}{list(idx)} differs outside the computed Q/K elements the call "
                f"writes: gpu {g[idx]:#06x} oracle {ref[idx]:#06x} ({int((~rot).sum())} such "
                f"elements)")
        gd, rd = g[where], ref[where]
        # computed NaN results match as NaN: IEEE 754 leaves the sign (and
        # payload) of a NaN produced by an invalid operation unspecified
        nan_pair = _is_nan16(gd) & _is_nan16(rd)
        if nan_pair.any():
            report[key + "_nan_bits_differ"] = int(nan_pair.sum())
            keep = ~nan_pair
            where = tuple(a[keep] for a in where)
            gd, rd = gd[keep], rd[keep]
            if gd.size == 0:
                report[key] = 0
                continue
        tol_ok = _within_tol(gd, rd)
        if not tol_ok.all():
            k = int(np.argmin(tol_ok))
            idx = tuple(int(a[k]) for a in where)
            raise AssertionError(
                f"{w.name}: {key}{list(idx)} outside tolerance: gpu {gd[k]:#06x} "
                f"oracle {rd[k]:#06x}")
        report[key] = int(diff.sum())
        ulps = _ulps(gd, rd)
        report[key + "_max_ulp"] = int(ulps.max())
        big = np.abs(rd.view(np.float16).astype(np.float64)) >= 2.0 ** -6
        report[key + "_max_ulp_ge_2m6"] = int(ulps[big].max()) if big.any() else 0
    return report
