"""The parity harness's write sets, pinned to the oracle (CPU).

The GPU parity tests hold every element outside a call's computed Q/K
elements to bit equality, and find those elements through write sets the
harness derives from end lengths, position ids and page ids (harness.
``written_slots``, ``written_tokens``, ``written_pool_rows``).  Here each
derivation is checked against what the oracle itself writes: the oracle runs
twice, on an output buffer filled with F and on one filled with the bitwise
complement of F; the calls only write their outputs, never read them, so an
element is written exactly when both runs leave the same value there.  The
workloads cover every skip rule: end lengths and positions outside the
cache and the table, padding rows, inactive sequences, positions past the
page table, unmapped and other-plane page ids, missing rope-table states.
"""
import copy

import numpy as np
import pytest

import oracle
import workloads as W
from harness import written_pool_rows, written_slots, written_tokens

NEOX, GPTJ = W.NEOX, W.GPTJ


def _twice(w, key):
    """Oracle output `key` for fill F and for fill ~F, and the written mask."""
    fill = getattr(w, "pool" if key == "pool" else key)
    a = copy.copy(w)
    b = copy.copy(w)
    setattr(b, "pool" if key == "pool" else key, np.invert(fill))
    if key == "q_out":
        ra, rb = oracle.run(a)["q_out"], oracle.run(b)["q_out"]
    else:
        k = "pool" if key == "pool" else "cache"
        ra, rb = oracle.run(a)[k], oracle.run(b)[k]
    return ra == rb


def _contig_cases():
    r = np.random.default_rng(44)
    B, S, Hq, Hkv, D, cap = 6, 8, 4, 2, 64, 20
    out = [W.packed(2, 24, 4, 2, 64, 64, 40, NEOX, 3, name="packed")]
    w = W.continuous(B, S, Hq, Hkv, D, D, cap, NEOX, 45, 8, 20, table_len=16, name="cont_oor")
    w.end_lens[:] = np.array([3, 8, 20, 25, -100, 2 ** 31 - 1], dtype=np.int32)
    out.append(w)
    w = W.tree(B, S, Hq, Hkv, D, 32, cap, GPTJ, 46, 8, 20, name="tree_oor")
    w.end_lens[:] = np.array([3, 8, 20, 25, -2 ** 31, 12], dtype=np.int32)
    w.pos_ids[0, :] = r.integers(-5, 5, S)
    w.pos_ids[1, :] = np.array([-1, 0, 19, 20, 21, 2 ** 31 - 1, -2 ** 31, 5])
    out.append(w)
    w = W.with_qk_norm(W.continuous(B, S, Hq, Hkv, D, 32, cap, GPTJ, 47, 4, 22, table_len=18,
                                    name="cont_norm_q_only"), 48, k_weight=False)
    out.append(w)
    out.append(W.with_fp8_cache(W.tree(B, S, Hq, Hkv, D, 64, cap, NEOX, 49, 2, 24,
                                       name="tree_fp8"), 50))
    return out


@pytest.mark.parametrize("w", _contig_cases(), ids=lambda w: w.name)
def test_contiguous_write_set(w):
    written = _twice(w, "cache")                       # [B, 2, Hkv, cap, D]
    rows = written.all(axis=(1, 2, 4))
    assert np.array_equal(rows, written.any(axis=(1, 2, 4))), "partly written slot"
    assert np.array_equal(rows, written_slots(w))
    assert rows.any() and not rows.all() or w.call == "packed"
    if w.call != "packed":
        q = _twice(w, "q_out")                         # [B, S, Hq, D]
        ok, _ = written_tokens(w)
        assert np.array_equal(q.all(axis=(2, 3)), ok)
        assert np.array_equal(q.any(axis=(2, 3)), ok)


def _paged_cases():
    out = []
    w = W.paged(512, 8, 2, 64, 64, 96, 8, NEOX, 77, width=64, name="paged_skips")
    r = np.random.default_rng(78)
    k = r.choice(w.N, 60, replace=False)
    w.positions[k[:10]] = -1
    w.seq[k[10:20]] = -3
    w.seq[k[20:30]] = 6
    w.positions[k[30:40]] = w.max_pages * 64
    w.positions[k[40:50]] = 2 ** 31 - 1
    w.batch = 6
    out.append(w)
    out.append(W.paged(300, 7, 3, 64, 32, 64, 9, GPTJ, 5064, width=43, pad_frac=0.2,
                       bad_frac=0.2, name="paged_bad_ids"))
    w = W.paged_gather(300, 7, 3, 64, 64, 64, 9, NEOX, 6064, rope_states=3, rope_rows=9 * 64 - 50,
                       width=43, pad_frac=0.2, bad_frac=0.2, name="gather_states")
    w.extra["state_indices"][1] = 3
    w.extra["state_indices"][2] = -1
    out.append(w)
    out.append(W.with_fp8_cache(W.paged(300, 7, 2, 64, 64, 64, 9, NEOX, 5065, width=43,
                                        pad_frac=0.2, bad_frac=0.2, name="paged_fp8"), 51))
    return out


@pytest.mark.parametrize("w", _paged_cases(), ids=lambda w: w.name)
def test_paged_write_set(w):
    written = _twice(w, "pool")                         # [2, P, 64, Hkv, D]
    rows = written.all(axis=(3, 4))
    assert np.array_equal(rows, written.any(axis=(3, 4))), "partly written pool row"
    tk, tv = written_pool_rows(w)
    assert np.array_equal(rows[0], tk)
    assert np.array_equal(rows[1], tv)
    assert tk.any() and tv.any()


def _bump(a, idx):
    """One fp16 ulp away (toward larger magnitude), as a stray write would be."""
    b = a.copy()
    b[idx] = np.uint16(int(b[idx]) + 1)
    return b


def test_compare_holds_unwritten_k_slots_to_bit_equality():
    """A one-ulp change passes inside the write set (default arithmetic's
    tolerance) and fails in a K-plane slot, a qOut row or a pool K row the
    call does not write."""
    from harness import compare, expected
    w = _contig_cases()[1]                                 # continuous, tokens skipped
    want = expected(w)
    ok, slot = written_tokens(w)
    rows = written_slots(w)
    b_w, s_w = map(int, np.argwhere(ok)[0])
    inside = (b_w, 0, 1, int(slot[b_w, s_w]), 3)
    rep = compare(w, {**want, "cache": _bump(want["cache"], inside)}, want)
    assert rep["cache"] == 1 and rep["cache_max_ulp"] == 1
    b_u, c_u = map(int, np.argwhere(~rows)[0])
    with pytest.raises(AssertionError, match="outside the computed"):
        compare(w, {**want, "cache": _bump(want["cache"], (b_u, 0, 1, c_u, 3))}, want)
    b_s, s_s = map(int, np.argwhere(~ok)[0])
    with pytest.raises(AssertionError, match="outside the computed"):
        compare(w, {**want, "q_out": _bump(want["q_out"], (b_s, s_s, 0, 0))}, want)
    p = _paged_cases()[0]
    want = expected(p)
    tk, _ = written_pool_rows(p)
    pg, off = map(int, np.argwhere(~tk)[0])
    with pytest.raises(AssertionError, match="outside the computed"):
        compare(p, {"pool": _bump(want["pool"], (0, pg, off, 0, 0))}, want)
    pg, off = map(int, np.argwhere(tk)[0])
    assert compare(p, {"pool": _bump(want["pool"], (0, pg, off, 0, 0))}, want)["pool"] == 1
