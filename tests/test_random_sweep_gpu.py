"""Seeded random combinations of every call's options against the CPU oracle.

The other GPU tests walk one option at a time; here each case draws all of
them at once from its own seed: the call (1-4, or 4 with the gather fused),
head dimension, rotary dimension, layout, head counts, batch and length, a
shared or per-sequence table, a table shorter than the cache, end lengths
that push some tokens out of range, the cache dtype (fp16 or E4M3, with or
without scales), the Q/K norm (either weight absent, several epsilons and
input scales) and, for the paged update, page tables with unmapped ids,
positions past the table, rope states with and without state indices.
Every case runs in both arithmetic modes under the parity bar of the other
GPU tests: bit-identical with RKV_ROUND_EXACT, within one fp16 ulp (one
E4M3 code step) in the default mode (for Q/K-norm cases, one ulp wherever
|ref| >= 2^-6).
"""
import numpy as np
import pytest

import workloads as W
from harness import compare, exact_diffs, expected, run_gpu

pytestmark = pytest.mark.gpu

N_CASES = 10000


def _rotary_dim(r, D):
    return int(r.choice(np.arange(0, D + 1, 16)))


def _contig_case(r, k, call):
    D = int(r.choice([64, 128, 256]))
    R = _rotary_dim(r, D)
    style = int(r.integers(0, 2))
    B, S = int(r.integers(1, 5)), int(r.integers(1, 41))
    Hq, Hkv = int(r.integers(0, 11)), int(r.integers(0, 5))
    if Hq + Hkv == 0:
        Hq = 1
    tb = int(r.choice([1, B]))
    seed = 12000 + k
    name = f"sweep{k}_{call}_B{B}_S{S}_Hq{Hq}_Hkv{Hkv}_D{D}_R{R}_s{style}_tb{tb}"
    if call == "packed":
        cap = S + int(r.integers(0, 31))
        tlen = int(r.integers(S, cap + 11))
        offs = r.integers(0, 50, size=tb)
        w = W.packed(B, S, Hq, Hkv, D, R, cap, style, seed, table_batch=tb, table_len=tlen,
                     offsets=offs, name=name)
    elif call == "continuous":
        cap = S + int(r.integers(0, 61))
        tlen = cap if r.integers(0, 3) else int(r.integers(1, cap + 6))
        w = W.continuous(B, S, Hq, Hkv, D, R, cap, style, seed, max(0, S - 6), cap + 3,
                         table_len=tlen, table_batch=tb, name=name)
    else:
        cap = S + int(r.integers(0, 61))
        w = W.tree(B, S, Hq, Hkv, D, R, cap, style, seed, max(0, S - 6), cap + 3,
                   table_batch=tb, name=name)
    flavour = str(r.choice(["fp16", "fp8", "norm", "norm_fp8"]))
    if flavour.startswith("norm"):
        W.with_qk_norm(w, seed + 1, eps=float(r.choice([0.0, 1e-6, 1e-2])),
                       q_weight=bool(r.integers(0, 4)), k_weight=bool(r.integers(0, 4)),
                       scale=float(r.choice([0.25, 1.0, 8.0])))
    if flavour.endswith("fp8"):
        _fp8(r, w, seed)
    return w, flavour


def _fp8(r, w, seed):
    ks = None if r.integers(0, 4) == 0 else float(r.uniform(1e-3, 1.0))
    vs = None if r.integers(0, 4) == 0 else float(r.uniform(1e-3, 1.0))
    W.with_fp8_cache(w, seed + 2, ks, vs, fill="sentinel")


def _paged_case(r, k, gather):
    D = int(r.choice([64, 128, 256]))
    R = _rotary_dim(r, D)
    style = int(r.integers(0, 2))
    batch, Hkv = int(r.integers(1, 7)), int(r.integers(1, 6))
    max_pages = int(r.integers(1, 7))
    num_pages = batch * max_pages + int(r.integers(0, 4))
    N = int(r.integers(0, 301))
    seed = 12500 + k
    name = f"sweep{k}_paged{'_gather' if gather else ''}_N{N}_b{batch}_Hkv{Hkv}_D{D}_R{R}_s{style}"
    if gather:
        states = int(r.integers(1, 4))
        rows = int(r.integers(1, max_pages * W.TOKENS_PER_PAGE + 1))
        w = W.paged_gather(N, batch, Hkv, D, R, num_pages, max_pages, style, seed,
                           rope_states=states, rope_rows=rows,
                           state_indices=bool(r.integers(0, 2)), name=name)
    else:
        w = W.paged(N, batch, Hkv, D, R, num_pages, max_pages, style, seed, name=name)
    flavour = "fp16"
    if r.integers(0, 2):
        flavour = "fp8"
        _fp8(r, w, seed)
    return w, flavour


def _case(k):
    r = np.random.default_rng(12000 + k)
    kind = ["packed", "continuous", "tree", "paged", "paged_gather"][k % 5]
    if kind.startswith("paged"):
        return _paged_case(r, k, kind == "paged_gather")
    return _contig_case(r, k, kind)


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_case(k):
    w, flavour = _case(k)
    print(f"[sweep] {w.name} {flavour} tokens={w.tokens}", flush=True)
    want = expected(w)
    for mode in ("fast", "exact"):
        got = run_gpu(w, exact=(mode == "exact"))
        rep = compare(w, got, want)
        print(f"[sweep] {w.name} {mode}: {rep}", flush=True)
        if mode == "exact":
            assert not exact_diffs(rep), f"exact mode not bit-identical: {rep}"
        else:
            keys = ("_max_ulp_ge_2m6", "_max_code_step") if "norm" in flavour else \
                ("_max_ulp", "_max_code_step")
            assert all(v <= 1 for key, v in rep.items() if key.endswith(keys)), rep
