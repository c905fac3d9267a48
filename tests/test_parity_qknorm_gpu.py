"""GPU parity of the Q/K-norm calls (RMS norm of Q and K heads before the
rotation, fp16 or E4M3 cache) against the CPU oracle.

Bars: the exact mode (RKV_ROUND_EXACT) is bit-identical to the oracle; the
default binary32 mode meets the harness tolerance everywhere and is within
one fp16 ulp wherever |ref| >= 2^-6 (its error is about 2^-21 relative to the
row's scale plus 2^-23 of each normalised value, so only results much
smaller than their pair can lose more than an ulp); E4M3 bytes are within
one code step.
"""
import numpy as np
import pytest

import workloads as W
from harness import compare, exact_diffs, expected, run_gpu

pytestmark = pytest.mark.gpu

NEOX, GPTJ = W.NEOX, W.GPTJ


def _say(*a):
    print(*a, flush=True)


def check(w, modes=("fast", "exact")):
    _say(f"[parity-qknorm] {w.name} tokens={w.tokens}")
    want = expected(w)
    for mode in modes:
        got = run_gpu(w, exact=(mode == "exact"))
        rep = compare(w, got, want)
        _say(f"[parity-qknorm] {w.name} {mode}: {rep}")
        if mode == "exact":
            diffs = exact_diffs(rep)
            assert not diffs, f"exact mode not bit-identical: {rep}"
        else:
            assert all(v <= 1 for k, v in rep.items()
                       if k.endswith(("_max_ulp_ge_2m6", "_max_code_step"))), rep


def norm(w, seed, fp8=False, **kw):
    W.with_qk_norm(w, seed, **kw)
    if fp8:
        W.with_fp8_cache(w, seed + 1, fill="sentinel")
    return w


@pytest.mark.parametrize("fp8", [False, True], ids=["fp16", "fp8"])
@pytest.mark.parametrize("idx,style", [(1, None), (2, NEOX), (2, GPTJ), (3, None), (5, None)],
                         ids=["prefill_tiny", "continuous_neox", "continuous_gptj", "tree",
                              "prefill_large"])
def test_config_qknorm(idx, style, fp8):
    w = W.config(idx, style) if idx == 2 else W.config(idx)
    check(norm(w, 8000 + idx, fp8=fp8, scale=3.0))


SMALL = []
for D in (64, 128, 256):
    for R in sorted({0, 16, D // 2, D}):
        for style in (NEOX, GPTJ):
            SMALL.append((D, R, style))


@pytest.mark.parametrize("D,R,style", SMALL, ids=lambda v: str(v))
@pytest.mark.parametrize("call", ["packed", "continuous", "tree"])
def test_small_shapes_qknorm(call, D, R, style):
    seed = 8100 + D + R * 3 + style * 7 + {"packed": 0, "continuous": 1, "tree": 2}[call] * 1000
    B, S, Hq, Hkv, cap = 3, 37, 5, 3, 96
    if call == "packed":
        w = W.packed(B, S, Hq, Hkv, D, R, cap, style, seed, table_batch=B, table_len=50,
                     offsets=np.array([0, 7, 40]), name=f"packed_D{D}_R{R}_s{style}")
    elif call == "continuous":
        w = W.continuous(B, S, Hq, Hkv, D, R, cap, style, seed, 20, 110, table_len=90,
                         name=f"continuous_D{D}_R{R}_s{style}")
    else:
        w = W.tree(B, S, Hq, Hkv, D, R, cap, style, seed, 20, 110, name=f"tree_D{D}_R{R}_s{style}")
    check(norm(w, seed, fp8=(seed % 2 == 1), scale=0.25))


@pytest.mark.parametrize("q,k,eps,scale", [(True, False, 1e-6, 1.0), (False, True, 1e-5, 40.0),
                                           (True, True, 0.0, 1.0), (True, True, 1.0, 0.01),
                                           (True, True, 1e-6, 1000.0)],
                         ids=["q_only", "k_only", "eps0", "eps1_small_x", "large_x"])
def test_weights_and_eps(q, k, eps, scale):
    w = W.continuous(4, 33, 6, 2, 128, 128, 64, GPTJ, 8300, 33, 64, name="continuous_norm_args")
    check(norm(w, 8301, q_weight=q, k_weight=k, eps=eps, scale=scale))
    w = W.packed(2, 40, 4, 4, 128, 64, 64, NEOX, 8302, name="packed_norm_args")
    check(norm(w, 8303, fp8=True, q_weight=q, k_weight=k, eps=eps, scale=scale))


def test_special_rows():
    """Rows of zeros (eps 0: 0/0 = NaN; eps > 0: zeros), rows holding an
    infinity or a NaN, rows at the fp16 maximum and rows of subnormals."""
    for eps in (0.0, 1e-6):
        w = W.packed(1, 8, 4, 2, 64, 64, 8, NEOX, 8400, name=f"packed_special_eps{eps}")
        H = w.Hq + 2 * w.Hkv
        w.qkv[0, 0, :, :] = 0                        # all heads of token 0 zero
        w.qkv[0, 1, 0, 5] = 0x7C00                   # +inf in a Q head
        w.qkv[0, 1, w.Hq, 9] = 0xFC00                # -inf in a K head
        w.qkv[0, 2, 1, 3] = 0x7E00                   # NaN in a Q head
        w.qkv[0, 3, :, :] = 0x7BFF                   # 65504 everywhere
        w.qkv[0, 4, :, :] = np.arange(1, 65, dtype=np.uint16)[None, :]   # subnormals
        w.qkv[0, 5, :, :] = 0x8001                   # -2^-24 everywhere
        assert H == 8
        check(norm(w, 8401, eps=eps))
