"""GPU parity: the HIP library against the CPU oracle on seeded inputs.

Every test calls the C ABI through the Python binding, on cuda:0.  Outputs
are compared with ``tests/harness.compare``: bit-exact everywhere except
rotated Q/K, which must meet |gpu - ref| <= 2^-10*|ref| + 1e-3.  Each case
runs in both arithmetic modes: the default binary32 mode must also stay
within one fp16 ulp of the oracle, and the RKV_ROUND_EXACT mode must be
bit-identical to it.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from harness import (compare, dev, download, exact_diffs, expected, host16, launch, run_gpu,
                     upload)

pytestmark = pytest.mark.gpu

NEOX, GPTJ = W.NEOX, W.GPTJ


def _say(*a):
    print(*a, flush=True)


def check(w, modes=("fast", "exact")):
    """Run the library in each arithmetic mode on fresh copies of the inputs
    and compare with one oracle run: the default (binary32) mode must stay
    within one fp16 ulp, the exact mode must be bit-identical."""
    _say(f"[parity] {w.name} tokens={w.tokens}")
    want = expected(w)
    reps = {}
    for mode in modes:
        got = run_gpu(w, exact=(mode == "exact"))
        rep = compare(w, got, want)
        _say(f"[parity] {w.name} {mode}: rotated elements differing from the oracle: {rep}")
        if mode == "exact":
            diffs = exact_diffs(rep)
            assert not diffs, f"exact mode not bit-identical: {rep}"
        else:
            ulps = {k: v for k, v in rep.items() if k.endswith("_max_ulp")}
            assert all(v <= 1 for v in ulps.values()), f"more than 1 ulp: {rep}"
        reps[mode] = rep
    return reps


# ------------------------------------------------------- the five configs --

@pytest.mark.parametrize("idx,style", [(1, None), (2, NEOX), (2, GPTJ), (3, None), (4, None),
                                       (5, None)],
                         ids=["prefill_tiny", "continuous_neox", "continuous_gptj", "tree",
                              "paged_delta", "prefill_large"])
def test_config(idx, style):
    w = W.config(idx, style) if idx == 2 else W.config(idx)
    check(w)


@pytest.mark.parametrize("tp", [4, 8])
def test_prefill_tensor_parallel_shard(tp):
    """One GPU's share of the large prefill under tensor parallelism: Hq/tp
    and Hkv/tp heads at the full batch and length, launched as the benchmark
    launches it."""
    check(W.prefill_tp_shard(tp))


def test_config4_gptj():
    w = W.paged(4096, 32, 8, 128, 128, 8192, 128, GPTJ, 1014, name="paged_delta_gptj")
    check(w)


# --------------------------------------------- shapes, styles, ragged tails --

SMALL = []
for D in (64, 128, 256):
    for R in sorted({0, 16, D // 2, D - 16, D}):
        for style in (NEOX, GPTJ):
            SMALL.append((D, R, style))


@pytest.mark.parametrize("D,R,style", SMALL, ids=lambda v: str(v))
@pytest.mark.parametrize("call", ["packed", "continuous", "tree"])
def test_small_shapes(call, D, R, style):
    seed = 2000 + D + R * 3 + style * 7 + {"packed": 0, "continuous": 1, "tree": 2}[call] * 1000
    B, S, Hq, Hkv, cap = 3, 37, 5, 3, 96       # H = 11: ragged against every row-set size
    if call == "packed":
        w = W.packed(B, S, Hq, Hkv, D, R, cap, style, seed, table_batch=B, table_len=50,
                     offsets=np.array([0, 7, 40]), name=f"packed_D{D}_R{R}_s{style}")
    elif call == "continuous":
        w = W.continuous(B, S, Hq, Hkv, D, R, cap, style, seed, 20, 110, table_len=90,
                         name=f"continuous_D{D}_R{R}_s{style}")
    else:
        w = W.tree(B, S, Hq, Hkv, D, R, cap, style, seed, 20, 110,
                   name=f"tree_D{D}_R{R}_s{style}")
    check(w)


@pytest.mark.parametrize("Hq,Hkv", [(0, 1), (1, 0), (0, 0), (1, 1), (7, 1), (32, 8), (64, 8),
                                    (17, 5)])
def test_head_counts(Hq, Hkv):
    w = W.packed(2, 9, Hq, Hkv, 128, 128, 12, GPTJ, 3000 + Hq * 13 + Hkv,
                 name=f"packed_Hq{Hq}_Hkv{Hkv}")
    check(w)
    w = W.continuous(2, 9, Hq, Hkv, 128, 64, 40, NEOX, 3100 + Hq * 13 + Hkv, 9, 40,
                     name=f"continuous_Hq{Hq}_Hkv{Hkv}")
    check(w)


def test_empty_inputs_launch_nothing():
    for B, S in [(0, 4), (3, 0)]:
        w = W.packed(B, S, 2, 1, 64, 64, 8, NEOX, 1, name=f"empty_{B}_{S}")
        check(w)
        w = W.continuous(B, S, 2, 1, 64, 64, 8, NEOX, 1, 4, 8, name=f"empty_c_{B}_{S}")
        check(w)
    w = W.paged(0, 2, 2, 64, 64, 4, 2, NEOX, 5, name="empty_paged")
    check(w)


def test_out_of_range_tokens_are_skipped():
    """Calls 2 and 3: end lengths and positions out of range on the device."""
    r = np.random.default_rng(44)
    B, S, Hq, Hkv, D, cap = 6, 8, 4, 2, 128, 20
    w = W.continuous(B, S, Hq, Hkv, D, D, cap, NEOX, 45, 8, 20, table_len=16,
                     name="continuous_out_of_range")
    w.end_lens[:] = np.array([3, 8, 20, 25, -100, 2 ** 31 - 1], dtype=np.int32)
    check(w)
    w = W.tree(B, S, Hq, Hkv, D, 64, cap, GPTJ, 46, 8, 20, name="tree_out_of_range")
    w.end_lens[:] = np.array([3, 8, 20, 25, -2 ** 31, 12], dtype=np.int32)
    w.pos_ids[0, :] = r.integers(-5, 5, S)
    w.pos_ids[1, :] = np.array([-1, 0, 19, 20, 21, 2 ** 31 - 1, -2 ** 31, 5])
    check(w)


# ---------------------------------------------------------------- paged --

@pytest.mark.parametrize("D,R,style,Hkv", [(64, 64, NEOX, 4), (64, 32, GPTJ, 3),
                                           (128, 64, NEOX, 8), (128, 128, GPTJ, 1),
                                           (256, 256, NEOX, 2), (256, 112, GPTJ, 5),
                                           (128, 0, NEOX, 2)])
def test_paged_shapes(D, R, style, Hkv):
    w = W.paged(300, 7, Hkv, D, R, 64, 9, style, 5000 + D + R + Hkv,
                width=43, pad_frac=0.2, bad_frac=0.2, name=f"paged_D{D}_R{R}_s{style}_H{Hkv}")
    check(w)


def test_paged_skip_reasons_and_inactive_batch():
    w = W.paged(512, 8, 2, 128, 128, 96, 8, NEOX, 77, width=64, pool_fill="sentinel",
                name="paged_skips")
    r = np.random.default_rng(78)
    # single-sided padding, inactive sequences, positions at and past capacity
    k = r.choice(w.N, 60, replace=False)
    w.positions[k[:10]] = -1
    w.seq[k[10:20]] = -3
    w.seq[k[20:30]] = 6           # >= batch below
    w.positions[k[30:40]] = w.max_pages * 64
    w.positions[k[40:50]] = 2 ** 31 - 1
    w.batch = 6                   # sequences 6 and 7 are inactive
    check(w)


# ------------------------------------------------ paged, gather fused in --

def test_config4_gather_fused():
    check(W.config(41))


@pytest.mark.parametrize("D,R,style,states,with_si", [
    (128, 128, NEOX, 3, True), (128, 64, GPTJ, 2, True), (64, 64, GPTJ, 1, False),
    (256, 112, NEOX, 4, False), (128, 0, NEOX, 2, True)])
def test_paged_gather_shapes(D, R, style, states, with_si):
    w = W.paged_gather(300, 7, 3, D, R, 64, 9, style, 6000 + D + R + states, rope_states=states,
                       rope_rows=9 * 64 - 50, state_indices=with_si, width=43, pad_frac=0.2,
                       bad_frac=0.2, name=f"paged_gather_D{D}_R{R}_s{style}_st{states}")
    if with_si:
        w.extra["state_indices"][1] = states        # a missing state
        w.extra["state_indices"][2] = -1
    check(w)


def test_paged_gather_equals_gather_then_update():
    """On the GPU, the fused call and the unfused call fed with the oracle's
    gathered rows write the same pool, bit for bit."""
    w = W.paged_gather(1024, 8, 4, 128, 128, 128, 16, NEOX, 6100, rope_states=2,
                       name="paged_gather_vs_unfused")
    rows = oracle.gather_delta_rope(w.extra["rope"], w.extra["state_indices"], w.positions, w.seq,
                                    w.batch)
    fused = run_gpu(w)["pool"]
    w.extra["gather"] = False
    w.cos_sin = rows
    unfused = run_gpu(w)["pool"]
    assert np.array_equal(fused, unfused)


# ------------------------------------------------------- 64-bit addressing --

def test_paged_pool_beyond_4g_elements():
    """A 10.5 GB pool (5.2e9 elements): the highest pages of both planes sit
    beyond 2^31 and 2^32 elements.  The oracle runs on the same rows with the
    used pages renamed into a compact pool; untouched pages are checked on
    the device."""
    Hkv, D, R, P, M, N = 8, 128, 128, 40000, 4, 48
    r = np.random.default_rng(90)
    batch = N // 16
    pos = np.tile(np.arange(16, dtype=np.int32) * 17 % (M * 64), batch)
    seq = np.repeat(np.arange(batch, dtype=np.int32), 16)
    k_ids = P - 1 - np.arange(batch * M)
    v_ids = 2 * P - 1 - np.arange(batch * M)
    pt = np.stack([k_ids.reshape(batch, M), v_ids.reshape(batch, M)], axis=1).astype(np.int32)
    k_delta = W.normal_f16(r, (N, Hkv, D))
    v_delta = W.normal_f16(r, (N, Hkv, D))
    cs = W.rope_rows(pos, R, 10000.0)
    # compact problem for the oracle: page id p -> its rank among used ids
    used_k, used_v = np.sort(k_ids), np.sort(v_ids)
    nc = used_k.size
    cpt = np.empty_like(pt)
    cpt[:, 0] = np.searchsorted(used_k, pt[:, 0])
    cpt[:, 1] = nc + np.searchsorted(used_v, pt[:, 1])
    small = W.sentinel_f16((2, nc, 64, Hkv, D))
    want = oracle.paged_delta(k_delta, v_delta, small, cs, pos, seq, cpt, batch, NEOX)
    _say("[parity] paged pool 10.5 GB")
    pool = torch.full((2, P, 64, Hkv, D), float("nan"), dtype=torch.float16, device="cuda")
    pool.view(torch.int16).fill_(W.SENTINEL)
    t = {"k_delta": dev(k_delta), "v_delta": dev(v_delta), "pool": pool, "cos_sin": dev(cs),
         "positions": dev(pos), "seq": dev(seq), "page_table": dev(pt)}
    import rope_kv_cache_amd as rkv
    rkv.dflash_target_kv_cache_update(t["k_delta"], t["v_delta"], pool, t["cos_sin"],
                                      t["positions"], t["seq"], t["page_table"], batch,
                                      NEOX | rkv.ROUND_EXACT)
    torch.cuda.synchronize()
    flat = pool.view(2 * P, 64 * Hkv * D)
    touched = (flat.view(torch.int16) != W.SENTINEL).any(dim=1).nonzero().flatten().cpu().numpy()
    assert set(touched.tolist()) <= set(used_k.tolist()) | set(used_v.tolist())
    wflat = want.reshape(2 * nc, 64, Hkv, D)
    for plane, used in ((0, used_k), (1, used_v)):
        for rank, pid in enumerate(used):
            g = host16(pool.view(2 * P, 64, Hkv, D)[pid])
            assert np.array_equal(g, wflat[plane * nc + rank]), (plane, pid)
    del pool
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,cap", [(8, 1 << 18), (2, 1 << 20)],
                         ids=["slice_1GiB_buffer_stores", "slice_4GiB_global_stores"])
def test_contiguous_cache_beyond_4g_elements(B, cap):
    """An 8 GiB cache [B, 2, 8, cap, 128] (2^32 elements) written near its
    end: the last rows lie beyond 2^31 and close to 2^32 elements.  With
    B = 8 each batch's slice is 1 GiB and its rows are stored through a
    buffer resource; with B = 2 a slice is 4 GiB, past a resource's 32-bit
    size, and the kernel stores the rows with global stores instead."""
    S, Hq, Hkv, D = 16, 4, 8, 128
    r = np.random.default_rng(91)
    qkv = W.normal_f16(r, (B, S, Hq + 2 * Hkv, D))
    end = (cap - np.arange(B) * 1000).astype(np.int32)
    tlen = cap
    cs_full = W.rope_table(1, tlen, D, 10000.0)
    # oracle on a compact cache covering the last 8000 + S slots of each row
    lo = int(end.min()) - S
    w_small = W.Contig("continuous", GPTJ, B, S, Hq, Hkv, D, D, cap - lo,
                       cs_full[:, lo:], qkv, W.sentinel_f16((B, 2, Hkv, cap - lo, D)),
                       q_out=W.sentinel_f16((B, S, Hq, D)), end_lens=(end - lo).astype(np.int32),
                       name="continuous_cache_8GiB_compact")
    want = expected(w_small)
    _say(f"[parity] contiguous cache 8 GiB, B={B}, cap={cap}")
    cache = torch.empty((B, 2, Hkv, cap, D), dtype=torch.float16, device="cuda")
    cache.view(torch.int16).fill_(W.SENTINEL)
    import rope_kv_cache_amd as rkv
    q_out = dev(W.sentinel_f16((B, S, Hq, D)))
    rkv.apply_rope_write_kv_continuous(dev(cs_full), dev(end), dev(qkv), cache, q_out,
                                       GPTJ | rkv.ROUND_EXACT)
    torch.cuda.synchronize()
    assert np.array_equal(host16(q_out), want["q_out"])
    tail = host16(cache[:, :, :, lo:])
    assert np.array_equal(tail, want["cache"])
    written = (cache.view(torch.int16) != W.SENTINEL).any(dim=-1).sum().item()
    assert written == B * S * 2 * Hkv
    del cache
    torch.cuda.empty_cache()


# -------------------------------------------------------------- streams --

def test_runs_on_the_current_stream_and_repeats():
    w = W.config(2, GPTJ)
    want = expected(w)
    t = upload(w)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):          # the continuous call is idempotent
            launch(w, t)
    s.synchronize()
    got = download(w, t)
    rep = compare(w, got, want)
    assert all(v <= 1 for k, v in rep.items() if k.endswith("ulp"))


def test_packed_twice_rotates_twice():
    w = W.packed(2, 24, 8, 2, 128, 128, 32, NEOX, 4242, name="packed_twice")
    once_q, once_c = oracle.packed_qkv(w.cos_sin, w.qkv, w.cache, NEOX)
    twice_q, twice_c = oracle.packed_qkv(w.cos_sin, once_q, once_c, NEOX)
    t = upload(w)
    launch(w, t, exact=True)
    launch(w, t, exact=True)
    got = download(w, t)
    assert np.array_equal(got["qkv"], twice_q)
    assert np.array_equal(got["cache"], twice_c)
