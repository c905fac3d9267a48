"""GPU parity of the fp8 (E4M3) cache calls against the CPU oracle.

Each workload is the fp16 workload with its cache (pool) replaced by E4M3
bytes filled with the E4M3 NaN code and per-tensor scales; the harness's
fp8 rule applies: bytes the oracle leaves untouched stay untouched, written
bytes are within one code step of the oracle in the default mode and equal
to it, bit for bit, with RKV_ROUND_EXACT.  Q (and call 1's in-place K) are
fp16 outputs under the fp16 rules.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from harness import (compare, dev, download, exact_diffs, expected, host8, host16, launch, run_gpu,
                     upload)

pytestmark = pytest.mark.gpu

NEOX, GPTJ = W.NEOX, W.GPTJ


def _say(*a):
    print(*a, flush=True)


def fp8(w, seed, k_scale=W.K_SCALE, v_scale=W.V_SCALE):
    return W.with_fp8_cache(w, seed, k_scale, v_scale, fill="sentinel")


def check(w, modes=("fast", "exact")):
    _say(f"[parity-fp8] {w.name} tokens={w.tokens}")
    want = expected(w)
    for mode in modes:
        got = run_gpu(w, exact=(mode == "exact"))
        rep = compare(w, got, want)
        _say(f"[parity-fp8] {w.name} {mode}: {rep}")
        if mode == "exact":
            diffs = exact_diffs(rep)
            assert not diffs, f"exact mode not bit-identical: {rep}"
        else:
            assert all(v <= 1 for k, v in rep.items() if k.endswith(("_max_ulp",
                                                                      "_max_code_step"))), rep


@pytest.mark.parametrize("idx,style", [(1, None), (2, NEOX), (2, GPTJ), (3, None), (4, None),
                                       (41, None), (5, None)],
                         ids=["prefill_tiny", "continuous_neox", "continuous_gptj", "tree",
                              "paged_delta", "paged_delta_gather", "prefill_large"])
def test_config_fp8(idx, style):
    w = W.config(idx, style) if idx == 2 else W.config(idx)
    check(fp8(w, 7000 + idx))


SMALL = []
for D in (64, 128, 256):
    for R in sorted({0, 16, D // 2, D}):
        for style in (NEOX, GPTJ):
            SMALL.append((D, R, style))


@pytest.mark.parametrize("D,R,style", SMALL, ids=lambda v: str(v))
@pytest.mark.parametrize("call", ["packed", "continuous", "tree"])
def test_small_shapes_fp8(call, D, R, style):
    seed = 7100 + D + R * 3 + style * 7 + {"packed": 0, "continuous": 1, "tree": 2}[call] * 1000
    B, S, Hq, Hkv, cap = 3, 37, 5, 3, 96
    if call == "packed":
        w = W.packed(B, S, Hq, Hkv, D, R, cap, style, seed, table_batch=B, table_len=50,
                     offsets=np.array([0, 7, 40]), name=f"packed_D{D}_R{R}_s{style}")
    elif call == "continuous":
        w = W.continuous(B, S, Hq, Hkv, D, R, cap, style, seed, 20, 110, table_len=90,
                         name=f"continuous_D{D}_R{R}_s{style}")
    else:
        w = W.tree(B, S, Hq, Hkv, D, R, cap, style, seed, 20, 110,
                   name=f"tree_D{D}_R{R}_s{style}")
    check(fp8(w, seed))


@pytest.mark.parametrize("k_scale,v_scale", [(None, None), (1.0, 0.5), (1e-3, 3e-3),
                                             (64.0, 0.0123), (0.0123, None),
                                             (2.0 ** -124, 2.0 ** -125), (2.0 ** 122, 2.0 ** 125),
                                             (0.0123, 2.0 ** -124)],
                         ids=["no_scale", "unit_half", "saturating", "subnormal", "k_only",
                              "tiny", "huge", "mixed_range"])
def test_scales(k_scale, v_scale):
    """Scales that leave values unscaled, saturate most of them (|x|/1e-3
    beyond 448) or push them into the E4M3 subnormals; scales outside
    [2^-120, 2^121), whose reciprocal the kernels take by binary64 division
    instead of the binary32 Newton step (every value saturates, or
    underflows to zero)."""
    w = W.continuous(4, 33, 6, 2, 128, 128, 64, GPTJ, 7300, 33, 64, name="continuous_scales")
    check(fp8(w, 7301, k_scale, v_scale))
    w = W.paged(200, 5, 3, 64, 48, 20, 4, NEOX, 7302, width=40, name="paged_scales")
    check(fp8(w, 7303, k_scale, v_scale))


def test_every_fp16_value_through_v():
    """All 65,536 fp16 bit patterns (NaN and infinities included) as V rows
    of the paged call, for three V scales."""
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    N, Hkv, D = 64, 16, 64
    for vs in (None, 2.0, 0.0109):
        w = W.Paged(NEOX, N, 1, Hkv, D, 0, 1, 1, np.zeros((N, Hkv, D), np.uint16),
                    allbits.reshape(N, Hkv, D).copy(), W.sentinel_f16((2, 1, 64, Hkv, D)),
                    np.zeros((N, 0), np.float32), np.arange(N, dtype=np.int32),
                    np.zeros(N, np.int32), np.array([[[0], [1]]], np.int32),
                    name=f"v_all_patterns_scale_{vs}")
        w = fp8(w, 1, None, vs)
        want = expected(w)["pool"]
        for exact in (False, True):
            got = run_gpu(w, exact=exact)["pool"]
            nan_w = (want & 0x7F) == 0x7F
            nan_g = (got & 0x7F) == 0x7F
            assert np.array_equal(nan_w, nan_g), vs
            _say(f"[parity-fp8] {w.name} exact={exact}: NaN codes whose sign bit differs: "
                 f"{int(((want ^ got) & 0x80)[nan_w].astype(bool).sum())}")
            same = ~nan_w
            assert np.array_equal(got[same], want[same]), \
                (vs, exact, int((got[same] != want[same]).sum()))


def test_paged_skips_and_gather_fp8():
    w = W.paged(512, 8, 2, 128, 128, 96, 8, NEOX, 7400, width=64, name="paged_skips_fp8")
    r = np.random.default_rng(7401)
    k = r.choice(w.N, 60, replace=False)
    w.positions[k[:10]] = -1
    w.seq[k[10:20]] = -3
    w.seq[k[20:30]] = 6
    w.positions[k[30:40]] = w.max_pages * 64
    w.positions[k[40:50]] = 2 ** 31 - 1
    w.batch = 6
    check(fp8(w, 7402))
    w = W.paged_gather(300, 7, 3, 128, 64, 64, 9, GPTJ, 7403, rope_states=3,
                       rope_rows=9 * 64 - 50, width=43, pad_frac=0.2, bad_frac=0.2,
                       name="paged_gather_fp8")
    w.extra["state_indices"][1] = 3
    w.extra["state_indices"][2] = -1
    check(fp8(w, 7404))


def test_empty_inputs_fp8():
    for B, S in [(0, 4), (3, 0)]:
        check(fp8(W.packed(B, S, 2, 1, 64, 64, 8, NEOX, 1, name=f"empty_{B}_{S}"), 1))
    check(fp8(W.paged(0, 2, 2, 64, 64, 4, 2, NEOX, 5, name="empty_paged"), 1))


def test_scale_is_read_when_the_kernel_runs():
    """The scales are device values: updating them on the stream between two
    launches changes the second launch's bytes."""
    w = fp8(W.continuous(2, 16, 4, 2, 128, 128, 32, NEOX, 7500, 16, 32, name="scale_update"),
            7501, 0.02, 0.02)
    t = upload(w)
    launch(w, t)
    first = download(w, t)
    t["k_scale"].fill_(0.04)
    t["v_scale"].fill_(0.01)
    t["cache"].fill_(W.SENTINEL8)
    launch(w, t, exact=True)
    second = download(w, t)
    w.extra["fp8"] = {"k_scale": np.float32(0.04), "v_scale": np.float32(0.01)}
    want = expected(w)
    assert np.array_equal(second["cache"], want["cache"])
    assert not np.array_equal(first["cache"], second["cache"])


def test_fp8_cache_tensor_may_be_float8_typed():
    """A torch.float8_e4m3fn cache is accepted and written like a uint8 one."""
    import rope_kv_cache_amd as rkv
    w = fp8(W.packed(2, 9, 3, 2, 64, 64, 12, GPTJ, 7600, name="packed_f8_dtype"), 7601)
    want = expected(w)
    t = upload(w)
    cache = t["cache"].view(torch.float8_e4m3fn)
    rkv.apply_rope_write_kv_packed_qkv_fp8(t["cos_sin"], t["qkv"], cache, t["k_scale"],
                                           t["v_scale"], GPTJ | rkv.ROUND_EXACT)
    torch.cuda.synchronize()
    assert np.array_equal(host8(t["cache"]), want["cache"])


@pytest.mark.parametrize("D,R,style,Hkv", [(64, 64, NEOX, 4), (64, 32, GPTJ, 3),
                                           (128, 0, NEOX, 2), (256, 256, GPTJ, 2),
                                           (256, 112, NEOX, 5)])
def test_paged_shapes_fp8(D, R, style, Hkv):
    w = W.paged(300, 7, Hkv, D, R, 64, 9, style, 7700 + D + R + Hkv, width=43, pad_frac=0.2,
                bad_frac=0.2, name=f"paged_fp8_D{D}_R{R}_s{style}_H{Hkv}")
    check(fp8(w, 7701 + D))


def test_fp8_pool_beyond_4g_elements():
    """An E4M3 pool of 5.2e9 bytes: the highest pages of both planes sit past
    2^31 and 2^32 elements.  The oracle runs on the used pages renamed into a
    compact pool; untouched pages are checked on the device."""
    import rope_kv_cache_amd as rkv
    Hkv, D, R, P, M, N = 8, 128, 128, 40000, 4, 48
    r = np.random.default_rng(7800)
    batch = N // 16
    pos = np.tile(np.arange(16, dtype=np.int32) * 17 % (M * 64), batch)
    seq = np.repeat(np.arange(batch, dtype=np.int32), 16)
    k_ids = P - 1 - np.arange(batch * M)
    v_ids = 2 * P - 1 - np.arange(batch * M)
    pt = np.stack([k_ids.reshape(batch, M), v_ids.reshape(batch, M)], axis=1).astype(np.int32)
    k_delta = W.normal_f16(r, (N, Hkv, D))
    v_delta = W.normal_f16(r, (N, Hkv, D))
    cs = W.rope_rows(pos, R, 10000.0)
    used_k, used_v = np.sort(k_ids), np.sort(v_ids)
    nc = used_k.size
    cpt = np.empty_like(pt)
    cpt[:, 0] = np.searchsorted(used_k, pt[:, 0])
    cpt[:, 1] = nc + np.searchsorted(used_v, pt[:, 1])
    small = np.full((2, nc, 64, Hkv, D), W.SENTINEL8, np.uint8)
    want = oracle.paged_delta_fp8(k_delta, v_delta, small, cs, pos, seq, cpt, batch, W.K_SCALE,
                                  W.V_SCALE, NEOX)
    _say("[parity-fp8] E4M3 pool 5.2 GB")
    pool = torch.full((2, P, 64, Hkv, D), W.SENTINEL8, dtype=torch.uint8, device="cuda")
    ks = torch.tensor([W.K_SCALE], dtype=torch.float32, device="cuda")
    vs = torch.tensor([W.V_SCALE], dtype=torch.float32, device="cuda")
    rkv.dflash_target_kv_cache_update_fp8(dev(k_delta), dev(v_delta), pool, ks, vs, dev(cs),
                                          dev(pos), dev(seq), dev(pt), batch,
                                          NEOX | rkv.ROUND_EXACT)
    torch.cuda.synchronize()
    flat = pool.view(2 * P, 64 * Hkv * D)
    touched = (flat != W.SENTINEL8).any(dim=1).nonzero().flatten().cpu().numpy()
    assert set(touched.tolist()) <= set(used_k.tolist()) | set(used_v.tolist())
    wflat = want.reshape(2 * nc, 64, Hkv, D)
    for plane, used in ((0, used_k), (1, used_v)):
        for rank, pid in enumerate(used):
            g = host8(pool.view(2 * P, 64, Hkv, D)[pid])
            assert np.array_equal(g, wflat[plane * nc + rank]), (plane, pid)
    del pool
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,cap", [(2, 1 << 20), (1, 1 << 21)],
                         ids=["slice_2GiB_buffer_stores", "slice_4GiB_global_stores"])
def test_fp8_cache_beyond_4g_elements(B, cap):
    """A 4 GiB E4M3 cache [B, 2, 8, cap, 128] (2^32 elements) written near
    its end.  With B = 2 each batch's slice is 2 GiB and its rows are stored
    through a buffer resource; with B = 1 the slice is 4 GiB, past a
    resource's 32-bit size, and the kernel stores the rows with global stores
    instead.  The oracle runs on a compact cache of the last slots."""
    import rope_kv_cache_amd as rkv
    S, Hq, Hkv, D = 16, 4, 8, 128
    r = np.random.default_rng(93)
    qkv = W.normal_f16(r, (B, S, Hq + 2 * Hkv, D))
    end = (cap - np.arange(B) * 1000).astype(np.int32)
    cs_full = W.rope_table(1, cap, D, 10000.0)
    lo = int(end.min()) - S
    w_small = W.Contig("continuous", GPTJ, B, S, Hq, Hkv, D, D, cap - lo, cs_full[:, lo:], qkv,
                       np.full((B, 2, Hkv, cap - lo, D), W.SENTINEL8, np.uint8),
                       q_out=W.sentinel_f16((B, S, Hq, D)), end_lens=(end - lo).astype(np.int32),
                       name="continuous_fp8_cache_compact")
    w_small.extra["fp8"] = {"k_scale": np.float32(W.K_SCALE), "v_scale": np.float32(W.V_SCALE)}
    want = expected(w_small)
    _say(f"[parity-fp8] E4M3 cache 4 GiB, B={B}, cap={cap}")
    cache = torch.full((B, 2, Hkv, cap, D), W.SENTINEL8, dtype=torch.uint8, device="cuda")
    q_out = dev(W.sentinel_f16((B, S, Hq, D)))
    ks = torch.tensor([W.K_SCALE], dtype=torch.float32, device="cuda")
    vs = torch.tensor([W.V_SCALE], dtype=torch.float32, device="cuda")
    rkv.apply_rope_write_kv_continuous_fp8(dev(cs_full), dev(end), dev(qkv), cache, q_out, ks, vs,
                                           GPTJ | rkv.ROUND_EXACT)
    torch.cuda.synchronize()
    assert np.array_equal(host16(q_out), want["q_out"])
    assert np.array_equal(host8(cache[:, :, :, lo:]), want["cache"])
    written = (cache != W.SENTINEL8).any(dim=-1).sum().item()
    assert written == B * S * 2 * Hkv
    del cache
    torch.cuda.empty_cache()
