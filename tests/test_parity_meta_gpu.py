"""GPU parity of the device metadata builders against the CPU oracle, and
the builders feeding the paged (call 4) and tree (call 3) writes on the
device.  All integer outputs: bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from harness import dev, download, expected, launch, upload

pytestmark = pytest.mark.gpu

NEOX, GPTJ = W.NEOX, W.GPTJ


def _say(*a):
    print(*a, flush=True)


def _delta_case(B, width, seed, old_hi=1 << 20, near_max=False):
    r = np.random.default_rng(seed)
    old = r.integers(0, old_hi, B).astype(np.int32)
    dl = r.integers(-2, width + 3, B).astype(np.int32)
    if near_max:
        old[: B // 2] = (2 ** 31 - 1) - r.integers(0, width, B // 2)
    return old, dl


@pytest.mark.parametrize("B,width,near_max", [(1, 1, False), (3, 7, False), (32, 128, False),
                                              (4096, 128, False), (64, 33, True),
                                              (1000, 1, True)])
def test_delta_metadata(B, width, near_max):
    import rope_kv_cache_amd as rkv
    _say(f"[parity-meta] delta metadata B={B} width={width}")
    old, dl = _delta_case(B, width, 9000 + B + width, near_max=near_max)
    want_p, want_s = oracle.prepare_delta_metadata(old, dl, width)
    pos = torch.full((B * width,), 12345, dtype=torch.int32, device="cuda")
    seq = torch.full((B * width,), 12345, dtype=torch.int32, device="cuda")
    rkv.dflash_prepare_delta_metadata(dev(old), dev(dl), width, pos, seq)
    torch.cuda.synchronize()
    assert np.array_equal(pos.cpu().numpy(), want_p)
    assert np.array_equal(seq.cpu().numpy(), want_s)


@pytest.mark.parametrize("B,V", [(1, 1), (2, 16), (16, 64), (3, 1000), (4096, 8)])
def test_linear_tree(B, V):
    import rope_kv_cache_amd as rkv
    _say(f"[parity-meta] linear tree B={B} V={V}")
    par = torch.full((B, V), 777, dtype=torch.int32, device="cuda")
    dep = torch.full((B, V), 777, dtype=torch.int32, device="cuda")
    rkv.dflash_build_linear_tree_metadata(par, dep)
    torch.cuda.synchronize()
    wp, wd = oracle.linear_tree_metadata(B, V)
    assert np.array_equal(par.cpu().numpy(), wp)
    assert np.array_equal(dep.cpu().numpy(), wd)


def test_empty_builders_enqueue_nothing():
    import rope_kv_cache_amd as rkv
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    rkv.dflash_prepare_delta_metadata(e, e, 4, e, e)
    rkv.dflash_build_linear_tree_metadata(e.view(0, 3), e.view(0, 3))
    torch.cuda.synchronize()


@pytest.mark.parametrize("fp8", [False, True], ids=["fp16", "fp8"])
def test_delta_metadata_drives_the_paged_update(fp8):
    """Metadata built on the device, then the paged update from it, equals
    the oracle's builder followed by the oracle's update."""
    import rope_kv_cache_amd as rkv
    B, width, Hkv, D, P, M = 32, 128, 8, 128, 2048, 32
    w = W.paged(B * width, B, Hkv, D, D, P, M, NEOX, 9100, width=width, name="paged_from_meta")
    r = np.random.default_rng(9101)
    old = r.integers(0, M * 64 - width, B).astype(np.int32)
    dl = r.integers(0, width + 1, B).astype(np.int32)
    pos, seq = oracle.prepare_delta_metadata(old, dl, width)
    w.positions, w.seq = pos, seq
    w.cos_sin = W.rope_rows(pos, D, 10000.0)
    if fp8:
        W.with_fp8_cache(w, 9102, fill="sentinel")
    want = expected(w)
    t = upload(w)
    t["positions"].fill_(-7)
    t["seq"].fill_(-7)
    rkv.dflash_prepare_delta_metadata(dev(old), dev(dl), width, t["positions"], t["seq"])
    launch(w, t, exact=True)
    got = download(w, t)
    assert np.array_equal(got["pool"], want["pool"])


def test_linear_tree_depths_make_call_3_equal_call_2():
    """tokenPosIds = endLens - S + depth from the device builder: the tree
    call writes what the continuous call writes, bit for bit."""
    import rope_kv_cache_amd as rkv
    w2 = W.config(2, NEOX)
    B, S = w2.B, w2.S
    t2 = upload(w2)
    launch(w2, t2, exact=True)
    out2 = download(w2, t2)
    par = torch.empty((B, S), dtype=torch.int32, device="cuda")
    dep = torch.empty((B, S), dtype=torch.int32, device="cuda")
    rkv.dflash_build_linear_tree_metadata(par, dep)
    w3 = W.Contig("tree", w2.style, B, S, w2.Hq, w2.Hkv, w2.D, w2.R, w2.cap, w2.cos_sin, w2.qkv,
                  w2.cache, q_out=w2.q_out, end_lens=w2.end_lens,
                  pos_ids=np.zeros((B, S), np.int32), name="tree_from_linear_depths")
    t3 = upload(w3)
    t3["pos_ids"].copy_(t3["end_lens"][:, None] - S + dep)
    launch(w3, t3, exact=True)
    out3 = download(w3, t3)
    for k in ("cache", "q_out"):
        assert np.array_equal(out3[k], out2[k]), k
