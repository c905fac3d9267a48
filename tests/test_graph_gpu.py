"""The calls inside HIP graphs: each call enqueues one kernel on the
caller's stream, with no allocation, host synchronisation or memset, so it
can be captured (torch.cuda.CUDAGraph drives hipStreamBeginCapture on ROCm).
Each graph is replayed several times with the program's own eager work and
synchronisations in between, and every replay is checked against the eager
result (or the oracle)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from harness import compare, dev, download, expected, launch, upload

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def test_paged_step_graph_replays():
    """Metadata builder -> paged update (E4M3 pool) captured as one graph;
    the pool is reset eagerly (a copy kernel outside the graph) before each
    replay and compared with the oracle after it."""
    import rope_kv_cache_amd as rkv
    B, width, Hkv, D, P, M = 8, 64, 4, 128, 256, 8
    w = W.paged(B * width, B, Hkv, D, D, P, M, W.NEOX, 9500, width=width, name="graph_paged")
    r = np.random.default_rng(9501)
    old = r.integers(0, M * 64 - width, B).astype(np.int32)
    dl = r.integers(1, width + 1, B).astype(np.int32)
    w.positions, w.seq = oracle.prepare_delta_metadata(old, dl, width)
    w.cos_sin = W.rope_rows(w.positions, D, 10000.0)
    W.with_fp8_cache(w, 9502, fill="bits")
    want = expected(w)["pool"]
    t = upload(w)
    pool0 = t["pool"].clone()
    old_d, dl_d = dev(old), dev(dl)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):           # warm up on the capture stream
        rkv.dflash_prepare_delta_metadata(old_d, dl_d, width, t["positions"], t["seq"])
        launch(w, t, exact=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rkv.dflash_prepare_delta_metadata(old_d, dl_d, width, t["positions"], t["seq"])
        launch(w, t, exact=True)
    for k in range(4):
        t["pool"].copy_(pool0)
        t["positions"].fill_(-9)
        t["seq"].fill_(-9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = download(w, t)["pool"]
        _say(f"[graph] paged replay {k}: equal = {np.array_equal(got, want)}")
        assert np.array_equal(got, want), k


def test_continuous_qknorm_graph_replays():
    """The continuous call with Q/K norm (idempotent) captured and replayed;
    every replay equals the eager launch bit for bit."""
    w = W.with_qk_norm(W.config(2, W.GPTJ), 9600, scale=2.0)
    t_eager = upload(w)
    launch(w, t_eager)
    eager = download(w, t_eager)
    rep = compare(w, eager, expected(w))
    assert all(v <= 1 for k, v in rep.items() if k.endswith("_max_ulp_ge_2m6")), rep
    t = upload(w)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        launch(w, t)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch(w, t)
    for k in range(4):
        t["cache"].zero_()
        t["q_out"].zero_()
        torch.cuda.synchronize()
        t["cache"].copy_(dev(w.cache))
        t["q_out"].copy_(dev(w.q_out))
        g.replay()
        got = download(w, t)
        for key in ("cache", "q_out", "qkv"):
            assert np.array_equal(got[key], eager[key]), (k, key)
        _say(f"[graph] continuous qknorm replay {k}: equal to eager")
