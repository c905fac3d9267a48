"""Benchmark of the fused RoPE + KV-cache write on one MI355X.

A step is one call of the library on the headline workload: empty-cache
prefill of packed QKV in place, B=4, S=8192, Hq=64, Hkv=8, D=R=128, GPT-J,
per-sequence cos/sin tables (1.43 GB of algorithmic traffic).  Inputs are
seeded synthetic data already resident in HBM.  W warm-up steps, then K timed
steps back to back, bracketed by device synchronisation and by one pair of
HIP events on the launch stream, whose span / K is the kernel's average
duration for the roofline.  The same workload in the library's
RKV_ROUND_EXACT mode, the NeoX layout, into an E4M3 cache and with Q/K RMS
norm, and the other workloads (continuous write, tree write, paged delta
update, the paged update with the cos/sin gather fused in, the continuous
and paged calls into an E4M3 cache, the continuous call with Q/K RMS norm,
the prefill's TP=8 shard, a 65,536-row paged update, a 16-sequence
continuous write, and the two device index builders) are reported under
"workloads".  The small workloads' inputs fit the 256 MB MALL: their figure
of record is timed like the headline, back to back, cycling through enough
full copies of every tensor they touch that each launch reads from and
writes back to HBM (``full_copies``, ``time_rotated``); warm launches on the
same tensors are reported beside it.

``--workload NAME`` times single small workloads and ``--ceilings`` the
measurement kernels of ``ceilings/`` (stream ceilings, empty kernels, an
index-free floor of the paged update, the LDS-staged prefill) beside the
library's kernels; both exist for rocprofv3 runs.

Prints one JSON line on stdout; progress goes to stderr.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]
                      [--calib] [--paged-large [fp16|fp8|both]] [--workload NAME]...
                      [--ceilings [PARTS]]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
HEADLINE = 5


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------- algorithmic bytes --

def bytes_contig(w) -> int:
    """Bytes the method must move for calls 1-3: per written token, its packed
    Q/K/V rows read, Q (and for call 1, K in place) written, K and V cache
    rows written (D bytes each for an E4M3 cache, 2D for fp16); each
    distinct cos/sin row read once; the index arrays (and the two fp8
    scales, and the Q/K norm weights)."""
    D, R, Hq, Hkv = w.D, w.R, w.Hq, w.Hkv
    fp8 = bool(w.extra.get("fp8"))
    cb = 1 if fp8 else 2
    H = Hq + 2 * Hkv
    tb, tlen = w.cos_sin.shape[0], w.cos_sin.shape[1]
    if w.call == "packed":
        valid = np.ones((w.B, w.S), dtype=bool)
        slot = pos = np.broadcast_to(np.arange(w.S), (w.B, w.S))
        write_q = (Hq + Hkv) * D * 2
        index = 0
    else:
        slot = w.end_lens[:, None].astype(np.int64) - w.S + np.arange(w.S)[None, :]
        pos = slot if w.call == "continuous" else w.pos_ids.astype(np.int64)
        valid = (slot >= 0) & (slot < w.cap) & (pos >= 0) & (pos < tlen)
        write_q = Hq * D * 2
        index = w.B * 4 + (w.B * w.S * 4 if w.call == "tree" else 0)
    n = int(valid.sum())
    rows = set()
    for b in range(w.B):
        t = 0 if tb == 1 else b
        rows.update((t, int(p)) for p in np.asarray(pos[b])[valid[b]])
    per_token = H * D * 2 + write_q + 2 * Hkv * D * cb
    norm = w.extra.get("qknorm") or {}
    weights = sum(D * 4 for k in ("q_weight", "k_weight") if norm.get(k) is not None)
    return n * per_token + len(rows) * R * 4 + index + (8 if fp8 else 0) + weights


def bytes_paged(w) -> int:
    """Call 4: per non-skipped row its two page-table entries; per mapped K
    its delta row read, rotated row written and cos/sin row read; per mapped
    V its delta row read and written (an E4M3 pool row is half the fp16 row);
    the two metadata arrays of all rows (and the two fp8 scales)."""
    D, R, Hkv, P = w.D, w.R, w.Hkv, w.num_pages
    fp8 = bool(w.extra.get("fp8"))
    wrow = Hkv * D * (1 if fp8 else 2)
    scales = 8 if fp8 else 0
    p, q = w.positions.astype(np.int64), w.seq.astype(np.int64)
    live = (p >= 0) & (q >= 0) & (q < w.batch) & (p < w.max_pages * 64)
    lp = np.where(live, p // 64, 0)
    qq = np.where(live, q, 0)
    kid = w.page_table[qq, 0, lp].astype(np.int64)
    vid = w.page_table[qq, 1, lp].astype(np.int64)
    k_ok = live & (kid >= 0) & (kid < P)
    v_ok = live & (vid >= P) & (vid < 2 * P)
    row = Hkv * D * 2
    if w.extra.get("gather"):
        # cos/sin come from the rope table: each distinct (state, position) row once,
        # for rows whose K is written; plus the state indices when given
        rope = w.extra["rope"]
        si = w.extra["state_indices"]
        st = si[qq] if si is not None else (np.zeros_like(qq) if rope.shape[0] == 1 else qq)
        has_row = (st >= 0) & (st < rope.shape[0]) & (p < rope.shape[1])
        k_ok = k_ok & has_row
        rows_read = len({(int(a), int(b)) for a, b in zip(st[k_ok], p[k_ok])})
        return int(k_ok.sum()) * (row + wrow) + rows_read * R * 4 \
            + int(v_ok.sum()) * (row + wrow) + w.N * 8 + int(live.sum()) * 8 \
            + (0 if si is None else si.size * 4) + scales
    return int(k_ok.sum()) * (row + wrow + R * 4) + int(v_ok.sum()) * (row + wrow) \
        + w.N * 8 + int(live.sum()) * 8 + scales


def algorithmic_bytes(w) -> int:
    import workloads as W
    return bytes_paged(w) if isinstance(w, W.Paged) else bytes_contig(w)


# ----------------------------------------------------------------- timing --

_SPIN_CYCLES_PER_US = None


def gpu_busy_wait(us):
    """Keep the current stream busy for about `us` microseconds with torch's
    spin kernel (it touches no memory), so that the host queues the launches
    that follow before the GPU reaches them; the spin's rate is measured
    once."""
    global _SPIN_CYCLES_PER_US
    import torch
    if _SPIN_CYCLES_PER_US is None:
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        start.record()
        torch.cuda._sleep(1_000_000)
        end.record()
        torch.cuda.synchronize()
        _SPIN_CYCLES_PER_US = 1_000_000 / max(start.elapsed_time(end) * 1e3, 1.0)
    torch.cuda._sleep(int(us * _SPIN_CYCLES_PER_US))


ROTATIONS = 4


def written_keys(w):
    """The launch arguments a call writes."""
    import workloads as W
    if isinstance(w, W.Paged):
        return ("pool",)
    return ("qkv", "cache") if w.call == "packed" else ("cache", "q_out")


def rotated(w, t, n):
    """`n` argument sets for back-to-back launches: the read-only tensors
    shared, each set with its own copy of every tensor the call writes.
    Launches that rewrite the lines the previous launch wrote can be partly
    absorbed by the 256 MB MALL (lines still dirty there are overwritten
    before they reach HBM); cycling through the copies leaves several
    launches' traffic between two writes of a line, as a real model's
    launches (new tokens, new cache slots) do."""
    sets = [t]
    for _ in range(n - 1):
        u = dict(t)
        for k in written_keys(w):
            u[k] = t[k].clone()
        sets.append(u)
    return sets


def time_launches(w, t, steps, warmup, exact=False):
    """Kernel duration and wall time of `steps` launches back to back on the
    current stream, bracketed by one pair of HIP events and by device
    synchronisations, so that nothing but the launches is timed; the kernel
    duration is the events' span divided by the launch count (the gaps
    between back-to-back launches, a few tenths of a microsecond, are
    included).  They cycle through ROTATIONS copies of the written tensors
    (`rotated`)."""
    import torch
    from harness import launch

    stream = torch.cuda.current_stream()
    sets = rotated(w, t, ROTATIONS)
    for k in range(warmup):
        launch(w, sets[k % len(sets)], exact)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for k in range(steps):
        launch(w, sets[k % len(sets)], exact)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del sets
    return start.elapsed_time(end) / steps, wall


def time_flushed(launch, flush, steps, pairs=5):
    """Cost of one launch whose inputs start in HBM, write-back included.

    Two series run back to back on the current stream, each between one
    pair of HIP events: `steps` x (flush, launch) and `steps` x flush alone;
    their difference / `steps` is the launch's cost.  The flush (a 1 GiB
    read) evicts the launch's inputs from L2 and MALL before it, and the
    next flush pays for writing back whatever lines the launch left dirty,
    so the figure covers the launch's writes reaching memory; it also
    covers the dispatch gap between two queued kernels (a few tenths of a
    microsecond).  Median over `pairs` pairs of series.  Returns ms."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(3):
        flush()
        launch()
    torch.cuda.synchronize()
    diffs = []
    for _ in range(pairs):
        spans = []
        for with_launch in (True, False):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(steps):
                flush()
                if with_launch:
                    launch()
            b.record(stream)
            torch.cuda.synchronize()
            spans.append(a.elapsed_time(b))
        diffs.append((spans[0] - spans[1]) / steps)
    return float(np.median(diffs))


def time_cold(launch, flush, steps):
    """Duration of one launch whose inputs start in HBM, without the timer's
    own cost (ms), and that cost.

    Everything is queued behind a GPU spin, so the host's launch rate is not
    timed: `steps` x (flush, event A, launch, event B, flush, event C,
    event D).  B - A covers the launch and the processing of one event; D - C
    the processing of one event alone, under the same conditions; the
    launch's duration is median(B - A) - median(D - C).  The flush (a 1 GiB
    read) evicts the launch's inputs from L2 and MALL; the launch's stores
    have left L2 when it completes (rocprofv3's WRITE_SIZE over a dispatch
    equals the bytes the kernel writes)."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(3):
        flush()
        launch()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    gpu_busy_wait(500)
    for a, b, c, d in ev:
        flush()
        a.record(stream)
        launch()
        b.record(stream)
        flush()
        c.record(stream)
        d.record(stream)
    torch.cuda.synchronize()
    with_launch = float(np.median([a.elapsed_time(b) for a, b, _, _ in ev]))
    alone = float(np.median([c.elapsed_time(d) for _, _, c, d in ev]))
    return with_launch - alone, alone


MALL_BYTES = 256 << 20


def full_copies(t, nbytes_per_launch, min_span=3 * MALL_BYTES, most=64):
    """Copies of every tensor a launch touches (inputs and outputs), enough
    of them that consecutive uses of one copy are separated by at least
    `min_span` bytes of other launches' traffic (three times the 256 MB
    MALL): cycling through them, no launch finds its inputs in the caches
    and every launch's writes are written back to HBM in steady state."""
    n = max(2, min(most, -(-min_span // max(nbytes_per_launch, 1)) + 1))
    return [t] + [{k: (None if v is None else v.clone()) for k, v in t.items()}
                  for _ in range(n - 1)]


def time_rotated(launch_set, sets, steps, warmup=None):
    """Steady state of back-to-back launches that cycle through `sets`: the
    GPU first spins long enough for the host to queue every launch, then
    the launches run; event span / count (ms).  With `full_copies` sets this
    is the HBM-bound cost per launch, as the headline is timed."""
    import torch
    stream = torch.cuda.current_stream()
    warmup = len(sets) if warmup is None else warmup
    for k in range(warmup):
        launch_set(sets[k % len(sets)])
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    gpu_busy_wait(2000 + 50 * steps)
    a.record(stream)
    for k in range(steps):
        launch_set(sets[(warmup + k) % len(sets)])
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def time_graph(launch_k, n, reps=5):
    """`launch_k(k)` for k < n captured as one HIP graph (torch's CUDAGraph
    drives hipStreamBeginCapture), replayed after a GPU spin: event span of
    one replay / n, the median over `reps` replays (ms).  The per-launch cost
    a step captured in a graph pays."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm up on the capture stream
        for k in range(n):
            launch_k(k)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(n):
            launch_k(k)
    g.replay()
    torch.cuda.synchronize()
    spans = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        gpu_busy_wait(3000)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        spans.append(a.elapsed_time(b) / n)
    del g
    return float(np.median(spans))


def time_queued(launch, steps, warmup=3):
    """Back to back: the GPU first spins long enough for the host to queue
    every launch, then the launches run; event span / count (ms)."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    gpu_busy_wait(2000 + 50 * steps)
    a.record(stream)
    for _ in range(steps):
        launch()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def make_flush():
    """A 1 GiB read (torch's sum into one float): leaves L2 and the 256 MB
    MALL holding clean lines of its own buffer."""
    import torch
    buf = torch.ones(1 << 29, dtype=torch.float16, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    def flush():
        torch.sum(buf, dim=0, dtype=torch.float32, out=sink)
    return flush


ROTATED_PROTOCOL = ("rotated: launches back to back, queued ahead behind a GPU spin, cycling "
                    "through full copies of every tensor the call reads or writes (at least 768 "
                    "MB of traffic between two uses of a copy, three times the MALL), event "
                    "span / count: every input comes from HBM and every write reaches HBM in "
                    "steady state, as for the headline")
COLD_PROTOCOL = ("cold: every launch follows a 1 GiB read that evicts its inputs from L2 and "
                 "MALL; all work queued behind a GPU spin; median over K launches of the event "
                 "pair around the launch minus the median of an event pair around nothing, "
                 "recorded the same way (an estimate from below: part of the pair's own cost "
                 "overlaps the launch; rocprofv3's trace of such launches reads up to about "
                 "2 us more)")
GRAPH_PROTOCOL = ("graph: the same launches (the same copies, in the same order) captured as "
                  "one HIP graph and replayed behind a GPU spin; event span of a replay / "
                  "launches, median of 5 replays")
MARGINAL_PROTOCOL = ("marginal: span of K x (1 GiB read, launch) minus span of K x (1 GiB "
                     "read), / K: the time one launch adds to a stream of HBM-bound work, its "
                     "dispatch and the write-back of the lines it leaves dirty included")


def metadata_builders(steps):
    """The two device index builders on the paged workload's shape (32
    sequences x 128 delta rows) and on a 16 x 64 linear verification tree."""
    import torch
    import rope_kv_cache_amd as rkv
    r = np.random.default_rng(7200)
    B, width = 32, 128
    old = torch.from_numpy(r.integers(0, 8064, B).astype(np.int32)).cuda()
    dl = torch.from_numpy(r.integers(100, 129, B).astype(np.int32)).cuda()
    pos = torch.empty(B * width, dtype=torch.int32, device="cuda")
    seq = torch.empty_like(pos)
    d_ms = time_queued(lambda: rkv.dflash_prepare_delta_metadata(old, dl, width, pos, seq), steps)
    par = torch.empty((16, 64), dtype=torch.int32, device="cuda")
    dep = torch.empty_like(par)
    t_ms = time_queued(lambda: rkv.dflash_build_linear_tree_metadata(par, dep), steps)
    note = "launch-bound; launches queued ahead and run back to back, event span / count"
    return {
        "delta_metadata_b32_w128": {"kernel_us": d_ms * 1e3,
                                    "algorithmic_bytes": 2 * B * 4 + 2 * B * width * 4,
                                    "note": "32 KB of output; " + note},
        "linear_tree_b16_v64": {"kernel_us": t_ms * 1e3,
                                "algorithmic_bytes": 2 * 16 * 64 * 4,
                                "note": "8 KB of output; " + note},
    }


def calibration_copy():
    """The counter runs' reference: torch.mul(src, 1.0, out=dst) on 1 GiB fp16
    tensors (1 GiB read, 1 GiB written per launch), three launches."""
    import torch
    src = torch.empty(1 << 29, dtype=torch.float16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def paged_large(steps, warmup=3, fp8=False):
    """The paged update at a size where bandwidth, not the launch, bounds
    it: 65,536 delta rows of the paged workload's shape (0.27 GB of deltas,
    beyond the 256 MB MALL) into the 2 GiB pool (1 GiB with `fp8`: an E4M3
    pool with per-tensor scales), launches back to back."""
    import torch
    import workloads as W
    from harness import upload
    label = "paged_delta_large_fp8" if fp8 else "paged_delta_large"
    log(f"[bench] generating {label}")
    x = W.paged(65536, 64, 8, 128, 128, 8192, 128, W.NEOX, 1044, pool_fill="none",
                name="paged_delta_n65536_p8192")
    if fp8:
        W.with_fp8_cache(x, 7044, fill="sentinel")
    xb = algorithmic_bytes(x)
    tx = upload(x)
    # the pool is filled on the device (its contents do not change the work)
    tx["pool"] = torch.zeros((2, x.num_pages, W.TOKENS_PER_PAGE, x.Hkv, x.D),
                             dtype=torch.uint8 if fp8 else torch.float16, device="cuda")
    k_ms, _ = time_launches(x, tx, steps, warmup)
    gbs = xb / (k_ms * 1e-3) / 1e9
    log(f"[bench] {label}: {k_ms * 1e3:.1f} us, {gbs:.0f} GB/s "
        f"({gbs / PEAK_HBM_GBS:.1%})")
    del tx, x
    torch.cuda.empty_cache()
    return {"workload": "paged_delta_n65536_p8192" + ("_fp8" if fp8 else ""),
            "kernel_us": k_ms * 1e3, "GB/s": gbs,
            "frac": gbs / PEAK_HBM_GBS, "tokens_per_s": 65536 / (k_ms * 1e-3),
            "algorithmic_bytes": xb, "note": "launches back to back over 4 copies of the written tensors, event span / count"}


def small_cases():
    """The workloads whose inputs fit the 256 MB MALL, by label."""
    import workloads as W
    return {
        "continuous_neox": lambda: W.config(2, W.NEOX),
        "continuous_gptj": lambda: W.config(2, W.GPTJ),
        "tree": lambda: W.config(3),
        "paged_delta": lambda: W.config(4),
        "paged_delta_gather_fused": lambda: W.config(41),
        "continuous_neox_fp8_cache":
            lambda: W.with_fp8_cache(W.config(2, W.NEOX), 7002, fill="sentinel"),
        "paged_delta_fp8_cache": lambda: W.with_fp8_cache(W.config(4), 7004, fill="sentinel"),
        "continuous_neox_qknorm": lambda: W.with_qk_norm(W.config(2, W.NEOX), 7102),
        # one GPU's share of the large prefill under 8-way tensor parallelism
        # (8 Q heads, 1 KV head; 193 MB, within the 256 MB MALL, hence flushed)
        "prefill_tp8_shard": lambda: W.prefill_tp_shard(8),
    }


def small_workload(label, make, steps):
    """One small workload: rotated (HBM steady state, the figure of record)
    and back-to-back warm times."""
    import torch
    import workloads as W
    from harness import launch, upload
    log(f"[bench] generating {label}")
    x = make()
    xb = algorithmic_bytes(x)
    tx = upload(x)
    sets = full_copies(tx, xb)
    r_ms = time_rotated(lambda s: launch(x, s), sets, steps)
    del sets
    torch.cuda.empty_cache()
    h_ms = time_queued(lambda: launch(x, tx), steps)
    gbs = xb / (r_ms * 1e-3) / 1e9
    log(f"[bench] {label}: {r_ms * 1e3:.2f} us rotated, {gbs:.0f} GB/s "
        f"({gbs / PEAK_HBM_GBS:.1%}); warm, back to back {h_ms * 1e3:.2f} us")
    name, tokens = x.name, x.tokens
    extra = {}
    if isinstance(x, W.Paged):
        # call 4 counts its N physical rows as tokens; the rows it writes are
        # those with a position, a sequence below the batch size and a page
        p, q = x.positions.astype(np.int64), x.seq.astype(np.int64)
        live = (p >= 0) & (q >= 0) & (q < x.batch) & (p < x.max_pages * W.TOKENS_PER_PAGE)
        valid = int(live.sum())
        extra = {"valid_rows": valid, "valid_rows_per_s": valid / (r_ms * 1e-3)}
    del tx, x
    torch.cuda.empty_cache()
    return {"workload": name, "kernel_us": r_ms * 1e3, "GB/s": gbs, "frac": gbs / PEAK_HBM_GBS,
            "tokens_per_s": tokens / (r_ms * 1e-3), **extra, "algorithmic_bytes": xb,
            "protocol": ROTATED_PROTOCOL,
            "hot_kernel_us": h_ms * 1e3,
            "hot_note": "not flushed: launches queued ahead and run back to back on the same "
                        "tensors (inputs left in MALL / L2 by the previous launch), event span / "
                        "count"}


def _device_paged(x):
    """Upload a paged workload whose pool is created on the device (its
    contents do not change the work)."""
    import torch
    import workloads as W
    from harness import upload
    t = upload(x)
    t["pool"] = torch.zeros((2, x.num_pages, W.TOKENS_PER_PAGE, x.Hkv, x.D),
                            dtype=torch.uint8 if x.extra.get("fp8") else torch.float16,
                            device="cuda")
    return t


CEILING_PARTS = ("streams", "persistent", "empty", "paged", "prefill", "shapes", "graph")


def ceilings_leg(steps, parts=CEILING_PARTS):
    """Ceilings and floors on this chip, from the kernels in ceilings/ timed
    beside the library's (rocprofv3's kernel trace of this run is the
    reference for the short ones):

    * copy and in-place streams over 1 GiB buffers, four buffers cycled, with
      the library's load and store policy (buffer loads nt, buffer stores nt
      sc1) and with plain accesses, XCDs taking 128-workgroup chunks in turn
      or contiguous eighths;
    * the in-place stream in persistent form (a fixed grid of workgroups
      looping over the buffer, 1, 2 or 4 chunks per step, with and without
      the next step's loads issued before the current stores, in plain or
      XCD-region order) beside the one-workgroup-per-chunk stream;
    * an empty kernel of 1 and of 2048 workgroups (the paged workload's
      grid), flushed and back to back;
    * the paged workload's shape (4096 delta rows, 8 KV heads, D = R = 128,
      NeoX, sequences of 128 rows of which 115 are written) moved by an
      index-free floor (every address computed from the row number), into
      contiguous rows and scattered over pool pages, in both access plans,
      beside the library's paged update on the paged workload;
    * the large prefill with its cos/sin row staged in LDS (one workgroup per
      token, 2 or 4 row groups per wave) beside the library's kernel;
    * launch shapes: each workload under every forced number of row groups
      per wave (and both load plans of the paged update), timed as its figure
      of record is;
    * graph: the empty kernel and the small workloads launched back to back
      on the stream and the same launches captured in one HIP graph."""
    out = {}
    flush = make_flush()
    if "streams" in parts:
        out.update(_stream_ceilings(steps))
    if "persistent" in parts:
        out["persistent_streams"] = _persistent_streams(steps)
    if "empty" in parts:
        out.update(_empty_kernels(steps, flush))
    if "paged" in parts:
        out.update(_paged_floors(steps, flush))
    if "prefill" in parts:
        out.update(_prefill_lds(steps))
    if "shapes" in parts:
        out["launch_shapes"] = _launch_shapes(steps)
    if "graph" in parts:
        out["graph_launches"] = _graph_launches(steps)
    return out


def _graph_launches(steps):
    """Per-launch cost on the stream and inside a HIP graph: the empty kernel
    (1 and 2048 workgroups) back to back, and every small workload over full
    copies of its tensors (the rotated protocol), each also captured as one
    graph of the same launches in the same order (time_graph).  Three
    rounds, stream and graph alternating; medians.  Returns {name: {...}}."""
    import torch
    import ceilings as C
    from harness import launch, upload
    out = {}

    def both(name, run_k, n, stream_ms):
        e, g = [], []
        for _ in range(3):
            e.append(stream_ms())
            g.append(time_graph(run_k, n))
        out[name] = {"stream_us": float(np.median(e)) * 1e3, "graph_us": float(np.median(g)) * 1e3,
                     "launches": n, "graph_protocol": GRAPH_PROTOCOL}
        log(f"[bench] {name}: {out[name]['stream_us']:.2f} us per launch on the stream, "
            f"{out[name]['graph_us']:.2f} us in a graph")

    for wg in (1, 2048):
        both(f"empty_kernel_{wg}wg", lambda k, wg=wg: C.empty(wg), steps,
             lambda wg=wg: time_queued(lambda: C.empty(wg), steps))
    for name, make in small_cases().items():
        w = make()
        t = upload(w)
        sets = full_copies(t, algorithmic_bytes(w))
        n = len(sets) * max(1, steps // len(sets))
        both(name, lambda k: launch(w, sets[k % len(sets)]), n,
             lambda: time_rotated(lambda s_: launch(w, s_), sets, n))
        del sets, t, w
        torch.cuda.empty_cache()
    return out


def _stream_ceilings(steps):
    import torch
    import ceilings as C
    out = {}
    GiB = 1 << 30
    bufs = [torch.ones(GiB // 2, dtype=torch.float16, device="cuda") for _ in range(8)]
    for policy, pname in ((1, "library policy (nt loads, nt sc1 stores)"), (0, "plain")):
        for chunk in (7, 0):
            tag = f"{'lib' if policy else 'plain'}_xcd{'chunk128' if chunk else 'eighths'}"
            for kind in ("copy", "narrow", "inplace"):
                k = [0]

                def run():
                    i = k[0] % 4
                    k[0] += 1
                    if kind == "copy":
                        C.stream_copy(bufs[i], bufs[4 + i], policy, chunk)
                    elif kind == "narrow":
                        C.stream_narrow(bufs[i], bufs[4 + i], policy, chunk)
                    else:
                        C.stream_inplace(bufs[i], policy, chunk)
                for _ in range(4):
                    run()
                torch.cuda.synchronize()
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(steps):
                    run()
                b.record()
                torch.cuda.synchronize()
                us = a.elapsed_time(b) / steps * 1e3
                moved = GiB + GiB // 2 if kind == "narrow" else 2 * GiB
                gbs = moved / (us * 1e-6) / 1e9
                out[f"stream_{kind}_{tag}"] = {"kernel_us": us, "bytes": moved, "GB/s": gbs,
                                               "frac": gbs / PEAK_HBM_GBS, "policy": pname,
                                               "timing": "back to back over 4 buffers"}
                log(f"[bench] ceiling stream_{kind}_{tag}: {us:.1f} us, {gbs:.0f} GB/s")
    del bufs
    torch.cuda.empty_cache()
    return out


PERSISTENT_FORMS = [  # (chunks per step, next loads before stores, XCD regions, workgroups per CU)
    (1, 0, 0, 8), (2, 0, 0, 4), (4, 0, 0, 2), (1, 1, 0, 4), (4, 1, 0, 2),
    (1, 0, 1, 4), (4, 0, 1, 2), (2, 1, 1, 2), (4, 1, 1, 2)]


def _persistent_streams(steps):
    """The in-place stream with the library's policy over 1 GiB, four
    buffers cycled, as the one-workgroup-per-chunk kernel (128-workgroup XCD
    chunks) and in each persistent form of PERSISTENT_FORMS; two rounds,
    interleaved; per form the round with the lower time."""
    import torch
    import ceilings as C
    GiB = 1 << 30
    bufs = [torch.ones(GiB // 2, dtype=torch.float16, device="cuda") for _ in range(4)]
    n = max(8, steps // 5)

    def timed(launch):
        for i in range(4):
            launch(bufs[i])
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n):
            launch(bufs[i % 4])
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3

    forms = {"one_workgroup_per_chunk": lambda buf: C.stream_inplace(buf, 1, 7)}
    for u, pipe, xcd, wpc in PERSISTENT_FORMS:
        forms[f"persistent_u{u}_pipe{pipe}_{'xcd' if xcd else 'plain'}_wg{wpc}"] = (
            lambda buf, u=u, pipe=pipe, xcd=xcd, wpc=wpc:
                C.stream_persistent(buf, u, pipe, xcd, 256 * wpc))
    times = {k: [] for k in forms}
    for _ in range(2):
        for k, launch in forms.items():
            times[k].append(timed(launch))
    out = {}
    for k, v in times.items():
        us = min(v)
        gbs = 2 * GiB / (us * 1e-6) / 1e9
        out[k] = {"kernel_us": us, "rounds_us": v, "GB/s": gbs, "frac": gbs / PEAK_HBM_GBS,
                  "launches": n}
        log(f"[bench] {k}: {us:.1f} us, {gbs:.0f} GB/s")
    del bufs
    torch.cuda.empty_cache()
    return out


def _four_ways(run_set, t, nbytes, flush, steps):
    """rotated (time_rotated over full copies of `t`), cold (time_cold),
    marginal (time_flushed) and back-to-back warm times of run_set(t), us."""
    import torch
    sets = full_copies(t, nbytes)
    r_ms = time_rotated(run_set, sets, steps)
    del sets
    torch.cuda.empty_cache()
    c_ms, ev_ms = time_cold(lambda: run_set(t), flush, steps)
    m_ms = time_flushed(lambda: run_set(t), flush, steps)
    h_ms = time_queued(lambda: run_set(t), steps)
    return {"kernel_us": r_ms * 1e3, "protocol": ROTATED_PROTOCOL, "cold_us": c_ms * 1e3,
            "event_pair_us": ev_ms * 1e3, "marginal_us": m_ms * 1e3, "hot_kernel_us": h_ms * 1e3,
            "cold_protocol": COLD_PROTOCOL, "marginal_protocol": MARGINAL_PROTOCOL}


def _empty_kernels(steps, flush):
    import ceilings as C
    out = {}
    for wg in (1, 2048):
        r = _four_ways(lambda t: C.empty(wg), {}, 1, flush, steps)
        out[f"empty_kernel_{wg}wg"] = r
        log(f"[bench] ceiling empty kernel {wg} workgroups: {r['kernel_us']:.2f} us back to back "
            f"(rotated protocol), {r['cold_us']:.2f} us cold, {r['marginal_us']:.2f} us marginal")
    return out


def _paged_floors(steps, flush):
    import torch
    import ceilings as C
    import workloads as W
    from harness import launch
    out = {}
    x = W.paged(4096, 32, 8, 128, 128, 8192, 128, W.NEOX, 1004, pool_fill="none",
                name="paged_delta_n4096_p8192")
    xb = algorithmic_bytes(x)
    tx = _device_paged(x)
    r = _four_ways(lambda t: launch(x, t), tx, xb, flush, steps)
    r.update(bytes=xb, **{"GB/s": xb / (r["kernel_us"] * 1e-6) / 1e9})
    out["paged_delta_library"] = r
    log(f"[bench] paged update (library): {r['kernel_us']:.2f} us rotated, {r['cold_us']:.2f} us "
        f"cold, {r['marginal_us']:.2f} us marginal, {r['hot_kernel_us']:.2f} us back to back")
    live, rows_log2 = 115, 7
    n_live = sum(min(live, 128) for _ in range(4096 // 128))
    floor_bytes = n_live * (8 * 128 * 2 * 4 + 128 * 4)
    for scatter, plan, g in [(sc, pl, g) for sc in (0, 1) for pl in (0, 1) for g in (2, 4)]:
        def run(t, scatter=scatter, plan=plan, g=g):
            C.paged_floor(t["k_delta"], t["v_delta"], t["pool"], t["cos_sin"],
                          x.num_pages, rows_log2, live, scatter, g, plan)
        r = _four_ways(run, tx, floor_bytes, flush, steps)
        r.update(bytes=floor_bytes, **{"GB/s": floor_bytes / (r["kernel_us"] * 1e-6) / 1e9})
        name = (f"paged_floor_{'scatter' if scatter else 'contiguous'}_"
                f"{'nt_policy' if plan else 'default_policy'}_g{g}")
        out[name] = r
        log(f"[bench] {name}: {r['kernel_us']:.2f} us rotated ({r['GB/s']:.0f} GB/s), "
            f"{r['cold_us']:.2f} us cold, {r['marginal_us']:.2f} us marginal, "
            f"{r['hot_kernel_us']:.2f} us back to back")
    del tx, x
    torch.cuda.empty_cache()
    return out


def _prefill_lds(steps):
    """Call 1 on the headline shape with one workgroup per token: the cos/sin
    row staged in LDS (lds_*) or fetched per wave as the library does
    (wave_*), and, on the same shape in NeoX style, the NeoX partners
    exchanged by ds_bpermute (the library's) or by DPP (wave_*_dpp).  Each
    variant back to back over four copies of the written tensors, two
    interleaved series; the library's own launch beside them."""
    import torch
    import ceilings as C
    import workloads as W
    from harness import launch, upload
    out = {}
    for style_name in ("gptj", "neox"):
        w = W.config(HEADLINE)
        if style_name == "neox":
            w = _styled(w, W.NEOX)
        nbytes = algorithmic_bytes(w)
        t = upload(w)
        sets = rotated(w, t, ROTATIONS)
        variants = [("library", None, None, True, False)]
        variants += [(f"lds_g{g}_xcd{c}", g, c, True, False) for g in (2, 4) for c in (5, 0)]
        variants += [(f"wave_g{g}_xcd5", g, 5, False, False) for g in (2, 4)]
        if style_name == "neox":
            variants += [(f"wave_g{g}_xcd5_dpp", g, 5, False, True) for g in (2, 4)]
        for rep in range(2):
            for name, g, c, lds, dpp in variants:
                k = [0]

                def run(g=g, c=c, lds=lds, dpp=dpp):
                    s = sets[k[0] % len(sets)]
                    k[0] += 1
                    if g is None:
                        launch(w, s)
                    else:
                        C.prefill_lds(s["cos_sin"], s["qkv"], s["cache"], w.style, g, c, lds, dpp)
                for _ in range(4):
                    run()
                torch.cuda.synchronize()
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(steps):
                    run()
                b.record()
                torch.cuda.synchronize()
                us = a.elapsed_time(b) / steps * 1e3
                key = f"prefill_{style_name}_{name}"
                prev = out.get(key, {}).get("kernel_us_series", [])
                out[key] = {"kernel_us_series": prev + [us], "bytes": nbytes,
                            "timing": "back to back over 4 copies of the written tensors; two "
                                      "interleaved series"}
                log(f"[bench] {key}: {us:.1f} us ({nbytes / (us * 1e-6) / 1e9:.0f} GB/s)")
        del sets, t
        torch.cuda.empty_cache()
    return out


def _launch_shapes(steps):
    """Every workload under each forced row-group count (rkv_set_launch_
    overrides; results are identical under all of them), and the paged
    update under both load plans: the large workloads back to back over four
    copies of the written tensors (time_launches), the small ones back to
    back over full copies (time_rotated).  The library's own choice is
    reported beside them.  Returns {workload: {setting: us}}."""
    import torch
    import rope_kv_cache_amd as rkv
    import workloads as W
    from harness import launch, upload
    out = {}

    def sweep(label, w, t, large, plans=(0,), exact=False):
        """Three rounds over the settings, each round in a rotated order (so
        that no setting always runs first); median per setting."""
        nb = algorithmic_bytes(w)
        sets = None if large else full_copies(t, nb)
        settings = [(g, plan) for plan in plans for g in (0, 1, 2, 4)]
        times = {}
        for rnd in range(3):
            k = rnd * len(settings) // 3
            for g, plan in settings[k:] + settings[:k]:
                rkv.set_launch_overrides(g, plan)
                try:
                    if large:
                        ms, _ = time_launches(w, t, max(10, steps // 2), 3, exact=exact)
                    else:
                        ms = time_rotated(lambda s_: launch(w, s_, exact), sets, steps)
                    chosen = rkv.last_launch_groups_per_wave()
                    loads = rkv.last_launch_paged_loads()
                finally:
                    rkv.set_launch_overrides(0, 0)
                key = (f"G{g}" if g else f"auto(G{chosen})") + \
                    (f"_{'early' if loads == 1 else 'late'}" if loads else "")
                times.setdefault(key, []).append(ms * 1e3)
        res = {k: float(np.median(v)) for k, v in times.items()}
        log(f"[bench] shapes {label}: " + ", ".join(f"{k} {v:.2f}" for k, v in res.items()))
        out[label] = {"median_us": res, "rounds_us": times}
        del sets
        torch.cuda.empty_cache()

    for label, make, large, plans in (
            ("prefill_gptj", lambda: W.config(HEADLINE), True, (0,)),
            ("prefill_gptj_exact", lambda: W.config(HEADLINE), True, (0,)),
            ("prefill_neox", lambda: _styled(W.config(HEADLINE), W.NEOX), True, (0,)),
            ("prefill_fp8_cache", lambda: W.with_fp8_cache(W.config(HEADLINE), 7005, fill="sentinel"), True, (0,)),
            ("prefill_qknorm", lambda: W.with_qk_norm(W.config(HEADLINE), 7105), True, (0,)),
            ("prefill_qknorm_neox", lambda: _styled(W.with_qk_norm(W.config(HEADLINE), 7105), W.NEOX), True, (0,)),
            ("prefill_neox_exact", lambda: _styled(W.config(HEADLINE), W.NEOX), True, (0,)),
            ("prefill_fp8_cache_exact", lambda: W.with_fp8_cache(W.config(HEADLINE), 7005, fill="sentinel"), True, (0,)),
            ("prefill_qknorm_fp8_cache", lambda: W.with_fp8_cache(W.with_qk_norm(W.config(HEADLINE), 7105), 7005, fill="sentinel"), True, (0,)),
            ("prefill_qknorm_fp8_cache_neox", lambda: _styled(W.with_fp8_cache(W.with_qk_norm(W.config(HEADLINE), 7105), 7005, fill="sentinel"), W.NEOX), True, (0,)),
            ("paged_delta_n65536", lambda: W.paged(65536, 64, 8, 128, 128, 8192, 128, W.NEOX, 1044,
                                                   pool_fill="none", name="paged_delta_n65536_p8192"),
             True, (1, 2)),
            ("paged_delta_n65536_gptj", lambda: W.paged(65536, 64, 8, 128, 128, 8192, 128, W.GPTJ, 1045,
                                                        pool_fill="none", name="paged_delta_n65536_gptj"),
             True, (2,)),
            ("paged_delta_n65536_fp8", lambda: W.with_fp8_cache(
                W.paged(65536, 64, 8, 128, 128, 8192, 128, W.NEOX, 1044, pool_fill="none",
                        name="paged_delta_n65536_p8192"), 7044, fill="sentinel"), True, (2,)),
            ("paged_delta_n65536_fp8_gptj", lambda: W.with_fp8_cache(
                W.paged(65536, 64, 8, 128, 128, 8192, 128, W.GPTJ, 1046, pool_fill="none",
                        name="paged_delta_n65536_gptj"), 7046, fill="sentinel"), True, (2,))):
        log(f"[bench] generating {label}")
        w = make()
        t = _device_paged(w) if isinstance(w, W.Paged) else upload(w)
        sweep(label, w, t, large, plans, exact=label.endswith("_exact"))
        del t, w
        torch.cuda.empty_cache()
    smalls = dict(small_cases())
    smalls["paged_delta_gptj"] = lambda: _styled(W.config(4), W.GPTJ)
    smalls["paged_delta_exact"] = lambda: W.config(4)
    smalls["continuous_neox_exact"] = lambda: W.config(2, W.NEOX)
    for label, make in smalls.items():
        log(f"[bench] generating {label}")
        w = make()
        t = upload(w)
        sweep(label, w, t, False, (1, 2) if isinstance(w, W.Paged) else (0,),
              exact=label.endswith("_exact"))
        del t, w
        torch.cuda.empty_cache()
    return out


def _styled(w, style):
    w.style = style
    return w


def traffic_from_profile(kernel_name: str):
    """HBM bytes per launch measured with rocprofv3 counters, if the recorded
    kernel source still matches the current one."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    h = re.search(r"^kernel_source_sha256:\s*([0-9a-f]+)", text, re.M)
    if not m or not h or h.group(1) != kernel_source_hash():
        return None
    return float(m.group(1))


def kernel_source_hash(d=None) -> str:
    """SHA-256 of the library's HIP sources (in `d`, by default the
    package's csrc) with comments and blank space removed: a traffic profile
    stays valid across comment edits and is void once any code changes."""
    d = d or os.path.join(ROOT, "rope_kv_cache_amd", "csrc")
    hsh = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp")):
            text = open(os.path.join(d, f)).read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            hsh.update(f.encode())
            hsh.update(" ".join(text.split()).encode())
    return hsh.hexdigest()


def host_cpus():
    """(threads to use, logical CPUs of the host, CPUs this process may run
    on, CPU model).  The threads are the CPUs this process may run on,
    capped by OMP_NUM_THREADS when the environment sets it (a machine's CPU
    share for this job)."""
    host = os.cpu_count() or 1
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = host
    use = allowed
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        use = min(use, int(env))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return use, host, allowed, model


def _oracle_parts(w, ranges):
    """Inputs of the oracle's call 1 for token ranges [t0, t1) of sequences
    b, made once, outside any timed region: the range's table rows (so that
    its first token sits at position t0, as in the whole call), its qkv rows
    and a cache of its own of capacity t1 - t0 that receives its K and V
    rows.  Each part computes exactly the values the whole call computes for
    those tokens."""
    tb = w.cos_sin.shape[0]
    parts = []
    for b, t0, t1 in ranges:
        table = np.ascontiguousarray(w.cos_sin[b if tb > 1 else 0, t0:t1][None])
        qkv = np.array(w.qkv[b:b + 1, t0:t1], order="C")
        cache = np.empty((1, 2, w.Hkv, t1 - t0, w.D), dtype=np.uint16)
        parts.append((table, qkv, cache))
    return parts


def _token_ranges(w, n_parts):
    """Split every sequence into ceil(n_parts / B) contiguous token ranges."""
    per_seq = max(1, -(-n_parts // w.B))
    step = -(-w.S // per_seq)
    return [(b, t0, min(w.S, t0 + step)) for b in range(w.B) for t0 in range(0, w.S, step)]


def _time_parts(w, parts, threads, budget_s):
    """One warm-up round of every part's oracle call (in place) on a pool of
    `threads` host threads, then timed rounds until the budget is spent; the
    oracle's C code runs outside Python's interpreter lock.  Returns (tokens
    per second at the median round, rounds, seconds)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    oracle.lib()
    tokens = sum(p[1].shape[1] for p in parts)
    rounds = []
    with ThreadPoolExecutor(max_workers=threads) as pool:
        list(pool.map(lambda p: oracle.packed_qkv_in_place(*p, w.style), parts))
        while sum(rounds) < budget_s or len(rounds) < 3:
            t0 = time.perf_counter()
            list(pool.map(lambda p: oracle.packed_qkv_in_place(*p, w.style), parts))
            rounds.append(time.perf_counter() - t0)
    return tokens / float(np.median(rounds)), len(rounds), sum(rounds)


def cpu_baseline(w, budget_s=15.0):
    """The oracle as it is (plain C, one call-1 evaluation per token range),
    partitioned over every CPU this process may use: all B x S tokens of the
    headline workload in contiguous token ranges, at least one per thread,
    repeated until the budget is spent; the rate of the median round, and
    the same in GB/s of the call's algorithmic bytes."""
    use, host, allowed, model = host_cpus()
    parts = _oracle_parts(w, _token_ranges(w, use))
    rate, n, secs = _time_parts(w, parts, use, budget_s)
    gbs = rate * algorithmic_bytes(w) / w.tokens / 1e9
    return {"value": rate, "unit": "tokens/s", "cores": use, "kind": "oracle", "GB/s": gbs,
            "host_logical_cpus": host, "cpus_allowed": allowed, "cpu_model": model,
            "sample": f"all {w.B * w.S} tokens of the workload in {len(parts)} token ranges on "
                      f"{use} threads, one warm-up round, then the median of {n} rounds of "
                      f"in-place oracle calls ({secs:.1f} s)"}


def cpu_baseline_single(w, budget_s=10.0):
    """The same oracle on one thread: sequence 0's first 2048 tokens, called
    in place repeatedly until the budget is spent."""
    parts = _oracle_parts(w, [(0, 0, min(w.S, 2048))])
    rate, n, secs = _time_parts(w, parts, 1, budget_s)
    return {"value": rate, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "GB/s": rate * algorithmic_bytes(w) / w.tokens / 1e9,
            "sample": f"tokens 0-{parts[0][1].shape[1] - 1} of sequence 0, one warm-up call, "
                      f"then the median of {n} in-place oracle calls ({secs:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--paged-large", nargs="?", const="fp16", default=None,
                    choices=("fp16", "fp8", "both"),
                    help="time only the 65,536-row paged update into an fp16 pool, an E4M3 "
                         "pool, or both (for counter runs; default fp16)")
    ap.add_argument("--workload", action="append", default=[], metavar="NAME",
                    help="time only this small workload (repeatable; for counter and trace "
                         "runs): " + ", ".join(small_cases()))
    ap.add_argument("--ceilings", nargs="?", const=",".join(CEILING_PARTS), default=None,
                    metavar="PARTS",
                    help="time only the ceilings and floors of ceilings/ beside the library's "
                         "kernels: a comma list of " + ", ".join(CEILING_PARTS) + " (default: all)")
    ap.add_argument("--calib", action="store_true",
                    help="also run a 1 GiB elementwise copy (1 GiB read + 1 GiB written per "
                         "launch) to scale HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the step "
              "needs no cross-GPU exchange, so each GPU would run this same kernel on its "
              "own shard of batches, heads or pages", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    from harness import upload
    import rope_kv_cache_amd  # noqa: F401  (fails loudly if the library is missing)

    assert torch.cuda.is_available(), "no GPU visible"
    torch.cuda.set_device(0)
    log(f"[bench] device: {torch.cuda.get_device_name(0)}")
    if args.ceilings is not None or args.workload:
        cases = small_cases()
        unknown = [n for n in args.workload if n not in cases]
        parts = [p for p in (args.ceilings or "").split(",") if p]
        unknown += [p for p in parts if p not in CEILING_PARTS]
        if unknown:
            sys.exit(f"unknown workload(s) or ceiling part(s) {unknown}; choose from "
                     f"{list(cases)} and {list(CEILING_PARTS)}")
        res = {}
        if args.workload:
            res["workloads"] = {n: small_workload(n, cases[n], args.steps)
                                for n in args.workload}
        if parts:
            res["ceilings"] = ceilings_leg(args.steps, parts)
        if args.calib:
            calibration_copy()
        print(json.dumps(res), flush=True)
        return
    if args.paged_large:
        res = {}
        if args.paged_large in ("fp16", "both"):
            res["paged_delta_large"] = paged_large(args.steps, args.warmup)
        if args.paged_large in ("fp8", "both"):
            res["paged_delta_large_fp8"] = paged_large(args.steps, args.warmup, fp8=True)
        if args.calib:
            calibration_copy()
        print(json.dumps(res), flush=True)
        return

    log("[bench] generating the headline workload")
    w = W.config(HEADLINE)
    nbytes = algorithmic_bytes(w)
    t = upload(w)
    log(f"[bench] {w.name}: {nbytes / 1e6:.1f} MB algorithmic per launch; timing "
        f"{args.warmup} + {args.steps} steps")
    kernel_ms, wall = time_launches(w, t, args.steps, args.warmup)
    ms_per_step = wall / args.steps * 1e3
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    traffic = traffic_from_profile("contig_packed_prefill_b4_s8192_h64_d128")
    result = {
        "metric": "tokens/s and achieved HBM GB/s (% of MI355X peak) for fused RoPE+KV write",
        "value": w.tokens / (wall / args.steps),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "call": "packed QKV prefill, in place", "B": w.B,
                   "S": w.S, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "R": w.R, "style": "gptj",
                   "io": "fp16 qkv/cache, fp32 cos/sin", "tokens_per_step": w.tokens,
                   "timing": f"launches back to back, cycling {ROTATIONS} copies of qkv and "
                             "the cache"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel_us": kernel_ms * 1e3, "algorithmic_bytes": nbytes},
    }
    log(f"[bench] headline kernel {kernel_ms * 1e3:.1f} us, {achieved:.0f} GB/s "
        f"({achieved / PEAK_HBM_GBS:.1%}), {result['value']:.3e} tokens/s")
    extra = {}
    if not args.no_extra:
        ex_ms, ex_wall = time_launches(w, t, max(10, args.steps // 2), 3, exact=True)
        ex_gbs = nbytes / (ex_ms * 1e-3) / 1e9
        extra["prefill_exact_rounding"] = {
            "workload": w.name, "mode": "RKV_ROUND_EXACT (binary64, bit-identical)",
            "kernel_us": ex_ms * 1e3, "GB/s": ex_gbs, "frac": ex_gbs / PEAK_HBM_GBS,
            "tokens_per_s": w.tokens / (ex_ms * 1e-3)}
        log(f"[bench] exact mode: {ex_ms * 1e3:.1f} us, {ex_gbs:.0f} GB/s")
        # the same data in the NeoX layout (same bytes; each lane fetches 8 cos/sin pairs)
        style0, w.style = w.style, W.NEOX
        nx_ms, _ = time_launches(w, t, max(10, args.steps // 2), 3)
        w.style = style0
        nx_gbs = nbytes / (nx_ms * 1e-3) / 1e9
        extra["prefill_neox"] = {
            "workload": w.name, "layout": "NeoX (rotate-half pairs)",
            "kernel_us": nx_ms * 1e3, "GB/s": nx_gbs, "frac": nx_gbs / PEAK_HBM_GBS,
            "tokens_per_s": w.tokens / (nx_ms * 1e-3)}
        log(f"[bench] NeoX layout: {nx_ms * 1e3:.1f} us, {nx_gbs:.0f} GB/s "
            f"({nx_gbs / PEAK_HBM_GBS:.1%})")
    del t
    torch.cuda.empty_cache()

    if not args.no_extra:
        # the same prefill into an E4M3 cache with per-tensor scales
        W.with_fp8_cache(w, 7005, fill="sentinel")
        f8_bytes = algorithmic_bytes(w)
        t = upload(w)
        f8_ms, f8_wall = time_launches(w, t, max(10, args.steps // 2), 3)
        f8_gbs = f8_bytes / (f8_ms * 1e-3) / 1e9
        extra["prefill_fp8_cache"] = {
            "workload": w.name, "cache": "E4M3, per-tensor k/v scales",
            "kernel_us": f8_ms * 1e3, "GB/s": f8_gbs, "frac": f8_gbs / PEAK_HBM_GBS,
            "tokens_per_s": w.tokens / (f8_ms * 1e-3), "algorithmic_bytes": f8_bytes}
        log(f"[bench] fp8 cache: {f8_ms * 1e3:.1f} us, {f8_gbs:.0f} GB/s "
            f"({f8_gbs / PEAK_HBM_GBS:.1%})")
        del t
        torch.cuda.empty_cache()
        # the same prefill with Q/K RMS norm before the rotation, fp16 cache
        w = W.config(HEADLINE)
        W.with_qk_norm(w, 7105)
        nb = algorithmic_bytes(w)
        t = upload(w)
        n_ms, _ = time_launches(w, t, max(10, args.steps // 2), 3)
        n_gbs = nb / (n_ms * 1e-3) / 1e9
        extra["prefill_qknorm"] = {
            "workload": w.name, "norm": "RMS norm of Q and K heads before the rotation",
            "kernel_us": n_ms * 1e3, "GB/s": n_gbs, "frac": n_gbs / PEAK_HBM_GBS,
            "tokens_per_s": w.tokens / (n_ms * 1e-3), "algorithmic_bytes": nb}
        log(f"[bench] Q/K norm: {n_ms * 1e3:.1f} us, {n_gbs:.0f} GB/s "
            f"({n_gbs / PEAK_HBM_GBS:.1%})")
        w.style = W.NEOX
        nn_ms, _ = time_launches(w, t, max(10, args.steps // 2), 3)
        nn_gbs = nb / (nn_ms * 1e-3) / 1e9
        extra["prefill_qknorm_neox"] = {
            "workload": w.name, "norm": "RMS norm of Q and K heads before the rotation",
            "layout": "NeoX (rotate-half pairs)",
            "kernel_us": nn_ms * 1e3, "GB/s": nn_gbs, "frac": nn_gbs / PEAK_HBM_GBS,
            "tokens_per_s": w.tokens / (nn_ms * 1e-3), "algorithmic_bytes": nb}
        log(f"[bench] Q/K norm, NeoX layout: {nn_ms * 1e3:.1f} us, {nn_gbs:.0f} GB/s "
            f"({nn_gbs / PEAK_HBM_GBS:.1%})")
        del t
        torch.cuda.empty_cache()

    if args.calib:
        calibration_copy()

    if not args.no_extra:
        for label, make in small_cases().items():
            extra[label] = small_workload(label, make, max(20, args.steps))
        torch.cuda.empty_cache()
        extra["paged_delta_large"] = paged_large(max(10, args.steps // 2))
        extra["paged_delta_large_fp8"] = paged_large(max(10, args.steps // 2), fp8=True)
        # call 2 at a size where bandwidth bounds it: 16 sequences x 1024 new tokens
        # (0.4 GB moved, beyond the 256 MB MALL)
        log("[bench] generating continuous_large")
        x = W.continuous(16, 1024, 32, 8, 128, 128, 2048, W.NEOX, 1062, 1024, 2048,
                         theta=500000.0, cache_fill="sentinel",
                         name="continuous_b16_s1024_d128_neox")
        xb = algorithmic_bytes(x)
        tx = upload(x)
        c_ms, _ = time_launches(x, tx, max(10, args.steps // 2), 3)
        gbs = xb / (c_ms * 1e-3) / 1e9
        extra["continuous_large"] = {
            "workload": x.name, "kernel_us": c_ms * 1e3, "GB/s": gbs,
            "frac": gbs / PEAK_HBM_GBS, "tokens_per_s": x.tokens / (c_ms * 1e-3),
            "algorithmic_bytes": xb, "note": "launches back to back over 4 copies of the written tensors, event span / count"}
        log(f"[bench] continuous_large: {c_ms * 1e3:.1f} us, {gbs:.0f} GB/s "
            f"({gbs / PEAK_HBM_GBS:.1%})")
        del tx, x
        torch.cuda.empty_cache()
        meta = metadata_builders(max(10, args.steps // 2))
        for k, v in meta.items():
            log(f"[bench] {k}: {v['kernel_us']:.2f} us")
        extra.update(meta)
        result["workloads"] = extra

    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a sample")
        w = W.config(HEADLINE)
        result["cpu_baseline"] = cpu_baseline(w)
        cb = result["cpu_baseline"]
        log(f"[bench] cpu oracle, {cb['cores']} threads ({cb['cpu_model']}, "
            f"{cb['host_logical_cpus']} logical CPUs): {cb['value']:.3e} tokens/s")
        result["cpu_baseline_single_thread"] = cpu_baseline_single(w)
        log(f"[bench] cpu oracle, 1 thread: "
            f"{result['cpu_baseline_single_thread']['value']:.3e} tokens/s")
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
