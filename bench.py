"""Benchmark of the fused RoPE + KV-cache write on one MI355X.

A step is one call of the library on the headline workload: empty-cache
prefill of packed QKV in place, B=4, S=8192, Hq=64, Hkv=8, D=R=128, GPT-J,
per-sequence cos/sin tables (1.43 GB of algorithmic traffic).  Inputs are
seeded synthetic data already resident in HBM.  W warm-up steps, then K timed
steps back to back, bracketed by device synchronisation and by one pair of
HIP events on the launch stream, whose span / K is the kernel's average
duration for the roofline.  The same workload in the library's RKV_ROUND_EXACT mode and the
other workloads (continuous write, tree write, paged delta update, the
paged update with the cos/sin gather fused in, the prefill, continuous
and paged calls into an E4M3 cache, the prefill and continuous calls
with Q/K RMS norm, the prefill in the NeoX layout, a 65,536-row paged update,
a 16-sequence continuous write, and the two device index builders) are
reported under "workloads".  The
small workloads' inputs fit the 256 MB
MALL, so a 1 GiB buffer is read before each of their timed launches to push
them back to HBM (a read leaves clean lines, so the timed kernel inherits no
write-back); their event-bracketed times include the events' own overhead
of a few microseconds, so rocprofv3's kernel trace is the reference there.

Prints one JSON line on stdout; progress goes to stderr.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]
                      [--calib] [--floors] [--paged-large]
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


def time_launches(w, t, steps, warmup, flush=None, exact=False, queue_ahead=False):
    """Kernel duration and wall time of `steps` launches.

    Without `flush`: the launches run back to back on the current stream,
    bracketed by one pair of HIP events and by device synchronisations, so
    that nothing but the launches is timed; the kernel duration is the
    events' span divided by the launch count (the gaps between back-to-back
    launches, about a microsecond, are included).  They cycle through
    ROTATIONS copies of the written tensors (`rotated`), except with
    `queue_ahead`, which times warm launches on purpose.  With `flush` (small
    workloads): a flush runs before each launch, so each launch has its own
    pair of events (their overhead included).  `queue_ahead` (short
    kernels, back to back): the GPU first spins long enough for the host to
    queue every launch, so the span measures the kernels, not the host's
    launch rate."""
    import torch
    from harness import launch as launch_exact

    def launch(w, t):
        launch_exact(w, t, exact)

    stream = torch.cuda.current_stream()
    sets = rotated(w, t, ROTATIONS) if flush is None and not queue_ahead else [t]
    for k in range(warmup):
        if flush is not None:
            flush()
        launch(w, sets[k % len(sets)])
    torch.cuda.synchronize()
    wall = 0.0
    if flush is None:
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        if queue_ahead:
            gpu_busy_wait(2000 + 50 * steps)
        t0 = time.perf_counter()
        start.record(stream)
        for k in range(steps):
            launch(w, sets[k % len(sets)])
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        del sets
        return start.elapsed_time(end) / steps, wall
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for k in range(steps):
        flush()
        starts[k].record(stream)
        launch(w, t)
        ends[k].record(stream)
    torch.cuda.synchronize()
    kernel_ms = float(np.mean([s.elapsed_time(e) for s, e in zip(starts, ends)]))
    return kernel_ms, wall


def time_calls(fn, steps, warmup=3):
    """Average duration of fn()'s launch, events on the current stream."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for k in range(steps):
        starts[k].record(stream)
        fn()
        ends[k].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([s.elapsed_time(e) for s, e in zip(starts, ends)]))


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
    d_ms = time_calls(lambda: rkv.dflash_prepare_delta_metadata(old, dl, width, pos, seq), steps)
    par = torch.empty((16, 64), dtype=torch.int32, device="cuda")
    dep = torch.empty_like(par)
    t_ms = time_calls(lambda: rkv.dflash_build_linear_tree_metadata(par, dep), steps)
    return {
        "delta_metadata_b32_w128": {"kernel_us_events": d_ms * 1e3,
                                    "algorithmic_bytes": 2 * B * 4 + 2 * B * width * 4,
                                    "note": "launch-bound: 32 KB of output"},
        "linear_tree_b16_v64": {"kernel_us_events": t_ms * 1e3,
                                "algorithmic_bytes": 2 * 16 * 64 * 4,
                                "note": "launch-bound: 8 KB of output"},
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


def floors(steps):
    """Lower bounds for the small workloads on this chip, timed like them (a
    1 GiB read before each launch pushes the inputs out of the MALL): a
    plain device copy moving the paged workload's bytes (15.2 MB read, 15.2
    MB written) and a near-empty kernel (one fp32 zeroed)."""
    import torch
    import workloads as W
    flush_buf = torch.ones(1 << 29, dtype=torch.float16, device="cuda")
    flush_sink = torch.empty((), dtype=torch.float32, device="cuda")

    def flush():
        torch.sum(flush_buf, dim=0, dtype=torch.float32, out=flush_sink)

    half = algorithmic_bytes(W.config(4)) // 2
    src = torch.ones(half // 2, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    tiny = torch.ones(1, dtype=torch.float32, device="cuda")
    out = {}
    for label, fn, nbytes in (("copy_paged_bytes", lambda: dst.copy_(src), 2 * src.numel() * 2),
                              ("near_empty_kernel", lambda: tiny.zero_(), 4)):
        stream = torch.cuda.current_stream()
        for _ in range(3):
            flush()
            fn()
        torch.cuda.synchronize()
        st = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        en = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for k in range(steps):
            flush()
            st[k].record(stream)
            fn()
            en[k].record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in zip(st, en)]))
        out[label] = {"kernel_us_events": ms * 1e3, "bytes": nbytes,
                      "GB/s": nbytes / (ms * 1e-3) / 1e9}
        log(f"[bench] floor {label}: {ms * 1e3:.2f} us by events")
    return {"floors": out, "note": "event-bracketed single launches after a 1 GiB read; "
                                   "rocprofv3 kernel durations are the reference"}


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


def _oracle_parts(w, batches):
    """Per-sequence copies of the headline inputs, made once, outside any
    timed region: (table rows, qkv, cache) of each listed sequence."""
    tb = w.cos_sin.shape[0]
    return [(np.ascontiguousarray(w.cos_sin[b:b + 1] if tb > 1 else w.cos_sin),
             np.array(w.qkv[b:b + 1], order="C"), np.array(w.cache[b:b + 1], order="C"))
            for b in batches]


def cpu_baseline(w, budget_s=10.0):
    """The oracle as it is (single-threaded C) on a bounded sample of the
    headline workload: sequence 0 (8192 tokens, all 80 heads), called on
    arrays prepared once (qkv is rotated in place again by each call, as on
    the GPU), repeated until the budget is spent."""
    import oracle
    oracle.lib()
    part = _oracle_parts(w, [0])[0]
    n, t_total = 0, 0.0
    while t_total < budget_s:
        t0 = time.perf_counter()
        oracle.packed_qkv_in_place(*part, w.style)
        t_total += time.perf_counter() - t0
        n += 1
    tokens = n * w.S
    return {"value": tokens / t_total, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"sequence 0 of the workload ({w.S} tokens x {w.Hq + 2 * w.Hkv} heads), "
                      f"{n} oracle calls in place, {t_total:.1f} s"}


def cpu_baseline_threads(w, budget_s=10.0):
    """The same oracle call on all sequences of the headline workload at
    once, one host thread per sequence (call 1 places each sequence's tokens
    from slot 0, so a sequence is its smallest independent piece), repeated
    until the budget is spent.  The oracle's C code runs outside Python's
    interpreter lock, so the threads run in parallel."""
    import threading

    import oracle
    oracle.lib()
    parts = _oracle_parts(w, range(w.B))
    errors = []

    def work(part):
        try:
            oracle.packed_qkv_in_place(*part, w.style)
        except Exception as e:      # surfaced after the join
            errors.append(e)

    n, t_total = 0, 0.0
    while t_total < budget_s:
        threads = [threading.Thread(target=work, args=(part,)) for part in parts]
        t0 = time.perf_counter()
        for th in threads:
            th.start()
        for th in threads:
            th.join()
        t_total += time.perf_counter() - t0
        if errors:
            raise errors[0]
        n += 1
    tokens = n * w.B * w.S
    return {"value": tokens / t_total, "unit": "tokens/s", "cores": len(parts), "kind": "oracle",
            "sample": f"all {w.B} sequences of the workload, one thread each, {n} rounds of "
                      f"in-place calls, {t_total:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--paged-large", action="store_true",
                    help="time only the 65,536-row paged update (for counter runs)")
    ap.add_argument("--floors", action="store_true",
                    help="only time the floors of the small workloads: a torch copy moving the "
                         "paged workload's bytes and a near-empty kernel, each after the same "
                         "MALL flush")
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
    if args.floors:
        print(json.dumps(floors(max(10, args.steps // 2))), flush=True)
        return
    if args.paged_large:
        res = paged_large(args.steps, args.warmup)
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
        flush_buf = torch.ones(1 << 29, dtype=torch.float16, device="cuda")   # 1 GiB
        flush_sink = torch.empty((), dtype=torch.float32, device="cuda")

        def flush():
            torch.sum(flush_buf, dim=0, dtype=torch.float32, out=flush_sink)

        cases = [("continuous_neox", lambda: W.config(2, W.NEOX)),
                 ("continuous_gptj", lambda: W.config(2, W.GPTJ)),
                 ("tree", lambda: W.config(3)),
                 ("paged_delta", lambda: W.config(4)),
                 ("paged_delta_gather_fused", lambda: W.config(41)),
                 ("continuous_neox_fp8_cache",
                  lambda: W.with_fp8_cache(W.config(2, W.NEOX), 7002, fill="sentinel")),
                 ("paged_delta_fp8_cache",
                  lambda: W.with_fp8_cache(W.config(4), 7004, fill="sentinel")),
                 ("continuous_neox_qknorm", lambda: W.with_qk_norm(W.config(2, W.NEOX), 7102)),
                 # one GPU's share of the large prefill under 8-way tensor parallelism
                 # (8 Q heads, 1 KV head; 193 MB, within the 256 MB MALL, hence flushed)
                 ("prefill_tp8_shard", lambda: W.prefill_tp_shard(8))]
        for label, make in cases:
            log(f"[bench] generating {label}")
            x = make()
            xb = algorithmic_bytes(x)
            tx = upload(x)
            steps = max(5, min(args.steps, 50))
            k_ms, _ = time_launches(x, tx, steps, 3, flush=flush)
            gbs = xb / (k_ms * 1e-3) / 1e9
            # hot: the same launches back to back, inputs left in MALL / L2 by the previous one
            h_ms, _ = time_launches(x, tx, steps, 3, queue_ahead=True)
            extra[label] = {"workload": x.name, "kernel_us_events": k_ms * 1e3, "GB/s": gbs,
                            "frac": gbs / PEAK_HBM_GBS, "tokens_per_s": x.tokens / (k_ms * 1e-3),
                            "algorithmic_bytes": xb, "mall_flushed": True,
                            "note": "event-bracketed single launches: includes event overhead",
                            "hot_kernel_us": h_ms * 1e3,
                            "hot_note": "not flushed: launches queued ahead and run back to "
                                        "back, event span / count"}
            log(f"[bench] {label}: {k_ms * 1e3:.2f} us, {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.1%}); "
                f"hot {h_ms * 1e3:.2f} us")
            del tx, x
            torch.cuda.empty_cache()
        del flush_buf
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
            log(f"[bench] {k}: {v['kernel_us_events']:.2f} us")
        extra.update(meta)
        result["workloads"] = extra

    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(w)
        log(f"[bench] cpu oracle {result['cpu_baseline']['value']:.3e} tokens/s")
        result["cpu_baseline_threads"] = cpu_baseline_threads(w)
        log(f"[bench] cpu oracle, {result['cpu_baseline_threads']['cores']} threads: "
            f"{result['cpu_baseline_threads']['value']:.3e} tokens/s")
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
