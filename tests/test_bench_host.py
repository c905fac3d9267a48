"""bench.py on the host: its algorithmic byte counts (the numerator of every
roofline figure) against closed forms written out by hand, and its refusal
of more than one GPU."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def _headline():
    """The large prefill's shapes only (the byte count needs no data)."""
    return W.Contig("packed", W.GPTJ, 4, 8192, 64, 8, 128, 128, 16384,
                    np.empty((4, 8192, 128), np.float32), None, None,
                    name="prefill_b4_s8192_h64_d128")


def test_headline_bytes():
    """Large prefill: per token, 80 head rows of 256 B read, 72 rotated rows
    written in place, 16 cache rows written; each of the 4 x 8192 table rows
    (512 B) read once."""
    w = _headline()
    per_token = 80 * 256 + 72 * 256 + 16 * 256
    assert bench.algorithmic_bytes(w) == 32768 * per_token + 32768 * 512 == 1426063360


def test_variant_bytes():
    w = _headline()
    w.cache = np.empty(0, np.uint16)
    w.extra["fp8"] = {"k_scale": np.float32(1), "v_scale": np.float32(1)}
    # cache rows of 128 B instead of 256 B, plus the two 4-byte scales
    assert bench.algorithmic_bytes(w) == 32768 * (80 * 256 + 72 * 256 + 16 * 128) \
        + 32768 * 512 + 8
    w = _headline()
    w.extra["qknorm"] = {"q_weight": np.ones(128, np.float32), "k_weight": np.ones(128, np.float32),
                         "eps": 1e-6}
    # plus the two fp32 weight vectors of 128 entries
    assert bench.algorithmic_bytes(w) == 1426063360 + 2 * 128 * 4


def test_paged_bytes_by_row():
    """Paged workload: the per-row rule applied row by row in a plain loop.
    (The workload's index arrays without its 2 GiB pool: the pool is drawn
    last, so they are those of the benchmarked workload.)"""
    w = W.paged(4096, 32, 8, 128, 128, 8192, 128, W.NEOX, 1004, pool_fill="none")
    row = w.Hkv * w.D * 2
    total = 0
    for i in range(w.N):
        p, q = int(w.positions[i]), int(w.seq[i])
        total += 8                                    # its position and sequence
        if p < 0 or q < 0 or q >= w.batch or p >= w.max_pages * 64:
            continue
        total += 8                                    # its two page-table entries
        kid = int(w.page_table[q, 0, p // 64])
        vid = int(w.page_table[q, 1, p // 64])
        if 0 <= kid < w.num_pages:
            total += 2 * row + w.R * 4                # K read + written, cos/sin row
        if w.num_pages <= vid < 2 * w.num_pages:
            total += 2 * row                          # V read + written
    assert bench.algorithmic_bytes(w) == total == 30381456


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_kernel_source_hash_ignores_comments_only(tmp_path):
    src = "// header\n__global__ void k(int* p) {  /* body */\n  p[0] = 1;   // store\n}\n"
    (tmp_path / "a.hip").write_text(src)
    h0 = bench.kernel_source_hash(str(tmp_path))
    (tmp_path / "a.hip").write_text(src.replace("// store", "// the store").replace("header", "x"))
    assert bench.kernel_source_hash(str(tmp_path)) == h0
    (tmp_path / "a.hip").write_text(src.replace("p[0] = 1", "p[0] = 2"))
    assert bench.kernel_source_hash(str(tmp_path)) != h0


def test_rotated_copies_only_the_written_tensors():
    """Back-to-back timings cycle through copies of what a call writes: call 1
    writes qkv and the cache, calls 2-3 the cache and qOut, call 4 the pool;
    everything else is shared."""
    import torch
    from harness import upload
    cases = [(W.config(1), ("qkv", "cache")), (W.config(2), ("cache", "q_out")),
             (W.config(3), ("cache", "q_out"))]
    for w, keys in cases:
        t = upload(w, device="cpu")
        sets = bench.rotated(w, t, 3)
        assert len(sets) == 3 and sets[0] is t
        assert bench.written_keys(w) == keys
        for u in sets[1:]:
            assert set(u) == set(t)
            for k, v in u.items():
                if k in keys:
                    assert v is not t[k] and v.data_ptr() != t[k].data_ptr()
                    assert torch.equal(v.view(torch.int16), t[k].view(torch.int16))
                else:
                    assert v is t[k]
    p = W.paged(64, 2, 2, 64, 64, 8, 4, W.NEOX, 5, name="p")
    assert bench.written_keys(p) == ("pool",)


def test_token_ranges_cover_every_token_once():
    w = _headline()
    for parts in (1, 3, 4, 16, 100, 257):
        ranges = bench._token_ranges(w, parts)
        assert len(ranges) >= min(parts, w.B * w.S)
        seen = np.zeros((w.B, w.S), dtype=np.int32)
        for b, t0, t1 in ranges:
            assert 0 <= t0 < t1 <= w.S
            seen[b, t0:t1] += 1
        assert (seen == 1).all()


def test_cpu_baseline_parts_reproduce_the_whole_call():
    """The CPU baseline's token-range parts compute exactly what one call on
    the whole workload computes: every part's in-place qkv rows and its own
    cache rows equal the whole call's, bit for bit."""
    import oracle
    w = W.packed(2, 40, 4, 2, 128, 128, 48, W.GPTJ, 77, table_batch=2, table_len=48,
                 offsets=np.array([0, 9]), name="t")
    whole_qkv, whole_cache = oracle.packed_qkv(w.cos_sin, w.qkv, w.cache, w.style)
    ranges = bench._token_ranges(w, 7)
    parts = bench._oracle_parts(w, ranges)
    for (b, t0, t1), (table, qkv, cache) in zip(ranges, parts):
        oracle.packed_qkv_in_place(table, qkv, cache, w.style)
        assert np.array_equal(qkv[0], whole_qkv[b, t0:t1])
        assert np.array_equal(cache[0], whole_cache[b, :, :, t0:t1])


def test_host_cpus():
    use, host, allowed, model = bench.host_cpus()
    assert 1 <= use <= allowed <= host and isinstance(model, str) and model


def test_ceilings_library_loads():
    """The measurement kernels' library is built and exports its entry points
    (no kernel is launched here)."""
    import ceilings as C
    for name in ("rkvc_stream_copy", "rkvc_stream_inplace", "rkvc_stream_narrow",
                 "rkvc_stream_persistent", "rkvc_check_reciprocal", "rkvc_check_f16_pair",
                 "rkvc_empty",
                 "rkvc_paged_floor", "rkvc_prefill_lds"):
        assert hasattr(C._L, name)


def test_cpu_baseline_reports_rate_bandwidth_and_cores():
    """The CPU leg times every CPU this process may use, reports the median
    round's rate and the same rate in GB/s of the call's algorithmic bytes."""
    import workloads as W
    w = W.config(1)
    cb = bench.cpu_baseline(w, budget_s=0.2)
    use, host, allowed, model = bench.host_cpus()
    assert cb["cores"] == use and cb["host_logical_cpus"] == host and cb["cpu_model"] == model
    assert cb["value"] > 0 and cb["kind"] == "oracle" and cb["unit"] == "tokens/s"
    per_token = bench.algorithmic_bytes(w) / w.tokens
    assert abs(cb["GB/s"] - cb["value"] * per_token / 1e9) < 1e-9 * max(1.0, cb["GB/s"])
    single = bench.cpu_baseline_single(w, budget_s=0.1)
    assert single["cores"] == 1 and single["value"] > 0
