"""The measurement kernels of ceilings/ do the work they stand in for.

bench.py --ceilings times them beside the library's kernels, so each must
move exactly what it claims: the streams copy (or xor in place) every byte;
the index-free paged floor writes the pool that the library's paged update
writes when its positions, sequences and page table encode the floor's
address arithmetic; the LDS-staged prefill produces the library's call-1
output bit for bit (both use the library's default arithmetic).
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def _lib():
    import ceilings as C
    import rope_kv_cache_amd as rkv
    return C, rkv


def test_streams_move_every_byte():
    C, _ = _lib()
    n = 1 << 22   # 8 MiB of fp16
    src = torch.from_numpy(W.normal_f16(W.rng(3), (n,)).view(np.float16)).cuda()
    for policy in (1, 0):
        for chunk in (7, 0):
            dst = torch.zeros_like(src)
            C.stream_copy(src, dst, policy, chunk)
            torch.cuda.synchronize()
            assert torch.equal(dst.view(torch.int16), src.view(torch.int16))
            buf = src.clone()
            C.stream_inplace(buf, policy, chunk, key=0x00010001)
            torch.cuda.synchronize()
            want = src.view(torch.int32) ^ 0x00010001
            assert torch.equal(buf.view(torch.int32), want)
            half = torch.zeros(n // 2, dtype=torch.float16, device="cuda")
            C.stream_narrow(src, half, policy, chunk)
            torch.cuda.synchronize()
            words = src.view(torch.int32)
            assert torch.equal(half.view(torch.int32), words[0::2] ^ words[1::2])


def test_reciprocal_is_the_rounded_binary64_quotient_for_every_fp32():
    """The fp32 reciprocal the fp8 kernels take of a scale (a binary32
    Newton step over the hardware estimate in the middle range, the binary64
    division elsewhere) equals 1/scale in binary64 rounded to binary32, for
    all 2^32 patterns."""
    C, _ = _lib()
    threads = 1 << 20
    counts = torch.zeros(2 * threads, dtype=torch.int32, device="cuda")
    C.check_reciprocal(counts)
    torch.cuda.synchronize()
    c = counts.cpu().numpy().view(np.uint32)
    bad = int(c[0::2].astype(np.uint64).sum())
    firsts = [hex(int(v)) for v in c[1::2][c[0::2] > 0][:8]]
    assert bad == 0, (bad, firsts)


def test_packed_fp16_conversion_equals_two_scalar_ones_for_every_fp32():
    """v_cvt_pk_f16_f32, which the kernels round their fp16 outputs with,
    gives bit for bit the two scalar conversions, for all 2^32 patterns in
    the low half (NaN payloads included)."""
    C, _ = _lib()
    threads = 1 << 20
    counts = torch.zeros(2 * threads, dtype=torch.int32, device="cuda")
    C.check_f16_pair(counts)
    torch.cuda.synchronize()
    c = counts.cpu().numpy().view(np.uint32)
    bad = int(c[0::2].astype(np.uint64).sum())
    firsts = [hex(int(v)) for v in c[1::2][c[0::2] > 0][:8]]
    assert bad == 0, (bad, firsts)


def test_persistent_stream_visits_every_chunk_once():
    """Every persistent form xors each 32-bit word exactly once: a chunk
    visited twice would come back unchanged, one never visited too."""
    C, _ = _lib()
    n = 1 << 22   # 8 MiB of fp16: 2048 chunks of 4 KB, two rounds of 8 x 128
    src = torch.from_numpy(W.normal_f16(W.rng(4), (n,)).view(np.float16)).cuda()
    want = src.view(torch.int32) ^ 0x00FF00FF
    for unroll in (1, 2, 4):
        for pipe in (0, 1):
            for xcd in (0, 1):
                for grid in (8, 64, 512):
                    buf = src.clone()
                    C.stream_persistent(buf, unroll, pipe, xcd, grid, key=0x00FF00FF)
                    torch.cuda.synchronize()
                    assert torch.equal(buf.view(torch.int32), want), (unroll, pipe, xcd, grid)


def _floor_as_paged(N, Hkv, num_pages, rows_log2, live, scatter, seed):
    """Delta rows, cos/sin rows, and the positions, sequences and page table
    under which the library's paged update writes what the floor writes."""
    r = W.rng(seed)
    per = 1 << rows_log2
    seqs = N // per
    i = np.arange(N)
    q, j = i >> rows_log2, i & (per - 1)
    live_row = j < live
    if scatter:
        pos = ((q * 37) & 63) + j
    else:
        pos = j
    positions = np.where(live_row, pos, -1).astype(np.int32)
    seq = np.where(live_row, q, -1).astype(np.int32)
    max_pages = 4
    pt = np.zeros((seqs, 2, max_pages), dtype=np.int32)
    for s in range(seqs):
        for lp in range(max_pages):
            if scatter:
                key = 4 * s + lp
                pt[s, 0, lp] = (key * 1021) & (num_pages - 1)
                pt[s, 1, lp] = num_pages + ((key * 2053) & (num_pages - 1))
            else:
                pt[s, 0, lp] = (per // 64) * s + lp
                pt[s, 1, lp] = num_pages + (per // 64) * s + lp
    k = W.normal_f16(r, (N, Hkv, 128))
    v = W.normal_f16(r, (N, Hkv, 128))
    cs = W.rope_rows(np.where(live_row, pos, 0), 128, 10000.0)
    return k, v, cs, positions, seq, pt, seqs, max_pages


@pytest.mark.parametrize("scatter", [0, 1])
@pytest.mark.parametrize("plan", [0, 1])
@pytest.mark.parametrize("groups", [1, 2, 4])
def test_paged_floor_equals_library_update(scatter, plan, groups):
    C, rkv = _lib()
    from harness import dev
    N, Hkv, num_pages, rows_log2, live = 512, 8, 64, 7, 115
    k, v, cs, positions, seq, pt, seqs, max_pages = _floor_as_paged(
        N, Hkv, num_pages, rows_log2, live, scatter, 40 + scatter)
    kd, vd, csd = dev(k), dev(v), dev(cs)
    fill = W.normal_f16(W.rng(9), (2, num_pages, 64, Hkv, 128))
    pool_floor, pool_lib = dev(fill), dev(fill)
    C.paged_floor(kd, vd, pool_floor, csd, num_pages, rows_log2, live, scatter, groups, plan)
    rkv.dflash_target_kv_cache_update(kd, vd, pool_lib, csd, dev(positions), dev(seq), dev(pt),
                                      seqs, rkv.ROPE_NEOX)
    torch.cuda.synchronize()
    a, b = pool_floor.view(torch.int16), pool_lib.view(torch.int16)
    written = (b != dev(fill).view(torch.int16)).sum().item()
    assert written > 0.9 * N * 2 * Hkv * 128 * (live / 128)
    assert torch.equal(a, b)


_TABLE_MODES = [(True, False), (False, False), (False, True)]   # (lds, dpp)


@pytest.mark.parametrize("style", [W.GPTJ, W.NEOX])
@pytest.mark.parametrize("R", [128, 64])
@pytest.mark.parametrize("groups", [2, 4])
@pytest.mark.parametrize("chunk", [0, 5])
@pytest.mark.parametrize("lds,dpp", _TABLE_MODES, ids=["lds", "per_wave", "per_wave_dpp"])
def test_lds_prefill_equals_library_call1(style, R, groups, chunk, lds, dpp):
    if dpp and (style != W.NEOX or R != 128):
        pytest.skip("the DPP exchange is the NeoX partner map for R = 128 only")
    C, rkv = _lib()
    from harness import upload
    w = W.packed(2, 96, 8, 2, 128, R, 128, style, 55 + R, table_batch=2, table_len=100,
                 offsets=np.array([0, 17]), name="lds")
    t_lib, t_lds = upload(w), upload(w)
    rkv.apply_rope_write_kv_packed_qkv(t_lib["cos_sin"], t_lib["qkv"], t_lib["cache"], style)
    C.prefill_lds(t_lds["cos_sin"], t_lds["qkv"], t_lds["cache"], style, groups, chunk, lds, dpp)
    torch.cuda.synchronize()
    for key in ("qkv", "cache"):
        assert torch.equal(t_lds[key].view(torch.int16), t_lib[key].view(torch.int16)), key
