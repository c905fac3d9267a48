"""The C ABI on the host, without a GPU.

* ``librkv.so`` loads and exports every function ``include/rope_kv_cache.h``
  declares.
* Host validation returns the documented status for every malformed call,
  before any HIP call (so these run on a machine without a GPU).
* The capacity check follows its truth table (tests/golden/capacity_check.txt).

The descriptors here carry fake device addresses that are never dereferenced:
every call below is invalid or empty, so it returns before any launch.  As a
guard against a validation bug turning one of them into a launch, the
fake-pointer tests are skipped when a GPU is visible.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rope_kv_cache.h")

rkv = pytest.importorskip("rope_kv_cache_amd")
L = rkv.lib
T = rkv.RkvTensor
F16, F32, I32 = 0, 1, 2


def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0


no_gpu = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer validation tests run on CPU only")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rkv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_calls():
    names = declared_functions()
    for want in ["rkv_apply_rope_write_kv_packed_qkv", "rkv_apply_rope_write_kv_continuous",
                 "rkv_apply_rope_write_kv_tree", "rkv_dflash_target_kv_cache_update",
                 "rkv_check_rope_capacity", "rkv_tokens_per_page", "rkv_last_error",
                 "rkv_status_string", "rkv_last_launch_groups_per_wave"]:
        assert want in names


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports(name):
    lib = ctypes.CDLL(rkv.LIB_PATH)
    assert hasattr(lib, name)


def test_status_strings_and_page_size():
    assert rkv.tokens_per_page() == 64
    for code, name in enumerate(["RKV_OK", "RKV_ERR_NULL", "RKV_ERR_DTYPE", "RKV_ERR_SHAPE",
                                 "RKV_ERR_UNSUPPORTED", "RKV_ERR_CAPACITY", "RKV_ERR_ALIGNMENT",
                                 "RKV_ERR_ALIAS", "RKV_ERR_HIP"]):
        assert rkv.status_string(code) == name


def test_capacity_truth_table():
    path = os.path.join(ROOT, "tests", "golden", "capacity_check.txt")
    for line in open(path):
        line = line.split("#")[0].split()
        if not line:
            continue
        a, b, want = int(line[0]), int(line[1]), line[2]
        st = L.rkv_check_rope_capacity(a, b)
        assert st == (rkv.OK if want == "ok" else rkv.ERR_CAPACITY), (a, b)
        if want != "ok":
            assert b"exceeds" in L.rkv_last_error()
        with pytest.raises(rkv.RkvError) if want != "ok" else _nullctx():
            rkv.check_rope_capacity(a, b)


class _nullctx:
    def __enter__(self):
        return None

    def __exit__(self, *a):
        return False


# --------------------------------------------------------------- helpers --

_next = [0x7F0000000000]


def fake(dtype, *shape, addr=None):
    t = T()
    if addr is None:
        _next[0] += 1 << 36
        addr = _next[0]
    t.data = addr
    t.dtype = dtype
    t.ndim = len(shape)
    for k, n in enumerate(shape):
        t.shape[k] = n
    return t


def packed_args(B=2, S=8, Hq=4, Hkv=2, D=128, R=128, cap=16, tb=1, tl=16):
    return [fake(F32, tb, tl, R), fake(F16, B, S, Hq + 2 * Hkv, D), fake(F16, B, 2, Hkv, cap, D)]


def call_packed(cs, qkv, cache, style=0):
    b = ctypes.byref
    return L.rkv_apply_rope_write_kv_packed_qkv(b(cs) if cs else None, b(qkv) if qkv else None,
                                                b(cache) if cache else None, style, None)


def cont_args(B=2, S=8, Hq=4, Hkv=2, D=128, R=128, cap=16, tb=1, tl=16):
    return [fake(F32, tb, tl, R), fake(I32, B), fake(F16, B, S, Hq + 2 * Hkv, D),
            fake(F16, B, 2, Hkv, cap, D), fake(F16, B, S, Hq, D)]


def call_cont(args, style=0):
    return L.rkv_apply_rope_write_kv_continuous(*[ctypes.byref(a) if a else None for a in args],
                                                style, None)


def tree_args(B=2, S=8, Hq=4, Hkv=2, D=128, R=64, cap=16):
    c = cont_args(B, S, Hq, Hkv, D, R, cap)
    return [c[0], c[1], fake(I32, B, S), c[2], c[3], c[4]]


def call_tree(args, style=0):
    return L.rkv_apply_rope_write_kv_tree(*[ctypes.byref(a) if a else None for a in args], style,
                                          None)


# ------------------------------------------------------------ call 1 ------

@no_gpu
@pytest.mark.parametrize("case,want", [
    ("null_cos_sin", rkv.ERR_NULL), ("null_qkv", rkv.ERR_NULL), ("null_cache", rkv.ERR_NULL),
    ("null_data", rkv.ERR_NULL), ("qkv_f32", rkv.ERR_DTYPE), ("table_f16", rkv.ERR_DTYPE),
    ("qkv_rank3", rkv.ERR_SHAPE), ("cache_B", rkv.ERR_SHAPE), ("cache_planes", rkv.ERR_SHAPE),
    ("cache_D", rkv.ERR_SHAPE), ("table_batch", rkv.ERR_SHAPE), ("too_few_heads", rkv.ERR_SHAPE),
    ("odd_R", rkv.ERR_SHAPE), ("R_gt_D", rkv.ERR_SHAPE), ("R_not_16", rkv.ERR_UNSUPPORTED),
    ("D_96", rkv.ERR_UNSUPPORTED), ("S_gt_cap", rkv.ERR_CAPACITY),
    ("S_gt_table", rkv.ERR_CAPACITY), ("misaligned", rkv.ERR_ALIGNMENT),
    ("cache_aliases_qkv", rkv.ERR_ALIAS), ("table_aliases_cache", rkv.ERR_ALIAS),
    ("bad_style", rkv.ERR_SHAPE), ("negative_extent", rkv.ERR_SHAPE),
])
def test_packed_validation(case, want):
    cs, qkv, cache = packed_args()
    style = 0
    if case == "null_cos_sin":
        cs = None
    elif case == "null_qkv":
        qkv = None
    elif case == "null_cache":
        cache = None
    elif case == "null_data":
        qkv.data = None
    elif case == "qkv_f32":
        qkv.dtype = F32
    elif case == "table_f16":
        cs.dtype = F16
    elif case == "qkv_rank3":
        qkv = fake(F16, 16, 8, 128)
    elif case == "cache_B":
        cache.shape[0] = 3
    elif case == "cache_planes":
        cache.shape[1] = 1
    elif case == "cache_D":
        cache.shape[4] = 64
    elif case == "table_batch":
        cs.shape[0] = 3
    elif case == "too_few_heads":
        qkv.shape[2] = 3
    elif case == "odd_R":
        cs.shape[2] = 63
    elif case == "R_gt_D":
        cs.shape[2] = 144
    elif case == "R_not_16":
        cs.shape[2] = 40
    elif case == "D_96":
        cs, qkv, cache = packed_args(D=96, R=96)
    elif case == "S_gt_cap":
        cs, qkv, cache = packed_args(S=8, cap=7)
    elif case == "S_gt_table":
        cs, qkv, cache = packed_args(S=8, tl=7)
    elif case == "misaligned":
        cache.data = cache.data + 2
    elif case == "cache_aliases_qkv":
        cache.data = qkv.data + 4096
    elif case == "table_aliases_cache":
        cs.data = cache.data
    elif case == "bad_style":
        style = 2
    elif case == "negative_extent":
        qkv.shape[1] = -1
    st = call_packed(cs, qkv, cache, style)
    assert st == want, (case, rkv.status_string(st), L.rkv_last_error())
    assert L.rkv_last_error() != b""
    assert rkv.last_launch_groups_per_wave() == 0


@no_gpu
def test_packed_empty_is_ok_without_launch():
    for B, S in [(0, 8), (2, 0)]:
        cs, qkv, cache = packed_args(B=B, S=S)
        assert call_packed(cs, qkv, cache) == rkv.OK
        assert rkv.last_launch_groups_per_wave() == 0
    # zero heads: nothing to do
    cs, qkv, cache = packed_args(Hq=0, Hkv=0)
    assert call_packed(cs, qkv, cache) == rkv.OK


@no_gpu
def test_more_waves_than_one_dispatch_is_unsupported():
    """2^24 tokens of 80 heads need 2^24 * 5 waves even at four row groups per
    wave: more than one dispatch's 2^32 - 1 work-items hold."""
    S = 1 << 24
    cs = fake(F32, 1, S, 128, addr=1 << 42)
    qkv = fake(F16, 1, S, 80, 128, addr=2 << 42)
    cache = fake(F16, 1, 2, 8, S, 128, addr=3 << 42)
    st = call_packed(cs, qkv, cache, style=1)
    assert st == rkv.ERR_UNSUPPORTED, (rkv.status_string(st), L.rkv_last_error())
    assert b"too many rows" in L.rkv_last_error()


@no_gpu
def test_token_rows_beyond_32bit_offsets_are_unsupported():
    """A token's head rows are addressed by 32-bit byte offsets: 2^23 heads
    of 256 values (4 GiB per token) are refused before any launch."""
    H = 1 << 23
    cs = fake(F32, 1, 4, 256, addr=1 << 42)
    qkv = fake(F16, 1, 1, H, 256, addr=2 << 42)
    cache = fake(F16, 1, 2, 1, 4, 256, addr=3 << 42)
    st = call_packed(cs, qkv, cache, style=1)
    assert st == rkv.ERR_UNSUPPORTED, (rkv.status_string(st), L.rkv_last_error())
    assert b"heads of 256 values per token" in L.rkv_last_error()


# -------------------------------------------------------- calls 2 and 3 ---

@no_gpu
@pytest.mark.parametrize("case,want", [
    ("null_end", rkv.ERR_NULL), ("null_qout", rkv.ERR_NULL), ("end_f32", rkv.ERR_DTYPE),
    ("qout_f32", rkv.ERR_DTYPE), ("end_len_B", rkv.ERR_SHAPE), ("qout_S", rkv.ERR_SHAPE),
    ("heads_mismatch", rkv.ERR_SHAPE), ("qout_aliases_qkv", rkv.ERR_ALIAS),
    ("qout_aliases_cache", rkv.ERR_ALIAS), ("cache_aliases_end", rkv.ERR_ALIAS),
])
def test_continuous_validation(case, want):
    a = cont_args()
    if case == "null_end":
        a[1] = None
    elif case == "null_qout":
        a[4] = None
    elif case == "end_f32":
        a[1].dtype = F32
    elif case == "qout_f32":
        a[4].dtype = F32
    elif case == "end_len_B":
        a[1].shape[0] = 3
    elif case == "qout_S":
        a[4].shape[1] = 7
    elif case == "heads_mismatch":
        a[4].shape[2] = 5
    elif case == "qout_aliases_qkv":
        a[4].data = a[2].data + 256
    elif case == "qout_aliases_cache":
        a[4].data = a[3].data
    elif case == "cache_aliases_end":
        a[3].data = a[1].data - 4096
    st = call_cont(a)
    assert st == want, (case, rkv.status_string(st), L.rkv_last_error())


@no_gpu
def test_continuous_does_not_check_capacity_on_host():
    # the token positions live on the device; S > cap is not a host error,
    # so the call gets past validation.  Make it fail on an unsupported D so
    # that nothing is launched.
    a = cont_args(S=8, cap=4, D=96, R=96)
    assert call_cont(a) == rkv.ERR_UNSUPPORTED


@no_gpu
@pytest.mark.parametrize("case,want", [
    ("null_pos", rkv.ERR_NULL), ("pos_f16", rkv.ERR_DTYPE), ("pos_shape", rkv.ERR_SHAPE),
    ("cache_aliases_pos", rkv.ERR_ALIAS),
])
def test_tree_validation(case, want):
    a = tree_args()
    if case == "null_pos":
        a[2] = None
    elif case == "pos_f16":
        a[2].dtype = F16
    elif case == "pos_shape":
        a[2].shape[1] = 9
    elif case == "cache_aliases_pos":
        a[4].data = a[2].data
    st = call_tree(a)
    assert st == want, (case, rkv.status_string(st), L.rkv_last_error())


@no_gpu
def test_continuous_and_tree_empty():
    assert call_cont(cont_args(B=0)) == rkv.OK
    assert call_tree(tree_args(S=0)) == rkv.OK


# ---------------------------------------------------------------- call 4 --

def paged_call(**kw):
    base = dict(k=1 << 40, v=2 << 40, pool=3 << 40, cs=4 << 40, pos=5 << 40, seq=6 << 40,
                pt=7 << 40, N=16, batch=2, Hkv=2, D=128, R=128, P=8, M=4, style=0)
    base.update(kw)
    b = base
    return L.rkv_dflash_target_kv_cache_update(b["k"], b["v"], b["pool"], b["cs"], b["pos"],
                                               b["seq"], b["pt"], b["N"], b["batch"], b["Hkv"],
                                               b["D"], b["R"], b["P"], b["M"], b["style"], None)


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(N=-1), rkv.ERR_SHAPE), (dict(batch=-2), rkv.ERR_SHAPE), (dict(Hkv=-1), rkv.ERR_SHAPE),
    (dict(P=-1), rkv.ERR_SHAPE), (dict(M=-1), rkv.ERR_SHAPE), (dict(style=5), rkv.ERR_SHAPE),
    (dict(R=130), rkv.ERR_SHAPE), (dict(R=7), rkv.ERR_SHAPE), (dict(R=24), rkv.ERR_UNSUPPORTED),
    (dict(D=32, R=32), rkv.ERR_UNSUPPORTED), (dict(k=0), rkv.ERR_NULL), (dict(pt=0), rkv.ERR_NULL),
    (dict(pool=0), rkv.ERR_NULL), (dict(cs=0), rkv.ERR_NULL), (dict(pos=0), rkv.ERR_NULL),
    (dict(cs=0, R=0, D=96), rkv.ERR_UNSUPPORTED),    # null cos/sin accepted when R = 0
    (dict(cs=(4 << 40) + 8), rkv.ERR_ALIGNMENT),
    (dict(pool=(1 << 40) + 4096), rkv.ERR_ALIAS), (dict(pt=(3 << 40) + 64), rkv.ERR_ALIAS),
    (dict(P=1 << 30, Hkv=1 << 20), rkv.ERR_SHAPE),
    (dict(N=1, P=0, Hkv=(1 << 30) + 1, D=64, R=64), rkv.ERR_UNSUPPORTED),
])
def test_paged_validation(kw, want):
    st = paged_call(**kw)
    assert st == want, (kw, rkv.status_string(st), L.rkv_last_error())


def gather_call(**kw):
    base = dict(k=1 << 40, v=2 << 40, pool=3 << 40, rope=4 << 40, states=2, rows=512, si=8 << 40,
                pos=5 << 40, seq=6 << 40, pt=7 << 40, N=16, batch=2, Hkv=2, D=128, R=128, P=8,
                M=4, style=0)
    base.update(kw)
    b = base
    return L.rkv_dflash_target_kv_cache_update_gather_rope(
        b["k"], b["v"], b["pool"], b["rope"], b["states"], b["rows"], b["si"], b["pos"], b["seq"],
        b["pt"], b["N"], b["batch"], b["Hkv"], b["D"], b["R"], b["P"], b["M"], b["style"], None)


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(states=-1), rkv.ERR_SHAPE), (dict(rows=-1), rkv.ERR_SHAPE), (dict(rope=0), rkv.ERR_NULL),
    (dict(si=(8 << 40) + 4), rkv.ERR_ALIGNMENT), (dict(pool=(4 << 40) + 1024), rkv.ERR_ALIAS),
    (dict(si=(3 << 40) + 64), rkv.ERR_ALIAS), (dict(R=24), rkv.ERR_UNSUPPORTED),
    (dict(style=0x102), rkv.ERR_SHAPE), (dict(N=0), rkv.OK), (dict(P=0), rkv.OK),
    # an empty rope table may be null: validation then stops at the unsupported D
    (dict(rope=0, states=0, D=96, R=96), rkv.ERR_UNSUPPORTED),
])
def test_gather_validation(kw, want):
    st = gather_call(**kw)
    assert st == want, (kw, rkv.status_string(st), L.rkv_last_error())


@no_gpu
def test_gather_null_state_indices_accepted_by_validation():
    # stateIndices may be null; stop before the launch with an empty pool
    assert gather_call(si=0, P=0) == rkv.OK


@no_gpu
def test_paged_empty():
    assert paged_call(N=0) == rkv.OK
    assert paged_call(Hkv=0) == rkv.OK
    assert paged_call(P=0) == rkv.OK         # an empty pool: nothing can be written
    assert paged_call(M=0) == rkv.OK
    assert paged_call(batch=0, M=0) == rkv.OK


def test_binding_rejects_host_tensors():
    import torch
    cs = torch.zeros(1, 16, 128)
    qkv = torch.zeros(1, 8, 8, 128, dtype=torch.float16)
    cache = torch.zeros(1, 2, 2, 16, 128, dtype=torch.float16)
    with pytest.raises(ValueError):
        rkv.apply_rope_write_kv_packed_qkv(cs, qkv, cache, rkv.ROPE_NEOX)


# ------------------------------------------------------------ fp8 calls ---

F8 = 3


def call_packed_fp8(cs, qkv, cache, ks=None, vs=None, style=0):
    b = ctypes.byref
    return L.rkv_apply_rope_write_kv_packed_qkv_fp8(b(cs), b(qkv), b(cache), ks, vs, style, None)


@no_gpu
@pytest.mark.parametrize("case,want", [
    ("fp16_cache", rkv.ERR_DTYPE), ("f32_cache", rkv.ERR_DTYPE),
    ("misaligned_k_scale", rkv.ERR_ALIGNMENT), ("misaligned_v_scale", rkv.ERR_ALIGNMENT),
    ("cache_covers_k_scale", rkv.ERR_ALIAS), ("qkv_covers_v_scale", rkv.ERR_ALIAS),
    ("null_scales_then_D_96", rkv.ERR_UNSUPPORTED), ("empty", rkv.OK),
    ("misaligned_cache", rkv.ERR_ALIGNMENT),
])
def test_packed_fp8_validation(case, want):
    cs, qkv, cache = packed_args()
    cache.dtype = F8
    ks, vs = 9 << 40, 10 << 40
    if case == "fp16_cache":
        cache.dtype = F16
    elif case == "f32_cache":
        cache.dtype = F32
    elif case == "misaligned_k_scale":
        ks += 2
    elif case == "misaligned_v_scale":
        vs += 1
    elif case == "cache_covers_k_scale":
        ks = cache.data + 1024
    elif case == "qkv_covers_v_scale":
        vs = qkv.data + 64      # qkv is an output of call 1
    elif case == "null_scales_then_D_96":
        cs, qkv, cache = packed_args(D=96, R=96)
        cache.dtype = F8
        ks = vs = None
    elif case == "empty":
        cs, qkv, cache = packed_args(B=0)
        cache.dtype = F8
    elif case == "misaligned_cache":
        cache.data = cache.data + 8
    st = call_packed_fp8(cs, qkv, cache, ks, vs)
    assert st == want, (case, rkv.status_string(st), L.rkv_last_error())


@no_gpu
def test_fp16_calls_reject_an_fp8_cache():
    cs, qkv, cache = packed_args()
    cache.dtype = F8
    assert call_packed(cs, qkv, cache) == rkv.ERR_DTYPE
    a = cont_args()
    a[3].dtype = F8
    assert call_cont(a) == rkv.ERR_DTYPE


@no_gpu
def test_continuous_and_tree_fp8_validation():
    a = cont_args()
    a[3].dtype = F8
    b = ctypes.byref
    st = L.rkv_apply_rope_write_kv_continuous_fp8(*[b(x) for x in a], a[3].data + 16, None, 0,
                                                  None)
    assert st == rkv.ERR_ALIAS, L.rkv_last_error()
    t = tree_args()
    t[4].dtype = F16
    st = L.rkv_apply_rope_write_kv_tree_fp8(*[b(x) for x in t], None, None, 0, None)
    assert st == rkv.ERR_DTYPE
    t[4].dtype = F8
    t[2].shape[1] = 3
    st = L.rkv_apply_rope_write_kv_tree_fp8(*[b(x) for x in t], None, None, 0, None)
    assert st == rkv.ERR_SHAPE
    c = cont_args(B=0)
    c[3].dtype = F8
    assert L.rkv_apply_rope_write_kv_continuous_fp8(*[b(x) for x in c], None, None, 0,
                                                    None) == rkv.OK


def paged_fp8_call(**kw):
    base = dict(k=1 << 40, v=2 << 40, pool=3 << 40, ks=11 << 40, vs=12 << 40, cs=4 << 40,
                pos=5 << 40, seq=6 << 40, pt=7 << 40, N=16, batch=2, Hkv=2, D=128, R=128, P=8,
                M=4, style=0)
    base.update(kw)
    b = base
    return L.rkv_dflash_target_kv_cache_update_fp8(
        b["k"], b["v"], b["pool"], b["ks"], b["vs"], b["cs"], b["pos"], b["seq"], b["pt"],
        b["N"], b["batch"], b["Hkv"], b["D"], b["R"], b["P"], b["M"], b["style"], None)


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(ks=(11 << 40) + 2), rkv.ERR_ALIGNMENT), (dict(ks=(3 << 40) + 4), rkv.ERR_ALIAS),
    (dict(vs=(3 << 40) + 262140), rkv.ERR_ALIAS),       # last byte of the 262,144-byte pool
    (dict(pool=0), rkv.ERR_NULL), (dict(R=24), rkv.ERR_UNSUPPORTED), (dict(N=0), rkv.OK),
    (dict(P=0), rkv.OK), (dict(ks=0, vs=0, P=0), rkv.OK),
])
def test_paged_fp8_validation(kw, want):
    st = paged_fp8_call(**kw)
    assert st == want, (kw, rkv.status_string(st), L.rkv_last_error())


@no_gpu
def test_gather_fp8_validation():
    def call(**kw):
        base = dict(k=1 << 40, v=2 << 40, pool=3 << 40, ks=11 << 40, vs=12 << 40, rope=4 << 40,
                    states=2, rows=512, si=8 << 40, pos=5 << 40, seq=6 << 40, pt=7 << 40, N=16,
                    batch=2, Hkv=2, D=128, R=128, P=8, M=4, style=0)
        base.update(kw)
        b = base
        return L.rkv_dflash_target_kv_cache_update_gather_rope_fp8(
            b["k"], b["v"], b["pool"], b["ks"], b["vs"], b["rope"], b["states"], b["rows"],
            b["si"], b["pos"], b["seq"], b["pt"], b["N"], b["batch"], b["Hkv"], b["D"], b["R"],
            b["P"], b["M"], b["style"], None)
    assert call(vs=(12 << 40) + 1) == rkv.ERR_ALIGNMENT
    assert call(vs=(3 << 40) + 8) == rkv.ERR_ALIAS
    assert call(rope=0) == rkv.ERR_NULL
    assert call(P=0) == rkv.OK


def test_fp8_binding_rejects_fp16_cache():
    import torch
    cs = torch.zeros(1, 16, 128)
    qkv = torch.zeros(1, 8, 8, 128, dtype=torch.float16)
    cache = torch.zeros(1, 2, 2, 16, 128, dtype=torch.float16)
    with pytest.raises(ValueError):
        rkv.apply_rope_write_kv_packed_qkv_fp8(cs, qkv, cache, None, None, rkv.ROPE_NEOX)


# ------------------------------------------------------ Q/K-norm calls ---

def call_packed_norm(cs, qkv, cache, qw=None, kw=None, eps=1e-6, ks=None, vs=None, style=0):
    b = ctypes.byref
    return L.rkv_apply_rope_write_kv_packed_qkv_qknorm(b(cs), b(qkv), b(cache), qw, kw,
                                                       ctypes.c_float(eps), ks, vs, style, None)


@no_gpu
@pytest.mark.parametrize("case,want", [
    ("eps_negative", rkv.ERR_SHAPE), ("eps_nan", rkv.ERR_SHAPE), ("eps_inf", rkv.ERR_SHAPE),
    ("q_weight_misaligned", rkv.ERR_ALIGNMENT), ("k_weight_misaligned", rkv.ERR_ALIGNMENT),
    ("cache_covers_k_weight", rkv.ERR_ALIAS), ("qkv_covers_q_weight", rkv.ERR_ALIAS),
    ("scales_with_fp16_cache", rkv.ERR_DTYPE), ("f32_cache", rkv.ERR_DTYPE),
    ("fp8_cache_then_D_96", rkv.ERR_UNSUPPORTED), ("no_weights_then_D_96", rkv.ERR_UNSUPPORTED),
    ("empty", rkv.OK), ("empty_fp8", rkv.OK),
])
def test_packed_qknorm_validation(case, want):
    cs, qkv, cache = packed_args()
    qw, kw, eps, ks, vs = 13 << 40, 14 << 40, 1e-6, None, None
    if case == "eps_negative":
        eps = -1e-6
    elif case == "eps_nan":
        eps = float("nan")
    elif case == "eps_inf":
        eps = float("inf")
    elif case == "q_weight_misaligned":
        qw += 4
    elif case == "k_weight_misaligned":
        kw += 8
    elif case == "cache_covers_k_weight":
        kw = cache.data + 4096
    elif case == "qkv_covers_q_weight":
        qw = qkv.data + 256
    elif case == "scales_with_fp16_cache":
        ks = 9 << 40
    elif case == "f32_cache":
        cache.dtype = F32
    elif case == "fp8_cache_then_D_96":
        cs, qkv, cache = packed_args(D=96, R=96)
        cache.dtype = F8
        ks, vs = 9 << 40, 10 << 40
    elif case == "no_weights_then_D_96":
        cs, qkv, cache = packed_args(D=96, R=96)
        qw = kw = None
    elif case == "empty":
        cs, qkv, cache = packed_args(B=0)
    elif case == "empty_fp8":
        cs, qkv, cache = packed_args(S=0)
        cache.dtype = F8
    st = call_packed_norm(cs, qkv, cache, qw, kw, eps, ks, vs)
    assert st == want, (case, rkv.status_string(st), L.rkv_last_error())


@no_gpu
def test_continuous_and_tree_qknorm_validation():
    b = ctypes.byref
    a = cont_args()
    st = L.rkv_apply_rope_write_kv_continuous_qknorm(*[b(x) for x in a], 13 << 40, a[4].data,
                                                     ctypes.c_float(1e-6), None, None, 0, None)
    assert st == rkv.ERR_ALIAS, L.rkv_last_error()          # k weight inside qOut
    t = tree_args()
    st = L.rkv_apply_rope_write_kv_tree_qknorm(*[b(x) for x in t], None, None,
                                               ctypes.c_float(-1.0), None, None, 0, None)
    assert st == rkv.ERR_SHAPE
    c = cont_args(B=0)
    assert L.rkv_apply_rope_write_kv_continuous_qknorm(*[b(x) for x in c], None, None,
                                                       ctypes.c_float(0.0), None, None, 0,
                                                       None) == rkv.OK
    assert L.rkv_apply_rope_write_kv_packed_qkv_qknorm(None, None, None, None, None,
                                                       ctypes.c_float(0.0), None, None, 0,
                                                       None) == rkv.ERR_NULL


def test_qknorm_binding_rejects_bad_weights():
    import torch
    cs = torch.zeros(1, 16, 128)
    qkv = torch.zeros(1, 8, 8, 128, dtype=torch.float16)
    cache = torch.zeros(1, 2, 2, 16, 128, dtype=torch.float16)
    with pytest.raises(ValueError):
        rkv.apply_rope_write_kv_packed_qkv_qknorm(cs, qkv, cache, None, None, 1e-6,
                                                  rkv.ROPE_NEOX, k_scale=torch.ones(1))


# ------------------------------------------------------ metadata builders ---

@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(B=-1), rkv.ERR_SHAPE), (dict(width=-1), rkv.ERR_SHAPE),
    (dict(B=1 << 20, width=1 << 12), rkv.ERR_UNSUPPORTED), (dict(old=0), rkv.ERR_NULL),
    (dict(pos=0), rkv.ERR_NULL), (dict(seq=(4 << 40) + 2), rkv.ERR_ALIGNMENT),
    (dict(pos=(1 << 40) + 8), rkv.ERR_ALIAS),          # positions start inside old lengths
    (dict(seq=(3 << 40) + 4 * 16 * 8 - 4), rkv.ERR_ALIAS),   # owners overlap positions' end
    (dict(B=0), rkv.OK), (dict(width=0), rkv.OK), (dict(B=0, old=0, pos=0), rkv.OK),
])
def test_delta_metadata_validation(kw, want):
    a = dict(old=1 << 40, dl=2 << 40, width=16, pos=3 << 40, seq=4 << 40, B=8)
    a.update(kw)
    st = L.rkv_dflash_prepare_delta_metadata(a["old"], a["dl"], a["width"], a["pos"], a["seq"],
                                             a["B"], None)
    assert st == want, (kw, rkv.status_string(st), L.rkv_last_error())


@no_gpu
@pytest.mark.parametrize("kw,want", [
    (dict(B=-1), rkv.ERR_SHAPE), (dict(V=-2), rkv.ERR_SHAPE), (dict(par=0), rkv.ERR_NULL),
    (dict(dep=(2 << 40) + 1), rkv.ERR_ALIGNMENT), (dict(dep=(1 << 40) + 64), rkv.ERR_ALIAS),
    (dict(B=1 << 16, V=1 << 16), rkv.ERR_UNSUPPORTED), (dict(V=0), rkv.OK), (dict(B=0), rkv.OK),
])
def test_linear_tree_validation(kw, want):
    a = dict(par=1 << 40, dep=2 << 40, B=4, V=64)
    a.update(kw)
    st = L.rkv_dflash_build_linear_tree_metadata(a["par"], a["dep"], a["B"], a["V"], None)
    assert st == want, (kw, rkv.status_string(st), L.rkv_last_error())


def test_launch_overrides_validation():
    """rkv_set_launch_overrides accepts 0/1/2/4 row groups and load plans 0-2,
    rejects anything else without changing the setting; a fresh thread's
    last-launch queries read 0."""
    L = rkv.lib
    assert L.rkv_last_launch_paged_loads() == 0
    for g, p in ((0, 0), (1, 1), (2, 2), (4, 0), (0, 2)):
        assert L.rkv_set_launch_overrides(g, p) == rkv.OK
    for g, p in ((3, 0), (8, 0), (-1, 0), (0, 3), (0, -1)):
        assert L.rkv_set_launch_overrides(g, p) == rkv.ERR_SHAPE
        assert "must be" in L.rkv_last_error().decode()
    with pytest.raises(rkv.RkvError):
        rkv.set_launch_overrides(5, 0)
    rkv.set_launch_overrides(0, 0)
