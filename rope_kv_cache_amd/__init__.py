"""Python binding of ``librkv.so``: fused RoPE + KV-cache write on MI355X.

Argument marshalling only.  Each function turns torch device tensors into the
C descriptors of ``include/rope_kv_cache.h``, passes torch's current HIP
stream of the tensors' device, and raises :class:`RkvError` with the
library's message when the call returns an error status.  All computation
happens in the HIP kernels of ``librkv.so``; there is no fallback: if the
library is missing, importing this package raises.

Functions (same names as the C entry points, without the ``rkv_`` prefix):
  apply_rope_write_kv_packed_qkv(cos_sin_cache, qkv, kv_cache, rope_style)
  apply_rope_write_kv_continuous(cos_sin_cache, kv_cache_end_lens, qkv, kv_cache, q_out, rope_style)
  apply_rope_write_kv_tree(cos_sin_cache, kv_cache_end_lens, token_pos_ids, qkv, kv_cache, q_out, rope_style)
  dflash_target_kv_cache_update(k_delta, v_delta, kv_cache, token_aligned_cos_sin, delta_positions,
                                delta_token_to_sequence, page_table, batch_size, rope_style)
  dflash_target_kv_cache_update_gather_rope(k_delta, v_delta, kv_cache, rope_cos_sin, state_indices,
                                            delta_positions, delta_token_to_sequence, page_table,
                                            batch_size, rope_style)
  apply_rope_write_kv_packed_qkv_fp8(cos_sin_cache, qkv, kv_cache, k_scale, v_scale, rope_style)
  apply_rope_write_kv_continuous_fp8(..., kv_cache, q_out, k_scale, v_scale, rope_style)
  apply_rope_write_kv_tree_fp8(..., kv_cache, q_out, k_scale, v_scale, rope_style)
  dflash_target_kv_cache_update_fp8(k_delta, v_delta, kv_cache, k_scale, v_scale, ...)
  dflash_target_kv_cache_update_gather_rope_fp8(k_delta, v_delta, kv_cache, k_scale, v_scale, ...)
  dflash_prepare_delta_metadata(old_draft_cache_lengths, delta_lengths, delta_width,
                                delta_positions, delta_token_to_sequence)
  dflash_build_linear_tree_metadata(tree_parent_ids, tree_depths)
  check_rope_capacity(cos_sin_seq_len, kv_capacity)
  tokens_per_page()
  last_launch_groups_per_wave()
  set_launch_overrides(groups_per_wave=0, paged_loads=0), last_launch_paged_loads()

  apply_rope_write_kv_packed_qkv_qknorm(cos_sin_cache, qkv, kv_cache, q_norm_weight, k_norm_weight,
                                        epsilon, rope_style, k_scale=None, v_scale=None)
  apply_rope_write_kv_continuous_qknorm(..., kv_cache, q_out, q_norm_weight, k_norm_weight, epsilon, ...)
  apply_rope_write_kv_tree_qknorm(..., kv_cache, q_out, q_norm_weight, k_norm_weight, epsilon, ...)

The ``_qknorm`` functions RMS-normalise Q and K heads before the rotation
(weights: float32 [D] GPU tensors or None); their cache may be fp16 or E4M3.
The ``_fp8`` functions take an E4M3 cache (a ``torch.uint8`` or
``torch.float8_e4m3fn`` tensor of the fp16 cache's shape) and per-tensor
scales (one-element float32 device tensors, or None for a scale of 1).
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librkv.so")

ROPE_NEOX = 0
ROPE_GPTJ = 1
ROUND_EXACT = 0x100   # OR into rope_style for correctly rounded (binary64) arithmetic

OK, ERR_NULL, ERR_DTYPE, ERR_SHAPE, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_ALIGNMENT, ERR_ALIAS, \
    ERR_HIP = range(9)

_F16, _F32, _I32, _F8 = 0, 1, 2, 3
_DTYPES = {torch.float16: _F16, torch.float32: _F32, torch.int32: _I32, torch.uint8: _F8,
           torch.float8_e4m3fn: _F8}
_FP8_CACHE = (torch.uint8, torch.float8_e4m3fn)


class RkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


class RkvTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 5)]


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() "
                          "or python rope_kv_cache_amd/_build.py")
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    T = ctypes.POINTER(RkvTensor)
    sig = {
        "rkv_apply_rope_write_kv_packed_qkv": [T, T, T, i32, P],
        "rkv_apply_rope_write_kv_continuous": [T, T, T, T, T, i32, P],
        "rkv_apply_rope_write_kv_tree": [T, T, T, T, T, T, i32, P],
        "rkv_dflash_target_kv_cache_update": [P, P, P, P, P, P, P] + [i32] * 8 + [P],
        "rkv_dflash_target_kv_cache_update_gather_rope": [P, P, P, P, i32, i32, P, P, P, P]
        + [i32] * 8 + [P],
        "rkv_apply_rope_write_kv_packed_qkv_fp8": [T, T, T, P, P, i32, P],
        "rkv_apply_rope_write_kv_continuous_fp8": [T, T, T, T, T, P, P, i32, P],
        "rkv_apply_rope_write_kv_tree_fp8": [T, T, T, T, T, T, P, P, i32, P],
        "rkv_dflash_target_kv_cache_update_fp8": [P] * 9 + [i32] * 8 + [P],
        "rkv_dflash_target_kv_cache_update_gather_rope_fp8": [P] * 6 + [i32, i32] + [P] * 4
        + [i32] * 8 + [P],
        "rkv_apply_rope_write_kv_packed_qkv_qknorm": [T, T, T, P, P, ctypes.c_float, P, P, i32,
                                                      P],
        "rkv_apply_rope_write_kv_continuous_qknorm": [T, T, T, T, T, P, P, ctypes.c_float, P, P,
                                                      i32, P],
        "rkv_apply_rope_write_kv_tree_qknorm": [T, T, T, T, T, T, P, P, ctypes.c_float, P, P, i32,
                                                P],
        "rkv_dflash_prepare_delta_metadata": [P, P, i32, P, P, i32, P],
        "rkv_dflash_build_linear_tree_metadata": [P, P, i32, i32, P],
        "rkv_check_rope_capacity": [i32, i32],
        "rkv_tokens_per_page": [],
        "rkv_last_launch_groups_per_wave": [],
        "rkv_set_launch_overrides": [i32, i32],
        "rkv_last_launch_paged_loads": [],
        "rkv_last_error": [],
        "rkv_status_string": [i32],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int32
    L.rkv_last_error.restype = ctypes.c_char_p
    L.rkv_status_string.restype = ctypes.c_char_p
    return L


lib = _load()


def status_string(status: int) -> str:
    return lib.rkv_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != OK:
        raise RkvError(status, lib.rkv_last_error().decode())


def _device_of(*tensors) -> torch.device:
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError("all tensors must be torch tensors in GPU memory")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices: {dev} and {t.device}")
    return dev


def _desc(t: torch.Tensor) -> RkvTensor:
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous (dense row-major)")
    if t.dim() > 5:
        raise ValueError("at most 5 dimensions")
    d = RkvTensor()
    d.data = t.data_ptr() if t.numel() else (t.data_ptr() or None)
    d.dtype = _DTYPES.get(t.dtype, -1)
    d.ndim = t.dim()
    for k, n in enumerate(t.shape):
        d.shape[k] = n
    return d


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _scale_ptr(t):
    """Device pointer of a one-element float32 scale tensor, or None."""
    if t is None:
        return None
    if t.dtype != torch.float32 or t.numel() != 1 or not t.is_cuda:
        raise ValueError("scales must be one-element float32 GPU tensors or None")
    return t.data_ptr()


def _cache_ok(kv_cache, fp8: bool) -> None:
    if fp8 and kv_cache.dtype not in _FP8_CACHE:
        raise ValueError("an fp8 cache must be torch.uint8 or torch.float8_e4m3fn")


def apply_rope_write_kv_packed_qkv(cos_sin_cache, qkv, kv_cache, rope_style: int) -> None:
    dev = _device_of(cos_sin_cache, qkv, kv_cache)
    a, b, c = _desc(cos_sin_cache), _desc(qkv), _desc(kv_cache)
    _check(lib.rkv_apply_rope_write_kv_packed_qkv(ctypes.byref(a), ctypes.byref(b),
                                                  ctypes.byref(c), int(rope_style), _stream(dev)))


def apply_rope_write_kv_packed_qkv_fp8(cos_sin_cache, qkv, kv_cache, k_scale, v_scale,
                                       rope_style: int) -> None:
    dev = _device_of(cos_sin_cache, qkv, kv_cache, k_scale, v_scale)
    _cache_ok(kv_cache, True)
    a, b, c = _desc(cos_sin_cache), _desc(qkv), _desc(kv_cache)
    _check(lib.rkv_apply_rope_write_kv_packed_qkv_fp8(
        ctypes.byref(a), ctypes.byref(b), ctypes.byref(c), _scale_ptr(k_scale),
        _scale_ptr(v_scale), int(rope_style), _stream(dev)))


def apply_rope_write_kv_continuous(cos_sin_cache, kv_cache_end_lens, qkv, kv_cache, q_out,
                                   rope_style: int) -> None:
    dev = _device_of(cos_sin_cache, kv_cache_end_lens, qkv, kv_cache, q_out)
    d = [_desc(t) for t in (cos_sin_cache, kv_cache_end_lens, qkv, kv_cache, q_out)]
    _check(lib.rkv_apply_rope_write_kv_continuous(*[ctypes.byref(x) for x in d], int(rope_style),
                                                  _stream(dev)))


def apply_rope_write_kv_continuous_fp8(cos_sin_cache, kv_cache_end_lens, qkv, kv_cache, q_out,
                                       k_scale, v_scale, rope_style: int) -> None:
    dev = _device_of(cos_sin_cache, kv_cache_end_lens, qkv, kv_cache, q_out, k_scale, v_scale)
    _cache_ok(kv_cache, True)
    d = [_desc(t) for t in (cos_sin_cache, kv_cache_end_lens, qkv, kv_cache, q_out)]
    _check(lib.rkv_apply_rope_write_kv_continuous_fp8(
        *[ctypes.byref(x) for x in d], _scale_ptr(k_scale), _scale_ptr(v_scale),
        int(rope_style), _stream(dev)))


def apply_rope_write_kv_tree(cos_sin_cache, kv_cache_end_lens, token_pos_ids, qkv, kv_cache,
                             q_out, rope_style: int) -> None:
    dev = _device_of(cos_sin_cache, kv_cache_end_lens, token_pos_ids, qkv, kv_cache, q_out)
    d = [_desc(t) for t in (cos_sin_cache, kv_cache_end_lens, token_pos_ids, qkv, kv_cache,
                            q_out)]
    _check(lib.rkv_apply_rope_write_kv_tree(*[ctypes.byref(x) for x in d], int(rope_style),
                                            _stream(dev)))


def apply_rope_write_kv_tree_fp8(cos_sin_cache, kv_cache_end_lens, token_pos_ids, qkv, kv_cache,
                                 q_out, k_scale, v_scale, rope_style: int) -> None:
    dev = _device_of(cos_sin_cache, kv_cache_end_lens, token_pos_ids, qkv, kv_cache, q_out,
                     k_scale, v_scale)
    _cache_ok(kv_cache, True)
    d = [_desc(t) for t in (cos_sin_cache, kv_cache_end_lens, token_pos_ids, qkv, kv_cache,
                            q_out)]
    _check(lib.rkv_apply_rope_write_kv_tree_fp8(
        *[ctypes.byref(x) for x in d], _scale_ptr(k_scale), _scale_ptr(v_scale),
        int(rope_style), _stream(dev)))


def _weight_ptr(t, D):
    """Device pointer of a float32 [D] norm weight, or None."""
    if t is None:
        return None
    if t.dtype != torch.float32 or t.numel() != D or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"norm weights must be contiguous float32 GPU tensors of {D} elements")
    return t.data_ptr()


def _norm_scales(kv_cache, k_scale, v_scale):
    if kv_cache.dtype == torch.float16:
        if k_scale is not None or v_scale is not None:
            raise ValueError("k_scale / v_scale apply to an E4M3 cache only")
        return None, None
    _cache_ok(kv_cache, True)
    return _scale_ptr(k_scale), _scale_ptr(v_scale)


def apply_rope_write_kv_packed_qkv_qknorm(cos_sin_cache, qkv, kv_cache, q_norm_weight,
                                          k_norm_weight, epsilon: float, rope_style: int,
                                          k_scale=None, v_scale=None) -> None:
    dev = _device_of(cos_sin_cache, qkv, kv_cache, q_norm_weight, k_norm_weight, k_scale,
                     v_scale)
    ks, vs = _norm_scales(kv_cache, k_scale, v_scale)
    D = qkv.shape[-1]
    a, b, c = _desc(cos_sin_cache), _desc(qkv), _desc(kv_cache)
    _check(lib.rkv_apply_rope_write_kv_packed_qkv_qknorm(
        ctypes.byref(a), ctypes.byref(b), ctypes.byref(c), _weight_ptr(q_norm_weight, D),
        _weight_ptr(k_norm_weight, D), float(epsilon), ks, vs, int(rope_style), _stream(dev)))


def apply_rope_write_kv_continuous_qknorm(cos_sin_cache, kv_cache_end_lens, qkv, kv_cache, q_out,
                                          q_norm_weight, k_norm_weight, epsilon: float,
                                          rope_style: int, k_scale=None, v_scale=None) -> None:
    dev = _device_of(cos_sin_cache, kv_cache_end_lens, qkv, kv_cache, q_out, q_norm_weight,
                     k_norm_weight, k_scale, v_scale)
    ks, vs = _norm_scales(kv_cache, k_scale, v_scale)
    D = qkv.shape[-1]
    d = [_desc(t) for t in (cos_sin_cache, kv_cache_end_lens, qkv, kv_cache, q_out)]
    _check(lib.rkv_apply_rope_write_kv_continuous_qknorm(
        *[ctypes.byref(x) for x in d], _weight_ptr(q_norm_weight, D),
        _weight_ptr(k_norm_weight, D), float(epsilon), ks, vs, int(rope_style), _stream(dev)))


def apply_rope_write_kv_tree_qknorm(cos_sin_cache, kv_cache_end_lens, token_pos_ids, qkv,
                                    kv_cache, q_out, q_norm_weight, k_norm_weight,
                                    epsilon: float, rope_style: int, k_scale=None,
                                    v_scale=None) -> None:
    dev = _device_of(cos_sin_cache, kv_cache_end_lens, token_pos_ids, qkv, kv_cache, q_out,
                     q_norm_weight, k_norm_weight, k_scale, v_scale)
    ks, vs = _norm_scales(kv_cache, k_scale, v_scale)
    D = qkv.shape[-1]
    d = [_desc(t) for t in (cos_sin_cache, kv_cache_end_lens, token_pos_ids, qkv, kv_cache,
                            q_out)]
    _check(lib.rkv_apply_rope_write_kv_tree_qknorm(
        *[ctypes.byref(x) for x in d], _weight_ptr(q_norm_weight, D),
        _weight_ptr(k_norm_weight, D), float(epsilon), ks, vs, int(rope_style), _stream(dev)))


def _paged_checks(k_delta, v_delta, kv_cache, cos_sin, delta_positions, delta_token_to_sequence,
                  page_table, batch_size, fp8: bool, gather: bool):
    ts = (k_delta, v_delta, kv_cache, cos_sin, delta_positions, delta_token_to_sequence,
          page_table)
    cache_types = _FP8_CACHE if fp8 else (torch.float16,)
    for t, dts in zip(ts, ((torch.float16,), (torch.float16,), cache_types, (torch.float32,),
                           (torch.int32,), (torch.int32,), (torch.int32,))):
        if t.dtype not in dts or not t.is_contiguous():
            raise ValueError(f"expected a contiguous {' or '.join(map(str, dts))} tensor, "
                             f"got {t.dtype}")
    cs_rank = 3 if gather else 2
    if k_delta.dim() != 3 or v_delta.shape != k_delta.shape or kv_cache.dim() != 5 \
            or cos_sin.dim() != cs_rank or page_table.dim() != 3:
        raise ValueError("shapes must be k/v_delta [N,Hkv,D], kv_cache [2,P,64,Hkv,D], "
                         + ("rope_cos_sin [states,rows,R]" if gather else
                            "token_aligned_cos_sin [N,R]") + ", page_table [B,2,M]")
    N, Hkv, D = k_delta.shape
    if tuple(kv_cache.shape[::2]) != (2, 64, D) or kv_cache.shape[3] != Hkv \
            or (not gather and cos_sin.shape[0] != N) or delta_positions.numel() != N \
            or delta_token_to_sequence.numel() != N or page_table.shape[1] != 2 \
            or batch_size > page_table.shape[0]:
        raise ValueError("inconsistent shapes")
    return N, Hkv, D


def _state_ptr(state_indices, batch_size):
    if state_indices is None:
        return None
    if state_indices.dtype != torch.int32 or not state_indices.is_contiguous() \
            or state_indices.numel() < batch_size:
        raise ValueError("state_indices must be a contiguous int32 tensor of batch_size entries")
    return state_indices.data_ptr()


def dflash_target_kv_cache_update(k_delta, v_delta, kv_cache, token_aligned_cos_sin,
                                  delta_positions, delta_token_to_sequence, page_table,
                                  batch_size: int, rope_style: int) -> None:
    """Sizes come from the shapes: k_delta [N, Hkv, D], token_aligned_cos_sin
    [N, R], kv_cache [2, numPages, 64, Hkv, D], page_table [B, 2, maxPagesPerSeq].
    ``batch_size`` is the active batch size, which may be below B."""
    ts = (k_delta, v_delta, kv_cache, token_aligned_cos_sin, delta_positions,
          delta_token_to_sequence, page_table)
    dev = _device_of(*ts)
    N, Hkv, D = _paged_checks(*ts, batch_size, fp8=False, gather=False)
    _check(lib.rkv_dflash_target_kv_cache_update(
        *[t.data_ptr() for t in ts], N, int(batch_size), Hkv, D, token_aligned_cos_sin.shape[1],
        kv_cache.shape[1], page_table.shape[2], int(rope_style), _stream(dev)))


def dflash_target_kv_cache_update_fp8(k_delta, v_delta, kv_cache, k_scale, v_scale,
                                      token_aligned_cos_sin, delta_positions,
                                      delta_token_to_sequence, page_table, batch_size: int,
                                      rope_style: int) -> None:
    """Call 4 into an E4M3 pool [2, numPages, 64, Hkv, D] with per-tensor scales."""
    ts = (k_delta, v_delta, kv_cache, token_aligned_cos_sin, delta_positions,
          delta_token_to_sequence, page_table)
    dev = _device_of(*ts, k_scale, v_scale)
    N, Hkv, D = _paged_checks(*ts, batch_size, fp8=True, gather=False)
    _check(lib.rkv_dflash_target_kv_cache_update_fp8(
        k_delta.data_ptr(), v_delta.data_ptr(), kv_cache.data_ptr(), _scale_ptr(k_scale),
        _scale_ptr(v_scale), token_aligned_cos_sin.data_ptr(), delta_positions.data_ptr(),
        delta_token_to_sequence.data_ptr(), page_table.data_ptr(), N, int(batch_size), Hkv, D,
        token_aligned_cos_sin.shape[1], kv_cache.shape[1], page_table.shape[2], int(rope_style),
        _stream(dev)))


def dflash_target_kv_cache_update_gather_rope(k_delta, v_delta, kv_cache, rope_cos_sin,
                                              state_indices, delta_positions,
                                              delta_token_to_sequence, page_table,
                                              batch_size: int, rope_style: int) -> None:
    """Call 4 with the cos/sin rows read from ``rope_cos_sin`` [states, rows, R]
    by (state of the row's sequence, its position); ``state_indices`` is an
    int32 [batch_size] tensor or None."""
    ts = (k_delta, v_delta, kv_cache, rope_cos_sin, delta_positions, delta_token_to_sequence,
          page_table)
    dev = _device_of(*ts, state_indices)
    N, Hkv, D = _paged_checks(*ts, batch_size, fp8=False, gather=True)
    states, rows, R = rope_cos_sin.shape
    _check(lib.rkv_dflash_target_kv_cache_update_gather_rope(
        k_delta.data_ptr(), v_delta.data_ptr(), kv_cache.data_ptr(), rope_cos_sin.data_ptr(),
        states, rows, _state_ptr(state_indices, batch_size), delta_positions.data_ptr(),
        delta_token_to_sequence.data_ptr(), page_table.data_ptr(), N, int(batch_size), Hkv, D, R,
        kv_cache.shape[1], page_table.shape[2], int(rope_style), _stream(dev)))


def dflash_target_kv_cache_update_gather_rope_fp8(k_delta, v_delta, kv_cache, k_scale, v_scale,
                                                  rope_cos_sin, state_indices, delta_positions,
                                                  delta_token_to_sequence, page_table,
                                                  batch_size: int, rope_style: int) -> None:
    """The fused-gather call 4 into an E4M3 pool with per-tensor scales."""
    ts = (k_delta, v_delta, kv_cache, rope_cos_sin, delta_positions, delta_token_to_sequence,
          page_table)
    dev = _device_of(*ts, state_indices, k_scale, v_scale)
    N, Hkv, D = _paged_checks(*ts, batch_size, fp8=True, gather=True)
    states, rows, R = rope_cos_sin.shape
    _check(lib.rkv_dflash_target_kv_cache_update_gather_rope_fp8(
        k_delta.data_ptr(), v_delta.data_ptr(), kv_cache.data_ptr(), _scale_ptr(k_scale),
        _scale_ptr(v_scale), rope_cos_sin.data_ptr(), states, rows,
        _state_ptr(state_indices, batch_size), delta_positions.data_ptr(),
        delta_token_to_sequence.data_ptr(), page_table.data_ptr(), N, int(batch_size), Hkv, D, R,
        kv_cache.shape[1], page_table.shape[2], int(rope_style), _stream(dev)))


def _int32_vec(t, n, name):
    if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() != n:
        raise ValueError(f"{name} must be a contiguous int32 tensor of {n} elements")


def dflash_prepare_delta_metadata(old_draft_cache_lengths, delta_lengths, delta_width: int,
                                  delta_positions, delta_token_to_sequence) -> None:
    """Fill delta_positions / delta_token_to_sequence (int32 [B * delta_width])
    from the per-sequence old lengths and delta lengths (int32 [B])."""
    dev = _device_of(old_draft_cache_lengths, delta_lengths, delta_positions,
                     delta_token_to_sequence)
    B = old_draft_cache_lengths.numel()
    _int32_vec(old_draft_cache_lengths, B, "old_draft_cache_lengths")
    _int32_vec(delta_lengths, B, "delta_lengths")
    _int32_vec(delta_positions, B * delta_width, "delta_positions")
    _int32_vec(delta_token_to_sequence, B * delta_width, "delta_token_to_sequence")
    _check(lib.rkv_dflash_prepare_delta_metadata(
        old_draft_cache_lengths.data_ptr(), delta_lengths.data_ptr(), int(delta_width),
        delta_positions.data_ptr(), delta_token_to_sequence.data_ptr(), B, _stream(dev)))


def dflash_build_linear_tree_metadata(tree_parent_ids, tree_depths) -> None:
    """Fill int32 [B, verify_size] parent ids and depths of a linear path."""
    dev = _device_of(tree_parent_ids, tree_depths)
    if tree_parent_ids.dim() != 2 or tree_depths.shape != tree_parent_ids.shape:
        raise ValueError("tree_parent_ids and tree_depths must be [B, verify_size]")
    B, V = tree_parent_ids.shape
    _int32_vec(tree_parent_ids, B * V, "tree_parent_ids")
    _int32_vec(tree_depths, B * V, "tree_depths")
    _check(lib.rkv_dflash_build_linear_tree_metadata(tree_parent_ids.data_ptr(),
                                                     tree_depths.data_ptr(), B, V, _stream(dev)))


def check_rope_capacity(cos_sin_seq_len: int, kv_capacity: int) -> None:
    _check(lib.rkv_check_rope_capacity(int(cos_sin_seq_len), int(kv_capacity)))


def tokens_per_page() -> int:
    return lib.rkv_tokens_per_page()


def last_launch_groups_per_wave() -> int:
    """Row groups per wave (1, 2 or 4) of the kernel this thread's last
    rope / KV-cache call launched; 0 if it launched none."""
    return lib.rkv_last_launch_groups_per_wave()


def set_launch_overrides(groups_per_wave: int = 0, paged_loads: int = 0) -> None:
    """Force the row groups per wave (0 = the library's choice, 1, 2, 4) and
    the paged update's load plan (0 = the library's choice, 1 early, 2 late)
    for this thread's later calls."""
    _check(lib.rkv_set_launch_overrides(int(groups_per_wave), int(paged_loads)))


def last_launch_paged_loads() -> int:
    """Load plan of this thread's last call: 1 early, 2 late, 0 if it was
    not a paged update or launched nothing."""
    return lib.rkv_last_launch_paged_loads()
