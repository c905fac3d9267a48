"""Measurement kernels timed by ``bench.py --ceilings`` beside the library.

Streams with the library's memory policy (also in persistent form), an empty kernel, an index-free
floor of the paged update and the packed prefill with its cos/sin row staged
in LDS (``rkv_ceilings.hip`` says what each one bounds).  Argument
marshalling from torch tensors and torch's current stream only; importing
this package fails if ``libceilings.so`` is not built.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libceilings.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")

_L = ctypes.CDLL(LIB_PATH)
_P, _I, _LL, _U = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_uint
_L.rkvc_stream_copy.argtypes = [_P, _P, _LL, _I, _I, _P]
_L.rkvc_stream_inplace.argtypes = [_P, _LL, _U, _I, _I, _P]
_L.rkvc_stream_narrow.argtypes = [_P, _P, _LL, _I, _I, _P]
_L.rkvc_stream_persistent.argtypes = [_P, _LL, _U, _I, _I, _I, _I, _P]
_L.rkvc_check_reciprocal.argtypes = [_P, _I, _P]
_L.rkvc_check_f16_pair.argtypes = [_P, _I, _P]
_L.rkvc_empty.argtypes = [_I, _P]
_L.rkvc_paged_floor.argtypes = [_P, _P, _P, _P] + [_I] * 9 + [_P]
_L.rkvc_prefill_lds.argtypes = [_P, _I, _I, _P, _P] + [_I] * 11 + [_P]
for _f in ("rkvc_stream_copy", "rkvc_stream_inplace", "rkvc_stream_narrow",
           "rkvc_stream_persistent", "rkvc_check_reciprocal", "rkvc_check_f16_pair", "rkvc_empty",
           "rkvc_paged_floor", "rkvc_prefill_lds"):
    getattr(_L, _f).restype = _I


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc, what):
    if rc:
        raise RuntimeError(f"{what}: hip error {rc}")


def stream_copy(src: torch.Tensor, dst: torch.Tensor, policy: int = 1, chunk_log2: int = 7):
    n = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() == n and src.is_contiguous() and dst.is_contiguous()
    _check(_L.rkvc_stream_copy(src.data_ptr(), dst.data_ptr(), n, policy, chunk_log2, _stream()),
           "stream_copy")


def stream_narrow(src: torch.Tensor, dst: torch.Tensor, policy: int = 1, chunk_log2: int = 7):
    """dst (int32 words) = src word 2i ^ src word 2i+1: reads all of src,
    writes half as many bytes."""
    n = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= n // 2 and src.is_contiguous() and dst.is_contiguous()
    _check(_L.rkvc_stream_narrow(src.data_ptr(), dst.data_ptr(), n, policy, chunk_log2, _stream()),
           "stream_narrow")


def stream_inplace(buf: torch.Tensor, policy: int = 1, chunk_log2: int = 7, key: int = 0):
    assert buf.is_contiguous()
    _check(_L.rkvc_stream_inplace(buf.data_ptr(), buf.numel() * buf.element_size(), key, policy,
                                  chunk_log2, _stream()), "stream_inplace")


def stream_persistent(buf: torch.Tensor, unroll: int, pipe: int, xcd: int, workgroups: int,
                      key: int = 0):
    """buf ^= key (per 32-bit word) by a fixed grid of `workgroups` that loop
    over it, `unroll` 4 KB chunks per step (see rkv_ceilings.hip)."""
    assert buf.is_contiguous()
    _check(_L.rkvc_stream_persistent(buf.data_ptr(), buf.numel() * buf.element_size(), key,
                                     unroll, pipe, xcd, workgroups, _stream()),
           "stream_persistent")


def check_reciprocal(counts: torch.Tensor):
    """The library's fp32 reciprocal of a scale against the rounded binary64
    quotient for every fp32 pattern; `counts` (int32, even length 2t with t a
    power of two >= 256) receives per thread its mismatch count and first
    mismatching pattern."""
    assert counts.dtype == torch.int32 and counts.is_contiguous() and counts.numel() % 2 == 0
    _check(_L.rkvc_check_reciprocal(counts.data_ptr(), counts.numel() // 2, _stream()),
           "check_reciprocal")


def check_f16_pair(counts: torch.Tensor):
    """The library's packed fp16 conversion against two scalar conversions
    for every fp32 pattern; `counts` as for check_reciprocal."""
    assert counts.dtype == torch.int32 and counts.is_contiguous() and counts.numel() % 2 == 0
    _check(_L.rkvc_check_f16_pair(counts.data_ptr(), counts.numel() // 2, _stream()),
           "check_f16_pair")


def empty(workgroups: int):
    _check(_L.rkvc_empty(workgroups, _stream()), "empty")


def paged_floor(k_delta, v_delta, pool, cos_sin, num_pages: int, rows_per_seq_log2: int,
                live_per_seq: int, scatter: int, groups: int = 2, stream_plan: int = 0):
    """k/v deltas fp16 [N, Hkv, 128], pool fp16 [2, num_pages, 64, Hkv, 128],
    cos_sin fp32 [N, R] (NeoX)."""
    N, Hkv, D = k_delta.shape
    assert D == 128 and v_delta.shape == k_delta.shape and cos_sin.shape[0] == N
    assert pool.shape == (2, num_pages, 64, Hkv, D) and pool.dtype == torch.float16
    _check(_L.rkvc_paged_floor(k_delta.data_ptr(), v_delta.data_ptr(), pool.data_ptr(),
                               cos_sin.data_ptr(), N, Hkv, cos_sin.shape[1], num_pages,
                               rows_per_seq_log2, live_per_seq, scatter, groups, stream_plan,
                               _stream()), "paged_floor")


def prefill_lds(cos_sin, qkv, cache, style: int, groups: int = 2, chunk_log2: int = 5,
                lds: bool = True, dpp: bool = False):
    """Call 1 with one workgroup per token: cos_sin fp32 [TB, TL, R], qkv fp16
    [B, S, Hq + 2 Hkv, 128] (rotated in place), cache fp16 [B, 2, Hkv, cap,
    128]; `lds` stages the cos/sin row in LDS, `dpp` exchanges NeoX partners
    by DPP (NeoX, R = 128)."""
    TB, TL, R = cos_sin.shape
    B, S, H, D = qkv.shape
    Hkv, cap = cache.shape[2], cache.shape[3]
    assert D == 128 and cache.shape == (B, 2, Hkv, cap, D)
    _check(_L.rkvc_prefill_lds(cos_sin.data_ptr(), TB, TL, qkv.data_ptr(), cache.data_ptr(), B, S,
                               H - 2 * Hkv, Hkv, cap, R, style, groups, chunk_log2, int(lds),
                               int(dpp), _stream()), "prefill_lds")
