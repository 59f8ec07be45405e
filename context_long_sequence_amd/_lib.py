"""ctypes binding of libringattn.so: one Python function per C entry point, same
names, argument marshalling only (shape/dtype/device checks, pointers, stream).

PyTorch provides device memory and streams; every step runs in the HIP library.
If the library is missing the binding raises — there is no other implementation.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libringattn.so")

RA_OK = 0
RA_DTYPE_F32 = 0
RA_DTYPE_BF16 = 1

EXPORTED = (
    "ring_attn_fwd_step",
    "ring_attn_fwd_step_merge",
    "lse_merge",
    "segment_mask_from_pos",
    "ring_attn_bwd_preprocess",
    "ring_attn_bwd_step",
    "ring_attn_bwd_step_noalloc",
    "ring_recv_copy",
    "ra_status_string",
    "ra_last_error",
    "ra_abi_version",
)


class RaShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("kv_len", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("q_offset", ctypes.c_int64),
        ("kv_offset", ctypes.c_int64),
        ("causal", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


class RingAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def library_path() -> str:
    return LIB_PATH


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises FileNotFoundError if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} not found: build the HIP library first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(p)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sp = ctypes.POINTER(RaShape)
    lib.ring_attn_fwd_step.argtypes = [sp, vp, vp, vp, vp, i64, vp, vp, vp]
    lib.ring_attn_fwd_step_merge.argtypes = [sp, vp, vp, vp, vp, i64, vp, vp, vp, i32, vp]
    lib.lse_merge.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, i32, vp]
    lib.segment_mask_from_pos.argtypes = [i32, i64, vp, vp, vp]
    lib.ring_attn_bwd_preprocess.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.ring_attn_bwd_step.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp]
    lib.ring_attn_bwd_step_noalloc.argtypes = lib.ring_attn_bwd_step.argtypes
    lib.ring_recv_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
    for fn in ("ring_attn_fwd_step", "ring_attn_fwd_step_merge", "lse_merge", "segment_mask_from_pos", "ring_attn_bwd_preprocess",
               "ring_attn_bwd_step", "ring_attn_bwd_step_noalloc", "ring_recv_copy"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.ra_status_string.argtypes = [ctypes.c_int]
    lib.ra_status_string.restype = ctypes.c_char_p
    lib.ra_last_error.argtypes = []
    lib.ra_last_error.restype = ctypes.c_char_p
    lib.ra_abi_version.argtypes = []
    lib.ra_abi_version.restype = ctypes.c_int32
    if path is None:
        _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != RA_OK:
        lib = load()
        msg = lib.ra_last_error().decode()
        raise RingAttnError(fn, status, f"{lib.ra_status_string(status).decode()}: {msg}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return RA_DTYPE_BF16
    if t.dtype == torch.float32:
        return RA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _need(t: torch.Tensor, name: str, shape, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_shape(q: torch.Tensor, k: torch.Tensor, q_offset: int, kv_offset: int, causal: bool,
               scale: float) -> RaShape:
    B, Sq, Hq, d = q.shape
    Bk, Sk, Hkv, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError("q and k disagree on batch or head_dim")
    return RaShape(B, Sq, Sk, Hq, Hkv, d, int(q_offset), int(kv_offset), int(bool(causal)), float(scale),
                   _dtype_code(q))


def ring_attn_fwd_step(q, k, v, o_step, lse_step, *, q_offset: int, kv_offset: int, causal: bool,
                       scale: float, seg_ids: Optional[torch.Tensor] = None, stream=None) -> None:
    """Partial attention of q [B,Sq,Hq,d] against one KV chunk k,v [B,Sk,Hkv,d] ->
    o_step [B,Sq,Hq,d] fp32, lse_step [B,Hq,Sq] fp32 (see include/ringattn.h)."""
    B, Sq, Hq, d = q.shape
    _need(q, "q", q.shape)
    _need(k, "k", k.shape, q.dtype)
    _need(v, "v", k.shape, q.dtype)
    _need(o_step, "o_step", (B, Sq, Hq, d), torch.float32)
    _need(lse_step, "lse_step", (B, Hq, Sq), torch.float32)
    seg_len = 0
    if seg_ids is not None:
        _need(seg_ids, "seg_ids", seg_ids.shape, torch.int32)
        if seg_ids.dim() != 2 or seg_ids.shape[0] != B:
            raise ValueError("seg_ids must be [B, seg_len]")
        seg_len = seg_ids.shape[1]
    shape = make_shape(q, k, q_offset, kv_offset, causal, scale)
    lib = load()
    _check("ring_attn_fwd_step", lib.ring_attn_fwd_step(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                                        _ptr(seg_ids), seg_len, _ptr(o_step),
                                                        _ptr(lse_step), _stream(stream)))


def ring_attn_fwd_step_merge(q, k, v, o_acc, lse_acc, *, q_offset: int, kv_offset: int, causal: bool,
                             scale: float, seg_ids: Optional[torch.Tensor] = None, o_out=None,
                             stream=None) -> None:
    """One ring step folded into the running result: (o_acc [B,Sq,Hq,d] fp32, lse_acc
    [B,Hq,Sq] fp32) <- merge with the step's partial attention of q against k, v;
    optionally the merged O converted to o_out's dtype (see include/ringattn.h)."""
    B, Sq, Hq, d = q.shape
    _need(q, "q", q.shape)
    _need(k, "k", k.shape, q.dtype)
    _need(v, "v", k.shape, q.dtype)
    _need(o_acc, "o_acc", (B, Sq, Hq, d), torch.float32)
    _need(lse_acc, "lse_acc", (B, Hq, Sq), torch.float32)
    out_dtype = RA_DTYPE_F32
    if o_out is not None:
        _need(o_out, "o_out", (B, Sq, Hq, d))
        out_dtype = _dtype_code(o_out)
    seg_len = 0
    if seg_ids is not None:
        _need(seg_ids, "seg_ids", seg_ids.shape, torch.int32)
        if seg_ids.dim() != 2 or seg_ids.shape[0] != B:
            raise ValueError("seg_ids must be [B, seg_len]")
        seg_len = seg_ids.shape[1]
    shape = make_shape(q, k, q_offset, kv_offset, causal, scale)
    lib = load()
    _check("ring_attn_fwd_step_merge",
           lib.ring_attn_fwd_step_merge(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(seg_ids), seg_len,
                                        _ptr(o_acc), _ptr(lse_acc), _ptr(o_out), out_dtype, _stream(stream)))


def lse_merge(o_acc, lse_acc, o_step=None, lse_step=None, o_out=None, stream=None) -> None:
    """(o_acc, lse_acc) <- merge with (o_step, lse_step), in place; optionally write the
    merged O converted to o_out's dtype.  o_step = lse_step = None: conversion only."""
    B, Sq, Hq, d = o_acc.shape
    _need(o_acc, "o_acc", o_acc.shape, torch.float32)
    _need(lse_acc, "lse_acc", (B, Hq, Sq), torch.float32)
    if o_step is not None:
        _need(o_step, "o_step", o_acc.shape, torch.float32)
    if lse_step is not None:
        _need(lse_step, "lse_step", (B, Hq, Sq), torch.float32)
    out_dtype = RA_DTYPE_F32
    if o_out is not None:
        _need(o_out, "o_out", o_acc.shape)
        out_dtype = _dtype_code(o_out)
    lib = load()
    _check("lse_merge", lib.lse_merge(B, Sq, Hq, d, _ptr(o_acc), _ptr(lse_acc), _ptr(o_step), _ptr(lse_step),
                                      _ptr(o_out), out_dtype, _stream(stream)))


def segment_mask_from_pos(position_ids, seg_ids, stream=None) -> None:
    """seg_ids[b,t] = #{t'<=t : position_ids[b,t'] == 0} - 1 over the global row ([B,S] int32)."""
    B, S = position_ids.shape
    _need(position_ids, "position_ids", (B, S), torch.int32)
    _need(seg_ids, "seg_ids", (B, S), torch.int32)
    lib = load()
    _check("segment_mask_from_pos", lib.segment_mask_from_pos(B, S, _ptr(position_ids), _ptr(seg_ids),
                                                              _stream(stream)))


def ring_attn_bwd_preprocess(o, d_o, delta, stream=None) -> None:
    """delta[b,h,i] = sum_d dO[b,i,h,:] * O[b,i,h,:]."""
    B, Sq, Hq, d = o.shape
    _need(o, "o", o.shape)
    _need(d_o, "d_o", o.shape, o.dtype)
    _need(delta, "delta", (B, Hq, Sq), torch.float32)
    lib = load()
    _check("ring_attn_bwd_preprocess", lib.ring_attn_bwd_preprocess(B, Sq, Hq, d, _dtype_code(o), _ptr(o),
                                                                    _ptr(d_o), _ptr(delta), _stream(stream)))


def _bwd_step(fn, q, k, v, d_o, lse, delta, dq_acc, dk_acc, dv_acc, q_offset, kv_offset, causal, scale, seg_ids,
              stream) -> None:
    B, Sq, Hq, d = q.shape
    _need(q, "q", q.shape)
    _need(k, "k", k.shape, q.dtype)
    _need(v, "v", k.shape, q.dtype)
    _need(d_o, "d_o", q.shape, q.dtype)
    _need(lse, "lse", (B, Hq, Sq), torch.float32)
    _need(delta, "delta", (B, Hq, Sq), torch.float32)
    _need(dq_acc, "dq_acc", q.shape, torch.float32)
    _need(dk_acc, "dk_acc", k.shape, torch.float32)
    _need(dv_acc, "dv_acc", k.shape, torch.float32)
    seg_len = 0
    if seg_ids is not None:
        _need(seg_ids, "seg_ids", seg_ids.shape, torch.int32)
        if seg_ids.dim() != 2 or seg_ids.shape[0] != B:
            raise ValueError("seg_ids must be [B, seg_len]")
        seg_len = seg_ids.shape[1]
    shape = make_shape(q, k, q_offset, kv_offset, causal, scale)
    lib = load()
    _check(fn, getattr(lib, fn)(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(d_o), _ptr(lse), _ptr(delta),
                                _ptr(seg_ids), seg_len, _ptr(dq_acc), _ptr(dk_acc), _ptr(dv_acc), _stream(stream)))


def ring_attn_bwd_step(q, k, v, d_o, lse, delta, dq_acc, dk_acc, dv_acc, *, q_offset: int, kv_offset: int,
                       causal: bool, scale: float, seg_ids: Optional[torch.Tensor] = None, stream=None) -> None:
    """One backward ring step for one KV chunk; accumulates into dq_acc, dk_acc, dv_acc (fp32)."""
    _bwd_step("ring_attn_bwd_step", q, k, v, d_o, lse, delta, dq_acc, dk_acc, dv_acc, q_offset, kv_offset, causal,
              scale, seg_ids, stream)


def ring_attn_bwd_step_noalloc(q, k, v, d_o, lse, delta, dq_acc, dk_acc, dv_acc, *, q_offset: int, kv_offset: int,
                               causal: bool, scale: float, seg_ids: Optional[torch.Tensor] = None,
                               stream=None) -> None:
    """ring_attn_bwd_step without any device allocation (the library's static scratch;
    both kernels on `stream`).  Calls that overlap on one GPU must not be issued."""
    _bwd_step("ring_attn_bwd_step_noalloc", q, k, v, d_o, lse, delta, dq_acc, dk_acc, dv_acc, q_offset, kv_offset,
              causal, scale, seg_ids, stream)


def ring_recv_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    """Receive `src` into `dst` (same shape and dtype, contiguous) with the DMA engines."""
    if dst.shape != src.shape or dst.dtype != src.dtype:
        raise ValueError(f"ring_recv_copy: {tuple(src.shape)} {src.dtype} into {tuple(dst.shape)} {dst.dtype}")
    if not (dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("ring_recv_copy: tensors must be contiguous")
    lib = load()
    _check("ring_recv_copy", lib.ring_recv_copy(_ptr(dst), _ptr(src), src.numel() * src.element_size(),
                                                _stream(stream)))
