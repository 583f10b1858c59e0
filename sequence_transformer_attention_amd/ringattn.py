"""Python binding of libringattn (ctypes; argument marshalling only).

Every function here has the name and meaning of the C entry point in
include/libringattn.h: it turns torch tensors into ra_tensor descriptors
(device pointer, dtype, shape, element strides), passes the current torch
stream, calls the library and raises RaError on a negative status.  All
computation runs in the library's HIP kernels; nothing falls back to the CPU.
The library must have been built (python -m sequence_transformer_attention_amd.build);
loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libringattn.so")

RA_OK = 0
RA_E_NULL, RA_E_DTYPE, RA_E_SHAPE, RA_E_LAYOUT, RA_E_RANGE, RA_E_UNSUPPORTED, RA_E_HIP = -1, -2, -3, -4, -5, -6, -7
RA_BF16, RA_F32 = 0, 1
SKIP, FULL, PARTIAL = 0, 1, 2

_DT = {torch.bfloat16: RA_BF16, torch.float32: RA_F32}


class RaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class RaOpts(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("scale", ctypes.c_float),
                ("m", ctypes.POINTER(RaTensor)), ("o_out", ctypes.POINTER(RaTensor)),
                ("lse_out", ctypes.POINTER(RaTensor))]


class RaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libringattn error {status}: {message}")
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libringattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m sequence_transformer_attention_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    T = ctypes.POINTER(RaTensor)
    O = ctypes.POINTER(RaOpts)
    i64 = ctypes.c_int64
    L.ra_state_init.argtypes = [T, T, T, O]
    L.ra_step.argtypes = [T, T, T, T, T, T, i64, i64, ctypes.c_int, O]
    L.ra_finalize.argtypes = [T, T, O]
    L.ra_merge.argtypes = [T, T, T, T, T, T, O]
    L.ra_rank_share.argtypes = [T, T, T, ctypes.c_int, ctypes.c_int, ctypes.c_int, O]
    L.ra_rank_share_zigzag.argtypes = [T, T, T, ctypes.c_int, ctypes.c_int, ctypes.c_int, O]
    L.ra_rank_share_padded.argtypes = [T, T, T, ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, O]
    L.ra_rank_share_bwd.argtypes = [T, T, T, T, T, T, ctypes.c_int, ctypes.c_int, ctypes.c_int, T, T, T, T, O]
    L.ra_rank_share_zigzag_bwd.argtypes = L.ra_rank_share_bwd.argtypes
    L.ra_rank_share_bwd_noalloc.argtypes = [T, T, T, T, T, T, ctypes.c_int, ctypes.c_int, ctypes.c_int, T, T, T, O]
    L.ra_rank_share_padded_bwd.argtypes = [T, T, T, T, T, T, ctypes.c_int, ctypes.c_int, ctypes.c_int, i64,
                                           T, T, T, T, O]
    for f in (L.ra_state_init, L.ra_step, L.ra_finalize, L.ra_merge, L.ra_rank_share, L.ra_rank_share_zigzag,
              L.ra_rank_share_bwd, L.ra_rank_share_bwd_noalloc, L.ra_rank_share_padded, L.ra_rank_share_zigzag_bwd,
              L.ra_rank_share_padded_bwd):
        f.restype = ctypes.c_int
    L.ra_ring_block.argtypes = [i64, i64, i64]
    L.ra_ring_block.restype = i64
    L.ra_classify.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    L.ra_classify.restype = ctypes.c_int
    L.ra_plan_tiles.argtypes = [i64, i64, i64, i64, ctypes.c_int, i64, i64, ctypes.POINTER(ctypes.c_int8), i64]
    L.ra_plan_tiles.restype = i64
    L.ra_tile_shape.argtypes = [ctypes.c_int32, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.ra_tile_shape.restype = ctypes.c_int
    L.ra_flops.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int]
    L.ra_flops.restype = ctypes.c_double
    L.ra_share_flops.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int]
    L.ra_share_flops.restype = ctypes.c_double
    L.ra_share_flops_zigzag.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int]
    L.ra_share_flops_zigzag.restype = ctypes.c_double
    L.ra_last_error.argtypes = []
    L.ra_last_error.restype = ctypes.c_char_p
    L.ra_version.argtypes = []
    L.ra_version.restype = ctypes.c_char_p
    _lib = L
    return L


# ------------------------------------------------------------------ marshalling
def _desc(t: torch.Tensor, rows: bool = False) -> RaTensor:
    """[B, S, H, d] tensor -> ra_tensor; rows=True: [B, H, S] fp32 -> [B, H, S, 1]."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("libringattn works on device tensors only (got a CPU tensor)")
    if t.dtype not in _DT:
        raise ValueError(f"unsupported dtype {t.dtype}")
    d = RaTensor()
    d.data = t.data_ptr()
    d.dtype = _DT[t.dtype]
    if rows:
        if t.dim() != 3:
            raise ValueError("row statistics must be [B, H, S]")
        shape, stride = list(t.shape) + [1], list(t.stride()) + [1]
    else:
        if t.dim() != 4:
            raise ValueError("tensors must be [B, S, H, d]")
        shape, stride = list(t.shape), list(t.stride())
    for i in range(4):
        d.shape[i] = shape[i]
        d.stride[i] = stride[i]
    return d


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _opts(stream=None, scale: Optional[float] = None, m=None, o_out=None, lse_out=None):
    o = RaOpts()
    o.stream = _stream(stream)
    o.scale = float(scale) if scale is not None else 0.0
    keep = []
    if m is not None:
        keep.append(_desc(m, rows=True)); o.m = ctypes.pointer(keep[-1])
    if o_out is not None:
        keep.append(_desc(o_out)); o.o_out = ctypes.pointer(keep[-1])
    if lse_out is not None:
        keep.append(_desc(lse_out, rows=True)); o.lse_out = ctypes.pointer(keep[-1])
    return o, keep


def _check(status: int) -> None:
    if status != RA_OK:
        raise RaError(status, lib().ra_last_error().decode())


# ------------------------------------------------------------------ entry points
def ra_state_init(o_acc, m, l, stream=None) -> None:
    """o_acc [B, Nq, H, d] fp32 = 0; m [B, H, Nq] = -inf; l [B, H, Nq] = 0."""
    opts, keep = _opts(stream)
    _check(lib().ra_state_init(_desc(o_acc), _desc(m, True), _desc(l, True), ctypes.byref(opts)))


def ra_step(q, k_blk, v_blk, o_acc, m, l, q_off: int, kv_off: int, causal: bool,
            scale: Optional[float] = None, stream=None) -> None:
    """Fold one key/value block into the running state (o_acc, m, l) in place."""
    opts, keep = _opts(stream, scale)
    _check(lib().ra_step(_desc(q), _desc(k_blk), _desc(v_blk), _desc(o_acc), _desc(m, True),
                         _desc(l, True), int(q_off), int(kv_off), int(bool(causal)), ctypes.byref(opts)))


def ra_finalize(o_acc, l, m=None, o_out=None, lse_out=None, stream=None) -> None:
    """O = o_acc / l into o_out (or in place); LSE = m + ln l into lse_out."""
    opts, keep = _opts(stream, None, m=m, o_out=o_out, lse_out=lse_out)
    _check(lib().ra_finalize(_desc(o_acc), _desc(l, True), ctypes.byref(opts)))


def ra_merge(o_acc, m, l, o_b, m_b, l_b, stream=None) -> None:
    """Fold the partial state (o_b, m_b, l_b) into (o_acc, m, l) in place
    (log-sum-exp rescaling to the common maximum); o fp32 [B, S, H, d],
    m, l fp32 [B, H, S]."""
    opts, keep = _opts(stream)
    _check(lib().ra_merge(_desc(o_acc), _desc(m, True), _desc(l, True), _desc(o_b), _desc(m_b, True),
                          _desc(l_b, True), ctypes.byref(opts)))


def ra_rank_share(q, k, v, P: int, rank: int, causal: bool, o_out, lse_out=None,
                  scale: Optional[float] = None, stream=None) -> None:
    """One rank's share of ring attention in one launch: O -> o_out, LSE -> lse_out."""
    opts, keep = _opts(stream, scale, o_out=o_out, lse_out=lse_out)
    _check(lib().ra_rank_share(_desc(q), _desc(k), _desc(v), int(P), int(rank), int(bool(causal)),
                               ctypes.byref(opts)))


def ra_rank_share_padded(q, k, v, P: int, rank: int, causal: bool, n_valid: int, o_out, lse_out=None,
                         scale: Optional[float] = None, stream=None) -> None:
    """One rank's share of a sequence padded to N = P * ceil(n_valid / P) rows:
    keys at positions >= n_valid are masked out."""
    opts, keep = _opts(stream, scale, o_out=o_out, lse_out=lse_out)
    _check(lib().ra_rank_share_padded(_desc(q), _desc(k), _desc(v), int(P), int(rank), int(bool(causal)),
                                      int(n_valid), ctypes.byref(opts)))


def ra_rank_share_zigzag(q, k, v, P: int, rank: int, causal: bool, o_out, lse_out=None,
                         scale: Optional[float] = None, stream=None) -> None:
    """One rank's load-balanced share (local rows = chunks rank and 2P-1-rank of
    2P) in one launch: O -> o_out, LSE -> lse_out."""
    opts, keep = _opts(stream, scale, o_out=o_out, lse_out=lse_out)
    _check(lib().ra_rank_share_zigzag(_desc(q), _desc(k), _desc(v), int(P), int(rank), int(bool(causal)),
                                      ctypes.byref(opts)))


def ra_rank_share_bwd(q, k, v, o, lse, dout, P: int, rank: int, causal: bool, dq, dk, dv, delta,
                      scale: Optional[float] = None, stream=None) -> None:
    """Backward of one rank's share: dq [B, N/P, Hq, d], this rank's dk, dv
    [B, N, Hkv, d] (all fp32, written); delta [B, Hq, N/P] fp32 workspace."""
    opts, keep = _opts(stream, scale)
    _check(lib().ra_rank_share_bwd(_desc(q), _desc(k), _desc(v), _desc(o), _desc(lse, True), _desc(dout),
                                   int(P), int(rank), int(bool(causal)), _desc(dq), _desc(dk), _desc(dv),
                                   _desc(delta, True), ctypes.byref(opts)))


def ra_rank_share_bwd_noalloc(q, k, v, o, lse, dout, P: int, rank: int, causal: bool, dq, dk, dv,
                              scale: Optional[float] = None, stream=None) -> None:
    """ra_rank_share_bwd with the D workspace held by the library (a static
    device array of 2^20 rows per device): the call allocates nothing;
    calls overlapping on one device race."""
    opts, keep = _opts(stream, scale)
    _check(lib().ra_rank_share_bwd_noalloc(_desc(q), _desc(k), _desc(v), _desc(o), _desc(lse, True), _desc(dout),
                                           int(P), int(rank), int(bool(causal)), _desc(dq), _desc(dk), _desc(dv),
                                           ctypes.byref(opts)))


def ra_rank_share_zigzag_bwd(q, k, v, o, lse, dout, P: int, rank: int, causal: bool, dq, dk, dv, delta,
                             scale: Optional[float] = None, stream=None) -> None:
    """Backward of the load-balanced share (local rows = chunks rank and
    2P-1-rank of 2P; o, lse from ra_rank_share_zigzag); outputs as
    ra_rank_share_bwd."""
    opts, keep = _opts(stream, scale)
    _check(lib().ra_rank_share_zigzag_bwd(_desc(q), _desc(k), _desc(v), _desc(o), _desc(lse, True), _desc(dout),
                                          int(P), int(rank), int(bool(causal)), _desc(dq), _desc(dk), _desc(dv),
                                          _desc(delta, True), ctypes.byref(opts)))


def ra_rank_share_padded_bwd(q, k, v, o, lse, dout, P: int, rank: int, causal: bool, n_valid: int, dq, dk, dv,
                             delta, scale: Optional[float] = None, stream=None) -> None:
    """Backward of the padded share (o, lse from ra_rank_share_padded with the
    same n_valid); outputs as ra_rank_share_bwd, zero dk, dv past n_valid."""
    opts, keep = _opts(stream, scale)
    _check(lib().ra_rank_share_padded_bwd(_desc(q), _desc(k), _desc(v), _desc(o), _desc(lse, True), _desc(dout),
                                          int(P), int(rank), int(bool(causal)), int(n_valid), _desc(dq), _desc(dk),
                                          _desc(dv), _desc(delta, True), ctypes.byref(opts)))


def ra_ring_block(P: int, rank: int, s: int) -> int:
    return int(lib().ra_ring_block(P, rank, s))


def ra_classify(q_off: int, nq: int, kv_off: int, nkv: int, causal: bool) -> int:
    return int(lib().ra_classify(q_off, nq, kv_off, nkv, int(bool(causal))))


def ra_plan_tiles(q_off: int, nq: int, kv_off: int, nkv: int, causal: bool, bm: int, bn: int):
    n = (-(-nq // bm)) * (-(-nkv // bn))
    buf = (ctypes.c_int8 * max(n, 1))()
    r = int(lib().ra_plan_tiles(q_off, nq, kv_off, nkv, int(bool(causal)), bm, bn, buf, n))
    if r < 0:
        raise RaError(r, lib().ra_last_error().decode())
    return [buf[i] for i in range(r)]


def ra_tile_shape(dtype: torch.dtype, d: int):
    bm, bn = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().ra_tile_shape(_DT[dtype], d, ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value


def ra_flops(nq: int, nkv: int, q_off: int, kv_off: int, Hq: int, d: int, causal: bool) -> float:
    return float(lib().ra_flops(nq, nkv, q_off, kv_off, Hq, d, int(bool(causal))))


def ra_share_flops(B: int, N: int, P: int, rank: int, Hq: int, d: int, causal: bool) -> float:
    return float(lib().ra_share_flops(B, N, P, rank, Hq, d, int(bool(causal))))


def ra_share_flops_zigzag(B: int, N: int, P: int, rank: int, Hq: int, d: int, causal: bool) -> float:
    return float(lib().ra_share_flops_zigzag(B, N, P, rank, Hq, d, int(bool(causal))))


def ra_last_error() -> str:
    return lib().ra_last_error().decode()


def ra_version() -> str:
    return lib().ra_version().decode()
