"""fp64 CPU oracle for one rank's share of ring (blockwise) attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library.  It shares no code with
the HIP path.  The arithmetic lives in ra_oracle.c (plain C, fp64); this file
converts arrays and calls it.  What each function follows on the pages is
stated in ra_oracle.c.

Inputs may be torch tensors (any dtype, converted exactly to fp64) or numpy
arrays, in the [B, S, H, d] layout.  Rows are (b, h, i) triples.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ra_oracle.c")
_LIB = os.path.join(_HERE, "libraoracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def build() -> str:
    """Compile ra_oracle.c with gcc (plain C11, pthreads)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                           _SRC, "-o", tmp, "-lpthread", "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def _load(path: Optional[str] = None):
    """Load the oracle library (building it first if absent).  `path` loads
    another build of ra_oracle.c instead; the tests use it to run the pins on
    deliberately broken copies."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    if path is None:
        path = _LIB
        if not os.path.exists(path):
            build()
    lib = ctypes.CDLL(path)
    common = [_dp, _dp, _dp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
              ctypes.c_int, ctypes.c_double, _ip, _i64]
    lib.orc_attention.argtypes = common + [_dp, _dp, ctypes.c_int]
    lib.orc_attention.restype = ctypes.c_int
    lib.orc_block_partial.argtypes = common + [_dp, _dp, _dp, ctypes.c_int]
    lib.orc_block_partial.restype = ctypes.c_int
    lib.orc_merge.argtypes = [_i64, _i64, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
    lib.orc_merge.restype = None
    lib.orc_finalize.argtypes = [_i64, _i64, _dp, _dp, _dp, _dp, _dp]
    lib.orc_finalize.restype = None
    lib.orc_rank_share.argtypes = [_dp, _dp, _dp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                   ctypes.c_int, ctypes.c_double, _ip, _i64, _dp, _dp, ctypes.c_int]
    lib.orc_rank_share.restype = ctypes.c_int
    lib.orc_rank_share_padded.argtypes = [_dp, _dp, _dp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                          ctypes.c_int, ctypes.c_double, _i64, _ip, _i64, _dp, _dp, ctypes.c_int]
    lib.orc_rank_share_padded.restype = ctypes.c_int
    lib.orc_rank_share_zigzag.argtypes = lib.orc_rank_share.argtypes
    lib.orc_rank_share_zigzag.restype = ctypes.c_int
    lib.orc_share_flops_zigzag.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int]
    lib.orc_share_flops_zigzag.restype = ctypes.c_double
    lib.orc_rank_share_bwd.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                       ctypes.c_int, ctypes.c_double, _ip, _i64, _ip, _i64, _dp, _dp, _dp,
                                       ctypes.c_int]
    lib.orc_rank_share_bwd.restype = ctypes.c_int
    lib.orc_rank_share_zigzag_bwd.argtypes = lib.orc_rank_share_bwd.argtypes
    lib.orc_rank_share_zigzag_bwd.restype = ctypes.c_int
    lib.orc_rank_share_padded_bwd.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                              ctypes.c_int, ctypes.c_double, _i64, _ip, _i64, _ip, _i64,
                                              _dp, _dp, _dp, ctypes.c_int]
    lib.orc_rank_share_padded_bwd.restype = ctypes.c_int
    lib.orc_ring_block.argtypes = [_i64, _i64, _i64]
    lib.orc_ring_block.restype = _i64
    lib.orc_classify.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int]
    lib.orc_classify.restype = ctypes.c_int
    lib.orc_visible_pairs.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int]
    lib.orc_visible_pairs.restype = _i64
    lib.orc_share_flops.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int]
    lib.orc_share_flops.restype = ctypes.c_double
    _lib = lib
    return lib


def _reset() -> None:
    global _lib
    _lib = None


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def all_rows(B: int, H: int, nq: int) -> np.ndarray:
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(nq), indexing="ij")
    return np.ascontiguousarray(np.stack([b.ravel(), h.ravel(), i.ravel()], 1).astype(np.int64))


def _rows(rows, B, H, nq) -> np.ndarray:
    if rows is None:
        return all_rows(B, H, nq)
    r = np.asarray(rows)
    if hasattr(rows, "numpy"):
        r = rows.numpy()
    return np.ascontiguousarray(r.astype(np.int64).reshape(-1, 3))


def _args(q, k, v, q_off, kv_off, causal, scale, rows):
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, nq, hq, d = q.shape
    _, nkv, hkv, _ = k.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    r = _rows(rows, B, hq, nq)
    return q, k, v, B, nq, nkv, hq, hkv, d, r, float(scale)


def attention(q, k, v, q_off: int = 0, kv_off: int = 0, causal: bool = False,
              scale: Optional[float] = None, rows=None, nthreads: Optional[int] = None
              ) -> Tuple[np.ndarray, np.ndarray]:
    """Full softmax attention (the plain definition).  Returns O [n, d], LSE [n]."""
    lib = _load()
    q, k, v, B, nq, nkv, hq, hkv, d, r, scale = _args(q, k, v, q_off, kv_off, causal, scale, rows)
    n = r.shape[0]
    o = np.zeros((n, d)); lse = np.zeros(n)
    e = lib.orc_attention(_ptr(q), _ptr(k), _ptr(v), B, nq, nkv, nq, nkv, hq, hkv, d, q_off, kv_off,
                          int(causal), scale, r.ctypes.data_as(_ip), n, _ptr(o), _ptr(lse),
                          nthreads or default_threads())
    if e:
        raise ValueError(f"orc_attention failed ({e})")
    return o, lse


def block_partial(q, k, v, q_off: int = 0, kv_off: int = 0, causal: bool = False,
                  scale: Optional[float] = None, rows=None, nthreads: Optional[int] = None):
    """Unnormalised partial state (m [n], l [n], o [n, d]) against one key/value block."""
    lib = _load()
    q, k, v, B, nq, nkv, hq, hkv, d, r, scale = _args(q, k, v, q_off, kv_off, causal, scale, rows)
    n = r.shape[0]
    m = np.zeros(n); l = np.zeros(n); o = np.zeros((n, d))
    e = lib.orc_block_partial(_ptr(q), _ptr(k), _ptr(v), B, nq, nkv, nq, nkv, hq, hkv, d, q_off,
                              kv_off, int(causal), scale, r.ctypes.data_as(_ip), n, _ptr(m), _ptr(l),
                              _ptr(o), nthreads or default_threads())
    if e:
        raise ValueError(f"orc_block_partial failed ({e})")
    return m, l, o


def identity_state(n: int, d: int):
    return np.full(n, -np.inf), np.zeros(n), np.zeros((n, d))


def merge(a, b):
    """Merge two partial states (m, l, o) over disjoint key sets."""
    lib = _load()
    ma, la, oa = (_f64(x) for x in a)
    mb, lb, ob = (_f64(x) for x in b)
    n, d = oa.shape
    m = np.zeros(n); l = np.zeros(n); o = np.zeros((n, d))
    lib.orc_merge(n, d, _ptr(ma), _ptr(la), _ptr(oa), _ptr(mb), _ptr(lb), _ptr(ob),
                  _ptr(m), _ptr(l), _ptr(o))
    return m, l, o


def finalize(state):
    """O = o / l, LSE = m + ln l."""
    lib = _load()
    m, l, o = (_f64(x) for x in state)
    n, d = o.shape
    out = np.zeros((n, d)); lse = np.zeros(n)
    lib.orc_finalize(n, d, _ptr(m), _ptr(l), _ptr(o), _ptr(out), _ptr(lse))
    return out, lse


def rank_share(q, k, v, P: int, rank: int, causal: bool, scale: Optional[float] = None,
               rows=None, nthreads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """One rank's share: local Q [B, N/P, Hq, d] vs the P blocks of K, V [B, N, Hkv, d]
    in ring order, merged, normalised.  Returns O [n, d], LSE [n]."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, nq, hq, d = q.shape
    N, hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    r = _rows(rows, B, hq, nq)
    n = r.shape[0]
    out = np.zeros((n, d)); lse = np.zeros(n)
    e = lib.orc_rank_share(_ptr(q), _ptr(k), _ptr(v), B, N, P, rank, hq, hkv, d, int(causal),
                           float(scale), r.ctypes.data_as(_ip), n, _ptr(out), _ptr(lse),
                           nthreads or default_threads())
    if e:
        raise ValueError(f"orc_rank_share failed ({e})")
    return out, lse


def rank_share_padded(q, k, v, P: int, rank: int, causal: bool, n_valid: int, scale: Optional[float] = None,
                      rows=None, nthreads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Share of a padded sequence: K, V [B, N, Hkv, d] with the first n_valid
    rows real; keys at positions >= n_valid are masked out.  O [n, d], LSE [n]."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, nq, hq, d = q.shape
    N, hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    r = _rows(rows, B, hq, nq)
    n = r.shape[0]
    out = np.zeros((n, d)); lse = np.zeros(n)
    e = lib.orc_rank_share_padded(_ptr(q), _ptr(k), _ptr(v), B, N, P, rank, hq, hkv, d, int(causal), float(scale),
                                  int(n_valid), r.ctypes.data_as(_ip), n, _ptr(out), _ptr(lse),
                                  nthreads or default_threads())
    if e:
        raise ValueError(f"orc_rank_share_padded failed ({e})")
    return out, lse


def rank_share_zigzag(q, k, v, P: int, rank: int, causal: bool, scale: Optional[float] = None,
                      rows=None, nthreads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Load-balanced share: local Q [B, 2c, Hq, d] = [chunk rank | chunk 2P-1-rank]
    (c = N/(2P)) against the P ring blocks of K, V [B, N, Hkv, d], block j being
    key chunks j and 2P-1-j.  Returns O [n, d], LSE [n] for the listed rows."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, nq, hq, d = q.shape
    N, hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    r = _rows(rows, B, hq, nq)
    n = r.shape[0]
    out = np.zeros((n, d)); lse = np.zeros(n)
    e = lib.orc_rank_share_zigzag(_ptr(q), _ptr(k), _ptr(v), B, N, P, rank, hq, hkv, d, int(causal),
                                  float(scale), r.ctypes.data_as(_ip), n, _ptr(out), _ptr(lse),
                                  nthreads or default_threads())
    if e:
        raise ValueError(f"orc_rank_share_zigzag failed ({e})")
    return out, lse


def zigzag_positions(N: int, P: int, rank: int) -> np.ndarray:
    """Global positions of the local rows of the load-balanced share."""
    c = N // (2 * P)
    return np.concatenate([rank * c + np.arange(c), (2 * P - 1 - rank) * c + np.arange(c)])


def rank_share_bwd(q, k, v, dout, P: int, rank: int, causal: bool, scale: Optional[float] = None,
                   qrows=None, krows=None, nthreads: Optional[int] = None, zigzag: bool = False,
                   n_valid: Optional[int] = None):
    """Gradients of one rank's share for the upstream gradient dout [B, N/P, Hq, d]:
    dQ of the listed (b, h, i) local rows [n, d] (default all), and this rank's
    contribution dK, dV to the listed (b, g, j) key rows [m, d] (default all).
    zigzag: the load-balanced share (local rows = chunks rank and 2P-1-rank of 2P).
    n_valid: the padded share's real length (keys at or after it are masked out)."""
    lib = _load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, nq, hq, d = q.shape
    N, hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    qr = _rows(qrows, B, hq, nq)
    kr = np.ascontiguousarray(all_rows(B, hkv, N) if krows is None else np.asarray(krows, dtype=np.int64))
    nq_r, nk_r = qr.shape[0], kr.shape[0]
    dq = np.zeros((max(nq_r, 1), d)); dk = np.zeros((max(nk_r, 1), d)); dv = np.zeros((max(nk_r, 1), d))
    tail = (qr.ctypes.data_as(_ip), nq_r, kr.ctypes.data_as(_ip), nk_r, _ptr(dq), _ptr(dk), _ptr(dv),
            nthreads or default_threads())
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, N, P, rank, hq, hkv, d, int(causal), float(scale))
    if n_valid is not None:
        if zigzag:
            raise ValueError("padding of the load-balanced share is not defined here")
        e = lib.orc_rank_share_padded_bwd(*head, int(n_valid), *tail)
    else:
        e = (lib.orc_rank_share_zigzag_bwd if zigzag else lib.orc_rank_share_bwd)(*head, *tail)
    if e:
        raise ValueError(f"backward oracle failed ({e})")
    return dq[:nq_r], dk[:nk_r], dv[:nk_r]


def ring_block(P: int, rank: int, s: int) -> int:
    return int(_load().orc_ring_block(P, rank, s))


def classify(q_off: int, nq: int, kv_off: int, nkv: int, causal: bool) -> int:
    """0 = SKIP, 1 = FULL, 2 = PARTIAL."""
    return int(_load().orc_classify(q_off, nq, kv_off, nkv, int(causal)))


def visible_pairs(q_off: int, nq: int, kv_off: int, nkv: int, causal: bool) -> int:
    return int(_load().orc_visible_pairs(q_off, nq, kv_off, nkv, int(causal)))


def share_flops(B: int, N: int, P: int, rank: int, Hq: int, d: int, causal: bool) -> float:
    return float(_load().orc_share_flops(B, N, P, rank, Hq, d, int(causal)))


def share_flops_zigzag(B: int, N: int, P: int, rank: int, Hq: int, d: int, causal: bool) -> float:
    return float(_load().orc_share_flops_zigzag(B, N, P, rank, Hq, d, int(causal)))
