"""C-ABI tests that need no GPU.

  * libringattn.so loads and exports every function include/libringattn.h declares;
  * argument validation returns the documented negative status before any HIP
    call (fake, never-dereferenced device addresses);
  * the host planner (ring order, block classes, tile plans, FLOP rule)
    matches the oracle and tests/golden/ring_schedules.txt bit-exactly.
"""
import ctypes
import itertools
import os
import re

import pytest
import torch

import oracle
from sequence_transformer_attention_amd import ringattn as ra
from sequence_transformer_attention_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libringattn.h")

# These tests hand the library fake device addresses and rely on validation
# rejecting the call first; never run them where a GPU could be reached.
pytestmark = pytest.mark.skipif(torch.cuda.is_available(), reason="CPU-only ABI checks")

FAKE = 0x100000  # 16-byte aligned, never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"ra_step", "ra_finalize", "ra_rank_share", "ra_state_init"} <= set(names)
    L = ctypes.CDLL(ra.library_path())
    for n in names:
        assert hasattr(L, n), f"{n} declared in libringattn.h but not exported"


def test_version_and_empty_error():
    assert "gfx950" in ra.ra_version()


# ----------------------------------------------------------------- validation
def T(shape, dtype=ra.RA_BF16, stride=None, data=FAKE):
    t = ra.RaTensor()
    t.data = data
    t.dtype = dtype
    if stride is None:
        stride = [0, 0, 0, 1]
        acc = 1
        for i in (3, 2, 1, 0):
            stride[i] = acc
            acc *= shape[i]
    for i in range(4):
        t.shape[i] = shape[i]
        t.stride[i] = stride[i]
    return t


def rows(B, H, S, data=FAKE):
    return T([B, H, S, 1], ra.RA_F32, [H * S, S, 1, 1], data)


def P(x):
    return ctypes.byref(x) if x is not None else None


def step(q, k, v, oacc, m, l, q_off=0, kv_off=0, causal=1, opts=None):
    L = ra.lib()
    return L.ra_step(P(q), P(k), P(v), P(oacc), P(m), P(l), q_off, kv_off, causal, P(opts))


def good_step_args(B=1, nq=256, nkv=256, hq=4, hkv=2, d=128, dt=ra.RA_BF16):
    return dict(q=T([B, nq, hq, d], dt), k=T([B, nkv, hkv, d], dt), v=T([B, nkv, hkv, d], dt),
                oacc=T([B, nq, hq, d], ra.RA_F32), m=rows(B, hq, nq), l=rows(B, hq, nq))


@pytest.mark.parametrize("mutate,status", [
    (lambda a: a.update(q=None), ra.RA_E_NULL),
    (lambda a: a.update(m=None), ra.RA_E_NULL),
    (lambda a: setattr(a["k"], "data", 0), ra.RA_E_NULL),
    (lambda a: setattr(a["q"], "dtype", 7), ra.RA_E_DTYPE),
    (lambda a: setattr(a["k"], "dtype", ra.RA_F32), ra.RA_E_DTYPE),
    (lambda a: setattr(a["oacc"], "dtype", ra.RA_BF16), ra.RA_E_DTYPE),
    (lambda a: a.update(v=T([1, 128, 2, 128])), ra.RA_E_SHAPE),
    (lambda a: a.update(k=T([1, 256, 3, 128]), v=T([1, 256, 3, 128])), ra.RA_E_SHAPE),
    (lambda a: a.update(oacc=T([1, 128, 4, 128], ra.RA_F32)), ra.RA_E_SHAPE),
    (lambda a: a.update(l=rows(1, 4, 255)), ra.RA_E_SHAPE),
    (lambda a: a.update(q=T([1, 256, 4, 128], stride=[256 * 4 * 128, 4 * 128, 128, 2])), ra.RA_E_LAYOUT),
    (lambda a: a.update(q=T([1, 256, 4, 128], stride=[256 * 4 * 130, 4 * 130, 130, 1])), ra.RA_E_LAYOUT),
    (lambda a: setattr(a["q"], "data", FAKE + 8), ra.RA_E_LAYOUT),
    # k row stride beyond 2^24 elements (the tile loads use 32-bit row offsets)
    (lambda a: a.update(k=T([1, 256, 2, 128], stride=[256 * (1 << 25), 1 << 25, 128, 1])), ra.RA_E_RANGE),
    # k/v blocks longer than 2^29 keys (32-bit key counters in the kernels)
    (lambda a: a.update(k=T([1, (1 << 29) + 1, 2, 128]), v=T([1, (1 << 29) + 1, 2, 128])), ra.RA_E_RANGE),
    (lambda a: a.update(q=T([1, 256, 4, 96]), k=T([1, 256, 2, 96]), v=T([1, 256, 2, 96]),
                        oacc=T([1, 256, 4, 96], ra.RA_F32)), ra.RA_E_UNSUPPORTED),
])
def test_ra_step_rejects_bad_arguments(mutate, status):
    a = good_step_args()
    mutate(a)
    assert step(**a) == status
    assert ra.ra_last_error() != ""


def test_ra_step_rejects_negative_offsets():
    assert step(**good_step_args(), q_off=-1) == ra.RA_E_RANGE
    assert step(**good_step_args(), kv_off=-5) == ra.RA_E_RANGE


def test_ra_step_skip_and_empty_return_ok_without_launch():
    # causal block entirely in the future of every query: SKIP, no launch
    assert step(**good_step_args(), q_off=0, kv_off=1000, causal=1) == ra.RA_OK
    assert step(**good_step_args(nq=0)) == ra.RA_OK
    assert step(**good_step_args(B=0)) == ra.RA_OK
    assert step(**good_step_args(nkv=0), causal=0) == ra.RA_OK   # an empty key block is SKIP


def share(q, k, v, Pn, rank, causal=1, o_out=None, lse=None, scale=0.0):
    opts = ra.RaOpts()
    opts.scale = scale
    if o_out is not None:
        opts.o_out = ctypes.pointer(o_out)
    if lse is not None:
        opts.lse_out = ctypes.pointer(lse)
    return ra.lib().ra_rank_share(P(q), P(k), P(v), Pn, rank, causal, ctypes.byref(opts))


def test_ra_rank_share_validation():
    q, k, v = T([1, 512, 4, 128]), T([1, 4096, 1, 128]), T([1, 4096, 1, 128])
    o = T([1, 512, 4, 128])
    assert share(q, k, v, 8, 7) == ra.RA_E_NULL                   # no o_out
    assert share(q, k, v, 0, 0, o_out=o) == ra.RA_E_RANGE         # P < 1
    assert share(q, k, v, 8, 8, o_out=o) == ra.RA_E_RANGE         # rank outside [0, P)
    assert share(q, k, v, 8, -1, o_out=o) == ra.RA_E_RANGE
    k3, v3 = T([1, 4095, 1, 128]), T([1, 4095, 1, 128])
    assert share(q, k3, v3, 8, 7, o_out=o) == ra.RA_E_SHAPE       # N % P != 0: no padding
    assert "divisible" in ra.ra_last_error()
    assert share(q, k, v, 4, 3, o_out=o) == ra.RA_E_SHAPE         # Nq != N / P
    assert share(q, k, v, 8, 7, o_out=T([1, 512, 4, 64])) == ra.RA_E_SHAPE
    assert share(q, k, v, 8, 7, o_out=o, lse=rows(1, 4, 511)) == ra.RA_E_SHAPE
    assert share(T([1, 0, 4, 128]), T([1, 0, 1, 128]), T([1, 0, 1, 128]), 8, 7, o_out=T([1, 0, 4, 128])) == ra.RA_OK


def test_ra_rank_share_zigzag_validation():
    def zz(q, k, v, Pn, rank, o_out=None, lse=None):
        opts = ra.RaOpts()
        if o_out is not None:
            opts.o_out = ctypes.pointer(o_out)
        if lse is not None:
            opts.lse_out = ctypes.pointer(lse)
        return ra.lib().ra_rank_share_zigzag(P(q), P(k), P(v), Pn, rank, 1, ctypes.byref(opts))
    q, k, v = T([1, 512, 4, 128]), T([1, 4096, 1, 128]), T([1, 4096, 1, 128])
    o = T([1, 512, 4, 128])
    assert zz(q, k, v, 8, 7) == ra.RA_E_NULL                      # no o_out
    assert zz(q, k, v, 0, 0, o_out=o) == ra.RA_E_RANGE            # P < 1
    assert zz(q, k, v, 8, 8, o_out=o) == ra.RA_E_RANGE            # rank outside [0, P)
    k3, v3 = T([1, 4104, 1, 128]), T([1, 4104, 1, 128])         # divisible by P = 8, not by 2P
    assert zz(T([1, 513, 4, 128]), k3, v3, 8, 7, o_out=T([1, 513, 4, 128])) == ra.RA_E_SHAPE
    assert "2P" in ra.ra_last_error()
    assert zz(q, k, v, 4, 3, o_out=o) == ra.RA_E_SHAPE            # Nq != 2 N/(2P)
    assert zz(q, k, v, 8, 7, o_out=o, lse=rows(1, 4, 511)) == ra.RA_E_SHAPE
    assert zz(T([1, 0, 4, 128]), T([1, 0, 1, 128]), T([1, 0, 1, 128]), 8, 7, o_out=T([1, 0, 4, 128])) == ra.RA_OK


def test_ra_rank_share_padded_validation():
    def pad(q, k, v, Pn, rank, n_valid, o_out=None):
        opts = ra.RaOpts()
        if o_out is not None:
            opts.o_out = ctypes.pointer(o_out)
        return ra.lib().ra_rank_share_padded(P(q), P(k), P(v), Pn, rank, 1, n_valid, ctypes.byref(opts))
    q, k, v = T([1, 512, 4, 128]), T([1, 4096, 1, 128]), T([1, 4096, 1, 128])
    o = T([1, 512, 4, 128])
    assert pad(q, k, v, 8, 7, 4000) == ra.RA_E_NULL               # no o_out
    for bad in (0, -1, 4097):                                     # n_valid outside [1, N]
        assert pad(q, k, v, 8, 7, bad, o_out=o) == ra.RA_E_RANGE, bad
        assert "n_valid" in ra.ra_last_error()
    assert pad(q, k, v, 8, 8, 4000, o_out=o) == ra.RA_E_RANGE     # rank outside [0, P)
    assert pad(q, k, v, 4, 3, 4000, o_out=o) == ra.RA_E_SHAPE     # Nq != N / P


def test_ra_rank_share_bwd_validation():
    def bwd(q, k, v, o, lse, dout, Pn, rank, dq, dk, dv, delta):
        return ra.lib().ra_rank_share_bwd(P(q), P(k), P(v), P(o), P(lse), P(dout), Pn, rank, 1, P(dq), P(dk),
                                          P(dv), P(delta), None)
    q, k, v = T([1, 512, 4, 128]), T([1, 4096, 1, 128]), T([1, 4096, 1, 128])
    o, do = T([1, 512, 4, 128]), T([1, 512, 4, 128])
    dq = T([1, 512, 4, 128], ra.RA_F32)
    dk, dv = T([1, 4096, 1, 128], ra.RA_F32), T([1, 4096, 1, 128], ra.RA_F32)
    st = rows(1, 4, 512)
    good = dict(q=q, k=k, v=v, o=o, lse=st, dout=do, Pn=8, rank=7, dq=dq, dk=dk, dv=dv, delta=rows(1, 4, 512))
    for key, bad, status in (("q", None, ra.RA_E_NULL), ("dq", T([1, 512, 4, 128]), ra.RA_E_DTYPE),
                             ("dk", T([1, 4096, 1, 64], ra.RA_F32), ra.RA_E_SHAPE),
                             ("o", T([1, 512, 4, 128], ra.RA_F32), ra.RA_E_DTYPE),
                             ("delta", rows(1, 4, 511), ra.RA_E_SHAPE), ("rank", 8, ra.RA_E_RANGE)):
        args = dict(good)
        args[key] = bad
        assert bwd(**args) == status, key
    assert bwd(**dict(good, Pn=4, rank=3)) == ra.RA_E_SHAPE        # Nq != N / P
    # q and dout tiles are addressed with 32-bit offsets: sequence stride at most 2^24
    big = [512 * (1 << 25), 1 << 25, 128, 1]
    assert bwd(**dict(good, q=T([1, 512, 4, 128], stride=big))) == ra.RA_E_RANGE
    assert bwd(**dict(good, dout=T([1, 512, 4, 128], stride=big))) == ra.RA_E_RANGE
    f32 = dict(good, q=T([1, 512, 4, 128], ra.RA_F32), k=T([1, 4096, 1, 128], ra.RA_F32),
               v=T([1, 4096, 1, 128], ra.RA_F32))
    assert bwd(**f32) == ra.RA_E_UNSUPPORTED


def test_ra_rank_share_zigzag_bwd_validation():
    def bwd(q, k, v, o, lse, dout, Pn, rank, dq, dk, dv, delta):
        return ra.lib().ra_rank_share_zigzag_bwd(P(q), P(k), P(v), P(o), P(lse), P(dout), Pn, rank, 1, P(dq),
                                                 P(dk), P(dv), P(delta), None)
    q, k, v = T([1, 512, 4, 128]), T([1, 4096, 1, 128]), T([1, 4096, 1, 128])
    o, do = T([1, 512, 4, 128]), T([1, 512, 4, 128])
    dq = T([1, 512, 4, 128], ra.RA_F32)
    dk, dv = T([1, 4096, 1, 128], ra.RA_F32), T([1, 4096, 1, 128], ra.RA_F32)
    good = dict(q=q, k=k, v=v, o=o, lse=rows(1, 4, 512), dout=do, Pn=8, rank=7, dq=dq, dk=dk, dv=dv,
                delta=rows(1, 4, 512))
    assert bwd(**dict(good, rank=8)) == ra.RA_E_RANGE
    assert bwd(**dict(good, q=None)) == ra.RA_E_NULL
    # N = 4104 is divisible by P = 8 but not by 2P
    k3, v3 = T([1, 4104, 1, 128]), T([1, 4104, 1, 128])
    q3 = T([1, 513, 4, 128])
    bad = dict(good, q=q3, k=k3, v=v3, o=T([1, 513, 4, 128]), dout=T([1, 513, 4, 128]),
               dq=T([1, 513, 4, 128], ra.RA_F32), dk=T([1, 4104, 1, 128], ra.RA_F32),
               dv=T([1, 4104, 1, 128], ra.RA_F32), lse=rows(1, 4, 513), delta=rows(1, 4, 513))
    assert bwd(**bad) == ra.RA_E_SHAPE
    assert "2P" in ra.ra_last_error()
    assert bwd(**dict(good, Pn=4, rank=3)) == ra.RA_E_SHAPE        # Nq != N / P


def test_ra_rank_share_padded_bwd_validation():
    def bwd(n_valid, Pn=8, rank=7):
        q, k, v = T([1, 512, 4, 128]), T([1, 4096, 1, 128]), T([1, 4096, 1, 128])
        o, do = T([1, 512, 4, 128]), T([1, 512, 4, 128])
        dq = T([1, 512, 4, 128], ra.RA_F32)
        dk, dv = T([1, 4096, 1, 128], ra.RA_F32), T([1, 4096, 1, 128], ra.RA_F32)
        return ra.lib().ra_rank_share_padded_bwd(P(q), P(k), P(v), P(o), P(rows(1, 4, 512)), P(do), Pn, rank, 1,
                                                 n_valid, P(dq), P(dk), P(dv), P(rows(1, 4, 512)), None)
    for bad in (0, -1, 4097):
        assert bwd(bad) == ra.RA_E_RANGE, bad
        assert "n_valid" in ra.ra_last_error()
    assert bwd(4000, rank=8) == ra.RA_E_RANGE
    assert bwd(4000, Pn=4, rank=3) == ra.RA_E_SHAPE


def test_ra_finalize_validation():
    L = ra.lib()
    oacc, l = T([1, 64, 2, 64], ra.RA_F32), rows(1, 2, 64)
    opts = ra.RaOpts()
    lse = rows(1, 2, 64)
    opts.lse_out = ctypes.pointer(lse)
    assert L.ra_finalize(P(oacc), P(l), ctypes.byref(opts)) == ra.RA_E_NULL   # lse needs m
    assert L.ra_finalize(P(T([1, 64, 2, 64])), P(l), None) == ra.RA_E_DTYPE  # o_acc must be fp32
    assert L.ra_finalize(P(oacc), P(rows(1, 2, 63)), None) == ra.RA_E_SHAPE
    assert L.ra_finalize(P(T([1, 0, 2, 64], ra.RA_F32)), P(rows(1, 2, 0)), None) == ra.RA_OK


def test_ra_state_init_validation():
    L = ra.lib()
    assert L.ra_state_init(P(T([1, 8, 2, 64])), P(rows(1, 2, 8)), P(rows(1, 2, 8)), None) == ra.RA_E_DTYPE
    assert L.ra_state_init(P(T([1, 8, 2, 64], ra.RA_F32)), P(rows(1, 2, 7)), P(rows(1, 2, 8)), None) == ra.RA_E_SHAPE


def test_ra_state_init_rejects_other_head_dims():
    L = ra.lib()
    assert L.ra_state_init(P(T([1, 8, 2, 96], ra.RA_F32)), P(rows(1, 2, 8)), P(rows(1, 2, 8)), None) == \
        ra.RA_E_UNSUPPORTED


def test_ra_merge_validation():
    L = ra.lib()
    oa, ob = T([1, 64, 2, 128], ra.RA_F32), T([1, 64, 2, 128], ra.RA_F32)
    m, l, mb, lb = rows(1, 2, 64), rows(1, 2, 64), rows(1, 2, 64), rows(1, 2, 64)

    def merge(oa=oa, m=m, l=l, ob=ob, mb=mb, lb=lb):
        return L.ra_merge(P(oa), P(m), P(l), P(ob), P(mb), P(lb), None)

    assert merge(oa=None) == ra.RA_E_NULL
    assert merge(lb=None) == ra.RA_E_NULL
    assert merge(ob=T([1, 64, 2, 128])) == ra.RA_E_DTYPE                   # bf16 state
    assert merge(ob=T([1, 63, 2, 128], ra.RA_F32)) == ra.RA_E_SHAPE         # shapes differ
    assert merge(mb=rows(1, 2, 63)) == ra.RA_E_SHAPE
    assert merge(l=T([1, 2, 64, 1], ra.RA_BF16, [128, 64, 1, 1])) == ra.RA_E_DTYPE
    assert merge(oa=T([1, 64, 2, 128], ra.RA_F32, data=FAKE + 8)) == ra.RA_E_LAYOUT
    assert merge(oa=T([1, 64, 2, 96], ra.RA_F32), ob=T([1, 64, 2, 96], ra.RA_F32)) == ra.RA_E_UNSUPPORTED
    e0, e1 = T([1, 0, 2, 128], ra.RA_F32), T([1, 0, 2, 128], ra.RA_F32)
    assert merge(oa=e0, ob=e1, m=rows(1, 2, 0), l=rows(1, 2, 0), mb=rows(1, 2, 0), lb=rows(1, 2, 0)) == ra.RA_OK


def test_empty_calls_return_ok_before_any_launch():
    """A zero batch or a zero-length sequence is a no-op for every entry
    point: each returns RA_OK after validation and before any HIP call (these
    run with no GPU)."""
    L = ra.lib()
    F32 = ra.RA_F32
    for B, N, Pn, rank in ((1, 0, 8, 7), (0, 4096, 8, 7), (0, 0, 1, 0)):
        nq = N // Pn
        q, k = T([B, nq, 4, 128]), T([B, N, 1, 128])
        g, gk = T([B, nq, 4, 128], F32), T([B, N, 1, 128], F32)
        st = rows(B, 4, nq)
        opts = ra.RaOpts()
        opts.o_out = ctypes.pointer(T([B, nq, 4, 128]))
        o = ctypes.byref(opts)
        case = f"B{B} N{N}"
        assert L.ra_rank_share(P(q), P(k), P(k), Pn, rank, 1, o) == ra.RA_OK, case
        assert L.ra_rank_share_zigzag(P(q), P(k), P(k), Pn, rank, 1, o) == ra.RA_OK, case
        assert L.ra_rank_share_padded(P(q), P(k), P(k), Pn, rank, 1, N, o) == ra.RA_OK, case
        bwd_args = (P(q), P(k), P(k), P(q), P(st), P(q), Pn, rank, 1)
        assert L.ra_rank_share_bwd(*bwd_args, P(g), P(gk), P(gk), P(st), None) == ra.RA_OK, case
        assert L.ra_rank_share_zigzag_bwd(*bwd_args, P(g), P(gk), P(gk), P(st), None) == ra.RA_OK, case
        assert L.ra_rank_share_padded_bwd(*bwd_args[:-1], 1, N, P(g), P(gk), P(gk), P(st), None) == ra.RA_OK, case
        assert L.ra_rank_share_bwd_noalloc(*bwd_args, P(g), P(gk), P(gk), None) == ra.RA_OK, case
        assert L.ra_state_init(P(g), P(st), P(st), None) == ra.RA_OK, case
        assert L.ra_merge(P(g), P(st), P(st), P(g), P(st), P(st), None) == ra.RA_OK, case
        assert L.ra_finalize(P(g), P(st), None) == ra.RA_OK, case
        assert step(q, k, k, g, st, st) == ra.RA_OK, case


def test_launches_beyond_the_work_item_limit_are_rejected():
    """A grid is at most 2^32 - 1 work-items along x: the bf16 forward runs
    256 threads per 256 query rows, the backward 256 per 128 rows, the state
    kernels 512 per 64 rows (d = 128)."""
    L = ra.lib()
    heads = (1 << 24) + 1                        # one 256-row tile each: > 2^32 / 256 workgroups
    q, k = T([1, 256, heads, 128]), T([1, 256, 1, 128])
    assert share(q, k, k, 1, 0, o_out=T([1, 256, heads, 128])) == ra.RA_E_RANGE
    assert "work-items" in ra.ra_last_error()
    assert step(q, k, k, T([1, 256, heads, 128], ra.RA_F32), rows(1, heads, 256), rows(1, heads, 256)) == \
        ra.RA_E_RANGE
    # backward: 128-row tiles of 256 threads
    hb = (1 << 24) + 1
    qb, ob = T([1, 128, hb, 128]), T([1, 128, hb, 128])
    g = T([1, 128, hb, 128], ra.RA_F32)
    dk = T([1, 128, 1, 128], ra.RA_F32)
    assert L.ra_rank_share_bwd(P(qb), P(k := T([1, 128, 1, 128])), P(k), P(ob), P(rows(1, hb, 128)), P(ob), 1, 0, 1,
                               P(g), P(dk), P(dk), P(rows(1, hb, 128)), None) == ra.RA_E_RANGE
    # state kernels: 64 rows of d = 128 per 512-thread workgroup
    big = T([1, 1 << 20, 1 << 10, 128], ra.RA_F32)
    st = rows(1, 1 << 10, 1 << 20)
    assert L.ra_state_init(P(big), P(st), P(st), None) == ra.RA_E_RANGE
    assert L.ra_finalize(P(big), P(st), None) == ra.RA_E_RANGE
    assert L.ra_merge(P(big), P(st), P(st), P(big), P(st), P(st), None) == ra.RA_E_RANGE


# ------------------------------------------------------------- host planner
def test_ring_block_and_classes_match_golden_schedules():
    path = os.path.join(ROOT, "tests", "golden", "ring_schedules.txt")
    names = {"SKIP": 0, "FULL": 1, "PARTIAL": 2}
    by = workloads.BY_NAME
    n = 0
    for line in open(path):
        if line.startswith("#"):
            continue
        wname, r, s, j, kv_off, cls = line.split()
        w = by[wname]
        r, s, j, kv_off = int(r), int(s), int(j), int(kv_off)
        nb = w.N // w.P
        assert ra.ra_ring_block(w.P, r, s) == j
        assert ra.ra_classify(r * nb, nb, j * nb, nb, w.causal) == names[cls]
        n += 1
    assert n > 100


def test_classify_matches_oracle_exhaustively():
    R = range(0, 13)
    for q_off, nq, kv_off, nkv in itertools.product(R, R, R, R):
        for causal in (0, 1):
            assert ra.ra_classify(q_off, nq, kv_off, nkv, causal) == oracle.classify(q_off, nq, kv_off, nkv, causal)


@pytest.mark.parametrize("bm,bn", [(128, 64), (64, 64), (3, 5), (16, 32)])
def test_tile_plan_matches_oracle_per_tile(bm, bn):
    for (q_off, nq, kv_off, nkv) in [(0, 300, 0, 300), (28672, 4096, 28672, 4096), (100, 77, 40, 190),
                                     (4096, 4096, 0, 4096), (0, 130, 130, 70)]:
        for causal in (0, 1):
            plan = ra.ra_plan_tiles(q_off, nq, kv_off, nkv, causal, bm, bn)
            tj = -(-nkv // bn)
            for i in range(-(-nq // bm)):
                for j in range(tj):
                    rq = min(bm, nq - i * bm)
                    rk = min(bn, nkv - j * bn)
                    assert plan[i * tj + j] == oracle.classify(q_off + i * bm, rq, kv_off + j * bn, rk, causal)


def test_share_flops_match_oracle():
    for w in workloads.ALL:
        for r in range(w.P):
            assert ra.ra_share_flops(w.B, w.N, w.P, r, w.Hq, w.d, w.causal) == \
                oracle.share_flops(w.B, w.N, w.P, r, w.Hq, w.d, w.causal)


def test_block_flops_sum_to_the_share_and_follow_the_classes():
    # per ring step, ra_flops of the (local block, arriving block) pair, times B,
    # sums to the share's FLOP (the oracle's rule)
    for w in workloads.ALL:
        nb = w.N // w.P
        for r in range(w.P):
            tot = sum(ra.ra_flops(nb, nb, r * nb, ra.ra_ring_block(w.P, r, s) * nb, w.Hq, w.d, w.causal)
                      for s in range(w.P))
            assert tot * w.B == oracle.share_flops(w.B, w.N, w.P, r, w.Hq, w.d, w.causal)
    # weights 1, 1/2, 0 by the oracle's class, on ragged blocks and offsets
    for q_off, nq, kv_off, nkv in ((0, 7, 0, 5), (10, 3, 2, 4), (3, 5, 6, 9), (0, 1, 1, 1), (100, 64, 0, 100)):
        for causal in (False, True):
            c = oracle.classify(q_off, nq, kv_off, nkv, causal)
            want = {0: 0.0, 1: 1.0, 2: 0.5}[c] * 4 * nq * nkv * 128 * 3
            assert ra.ra_flops(nq, nkv, q_off, kv_off, 3, 128, causal) == want
    assert ra.ra_flops(-1, 4, 0, 0, 1, 64, True) == -1.0


def test_zigzag_share_flops_match_oracle():
    for (B, N, P, H, d) in ((1, 32768, 8, 32, 128), (1, 131072, 16, 32, 128), (2, 1200, 3, 2, 64)):
        for r in range(P):
            for causal in (False, True):
                assert ra.ra_share_flops_zigzag(B, N, P, r, H, d, causal) == \
                    oracle.share_flops_zigzag(B, N, P, r, H, d, causal)
    assert ra.ra_share_flops_zigzag(1, 100, 8, 0, 1, 64, True) == -1.0   # N % 2P != 0


def test_tile_shape():
    assert ra.ra_tile_shape(torch.bfloat16, 128) == (256, 64)
    assert ra.ra_tile_shape(torch.float32, 64) == (64, 64)
    with pytest.raises(ra.RaError):
        ra.ra_tile_shape(torch.bfloat16, 96)


def test_ra_rank_share_bwd_noalloc_validation():
    """The allocation-free backward validates like ra_rank_share_bwd (without
    a workspace argument) and refuses more query rows than its 2^20-row
    workspace before any HIP call."""
    L = ra.lib()
    q, k = T([1, 512, 4, 128]), T([1, 4096, 1, 128])
    g, gk = T([1, 512, 4, 128], ra.RA_F32), T([1, 4096, 1, 128], ra.RA_F32)

    def call(q=q, k=k, o=q, lse=rows(1, 4, 512), dout=q, P_=8, rank=7, dq=g, dk=gk, dv=gk):
        return L.ra_rank_share_bwd_noalloc(P(q), P(k), P(k), P(o), P(lse), P(dout), P_, rank, 1, P(dq), P(dk),
                                           P(dv), None)

    assert call(q=None) == ra.RA_E_NULL
    assert call(rank=8) == ra.RA_E_RANGE
    assert call(lse=rows(1, 4, 511)) == ra.RA_E_SHAPE
    assert call(dq=T([1, 512, 4, 128])) == ra.RA_E_DTYPE
    big_q, big_g = T([1, 512, 2049, 128]), T([1, 512, 2049, 128], ra.RA_F32)   # 2^20 + 512 rows
    assert call(q=big_q, o=big_q, dout=big_q, dq=big_g, lse=rows(1, 2049, 512)) == ra.RA_E_RANGE
    assert "workspace" in ra.ra_last_error()
