"""GPU parity of the HIP path against the fp64 oracle (small and shrunken workloads).

Every case draws seeded inputs, runs libringattn through its C ABI on the
GPU and compares element by element with the oracle on the same bytes:
max |O - O_ref| <= 1e-2 and max |LSE - LSE_ref| <= 1e-3 for bf16 inputs,
<= 1e-5 for both on the fp32 path.
"""
import numpy as np
import pytest
import torch

import oracle
from sequence_transformer_attention_amd import inputs, workloads
from sequence_transformer_attention_amd import ringattn as ra
from tests.gpu_util import (assert_close, assert_grad_close, backward_gpu, gather, oracle_threads, rank_share_gpu,
                            padded_backward_gpu, padded_gpu, say, stepwise_gpu, zigzag_backward_gpu, zigzag_gpu,
                            zigzag_rows)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _dev(x):
    return {k: v.to(DEV) for k, v in x.items()}


# -------------------------------------------------------------- tiny fp32 workload
def test_tiny_f32_every_rank_fused():
    w = workloads.TINY_F32
    x = inputs.workload_inputs(w)
    d = _dev(x)
    for r in w.ranks:
        say(f"tiny_f32 fused rank {r}")
        ql = inputs.local_q(w, x["q"], r)
        O, lse = rank_share_gpu(inputs.local_q(w, d["q"], r).contiguous(), d["k"], d["v"], w.P, r, w.causal)
        torch.cuda.synchronize()
        rows = oracle.all_rows(w.B, w.Hq, w.nq)
        o_ref, l_ref = oracle.rank_share(ql, x["k"], x["v"], w.P, r, w.causal, rows=rows, nthreads=oracle_threads())
        assert_close(*gather(O, lse, rows), o_ref, l_ref, "f32", f"tiny rank {r}")


def test_tiny_f32_every_rank_stepwise_state_after_each_step():
    """Per-step running state (o_acc, m, l) against the oracle's merged partials."""
    w = workloads.TINY_F32
    x = inputs.workload_inputs(w)
    d = _dev(x)
    nb = w.nq
    rows = oracle.all_rows(w.B, w.Hq, nb)
    for r in w.ranks:
        say(f"tiny_f32 stepwise rank {r}")
        qd = inputs.local_q(w, d["q"], r).contiguous()
        qh = inputs.local_q(w, x["q"], r)
        oacc = torch.empty((w.B, nb, w.Hq, w.d), dtype=torch.float32, device=DEV)
        m = torch.empty((w.B, w.Hq, nb), dtype=torch.float32, device=DEV)
        l = torch.empty_like(m)
        ra.ra_state_init(oacc, m, l)
        st = oracle.identity_state(len(rows), w.d)
        for s in range(w.P):
            j = ra.ra_ring_block(w.P, r, s)
            ra.ra_step(qd, d["k"][:, j * nb:(j + 1) * nb], d["v"][:, j * nb:(j + 1) * nb], oacc, m, l,
                       r * nb, j * nb, w.causal)
            part = oracle.block_partial(qh, x["k"][:, j * nb:(j + 1) * nb], x["v"][:, j * nb:(j + 1) * nb],
                                        r * nb, j * nb, w.causal, rows=rows, nthreads=oracle_threads())
            st = oracle.merge(st, part)
            torch.cuda.synchronize()
            mg = m.permute(0, 1, 2).reshape(-1).double().cpu().numpy()
            lg = l.reshape(-1).double().cpu().numpy()
            og = oacc.permute(0, 2, 1, 3).reshape(-1, w.d).double().cpu().numpy()
            np.testing.assert_allclose(mg, st[0], atol=1e-5, rtol=0)
            # l and o_acc are relative to m: compare after bringing both to the oracle's m
            corr = np.exp(mg - st[0])
            np.testing.assert_allclose(lg * corr, st[1], rtol=1e-5, atol=0)
            np.testing.assert_allclose(og * corr[:, None], st[2], rtol=0, atol=1e-5 * st[1].max())
        O = torch.empty((w.B, nb, w.Hq, w.d), dtype=torch.float32, device=DEV)
        lse = torch.empty((w.B, w.Hq, nb), dtype=torch.float32, device=DEV)
        ra.ra_finalize(oacc, l, m=m, o_out=O, lse_out=lse)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.finalize(st)
        assert_close(*gather(O, lse, rows), o_ref, l_ref, "f32", f"tiny stepwise rank {r}")


# ------------------------------------------------------------ shrunken bf16 workloads
SHRUNK = [w.shrunk(16) for w in (workloads.RANK7_BF16, workloads.GQA_BF16,
                                 workloads.ULYSSES_BF16, workloads.STRESS_BF16)]


@pytest.mark.parametrize("w", SHRUNK, ids=[w.name for w in SHRUNK])
def test_shrunken_bf16_workloads_all_rows(w):
    x = inputs.workload_inputs(w)
    d = _dev(x)
    r = w.ranks[0]
    rows = oracle.all_rows(w.B, w.Hq, w.nq)
    say(f"{w.name} fused rank {r}")
    O, lse = rank_share_gpu(d["q"], d["k"], d["v"], w.P, r, w.causal, torch.float32)
    Ob, lseb = rank_share_gpu(d["q"], d["k"], d["v"], w.P, r, w.causal, torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.rank_share(x["q"], x["k"], x["v"], w.P, r, w.causal, rows=rows, nthreads=oracle_threads())
    assert_close(*gather(O, lse, rows), o_ref, l_ref, "bf16", f"{w.name} fp32 O")
    assert_close(*gather(Ob, lseb, rows), o_ref, l_ref, "bf16", f"{w.name} bf16 O", out_bf16=True)
    say(f"{w.name} stepwise rank {r}")
    Os, lses = stepwise_gpu(d["q"], d["k"], d["v"], w.P, r, w.causal)
    torch.cuda.synchronize()
    assert_close(*gather(Os, lses, rows), o_ref, l_ref, "bf16", f"{w.name} stepwise")


# -------------------------------------------------- load-balanced (zigzag) share
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,N,P,Hq,Hkv,d,causal,ranks", [
    (1, 4096, 4, 2, 1, 128, True, (0, 3)),     # chunks of 512 rows: two full bf16 query tiles each
    (2, 1200, 3, 2, 2, 64, True, (0, 1, 2)),   # chunks of 200: ragged query and key tiles, B = 2
    (1, 2048, 2, 4, 2, 128, False, (1,)),      # no mask, GQA
    (1, 192, 3, 1, 1, 64, True, (2,)),         # chunks of 32 rows
])
def test_zigzag_share(dt, B, N, P, Hq, Hkv, d, causal, ranks):
    x = inputs.draw_qkv(B, N, N, Hq, Hkv, d, seed=N + P, dtype=dt)
    dv = _dev(x)
    for r in ranks:
        pos = zigzag_rows(N, P, r)
        ql = x["q"][:, pos].contiguous()
        say(f"zigzag {dt} B{B} N{N} P{P} Hq{Hq} Hkv{Hkv} d{d} causal{int(causal)} rank {r}")
        O, lse = zigzag_gpu(ql.to(DEV), dv["k"], dv["v"], P, r, causal)
        torch.cuda.synchronize()
        rows = oracle.all_rows(B, Hq, len(pos))
        o_ref, l_ref = oracle.rank_share_zigzag(ql, x["k"], x["v"], P, r, causal, rows=rows,
                                                nthreads=oracle_threads())
        assert_close(*gather(O, lse, rows), o_ref, l_ref, dt, f"zigzag rank {r}")


# ------------------------------------------------ padded (uneven length) share
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,n_valid,P,Hq,Hkv,d,causal,ranks", [
    (1, 4000, 4, 2, 1, 128, True, (0, 3)),     # N 4000 = 4 x 1000: last block 1000 rows, 0 padding
    (1, 3990, 4, 2, 1, 128, True, (1, 3)),     # N 3992: last block holds 990 real keys of 998
    (2, 1133, 3, 2, 2, 64, False, (0, 2)),     # N 1134, no mask, B 2
    (1, 700, 4, 4, 2, 128, True, (2, 3)),      # N 700: nb 175, ragged key tiles everywhere
    (1, 1500, 4, 2, 1, 128, True, (3, 0)),     # N 1500 + padding block: n_valid < 3 nb + 1 for N 2000
])
def test_padded_share(dt, B, n_valid, P, Hq, Hkv, d, causal, ranks):
    """Keys past n_valid hold NaN: a kernel that lets any of them into a sum fails."""
    N = P * (-(-n_valid // P))
    if n_valid == 1500:
        N = 2000                               # the whole last block is padding
    x = inputs.draw_qkv(B, N, N, Hq, Hkv, d, seed=n_valid + P, dtype=dt)
    x["k"][:, n_valid:] = float("nan")
    x["v"][:, n_valid:] = float("nan")
    dv = _dev(x)
    nb = N // P
    for r in ranks:
        ql = x["q"][:, r * nb:(r + 1) * nb].contiguous()
        say(f"padded {dt} B{B} N{N} n_valid{n_valid} P{P} Hq{Hq} Hkv{Hkv} d{d} causal{int(causal)} rank {r}")
        O, lse = padded_gpu(ql.to(DEV), dv["k"], dv["v"], P, r, causal, n_valid)
        torch.cuda.synchronize()
        rows = oracle.all_rows(B, Hq, nb)
        o_ref, l_ref = oracle.rank_share_padded(ql, x["k"], x["v"], P, r, causal, n_valid, rows=rows,
                                                nthreads=oracle_threads())
        assert_close(*gather(O, lse, rows), o_ref, l_ref, dt, f"padded rank {r}")


def test_zigzag_shares_reassemble_full_attention():
    """All ranks' load-balanced shares, put back in sequence order, give the
    same result as the one-rank share over the whole sequence (P = 1)."""
    B, N, P, H, d = 1, 2048, 4, 2, 128
    x = _dev(inputs.draw_qkv(B, N, N, H, H, d, seed=77))
    full, full_lse = rank_share_gpu(x["q"], x["k"], x["v"], 1, 0, True)
    got = torch.empty_like(full)
    got_lse = torch.empty_like(full_lse)
    for r in range(P):
        pos = zigzag_rows(N, P, r).to(DEV)
        O, lse = zigzag_gpu(x["q"][:, pos].contiguous(), x["k"], x["v"], P, r, True)
        got[:, pos] = O
        got_lse[:, :, pos] = lse
    torch.cuda.synchronize()
    say(f"zigzag reassembled: max|dO| {float((got - full).abs().max()):.3e}")
    assert float((got - full).abs().max()) <= 1e-2 and float((got_lse - full_lse).abs().max()) <= 1e-3


# ---------------------------------------------------------------- backward
@pytest.mark.parametrize("B,N,P,Hq,Hkv,d,causal,ranks", [
    (1, 1024, 4, 2, 1, 128, True, (0, 3)),     # GQA; the first rank's keys past its queries get zero
    (2, 600, 3, 2, 2, 64, True, (1,)),         # blocks of 200: ragged query and key tiles, B = 2
    (1, 512, 2, 4, 2, 128, False, (1,)),       # no mask
])
def test_backward_share(B, N, P, Hq, Hkv, d, causal, ranks):
    x = inputs.draw_qkv(B, N, N, Hq, Hkv, d, seed=N + 3 * P)
    dv_ = _dev(x)
    nb = N // P
    g = torch.Generator().manual_seed(N)
    for r in ranks:
        ql = x["q"][:, r * nb:(r + 1) * nb].contiguous()
        dout = torch.randn(B, nb, Hq, d, generator=g).to(torch.bfloat16)
        say(f"backward B{B} N{N} P{P} Hq{Hq} Hkv{Hkv} d{d} causal{int(causal)} rank {r}")
        dq, dk, dv = backward_gpu(ql.to(DEV), dv_["k"], dv_["v"], P, r, causal, dout.to(DEV))
        torch.cuda.synchronize()
        dq_r, dk_r, dv_r = oracle.rank_share_bwd(ql, x["k"], x["v"], dout, P, r, causal, nthreads=oracle_threads())
        grid = lambda a, H, S: a.reshape(B, H, S, d).transpose(0, 2, 1, 3)
        assert_grad_close(dq.double().cpu().numpy(), grid(dq_r, Hq, nb), f"dQ rank {r}")
        assert_grad_close(dk.double().cpu().numpy(), grid(dk_r, Hkv, N), f"dK rank {r}")
        assert_grad_close(dv.double().cpu().numpy(), grid(dv_r, Hkv, N), f"dV rank {r}")


@pytest.mark.parametrize("B,N,P,Hq,Hkv,d,causal,ranks", [
    (1, 2048, 4, 2, 1, 128, True, (0, 3)),     # chunks of 256 rows, GQA
    (2, 1200, 3, 2, 2, 64, True, (1, 2)),      # chunks of 200: ragged tiles in both chunks, B = 2
    (1, 1024, 2, 2, 2, 128, False, (0,)),      # no mask
])
def test_zigzag_backward_share(B, N, P, Hq, Hkv, d, causal, ranks):
    x = inputs.draw_qkv(B, N, N, Hq, Hkv, d, seed=N + 5 * P)
    dv_ = _dev(x)
    g = torch.Generator().manual_seed(N + 1)
    for r in ranks:
        pos = zigzag_rows(N, P, r)
        ql = x["q"][:, pos].contiguous()
        nq = len(pos)
        dout = torch.randn(B, nq, Hq, d, generator=g).to(torch.bfloat16)
        say(f"zigzag backward B{B} N{N} P{P} Hq{Hq} Hkv{Hkv} d{d} causal{int(causal)} rank {r}")
        dq, dk, dv = zigzag_backward_gpu(ql.to(DEV), dv_["k"], dv_["v"], P, r, causal, dout.to(DEV))
        torch.cuda.synchronize()
        dq_r, dk_r, dv_r = oracle.rank_share_bwd(ql, x["k"], x["v"], dout, P, r, causal, nthreads=oracle_threads(),
                                                 zigzag=True)
        grid = lambda a, H, S: a.reshape(B, H, S, d).transpose(0, 2, 1, 3)
        assert_grad_close(dq.double().cpu().numpy(), grid(dq_r, Hq, nq), f"zigzag dQ rank {r}")
        assert_grad_close(dk.double().cpu().numpy(), grid(dk_r, Hkv, N), f"zigzag dK rank {r}")
        assert_grad_close(dv.double().cpu().numpy(), grid(dv_r, Hkv, N), f"zigzag dV rank {r}")


@pytest.mark.parametrize("B,n_valid,P,Hq,Hkv,d,causal,ranks", [
    (1, 3990, 4, 2, 1, 128, True, (1, 3)),     # N 3992: the last block ends in 2 padding keys
    (2, 1133, 3, 2, 2, 64, False, (0, 2)),     # N 1134, no mask, B 2
    (1, 1500, 4, 2, 1, 128, True, (3, 0)),     # N 2000: the last block is all padding
])
def test_padded_backward_share(B, n_valid, P, Hq, Hkv, d, causal, ranks):
    """Keys past n_valid hold NaN: any read of them poisons a gradient."""
    N = 2000 if n_valid == 1500 else P * (-(-n_valid // P))
    x = inputs.draw_qkv(B, N, N, Hq, Hkv, d, seed=n_valid + 7 * P)
    x["k"][:, n_valid:] = float("nan")
    x["v"][:, n_valid:] = float("nan")
    dv_ = _dev(x)
    nb = N // P
    g = torch.Generator().manual_seed(n_valid)
    for r in ranks:
        ql = x["q"][:, r * nb:(r + 1) * nb].contiguous()
        dout = torch.randn(B, nb, Hq, d, generator=g).to(torch.bfloat16)
        say(f"padded backward B{B} N{N} n_valid{n_valid} P{P} Hq{Hq} Hkv{Hkv} d{d} causal{int(causal)} rank {r}")
        dq, dk, dv = padded_backward_gpu(ql.to(DEV), dv_["k"], dv_["v"], P, r, causal, n_valid, dout.to(DEV))
        torch.cuda.synchronize()
        dq_r, dk_r, dv_r = oracle.rank_share_bwd(ql, x["k"], x["v"], dout, P, r, causal, nthreads=oracle_threads(),
                                                 n_valid=n_valid)
        grid = lambda a, H, S: a.reshape(B, H, S, d).transpose(0, 2, 1, 3)
        assert_grad_close(dq.double().cpu().numpy(), grid(dq_r, Hq, nb), f"padded dQ rank {r}")
        assert_grad_close(dk.double().cpu().numpy(), grid(dk_r, Hkv, N), f"padded dK rank {r}")
        assert_grad_close(dv.double().cpu().numpy(), grid(dv_r, Hkv, N), f"padded dV rank {r}")
        assert float(dk[:, n_valid:].abs().max()) == 0.0 and float(dv[:, n_valid:].abs().max()) == 0.0


# --------------------------------------------------------- seeded random shapes
def _random_case(seed):
    """Head dim, ring size, mask and rank cycle with the seed; sizes are drawn."""
    rng = np.random.default_rng(1000 + seed)
    d, P, causal = 128 if seed % 2 == 0 else 64, 2 + seed % 3, seed % 5 != 4
    r = P - 1 - (seed // 3) % P
    B, nb = int(rng.integers(1, 3)), int(rng.integers(20, 300))
    Hkv, G = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    return B, P, nb, G * Hkv, Hkv, d, causal, r


@pytest.mark.parametrize("seed", range(10))
def test_random_shapes_share_and_backward(seed):
    """Seeded random shapes (block lengths off every tile size, GQA, d 64 or 128,
    with and without the mask, any rank): the fused share and its backward
    against the oracle on every row."""
    B, P, nb, Hq, Hkv, d, causal, r = _random_case(seed)
    N = P * nb
    x = inputs.draw_qkv(B, N, N, Hq, Hkv, d, seed=2000 + seed)
    dv_ = _dev(x)
    ql = x["q"][:, r * nb:(r + 1) * nb].contiguous()
    say(f"random seed {seed}: B{B} N{N} P{P} Hq{Hq} Hkv{Hkv} d{d} causal{int(causal)} rank {r}")
    O, lse = rank_share_gpu(ql.to(DEV), dv_["k"], dv_["v"], P, r, causal, torch.float32)
    torch.cuda.synchronize()
    rows = oracle.all_rows(B, Hq, nb)
    o_ref, l_ref = oracle.rank_share(ql, x["k"], x["v"], P, r, causal, rows=rows, nthreads=oracle_threads())
    assert_close(*gather(O, lse, rows), o_ref, l_ref, "bf16", f"random {seed} share")
    dout = torch.randn(B, nb, Hq, d, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    dq, dk, dv = backward_gpu(ql.to(DEV), dv_["k"], dv_["v"], P, r, causal, dout.to(DEV))
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r = oracle.rank_share_bwd(ql, x["k"], x["v"], dout, P, r, causal, nthreads=oracle_threads())
    grid = lambda a, H, S: a.reshape(B, H, S, d).transpose(0, 2, 1, 3)
    assert_grad_close(dq.double().cpu().numpy(), grid(dq_r, Hq, nb), f"random {seed} dQ")
    assert_grad_close(dk.double().cpu().numpy(), grid(dk_r, Hkv, N), f"random {seed} dK")
    assert_grad_close(dv.double().cpu().numpy(), grid(dv_r, Hkv, N), f"random {seed} dV")


def _random_variant_case(seed):
    """Shapes for the load-balanced, padded and reordered stepwise shares."""
    rng = np.random.default_rng(3000 + seed)
    d, P, causal = 64 if seed % 2 == 0 else 128, 2 + seed % 3, seed % 4 != 3
    B, Hkv, G = int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.integers(1, 3))
    c = int(rng.integers(9, 170))                   # zigzag chunk: N = 2 P c
    n_valid = int(rng.integers(P + 1, 300 * P))      # padded: N = P ceil(n_valid / P)
    r = int(rng.integers(0, P))
    order = [int(j) for j in rng.permutation(P)]     # any fold order gives the same share
    dt = "f32" if seed % 4 == 1 else "bf16"
    return B, P, G * Hkv, Hkv, d, causal, r, c, n_valid, order, dt


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_zigzag_padded_and_reordered_steps(seed):
    """Seeded random shapes for the other entry points, every row against the
    oracle: the load-balanced share and its backward, the padded share (NaN
    padding keys) and its backward, and the plain share as P ra_step calls in
    a random block order (the merge is order-independent up to rounding)."""
    B, P, Hq, Hkv, d, causal, r, c, n_valid, order, dt = _random_variant_case(seed)
    grid = lambda a, H, S: a.reshape(B, H, S, d).transpose(0, 2, 1, 3)
    g = torch.Generator().manual_seed(4000 + seed)

    N = 2 * P * c
    say(f"random zigzag seed {seed}: {dt} B{B} N{N} P{P} Hq{Hq} Hkv{Hkv} d{d} causal{int(causal)} rank {r}")
    x = inputs.draw_qkv(B, N, N, Hq, Hkv, d, seed=5000 + seed, dtype=dt)
    xd = _dev(x)
    ql = x["q"][:, zigzag_rows(N, P, r)].contiguous()
    rows = oracle.all_rows(B, Hq, 2 * c)
    O, lse = zigzag_gpu(ql.to(DEV), xd["k"], xd["v"], P, r, causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.rank_share_zigzag(ql, x["k"], x["v"], P, r, causal, rows=rows, nthreads=oracle_threads())
    assert_close(*gather(O, lse, rows), o_ref, l_ref, dt, f"random {seed} zigzag")
    if dt == "bf16":
        dout = torch.randn(B, 2 * c, Hq, d, generator=g).to(torch.bfloat16)
        dq, dk, dv = zigzag_backward_gpu(ql.to(DEV), xd["k"], xd["v"], P, r, causal, dout.to(DEV))
        torch.cuda.synchronize()
        dq_r, dk_r, dv_r = oracle.rank_share_bwd(ql, x["k"], x["v"], dout, P, r, causal,
                                                 nthreads=oracle_threads(), zigzag=True)
        assert_grad_close(dq.double().cpu().numpy(), grid(dq_r, Hq, 2 * c), f"random {seed} zigzag dQ")
        assert_grad_close(dk.double().cpu().numpy(), grid(dk_r, Hkv, N), f"random {seed} zigzag dK")
        assert_grad_close(dv.double().cpu().numpy(), grid(dv_r, Hkv, N), f"random {seed} zigzag dV")

    nb = -(-n_valid // P)
    N = P * nb
    say(f"random padded seed {seed}: {dt} B{B} N{N} n_valid{n_valid} P{P} Hq{Hq} Hkv{Hkv} d{d} "
        f"causal{int(causal)} rank {r}")
    x = inputs.draw_qkv(B, N, N, Hq, Hkv, d, seed=6000 + seed, dtype=dt)
    x["k"][:, n_valid:] = float("nan")
    x["v"][:, n_valid:] = float("nan")
    xd = _dev(x)
    ql = x["q"][:, r * nb:(r + 1) * nb].contiguous()
    rows = oracle.all_rows(B, Hq, nb)
    O, lse = padded_gpu(ql.to(DEV), xd["k"], xd["v"], P, r, causal, n_valid)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.rank_share_padded(ql, x["k"], x["v"], P, r, causal, n_valid, rows=rows,
                                            nthreads=oracle_threads())
    assert_close(*gather(O, lse, rows), o_ref, l_ref, dt, f"random {seed} padded")
    if dt == "bf16":
        dout = torch.randn(B, nb, Hq, d, generator=g).to(torch.bfloat16)
        dq, dk, dv = padded_backward_gpu(ql.to(DEV), xd["k"], xd["v"], P, r, causal, n_valid, dout.to(DEV))
        torch.cuda.synchronize()
        dq_r, dk_r, dv_r = oracle.rank_share_bwd(ql, x["k"], x["v"], dout, P, r, causal,
                                                 nthreads=oracle_threads(), n_valid=n_valid)
        assert_grad_close(dq.double().cpu().numpy(), grid(dq_r, Hq, nb), f"random {seed} padded dQ")
        assert_grad_close(dk.double().cpu().numpy(), grid(dk_r, Hkv, N), f"random {seed} padded dK")
        assert_grad_close(dv.double().cpu().numpy(), grid(dv_r, Hkv, N), f"random {seed} padded dV")
        if n_valid < N:
            assert float(dk[:, n_valid:].abs().max()) == 0.0 and float(dv[:, n_valid:].abs().max()) == 0.0

    # the contiguous share folded block by block in a random order (padding
    # rows removed: every key real)
    x = inputs.draw_qkv(B, N, N, Hq, Hkv, d, seed=7000 + seed, dtype=dt)
    xd = _dev(x)
    ql = x["q"][:, r * nb:(r + 1) * nb].contiguous()
    say(f"random stepwise seed {seed}: {dt} B{B} N{N} P{P} order {order} rank {r}")
    O, lse = stepwise_gpu(ql.to(DEV), xd["k"], xd["v"], P, r, causal, order=order)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.rank_share(ql, x["k"], x["v"], P, r, causal, rows=rows, nthreads=oracle_threads())
    assert_close(*gather(O, lse, rows), o_ref, l_ref, dt, f"random {seed} stepwise")


# ------------------------------------------------------------------ edge cases
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,nq,nkv,Hq,Hkv,d,q_off,kv_off,causal", [
    (1, 200, 150, 2, 1, 128, 100, 60, True),     # ragged q and kv tails, diagonal inside
    (2, 77, 333, 4, 2, 64, 300, 0, True),        # d = 64, GQA, B = 2, many ragged tiles
    (1, 130, 70, 3, 3, 128, 0, 0, False),
    (1, 1, 1, 1, 1, 128, 0, 0, True),            # single query, single key
    (1, 64, 4096, 1, 1, 128, 5000, 1000, True),  # block partly in the future of the first rows
    (1, 256, 64, 2, 2, 128, 0, 192, True),       # rows 0..191 see nothing of this block
])
def test_ra_step_edge_cases(dt, B, nq, nkv, Hq, Hkv, d, q_off, kv_off, causal):
    say(f"edge {dt} B{B} nq{nq} nkv{nkv} Hq{Hq} Hkv{Hkv} d{d} q_off{q_off} kv_off{kv_off} causal{causal}")
    x = inputs.draw_qkv(B, nq, nkv, Hq, Hkv, d, seed=nq + nkv, dtype=dt)
    xd = _dev(x)
    oacc = torch.empty((B, nq, Hq, d), dtype=torch.float32, device=DEV)
    m = torch.empty((B, Hq, nq), dtype=torch.float32, device=DEV)
    l = torch.empty_like(m)
    ra.ra_state_init(oacc, m, l)
    ra.ra_step(xd["q"], xd["k"], xd["v"], oacc, m, l, q_off, kv_off, causal)
    rows = oracle.all_rows(B, Hq, nq)
    mr, lr, orr = oracle.block_partial(x["q"], x["k"], x["v"], q_off, kv_off, causal, rows=rows,
                                       nthreads=oracle_threads())
    torch.cuda.synchronize()
    mg = m.reshape(-1).double().cpu().numpy()
    vis = lr > 0
    # rows that see no key keep the empty state exactly
    assert np.all(mg[~vis] == -np.inf)
    assert np.all(l.reshape(-1).cpu().numpy()[~vis] == 0)
    if vis.any():
        O = torch.empty((B, nq, Hq, d), dtype=torch.float32, device=DEV)
        lse = torch.empty((B, Hq, nq), dtype=torch.float32, device=DEV)
        ra.ra_finalize(oacc, l, m=m, o_out=O, lse_out=lse)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.finalize((mr[vis], lr[vis], orr[vis]))
        assert_close(*gather(O, lse, rows[vis]), o_ref, l_ref, dt, "edge")


def test_bhsd_strided_views_and_skip_leaves_state_untouched():
    """[B, H, S, d] buffers passed as permuted views; a SKIP step launches nothing."""
    B, S, H, d = 1, 300, 2, 128
    x = inputs.draw_qkv(B, S, S, H, H, d, seed=99)
    qh = x["q"].permute(0, 2, 1, 3).contiguous().to(DEV)   # [B, H, S, d] storage
    kh = x["k"].permute(0, 2, 1, 3).contiguous().to(DEV)
    vh = x["v"].permute(0, 2, 1, 3).contiguous().to(DEV)
    q, k, v = (t.permute(0, 2, 1, 3) for t in (qh, kh, vh))   # [B, S, H, d] views
    say("bhsd strided rank share")
    O, lse = rank_share_gpu(q, k, v, 1, 0, True)
    torch.cuda.synchronize()
    rows = oracle.all_rows(B, H, S)
    o_ref, l_ref = oracle.rank_share(x["q"], x["k"], x["v"], 1, 0, True, rows=rows, nthreads=oracle_threads())
    assert_close(*gather(O, lse, rows), o_ref, l_ref, "bf16", "bhsd views")
    oacc = torch.randn((B, S, H, d), device=DEV)
    m = torch.randn((B, H, S), device=DEV)
    l = torch.rand((B, H, S), device=DEV)
    before = [t.clone() for t in (oacc, m, l)]
    ra.ra_step(q, k, v, oacc, m, l, 0, 10_000, True)    # every key after every query
    torch.cuda.synchronize()
    for a, b in zip((oacc, m, l), before):
        assert torch.equal(a, b)


def test_run_to_run_bitwise_determinism_and_nan_poison():
    w = workloads.RANK7_BF16.shrunk(16)
    d = _dev(inputs.workload_inputs(w))
    say("determinism")
    O1, l1 = rank_share_gpu(d["q"], d["k"], d["v"], w.P, w.ranks[0], w.causal, torch.bfloat16)
    O2, l2 = rank_share_gpu(d["q"], d["k"], d["v"], w.P, w.ranks[0], w.causal, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(l1, l2)
    assert not torch.isnan(O1.float()).any() and not torch.isnan(l1).any()   # outputs were NaN-filled


def test_backward_run_to_run_bitwise_determinism():
    """The backward has no atomics or order-dependent sums: two runs agree bit for bit."""
    w = workloads.RANK7_BF16.shrunk(16)
    d = _dev(inputs.workload_inputs(w))
    g = torch.Generator().manual_seed(5)
    dout = torch.randn(d["q"].shape, generator=g).to(torch.bfloat16).to(DEV)
    say("backward determinism")
    r1 = backward_gpu(d["q"], d["k"], d["v"], w.P, w.ranks[0], w.causal, dout)
    r2 = backward_gpu(d["q"], d["k"], d["v"], w.P, w.ranks[0], w.causal, dout)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b) and not torch.isnan(a).any()


def test_stepwise_resume_from_host_checkpoint():
    """Stop after k steps, copy the state to host memory and back, finish: bitwise equal."""
    w = workloads.GQA_BF16.shrunk(16)
    d = _dev(inputs.workload_inputs(w))
    r, nb = w.ranks[0], w.nq
    say("checkpoint/resume")

    def run(checkpoint_at):
        oacc = torch.empty((w.B, nb, w.Hq, w.d), dtype=torch.float32, device=DEV)
        m = torch.empty((w.B, w.Hq, nb), dtype=torch.float32, device=DEV)
        l = torch.empty_like(m)
        ra.ra_state_init(oacc, m, l)
        for s in range(w.P):
            if s == checkpoint_at:
                host = [t.cpu() for t in (oacc, m, l)]
                oacc, m, l = (t.to(DEV) for t in host)
            j = ra.ra_ring_block(w.P, r, s)
            ra.ra_step(d["q"], d["k"][:, j * nb:(j + 1) * nb], d["v"][:, j * nb:(j + 1) * nb], oacc, m, l,
                       r * nb, j * nb, w.causal)
        torch.cuda.synchronize()
        return oacc, m, l

    a = run(-1)
    b = run(w.P // 2)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
