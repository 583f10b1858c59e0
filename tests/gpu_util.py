"""Helpers of the GPU parity tests: run the HIP path, gather rows, compare with the oracle."""
import os
import sys

import numpy as np
import torch

import oracle
from sequence_transformer_attention_amd import ringattn as ra

# bf16 inputs with fp32 accumulation / fp32 path
TOL = {"bf16": (1e-2, 1e-3), "f32": (1e-5, 1e-5)}


def say(msg: str) -> None:
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def oracle_threads() -> int:
    return max(1, min(16, oracle.default_threads()))


def gather(O: torch.Tensor, lse: torch.Tensor, rows: np.ndarray):
    """O [B, S, H, d], lse [B, H, S] (device) -> (O rows [n, d], lse rows [n]) as fp64 numpy."""
    r = torch.as_tensor(rows, dtype=torch.long, device=O.device)
    o = O[r[:, 0], r[:, 2], r[:, 1]].double().cpu().numpy()
    l = lse[r[:, 0], r[:, 1], r[:, 2]].double().cpu().numpy()
    return o, l


def assert_close(o, l, o_ref, l_ref, dtype: str, what: str, out_bf16: bool = False):
    """max |O - O_ref| and max |LSE - LSE_ref| within the tolerance of `dtype`.

    out_bf16: O was stored as bf16.  Rounding a value y to bf16 (8
    significant bits, round to nearest even) moves it by at most half an ulp,
    2^-8 |y| (0.0156 for |y| just above 4), and the value rounded is within
    tol of O_ref, so each element may differ by tol + 2^-8 (|O_ref| + tol):
    the arithmetic tolerance plus the output format's own rounding."""
    tol_o, tol_l = TOL[dtype]
    assert np.isfinite(o).all() and np.isfinite(l).all(), f"{what}: non-finite output"
    allow = tol_o + ((np.abs(o_ref) + tol_o) * 2.0 ** -8 if out_bf16 else 0.0)
    excess = float((np.abs(o - o_ref) - allow).max()) if o.size else -1.0
    eo = float(np.abs(o - o_ref).max()) if o.size else 0.0
    el = float(np.abs(l - l_ref).max()) if l.size else 0.0
    say(f"{what}: max|dO| = {eo:.3e} (tol {tol_o}{' + bf16 output rounding' if out_bf16 else ''}), "
        f"max|dLSE| = {el:.3e} (tol {tol_l}), rows {len(l)}")
    assert excess <= 0, f"{what}: |O - O_ref| exceeds the tolerance by {excess}"
    assert el <= tol_l, f"{what}: max |LSE - LSE_ref| = {el} > {tol_l}"
    return eo, el


def rank_share_gpu(q, k, v, P, rank, causal, o_dtype=torch.float32, scale=None):
    """q, k, v on the device; returns (O [B, Nq, Hq, d], lse [B, Hq, Nq])."""
    B, nq, hq, d = q.shape
    O = torch.full((B, nq, hq, d), float("nan"), dtype=o_dtype, device=q.device)
    lse = torch.full((B, hq, nq), float("nan"), dtype=torch.float32, device=q.device)
    ra.ra_rank_share(q, k, v, P, rank, causal, O, lse, scale=scale)
    return O, lse


def stepwise_gpu(q, k, v, P, rank, causal, o_dtype=torch.float32, scale=None, order=None):
    """The same share as P ra_step calls (ring order unless `order`) + ra_finalize."""
    B, nq, hq, d = q.shape
    N = k.shape[1]
    nb = N // P
    dev = q.device
    oacc = torch.empty((B, nq, hq, d), dtype=torch.float32, device=dev)
    m = torch.empty((B, hq, nq), dtype=torch.float32, device=dev)
    l = torch.empty((B, hq, nq), dtype=torch.float32, device=dev)
    ra.ra_state_init(oacc, m, l)
    steps = order if order is not None else [ra.ra_ring_block(P, rank, s) for s in range(P)]
    for j in steps:
        ra.ra_step(q, k[:, j * nb:(j + 1) * nb], v[:, j * nb:(j + 1) * nb], oacc, m, l,
                   rank * nb, j * nb, causal, scale=scale)
    O = torch.full((B, nq, hq, d), float("nan"), dtype=o_dtype, device=dev)
    lse = torch.full((B, hq, nq), float("nan"), dtype=torch.float32, device=dev)
    ra.ra_finalize(oacc, l, m=m, o_out=O, lse_out=lse)
    return O, lse


def zigzag_rows(N: int, P: int, rank: int) -> torch.Tensor:
    """Sequence rows of rank `rank`'s load-balanced share: chunks rank and
    2P-1-rank of 2P (written out here, independently of both sides)."""
    c = N // (2 * P)
    return torch.cat([torch.arange(rank * c, (rank + 1) * c), torch.arange((2 * P - 1 - rank) * c, (2 * P - rank) * c)])


def zigzag_gpu(q, k, v, P, rank, causal, o_dtype=torch.float32, scale=None):
    """q = the rank's local rows (both chunks) on the device; returns (O, lse)."""
    B, nq, hq, d = q.shape
    O = torch.full((B, nq, hq, d), float("nan"), dtype=o_dtype, device=q.device)
    lse = torch.full((B, hq, nq), float("nan"), dtype=torch.float32, device=q.device)
    ra.ra_rank_share_zigzag(q, k, v, P, rank, causal, O, lse, scale=scale)
    return O, lse


def padded_gpu(q, k, v, P, rank, causal, n_valid, o_dtype=torch.float32, scale=None):
    """Share of a sequence padded to k.shape[1] rows, the first n_valid real."""
    B, nq, hq, d = q.shape
    O = torch.full((B, nq, hq, d), float("nan"), dtype=o_dtype, device=q.device)
    lse = torch.full((B, hq, nq), float("nan"), dtype=torch.float32, device=q.device)
    ra.ra_rank_share_padded(q, k, v, P, rank, causal, n_valid, O, lse, scale=scale)
    return O, lse


def backward_gpu(q, k, v, P, rank, causal, dout, scale=None):
    """Forward (bf16 O, LSE) then backward on the device; returns (dq, dk, dv) fp32."""
    B, nq, hq, d = q.shape
    O = torch.empty((B, nq, hq, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, hq, nq), dtype=torch.float32, device=q.device)
    ra.ra_rank_share(q, k, v, P, rank, causal, O, lse, scale=scale)
    dq = torch.full((B, nq, hq, d), float("nan"), dtype=torch.float32, device=q.device)
    dk = torch.full(k.shape, float("nan"), dtype=torch.float32, device=q.device)
    dv = torch.full(k.shape, float("nan"), dtype=torch.float32, device=q.device)
    delta = torch.empty((B, hq, nq), dtype=torch.float32, device=q.device)
    ra.ra_rank_share_bwd(q, k, v, O, lse, dout, P, rank, causal, dq, dk, dv, delta, scale=scale)
    return dq, dk, dv


def zigzag_backward_gpu(q, k, v, P, rank, causal, dout, scale=None):
    """Load-balanced forward (bf16 O, LSE) then its backward; returns (dq, dk, dv) fp32."""
    B, nq, hq, d = q.shape
    O = torch.empty((B, nq, hq, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, hq, nq), dtype=torch.float32, device=q.device)
    ra.ra_rank_share_zigzag(q, k, v, P, rank, causal, O, lse, scale=scale)
    dq = torch.full((B, nq, hq, d), float("nan"), dtype=torch.float32, device=q.device)
    dk = torch.full(k.shape, float("nan"), dtype=torch.float32, device=q.device)
    dv = torch.full(k.shape, float("nan"), dtype=torch.float32, device=q.device)
    delta = torch.empty((B, hq, nq), dtype=torch.float32, device=q.device)
    ra.ra_rank_share_zigzag_bwd(q, k, v, O, lse, dout, P, rank, causal, dq, dk, dv, delta, scale=scale)
    return dq, dk, dv


def padded_backward_gpu(q, k, v, P, rank, causal, n_valid, dout, scale=None):
    """Padded forward (bf16 O, LSE) then its backward; returns (dq, dk, dv) fp32."""
    B, nq, hq, d = q.shape
    O = torch.empty((B, nq, hq, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, hq, nq), dtype=torch.float32, device=q.device)
    ra.ra_rank_share_padded(q, k, v, P, rank, causal, n_valid, O, lse, scale=scale)
    dq = torch.full((B, nq, hq, d), float("nan"), dtype=torch.float32, device=q.device)
    dk = torch.full(k.shape, float("nan"), dtype=torch.float32, device=q.device)
    dv = torch.full(k.shape, float("nan"), dtype=torch.float32, device=q.device)
    delta = torch.empty((B, hq, nq), dtype=torch.float32, device=q.device)
    ra.ra_rank_share_padded_bwd(q, k, v, O, lse, dout, P, rank, causal, n_valid, dq, dk, dv, delta, scale=scale)
    return dq, dk, dv


# Gradients: bf16 operands (q, k, v, dO, the forward's bf16 O, and P and dS
# rounded to bf16 for the MFMAs) against the exact fp64 chain rule.  Each
# rounding is at most 2^-8 relative; a gradient row is a sum of such terms,
# so its error is bounded relative to the row's own scale.  The bound is
# taken per row (one query's dQ, one key's dK or dV): an error confined to
# the rows of small magnitude cannot hide behind the largest row of the
# tensor.
GRAD_TOL = 1e-2


def assert_grad_close(g, g_ref, what: str):
    """Per row: max |g - g_ref| <= GRAD_TOL * max(1, max |g_ref| of that
    row) (fp64 numpy arrays, rows = every index but the last); an absolute
    floor of GRAD_TOL."""
    assert np.isfinite(g).all(), f"{what}: non-finite gradient"
    if not g.size:
        return
    g, g_ref = g.reshape(-1, g.shape[-1]), g_ref.reshape(-1, g_ref.shape[-1])
    scale = np.maximum(1.0, np.abs(g_ref).max(axis=1))
    err = np.abs(g - g_ref).max(axis=1)
    worst = int(np.argmax(err / scale))
    say(f"{what}: max|d| = {float(err.max()):.3e}; worst row {worst}: {float(err[worst]):.3e} against "
        f"{GRAD_TOL} x {float(scale[worst]):.3g} ({len(err)} rows)")
    assert (err <= GRAD_TOL * scale).all(), \
        f"{what}: row {worst}: max |g - g_ref| = {float(err[worst])} > {GRAD_TOL * float(scale[worst])}"

