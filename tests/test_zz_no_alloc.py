"""The allocation-free backward (ra_rank_share_bwd_noalloc) against the
backward that takes the caller's workspace (ra_rank_share_bwd), through the
C ABI: the same kernels on the same D values, so the gradients must agree
bit for bit.  Two calls in a row, the second on a smaller input, so that the
library's workspace carries the first call's values into the second."""
import pytest
import torch

from sequence_transformer_attention_amd import inputs
from sequence_transformer_attention_amd import ringattn as ra
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _backward_both(B, Hq, Hkv, d, N, P, r, causal, seed):
    nb = N // P
    x = inputs.draw_qkv(B, nb, N, Hq, Hkv, d, seed=seed)
    q, k, v = (x[t].to(DEV) for t in "qkv")
    O = torch.empty((B, nb, Hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, nb), dtype=torch.float32, device=DEV)
    ra.ra_rank_share(q, k, v, P, r, causal, O, lse)
    g = torch.Generator().manual_seed(seed + 1)
    dout = torch.randn((B, nb, Hq, d), generator=g).to(torch.bfloat16).to(DEV)

    def grads():
        return (torch.full((B, nb, Hq, d), float("nan"), device=DEV),
                torch.full(k.shape, float("nan"), device=DEV), torch.full(k.shape, float("nan"), device=DEV))

    dq0, dk0, dv0 = grads()
    ra.ra_rank_share_bwd_noalloc(q, k, v, O, lse, dout, P, r, causal, dq0, dk0, dv0)
    dq1, dk1, dv1 = grads()
    delta = torch.full((B, Hq, nb), float("nan"), device=DEV)
    ra.ra_rank_share_bwd(q, k, v, O, lse, dout, P, r, causal, dq1, dk1, dv1, delta)
    torch.cuda.synchronize()
    return (dq0, dk0, dv0), (dq1, dk1, dv1)


def test_noalloc_backward_equals_the_workspace_backward_twice():
    cases = [(1, 8, 2, 128, 2048, 4, 3, True, 31),   # GQA, last rank
             (2, 2, 1, 64, 512, 2, 1, True, 32)]     # then smaller: B = 2, d = 64
    for B, Hq, Hkv, d, N, P, r, causal, seed in cases:
        say(f"noalloc backward B{B} Hq{Hq} Hkv{Hkv} d{d} N{N} P{P} rank {r} causal={causal}")
        got, want = _backward_both(B, Hq, Hkv, d, N, P, r, causal, seed)
        for name, a, b in zip(("dQ", "dK", "dV"), got, want):
            assert torch.isfinite(a).all(), f"{name}: non-finite"
            assert torch.equal(a, b), f"{name}: max diff {float((a - b).abs().max())}"


def test_noalloc_backward_rejects_rows_beyond_its_workspace():
    # 2^20 + 2^12 query rows: rejected on the host, nothing launched
    B, Hq, d, nb = 1, 257, 64, 4096
    q = torch.empty((B, nb, Hq, d), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((B, nb, 1, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq, nb), device=DEV)
    dq = torch.empty((B, nb, Hq, d), device=DEV)
    dk = torch.empty((B, nb, 1, d), device=DEV)
    with pytest.raises(ra.RaError) as e:
        ra.ra_rank_share_bwd_noalloc(q, k, k, q, lse, q, 1, 0, True, dq, dk, dk)
    assert e.value.status == ra.RA_E_RANGE
