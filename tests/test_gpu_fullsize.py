"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The oracle computes a seeded sample of rows one by one: every row of the first
and last query tiles of the first and last head, plus one random row per
(query tile, head).  Each sampled row attends to all of its key blocks, so
every block, the causal diagonal and the fully visible path are exercised.
"""
import pytest
import torch

import oracle
from sequence_transformer_attention_amd import inputs, workloads
from tests.gpu_util import (assert_close, assert_grad_close, backward_gpu, gather, oracle_threads, rank_share_gpu,
                            padded_backward_gpu, padded_gpu, say, stepwise_gpu, zigzag_backward_gpu, zigzag_gpu,
                            zigzag_rows)

pytestmark = pytest.mark.gpu


def kv_heads(hkv: int, n: int, g: torch.Generator) -> torch.Tensor:
    """n kv-head indices spread over four heads: the first, the last and two
    seeded others (the oracle's backward costs a full forward of every kv
    head a sampled dK/dV row belongs to, about 2 s per head here)."""
    pick = torch.unique(torch.cat([torch.tensor([0, hkv - 1]), torch.randint(0, hkv, (2,), generator=g)]))
    return pick[torch.arange(n) % len(pick)]

FULL = [workloads.RANK7_BF16, workloads.GQA_BF16, workloads.ULYSSES_BF16, workloads.STRESS_BF16]


@pytest.mark.parametrize("w", FULL, ids=[w.name for w in FULL])
def test_full_size_sampled_rows(w):
    say(f"{w.name}: drawing inputs")
    x = inputs.workload_inputs(w)
    d = {k: t.to("cuda") for k, t in x.items()}
    r = w.ranks[0]
    say(f"{w.name}: fused rank share (bf16 O, as timed; fp32 O)")
    O, lse = rank_share_gpu(d["q"], d["k"], d["v"], w.P, r, w.causal, torch.bfloat16)
    O32, lse32 = rank_share_gpu(d["q"], d["k"], d["v"], w.P, r, w.causal, torch.float32)
    say(f"{w.name}: stepwise ({w.P} steps + finalize)")
    Os, lses = stepwise_gpu(d["q"], d["k"], d["v"], w.P, r, w.causal, torch.float32)
    torch.cuda.synchronize()
    rows = inputs.sample_rows(w.B, w.Hq, w.nq, w.seed).numpy()
    say(f"{w.name}: oracle on {len(rows)} rows")
    o_ref, l_ref = oracle.rank_share(x["q"], x["k"], x["v"], w.P, r, w.causal, rows=rows,
                                     nthreads=oracle_threads())
    assert_close(*gather(O, lse, rows), o_ref, l_ref, "bf16", f"{w.name} fused bf16 O", out_bf16=True)
    assert_close(*gather(O32, lse32, rows), o_ref, l_ref, "bf16", f"{w.name} fused fp32 O")
    assert_close(*gather(Os, lses, rows), o_ref, l_ref, "bf16", f"{w.name} stepwise")


def test_full_size_zigzag_sampled_rows():
    """Load-balanced shares of the rank-7-of-8 shape (N 32768, 32 heads, d 128),
    first and last rank, bf16 O as timed."""
    w = workloads.RANK7_BF16
    say("zigzag full size: drawing inputs (whole-sequence Q)")
    x = inputs.draw_qkv(w.B, w.N, w.N, w.Hq, w.Hkv, w.d, w.seed + 100, w.dtype, w.dist)
    k, v = x["k"].to("cuda"), x["v"].to("cuda")
    for r in (0, w.P - 1):
        pos = zigzag_rows(w.N, w.P, r)
        ql = x["q"][:, pos].contiguous()
        say(f"zigzag full size rank {r}")
        O, lse = zigzag_gpu(ql.to("cuda"), k, v, w.P, r, w.causal, torch.bfloat16)
        torch.cuda.synchronize()
        rows = inputs.sample_rows(w.B, w.Hq, len(pos), w.seed + r).numpy()
        say(f"zigzag full size rank {r}: oracle on {len(rows)} rows")
        o_ref, l_ref = oracle.rank_share_zigzag(ql, x["k"], x["v"], w.P, r, w.causal, rows=rows,
                                                nthreads=oracle_threads())
        assert_close(*gather(O, lse, rows), o_ref, l_ref, "bf16", f"zigzag rank {r} bf16 O", out_bf16=True)




def test_full_size_padded_sampled_rows():
    """Rank-7-of-8 shape (N 32768, 32 heads, d 128) holding 32768 - 777 real
    tokens: the last rank's block ends in 777 NaN padding keys."""
    w = workloads.RANK7_BF16
    n_valid = w.N - 777
    say("padded full size: drawing inputs")
    x = inputs.workload_inputs(w)
    x["k"][:, n_valid:] = float("nan")
    x["v"][:, n_valid:] = float("nan")
    d = {k: t.to("cuda") for k, t in x.items()}
    r = w.ranks[0]
    O, lse = padded_gpu(d["q"], d["k"], d["v"], w.P, r, w.causal, n_valid, torch.bfloat16)
    torch.cuda.synchronize()
    rows = inputs.sample_rows(w.B, w.Hq, w.nq, w.seed + 7).numpy()
    say(f"padded full size rank {r}: oracle on {len(rows)} rows")
    o_ref, l_ref = oracle.rank_share_padded(x["q"], x["k"], x["v"], w.P, r, w.causal, n_valid, rows=rows,
                                            nthreads=oracle_threads())
    assert_close(*gather(O, lse, rows), o_ref, l_ref, "bf16", f"padded rank {r} bf16 O", out_bf16=True)


def test_full_size_backward_sampled_rows():
    """Backward of the rank-7-of-8 share (N 32768, 32 heads, d 128): sampled dQ
    rows, and dK/dV rows of four kv heads (first, last, two seeded) over the whole
    sequence."""
    w = workloads.RANK7_BF16
    x = inputs.workload_inputs(w)
    d = {k: t.to("cuda") for k, t in x.items()}
    r = w.ranks[0]
    dout = torch.randn(w.B, w.nq, w.Hq, w.d, generator=torch.Generator().manual_seed(w.seed)).to(torch.bfloat16)
    say("backward full size: forward + backward on the GPU")
    dq, dk, dv = backward_gpu(d["q"], d["k"], d["v"], w.P, r, w.causal, dout.to("cuda"))
    torch.cuda.synchronize()
    qrows = inputs.sample_rows(w.B, w.Hq, w.nq, w.seed).numpy()[:512]
    g = torch.Generator().manual_seed(w.seed + 1)
    krows = torch.stack([torch.zeros(256, dtype=torch.long), kv_heads(w.Hkv, 256, g),
                         torch.randint(0, w.N, (256,), generator=g)], 1).numpy()
    say(f"backward full size: oracle on {len(qrows)} dQ rows and {len(krows)} dK/dV rows")
    dq_r, dk_r, dv_r = oracle.rank_share_bwd(x["q"], x["k"], x["v"], dout, w.P, r, w.causal, qrows=qrows,
                                             krows=krows, nthreads=oracle_threads())
    qi = torch.as_tensor(qrows)
    ki = torch.as_tensor(krows)
    assert_grad_close(dq[qi[:, 0], qi[:, 2], qi[:, 1]].double().cpu().numpy(), dq_r, "dQ full size")
    assert_grad_close(dk[ki[:, 0], ki[:, 2], ki[:, 1]].double().cpu().numpy(), dk_r, "dK full size")
    assert_grad_close(dv[ki[:, 0], ki[:, 2], ki[:, 1]].double().cpu().numpy(), dv_r, "dV full size")


def test_full_size_zigzag_backward_sampled_rows():
    """Backward of the last rank's load-balanced share at the rank-7-of-8 size
    (N 32768, 32 heads, d 128): sampled dQ rows of both chunks and dK/dV rows
    of four kv heads (first, last, two seeded) over the whole sequence."""
    w = workloads.RANK7_BF16
    r = w.P - 1
    x = inputs.draw_qkv(w.B, w.N, w.N, w.Hq, w.Hkv, w.d, w.seed + 200, w.dtype, w.dist)
    pos = zigzag_rows(w.N, w.P, r)
    ql = x["q"][:, pos].contiguous()
    nq = len(pos)
    dout = torch.randn(w.B, nq, w.Hq, w.d, generator=torch.Generator().manual_seed(w.seed + 3)).to(torch.bfloat16)
    say("zigzag backward full size: forward + backward on the GPU")
    dq, dk, dv = zigzag_backward_gpu(ql.to("cuda"), x["k"].to("cuda"), x["v"].to("cuda"), w.P, r, w.causal,
                                     dout.to("cuda"))
    torch.cuda.synchronize()
    qrows = inputs.sample_rows(w.B, w.Hq, nq, w.seed + 4).numpy()[:512]
    g = torch.Generator().manual_seed(w.seed + 5)
    krows = torch.stack([torch.zeros(256, dtype=torch.long), kv_heads(w.Hkv, 256, g),
                         torch.randint(0, w.N, (256,), generator=g)], 1).numpy()
    say(f"zigzag backward full size: oracle on {len(qrows)} dQ rows and {len(krows)} dK/dV rows")
    dq_r, dk_r, dv_r = oracle.rank_share_bwd(ql, x["k"], x["v"], dout, w.P, r, w.causal, qrows=qrows, krows=krows,
                                             nthreads=oracle_threads(), zigzag=True)
    qi = torch.as_tensor(qrows)
    ki = torch.as_tensor(krows)
    assert_grad_close(dq[qi[:, 0], qi[:, 2], qi[:, 1]].double().cpu().numpy(), dq_r, "zigzag dQ full size")
    assert_grad_close(dk[ki[:, 0], ki[:, 2], ki[:, 1]].double().cpu().numpy(), dk_r, "zigzag dK full size")
    assert_grad_close(dv[ki[:, 0], ki[:, 2], ki[:, 1]].double().cpu().numpy(), dv_r, "zigzag dV full size")


def test_full_size_padded_backward_sampled_rows():
    """Backward of the rank-7-of-8 share holding 32768 - 777 real tokens (NaN
    padding keys): sampled dQ rows, dK/dV rows of four kv heads over the
    whole sequence, and exact zeros on every padding key row."""
    w = workloads.RANK7_BF16
    n_valid = w.N - 777
    x = inputs.workload_inputs(w)
    x["k"][:, n_valid:] = float("nan")
    x["v"][:, n_valid:] = float("nan")
    d = {k: t.to("cuda") for k, t in x.items()}
    r = w.ranks[0]
    dout = torch.randn(w.B, w.nq, w.Hq, w.d, generator=torch.Generator().manual_seed(w.seed + 9)).to(torch.bfloat16)
    say("padded backward full size: forward + backward on the GPU")
    dq, dk, dv = padded_backward_gpu(d["q"], d["k"], d["v"], w.P, r, w.causal, n_valid, dout.to("cuda"))
    torch.cuda.synchronize()
    assert float(dk[:, n_valid:].abs().max()) == 0.0 and float(dv[:, n_valid:].abs().max()) == 0.0
    qrows = inputs.sample_rows(w.B, w.Hq, w.nq, w.seed + 10).numpy()[:512]
    g = torch.Generator().manual_seed(w.seed + 11)
    krows = torch.stack([torch.zeros(256, dtype=torch.long), kv_heads(w.Hkv, 256, g),
                         torch.randint(0, n_valid, (256,), generator=g)], 1).numpy()
    say(f"padded backward full size: oracle on {len(qrows)} dQ rows and {len(krows)} dK/dV rows")
    dq_r, dk_r, dv_r = oracle.rank_share_bwd(x["q"], x["k"], x["v"], dout, w.P, r, w.causal, qrows=qrows,
                                             krows=krows, nthreads=oracle_threads(), n_valid=n_valid)
    qi = torch.as_tensor(qrows)
    ki = torch.as_tensor(krows)
    assert_grad_close(dq[qi[:, 0], qi[:, 2], qi[:, 1]].double().cpu().numpy(), dq_r, "padded dQ full size")
    assert_grad_close(dk[ki[:, 0], ki[:, 2], ki[:, 1]].double().cpu().numpy(), dk_r, "padded dK full size")
    assert_grad_close(dv[ki[:, 0], ki[:, 2], ki[:, 1]].double().cpu().numpy(), dv_r, "padded dV full size")
