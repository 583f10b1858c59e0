"""Benchmark of one rank's share of ring attention on one MI355X.

A step is one ra_rank_share call: the local query block against all P key/value
blocks in ring order plus the normalisation, inputs resident in HBM.  Prints
one JSON line (rank 0, N = 1):

  value        algorithmic TFLOP/s of the whole step (4 * Nq * Nkv * d * Hq per
               block, 1/2 for the causal diagonal block, 0 for skipped blocks)
  roofline     the fused attention kernel against the bf16 dense MFMA peak,
               its average duration taken with HIP events around every launch
  cpu_baseline the fp64 oracle on a bounded sample of the same share's rows,
               timed on this host's cores, in the same unit

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "rank7_of_8_bf16_causal"
KERNEL_SOURCES = ["sequence_transformer_attention_amd/csrc/ra_kernels.hip",
                  "sequence_transformer_attention_amd/csrc/ra_plan.h",
                  "sequence_transformer_attention_amd/csrc/ra_launch.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the attention kernel from the committed rocprofv3
    counter runs, or None when absent or taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("kernel_hash") != kernel_hash():
        return None
    return e.get("bytes_per_launch")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x, O_gpu, lse_gpu, target_s: float):
    """Oracle (fp64 C, pthreads) on a seeded sample of the share's rows."""
    import numpy as np
    import torch

    import oracle

    threads = max(1, min(16, oracle.default_threads()))
    r = w.ranks[0]
    g = torch.Generator().manual_seed(w.seed + 77)

    def sample(n):
        b = torch.randint(w.B, (n,), generator=g)
        h = torch.randint(w.Hq, (n,), generator=g)
        i = torch.randint(w.nq, (n,), generator=g)
        return torch.stack([b, h, i], 1).numpy()

    def row_flops(rows):
        # visible keys of each row over the whole share (rank r owns positions r*nq..)
        pos = rows[:, 2] + r * w.nq
        vis = np.minimum(pos + 1, w.N) if w.causal else np.full(len(rows), w.N)
        return float(4.0 * w.d * vis.sum())

    q64 = x["q"].to(torch.float64).numpy()
    k64 = x["k"].to(torch.float64).numpy()
    v64 = x["v"].to(torch.float64).numpy()
    probe = sample(2 * threads)
    t0 = time.perf_counter()
    oracle.rank_share(q64, k64, v64, w.P, r, w.causal, rows=probe, nthreads=threads)
    dt = time.perf_counter() - t0
    n = int(max(2 * threads, min(200000, len(probe) * target_s / max(dt, 1e-3))))
    rows = sample(n)
    log(f"cpu baseline: oracle on {n} sampled rows with {threads} threads")
    t0 = time.perf_counter()
    o_ref, l_ref = oracle.rank_share(q64, k64, v64, w.P, r, w.causal, rows=rows, nthreads=threads)
    dt = time.perf_counter() - t0
    flops = row_flops(rows)
    rt = torch.as_tensor(rows, dtype=torch.long, device=O_gpu.device)
    o = O_gpu[rt[:, 0], rt[:, 2], rt[:, 1]].double().cpu().numpy()
    lse = lse_gpu[rt[:, 0], rt[:, 1], rt[:, 2]].double().cpu().numpy()
    # O is timed as bf16: allow the format's own rounding (half a bf16 ulp,
    # at most 2^-8 of the value rounded) on top of 1e-2
    excess = float((np.abs(o - o_ref) - (1e-2 + (np.abs(o_ref) + 1e-2) * 2.0 ** -8)).max())
    parity = {"rows": n, "max_abs_dO": float(np.abs(o - o_ref).max()),
              "max_abs_dLSE": float(np.abs(lse - l_ref).max()), "tol_O": "1e-2 + bf16 output rounding",
              "tol_LSE": 1e-3, "pass": bool(excess <= 0 and np.abs(lse - l_ref).max() <= 1e-3)}
    # every row of the share, at the same rate (extrapolated, not run)
    pos_all = np.arange(w.nq, dtype=np.float64) + r * w.nq
    vis_all = np.minimum(pos_all + 1, w.N) if w.causal else np.full(w.nq, float(w.N))
    share_flops = 4.0 * w.d * w.B * w.Hq * float(vis_all.sum())
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} random (b, h, i) rows of the same share, each against all its visible "
                      f"keys in ring order; {flops:.3e} FLOP in {dt:.2f} s (fp64, plain C)",
            "extrapolated_share_s": round(share_flops / (flops / dt), 1), "cpu": cpu_model()}
    return base, parity


def stepwise_and_finalize(w, r, qd, kd, vd, flop, ra, torch, reps: int = 5):
    """The same share as P ra_step calls (ring order, state in HBM) plus
    ra_finalize, and ra_finalize alone (HBM-bound: rows x (6d + 12) bytes for
    bf16 O: o_acc fp32, m and l read, O and LSE written).  Both timed with
    HIP events on the launch stream; the median of `reps` runs."""
    dev = qd.device
    nkv = w.N // w.P
    o_acc = torch.empty((w.B, w.nq, w.Hq, w.d), dtype=torch.float32, device=dev)
    m = torch.empty((w.B, w.Hq, w.nq), dtype=torch.float32, device=dev)
    l = torch.empty_like(m)
    odt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    O = torch.empty((w.B, w.nq, w.Hq, w.d), dtype=odt, device=dev)
    lse = torch.empty_like(m)
    blocks = [(ra.ra_ring_block(w.P, r, s), ) for s in range(w.P)]
    kb = [kd[:, j * nkv:(j + 1) * nkv] for (j,) in blocks]
    vb = [vd[:, j * nkv:(j + 1) * nkv] for (j,) in blocks]

    def stepwise():
        ra.ra_state_init(o_acc, m, l)
        for (j,), kk, vv in zip(blocks, kb, vb):
            ra.ra_step(qd, kk, vv, o_acc, m, l, r * nkv, j * nkv, w.causal)
        ra.ra_finalize(o_acc, l, m=m, o_out=O, lse_out=lse)

    def timed(fn):
        stream = torch.cuda.current_stream()
        fn()
        torch.cuda.synchronize()
        per = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1))
        return sorted(per)[len(per) // 2]

    st_ms = timed(stepwise)
    fin_ms = timed(lambda: ra.ra_finalize(o_acc, l, m=m, o_out=O, lse_out=lse))
    rows = w.B * w.Hq * w.nq
    fin_bytes = rows * (6 * w.d + 12) if w.dtype == "bf16" else rows * (8 * w.d + 12)
    log(f"stepwise {w.P} x ra_step + ra_finalize: {st_ms:.3f} ms -> {flop / st_ms / 1e9:.1f} TFLOP/s; "
        f"ra_finalize alone {fin_ms * 1e3:.1f} us -> {fin_bytes / fin_ms / 1e6:.0f} GB/s")
    return {"stepwise": {"ms": round(st_ms, 4), "tflops": round(flop / st_ms / 1e9, 3), "launches": w.P + 2},
            "finalize": {"us": round(fin_ms * 1e3, 2), "bytes": fin_bytes,
                         "GB/s": round(fin_bytes / fin_ms / 1e6, 1),
                         "frac_of_hbm": round(fin_bytes / fin_ms / 1e6 / HBM_PEAK_GBS, 4)}}


def load_balance(w, r, qd, kd, vd, mean_ms, ra, torch, reps: int = 5):
    """Causal load balance across the ring: the contiguous share of rank 0
    against the timed rank's, and the load-balanced (zigzag) share of the
    first and last rank, same shapes (the local Q has N/P rows either way)."""
    if not w.causal or w.P < 2 or w.N % (2 * w.P) != 0:
        return None
    O = torch.empty((w.B, w.nq, w.Hq, w.d), dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32,
                    device=qd.device)
    lse = torch.empty((w.B, w.Hq, w.nq), dtype=torch.float32, device=qd.device)

    def timed(fn):
        stream = torch.cuda.current_stream()
        fn()
        torch.cuda.synchronize()
        per = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1))
        return sorted(per)[len(per) // 2]

    c0 = timed(lambda: ra.ra_rank_share(qd, kd, vd, w.P, 0, True, O, lse))
    zz = {}
    for rr in (0, w.P - 1):
        ms = timed(lambda: ra.ra_rank_share_zigzag(qd, kd, vd, w.P, rr, True, O, lse))
        f = ra.ra_share_flops_zigzag(w.B, w.N, w.P, rr, w.Hq, w.d, True)
        zz[f"rank{rr}"] = {"ms": round(ms, 4), "tflops": round(f / ms / 1e9, 3)}
    slow_contig = max(c0, mean_ms)
    slow_zz = max(v["ms"] for v in zz.values())
    log(f"load balance: contiguous rank 0 {c0:.3f} ms, rank {r} {mean_ms:.3f} ms; zigzag "
        + ", ".join(f"{k} {v['ms']:.3f} ms ({v['tflops']:.0f} TFLOP/s)" for k, v in zz.items())
        + f"; slowest rank {slow_contig / slow_zz:.2f}x faster")
    return {"contiguous_ms": {"rank0": round(c0, 4), f"rank{r}": round(mean_ms, 4)}, "zigzag": zz,
            "slowest_rank_speedup": round(slow_contig / slow_zz, 3)}


def backward(w, r, qd, kd, vd, flop, ra, torch, reps: int = 5):
    """ra_rank_share_bwd on the same share (bf16 only): the algorithmic FLOP
    of the backward is 2.5x the forward's (five products per visible pair:
    S, dP, dV, dQ, dK, against two).  Under causal masking also
    ra_rank_share_zigzag_bwd of the first and last rank."""
    if w.dtype != "bf16":
        return None
    dev = qd.device
    O = torch.empty((w.B, w.nq, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, w.nq), dtype=torch.float32, device=dev)
    ra.ra_rank_share(qd, kd, vd, w.P, r, w.causal, O, lse)
    g = torch.Generator(device=dev).manual_seed(w.seed)
    dout = torch.randn((w.B, w.nq, w.Hq, w.d), generator=g, device=dev).to(torch.bfloat16)
    dq = torch.empty((w.B, w.nq, w.Hq, w.d), dtype=torch.float32, device=dev)
    dk = torch.empty(kd.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(kd.shape, dtype=torch.float32, device=dev)
    delta = torch.empty((w.B, w.Hq, w.nq), dtype=torch.float32, device=dev)

    def run():
        ra.ra_rank_share_bwd(qd, kd, vd, O, lse, dout, w.P, r, w.causal, dq, dk, dv, delta)

    stream = torch.cuda.current_stream()
    run()
    torch.cuda.synchronize()
    per = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1))
    ms = sorted(per)[len(per) // 2]
    bf = 2.5 * flop
    log(f"backward (prep + dQ + dK/dV): {ms:.3f} ms -> {bf / ms / 1e9:.1f} TFLOP/s "
        f"({100 * bf / ms / 1e9 / PEAK_BF16_TFLOPS:.1f} % of peak)")
    out = {"ms": round(ms, 4), "flop": bf, "tflops": round(bf / ms / 1e9, 3),
           "frac_of_peak": round(bf / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
    # the load-balanced shares' backward (first and last rank), same sizes
    if w.causal and w.N % (2 * w.P) == 0 and w.P > 1:
        # (timing only: the local Q of the timed share stands in for the
        # load-balanced rows; the sizes are the same)
        zz = {}
        qz = qd
        for rz in (0, w.P - 1):
            ra.ra_rank_share_zigzag(qz, kd, vd, w.P, rz, w.causal, O, lse)

            def runz():
                ra.ra_rank_share_zigzag_bwd(qz, kd, vd, O, lse, dout, w.P, rz, w.causal, dq, dk, dv, delta)

            runz()
            torch.cuda.synchronize()
            perz = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                runz()
                e1.record(stream)
                torch.cuda.synchronize()
                perz.append(e0.elapsed_time(e1))
            mz = sorted(perz)[len(perz) // 2]
            fz = 2.5 * ra.ra_share_flops_zigzag(w.B, w.N, w.P, rz, w.Hq, w.d, w.causal)
            zz[f"rank{rz}"] = {"ms": round(mz, 4), "tflops": round(fz / mz / 1e9, 3)}
        log("load-balanced backward: " + ", ".join(f"{k} {v['ms']:.3f} ms ({v['tflops']:.0f} TFLOP/s)"
                                                   for k, v in zz.items()))
        out["zigzag"] = zz
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the rank share only (no stepwise, load-balance or backward measurements), "
                         "so that a profiler's per-kernel summary covers the timed launches alone")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: libringattn has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    from sequence_transformer_attention_amd import inputs, workloads
    from sequence_transformer_attention_amd import ringattn as ra

    dev = torch.device("cuda:0")
    if args.copy_calib_mib:
        n = args.copy_calib_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": n * 4, "launches": 5}))
        return 0

    w = workloads.BY_NAME[args.workload]
    r = w.ranks[0]
    log(f"workload {w.name}: drawing inputs")
    x = inputs.workload_inputs(w)
    q = inputs.local_q(w, x["q"], r).contiguous()
    xq = dict(x, q=q)
    qd, kd, vd = (t.to(dev) for t in (q, x["k"], x["v"]))
    odt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    O = torch.empty((w.B, w.nq, w.Hq, w.d), dtype=odt, device=dev)
    lse = torch.empty((w.B, w.Hq, w.nq), dtype=torch.float32, device=dev)
    flop = ra.ra_share_flops(w.B, w.N, w.P, r, w.Hq, w.d, w.causal)

    def step():
        ra.ra_rank_share(qd, kd, vd, w.P, r, w.causal, O, lse)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(a.elapsed_time(b) for a, b in ev)
    mean_ms = sum(per) / len(per)
    ms_per_step = wall * 1e3 / args.steps
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (mean_ms * 1e-3) / 1e12
    log(f"{w.name}: {ms_per_step:.3f} ms/step, kernel mean {mean_ms:.3f} ms "
        f"(median {per[len(per) // 2]:.3f}, min {per[0]:.3f}) -> {achieved:.1f} TFLOP/s")

    if args.no_extras:
        side, balance, bwd = {"stepwise": None, "finalize": None}, None, None
    else:
        side = stepwise_and_finalize(w, r, qd, kd, vd, flop, ra, torch)
        balance = load_balance(w, r, qd, kd, vd, mean_ms, ra, torch)
        bwd = backward(w, r, qd, kd, vd, flop, ra, torch)

    out = {
        "metric": "rank-share ring-attention TFLOP/s (bf16, causal) and % of MFMA bf16 peak",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "N": w.N,
                   "P": w.P, "rank": r, "causal": w.causal, "q_block": w.nq, "input": w.dist,
                   "seed": w.seed},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "flop_per_step": flop,
        "kernel_ms": {"mean": round(mean_ms, 4), "median": round(per[len(per) // 2], 4),
                      "min": round(per[0], 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(w.name)},
        "inputs_sha256": {t: inputs.sha256(xq[t])[:16] for t in "qkv"},
        "stepwise": side["stepwise"],
        "finalize": side["finalize"],
        "load_balance": balance,
        "backward": bwd,
    }
    if not args.no_cpu_baseline:
        base, parity = cpu_baseline(w, xq, O, lse, args.cpu_seconds)
        out["cpu_baseline"] = base
        out["parity_sample"] = parity
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
