"""Benchmark of one rank's share of ring attention on one MI355X.

A step is one ra_rank_share call: the local query block against all P key/value
blocks in ring order plus the normalisation, inputs resident in HBM.  Prints
one JSON line (rank 0, N = 1):

  value        algorithmic TFLOP/s of the whole step on the headline workload
               (4 * Nq * Nkv * d * Hq per block, 1/2 for the causal diagonal
               block, 0 for skipped blocks), wall clock over the timed steps
  roofline     the fused attention kernel against the bf16 dense MFMA peak,
               its average duration taken with HIP events around every launch
  configs      every workload (tiny fp32, rank 7 of 8, GQA, Ulysses, stress):
               kernel time, TFLOP/s, fraction of its peak, a parity sample
               against the fp64 oracle and the input hashes
  clock        the GPU's engine clock under this load (SMI), if readable
  finalize, merge, stepwise, load_balance, backward
               the other entry points on the headline workload
  cpu_baseline the fp64 oracle on a bounded sample of the headline share's
               rows, timed on every core this process may run on

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector (the fp32 path is VALU FMA)
HBM_PEAK_GBS = 8000.0
WARM_SECONDS = 0.3          # untimed back-to-back launches before the warm-up steps
LLC_BYTES = 256 << 20       # last-level (Infinity) cache: working sets above it stream from HBM
DEFAULT_WORKLOAD = "rank7_of_8_bf16_causal"
METRIC = "rank-share ring-attention TFLOP/s (bf16, causal) and % of MFMA bf16 peak"
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


# ------------------------------------------------------------------ timing
def per_launch_ms(torch, fn, reps: int):
    """HIP events around every launch on the current stream; per-launch ms."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def loop_ms(torch, fns, reps: int):
    """Average ms per launch of reps back-to-back launches (fns[i % len(fns)]),
    HIP events around the loop on the current stream."""
    stream = torch.cuda.current_stream()
    for f in fns[:2]:
        f()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(reps):
        fns[i % len(fns)]()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def warm(torch, fn, seconds: float = 0.3):
    """Back-to-back launches for about `seconds`, so that the clocks have
    left the idle state a CPU-side phase (input draws, the oracle) leaves
    them in before anything is timed."""
    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(5):
            fn()
        n += 5
        torch.cuda.synchronize()
    return n


def summary(per):
    s = sorted(per)
    return {"mean": round(sum(s) / len(s), 4), "median": round(s[len(s) // 2], 4), "min": round(s[0], 4)}


# ------------------------------------------------------------------ clock
class ClockSampler:
    """The engine clock and socket power read through amdsmi while the GPU
    runs; None when amdsmi is missing or the device cannot be matched."""

    def __init__(self, torch):
        self.handle, self.amdsmi, self.samples, self.why = None, None, [], None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            props = torch.cuda.get_device_properties(0)
            bus = getattr(props, "pci_bus_id", None)
            pick = None
            for h in handles:
                try:
                    bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                    if bus is not None and int(bdf.split(":")[1], 16) == int(bus):
                        pick = h
                except Exception:
                    pass
            if pick is None and len(handles) == 1:
                pick = handles[0]
            if pick is None:
                self.why = f"{len(handles)} SMI devices, none matched to cuda:0"
                return
            self.handle, self.amdsmi = pick, amdsmi
        except Exception as e:  # no SMI on this host
            self.why = f"amdsmi unavailable ({type(e).__name__})"

    def read(self):
        """(engine clock MHz, per-XCD clocks, socket power W, gfx activity %)."""
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)

        def num(v):
            return v if isinstance(v, (int, float)) and 0 <= v < 100000 else None

        xcd = [c for c in (m.get("current_gfxclks") or []) if num(c)]
        return num(m.get("current_gfxclk")), tuple(xcd), num(m.get("current_socket_power")), \
            num(m.get("average_gfx_activity"))

    def sample_during(self, torch, fn, seconds: float):
        """Back-to-back launches of fn for about `seconds` while a thread reads
        the metrics every 20 ms.  The SMI refreshes them about once a
        second: only fresh readings (not equal to the previous one) taken
        while the engine reports itself busy count."""
        if self.handle is None:
            return {"recorded": False, "why": self.why}
        stop = threading.Event()
        got = []

        def loop():
            last = None
            while not stop.is_set():
                try:
                    r = self.read()
                    if r != last:
                        got.append(r)
                    last = r
                except Exception:
                    pass
                time.sleep(0.02)

        th = threading.Thread(target=loop, daemon=True)
        t0 = time.perf_counter()
        th.start()
        n = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(20):
                fn()
            n += 20
            torch.cuda.synchronize()
        stop.set()
        th.join()
        busy = [g for g in got if g[0] and g[3] is not None and g[3] >= 50]
        if not busy:
            return {"recorded": False, "why": f"no busy reading among {len(got)} SMI updates"}
        clks = [g[0] for g in busy]
        xcd = [c for g in busy for c in g[1]]
        pws = [g[2] for g in busy if g[2]]
        out = {"recorded": True,
               "source": f"amdsmi gpu metrics (current_gfxclk, current_gfxclks, current_socket_power), "
                         f"{len(busy)} fresh readings with gfx activity >= 50 % during {n} back-to-back launches "
                         f"of the timed kernel ({seconds:.1f} s)",
               "gfxclk_mhz": {"median": statistics.median(clks), "min": min(clks), "max": max(clks)},
               "spec_mhz": 2400}
        if xcd:
            out["xcd_gfxclk_mhz"] = {"median": statistics.median(xcd), "min": min(xcd), "max": max(xcd)}
        if pws:
            out["socket_power_w"] = {"median": statistics.median(pws), "max": max(pws)}
        return out


# ------------------------------------------------------------------ parity
def parity_rows(w, nq_local, seed, n_random=64):
    """Rows (b, h, i) to compare with the oracle: the first 32 local rows of
    head 0 and the last 32 of head Hq - 1, plus n_random seeded rows."""
    import numpy as np
    import torch
    rows = set()
    for i in range(min(32, nq_local)):
        rows.add((0, 0, i))
        rows.add((w.B - 1, w.Hq - 1, nq_local - 1 - i))
    g = torch.Generator().manual_seed(seed)
    for _ in range(n_random):
        rows.add((int(torch.randint(w.B, (1,), generator=g)), int(torch.randint(w.Hq, (1,), generator=g)),
                  int(torch.randint(nq_local, (1,), generator=g))))
    return np.array(sorted(rows), dtype=np.int64)


def compare(O, lse, rows, o_ref, l_ref, tol_o, tol_l, out_bf16):
    """max |dO|, max |dLSE| on the rows; a bf16 O may also differ by its own
    rounding (half an ulp, at most 2^-8 of the value rounded)."""
    import numpy as np
    import torch
    rt = torch.as_tensor(rows, dtype=torch.long, device=O.device)
    o = O[rt[:, 0], rt[:, 2], rt[:, 1]].double().cpu().numpy()
    lg = lse[rt[:, 0], rt[:, 1], rt[:, 2]].double().cpu().numpy()
    allow = tol_o + ((np.abs(o_ref) + tol_o) * 2.0 ** -8 if out_bf16 else 0.0)
    eo, el = float(np.abs(o - o_ref).max()), float(np.abs(lg - l_ref).max())
    ok = bool(np.isfinite(o).all() and (np.abs(o - o_ref) <= allow).all() and el <= tol_l)
    return {"rows": int(len(rows)), "max_abs_dO": eo, "max_abs_dLSE": el,
            "tol_O": f"{tol_o}" + (" + bf16 output rounding" if out_bf16 else ""), "tol_LSE": tol_l, "pass": ok}


# ------------------------------------------------------------------ workloads
def run_config(w, steps, warmup, torch, ra, inputs, oracle, threads):
    """One workload: every rank in w.ranks per step; kernel ms from HIP events,
    TFLOP/s, fraction of the peak of its dtype, parity sample, input hashes."""
    dev = torch.device("cuda:0")
    log(f"{w.name}: drawing inputs")
    x = inputs.workload_inputs(w)
    kd, vd = x["k"].to(dev), x["v"].to(dev)
    qs = {r: inputs.local_q(w, x["q"], r).contiguous() for r in w.ranks}
    qd = {r: t.to(dev) for r, t in qs.items()}
    odt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    O = {r: torch.empty((w.B, w.nq, w.Hq, w.d), dtype=odt, device=dev) for r in w.ranks}
    lse = {r: torch.empty((w.B, w.Hq, w.nq), dtype=torch.float32, device=dev) for r in w.ranks}
    flop = sum(ra.ra_share_flops(w.B, w.N, w.P, r, w.Hq, w.d, w.causal) for r in w.ranks)

    def step():
        for r in w.ranks:
            ra.ra_rank_share(qd[r], kd, vd, w.P, r, w.causal, O[r], lse[r])

    for _ in range(warmup):
        step()
    warm(torch, step)
    per = per_launch_ms(torch, step, steps)
    ms = summary(per)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    tflops = flop / ms["mean"] / 1e9
    # parity: every row of every rank for the tiny workload, a sample otherwise
    tol = (1e-2, 1e-3) if w.dtype == "bf16" else (1e-5, 1e-5)
    checks = []
    for r in w.ranks:
        rows = oracle.all_rows(w.B, w.Hq, w.nq) if w.N <= 4096 else parity_rows(w, w.nq, w.seed + 500 + r)
        o_ref, l_ref = oracle.rank_share(qs[r], x["k"], x["v"], w.P, r, w.causal, rows=rows, nthreads=threads)
        checks.append(compare(O[r], lse[r], rows, o_ref, l_ref, *tol, out_bf16=odt == torch.bfloat16))
    par = {"rows": sum(c["rows"] for c in checks), "max_abs_dO": max(c["max_abs_dO"] for c in checks),
           "max_abs_dLSE": max(c["max_abs_dLSE"] for c in checks), "tol_O": checks[0]["tol_O"],
           "tol_LSE": tol[1], "pass": all(c["pass"] for c in checks)}
    log(f"{w.name}: kernel mean {ms['mean']:.4f} ms -> {tflops:.1f} TFLOP/s ({100 * tflops / peak:.1f} % of "
        f"{'bf16 MFMA' if w.dtype == 'bf16' else 'fp32 vector'} peak); parity {par['pass']} on {par['rows']} rows")
    entry = {"dtype": w.dtype, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "N": w.N, "P": w.P,
             "ranks": list(w.ranks), "causal": w.causal, "input": w.dist, "seed": w.seed,
             "flop": flop, "kernel_ms": ms, "steps": steps, "tflops": round(tflops, 3),
             "peak": peak, "frac": round(tflops / peak, 4), "parity_sample": par,
             "inputs_sha256": {"q": inputs.sha256(x["q"])[:16], "k": inputs.sha256(x["k"])[:16],
                               "v": inputs.sha256(x["v"])[:16]}}
    del x, kd, vd, qd, O, lse
    torch.cuda.empty_cache()
    return entry


def stepwise(w, r, qd, kd, vd, flop, ra, torch, reps: int = 5):
    """The same share as P ra_step calls (ring order, state in HBM) plus
    ra_state_init and ra_finalize: median of reps runs, HIP events."""
    dev = qd.device
    nkv = w.N // w.P
    o_acc = torch.empty((w.B, w.nq, w.Hq, w.d), dtype=torch.float32, device=dev)
    m = torch.empty((w.B, w.Hq, w.nq), dtype=torch.float32, device=dev)
    l = torch.empty_like(m)
    O = torch.empty((w.B, w.nq, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty_like(m)
    blocks = [ra.ra_ring_block(w.P, r, s) for s in range(w.P)]

    def run():
        ra.ra_state_init(o_acc, m, l)
        for j in blocks:
            ra.ra_step(qd, kd[:, j * nkv:(j + 1) * nkv], vd[:, j * nkv:(j + 1) * nkv], o_acc, m, l, r * nkv,
                       j * nkv, w.causal)
        ra.ra_finalize(o_acc, l, m=m, o_out=O, lse_out=lse)

    warm(torch, run)
    ms = sorted(per_launch_ms(torch, run, reps))[reps // 2]
    log(f"stepwise {w.P} x ra_step + init + finalize: {ms:.3f} ms -> {flop / ms / 1e9:.1f} TFLOP/s")
    return {"ms": round(ms, 4), "tflops": round(flop / ms / 1e9, 3), "launches": w.P + 2}


def state_kernels(w, torch, ra):
    """ra_finalize and ra_merge on the headline share's running state
    (B * Hq * Nq rows of d fp32).  Algorithmic bytes per row: finalize
    6d + 12 (o_acc, m, l read; bf16 O and LSE written), merge 3 (4d + 8)
    (two states read, one written).  Two rates each, as the average of 60
    back-to-back launches between HIP events:
      pipeline  the same buffers every launch, as after the step that wrote
                them (the state is resident in the 256 MB last-level cache)
      hbm       rotating over buffer sets whose total exceeds that cache, so
                every launch streams from HBM
    and, for reference, torch's device copy of one state's o (8d bytes per
    row) under both conditions."""
    dev = torch.device("cuda:0")
    shape, rshape = (w.B, w.nq, w.Hq, w.d), (w.B, w.Hq, w.nq)
    rows = w.B * w.Hq * w.nq
    set_bytes = rows * (2 * (4 * w.d + 8) + 2 * w.d + 4)
    nset = max(2, -(-2 * LLC_BYTES // set_bytes))
    g = torch.Generator(device=dev).manual_seed(11)
    sets = []
    for _ in range(nset):
        sets.append({"o": torch.randn(shape, generator=g, device=dev), "m": torch.randn(rshape, generator=g, device=dev),
                     "l": torch.rand(rshape, generator=g, device=dev) + 0.5,
                     "ob": torch.randn(shape, generator=g, device=dev), "mb": torch.randn(rshape, generator=g, device=dev),
                     "lb": torch.rand(rshape, generator=g, device=dev) + 0.5,
                     "O": torch.empty(shape, dtype=torch.bfloat16, device=dev),
                     "lse": torch.empty(rshape, device=dev)})

    def fin(s):
        return lambda: ra.ra_finalize(s["o"], s["l"], m=s["m"], o_out=s["O"], lse_out=s["lse"])

    def mer(s):
        return lambda: ra.ra_merge(s["o"], s["m"], s["l"], s["ob"], s["mb"], s["lb"])

    def cp(s):
        return lambda: s["ob"].copy_(s["o"])

    out = {}
    for name, mk, nbytes in (("finalize", fin, rows * (6 * w.d + 12)), ("merge", mer, rows * 3 * (4 * w.d + 8)),
                             ("copy_reference", cp, rows * 8 * w.d)):
        warm(torch, mk(sets[0]), 0.1)
        hot = loop_ms(torch, [mk(sets[0])], 60)
        cold = loop_ms(torch, [mk(s) for s in sets], 60)
        e = {"bytes": nbytes,
             "pipeline": {"us": round(hot * 1e3, 2), "GB/s": round(nbytes / hot / 1e6, 1),
                          "frac_of_hbm": round(nbytes / hot / 1e6 / HBM_PEAK_GBS, 4)},
             "hbm": {"us": round(cold * 1e3, 2), "GB/s": round(nbytes / cold / 1e6, 1),
                     "frac_of_hbm": round(nbytes / cold / 1e6 / HBM_PEAK_GBS, 4), "buffer_sets": nset}}
        out[name] = e
        log(f"{name}: {e['pipeline']['GB/s']:.0f} GB/s in the pipeline, {e['hbm']['GB/s']:.0f} GB/s from HBM "
            f"({nbytes / 1e6:.1f} MB per launch)")
    del sets
    torch.cuda.empty_cache()
    return out


def load_balance(w, r, qd, kd, vd, mean_ms, ra, torch, inputs, oracle, threads, reps: int = 5):
    """Causal load balance across the ring: the contiguous share of rank 0
    against the timed rank's, and the load-balanced share (chunks r and
    2P-1-r of 2P) of the first and last rank on their own rows of a
    whole-sequence Q (drawn with another seed, with its own K and V), each
    with a parity sample.  Returns the object and the zigzag inputs for the
    backward."""
    if not w.causal or w.P < 2 or w.N % (2 * w.P) != 0:
        return None, None
    dev = qd.device
    O = torch.empty((w.B, w.nq, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, w.nq), dtype=torch.float32, device=dev)
    warm(torch, lambda: ra.ra_rank_share(qd, kd, vd, w.P, 0, True, O, lse))
    c0 = sorted(per_launch_ms(torch, lambda: ra.ra_rank_share(qd, kd, vd, w.P, 0, True, O, lse), reps))[reps // 2]
    log(f"{w.name} load balance: drawing a whole-sequence Q")
    x = inputs.draw_qkv(w.B, w.N, w.N, w.Hq, w.Hkv, w.d, w.seed + 100, w.dtype, w.dist)
    kz, vz = x["k"].to(dev), x["v"].to(dev)
    c = w.N // (2 * w.P)
    zz, zin = {}, {}
    for rr in (0, w.P - 1):
        pos = list(range(rr * c, (rr + 1) * c)) + list(range((2 * w.P - 1 - rr) * c, (2 * w.P - rr) * c))
        ql = x["q"][:, pos].contiguous()
        qz = ql.to(dev)
        Oz = torch.empty((w.B, 2 * c, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
        lz = torch.empty((w.B, w.Hq, 2 * c), dtype=torch.float32, device=dev)
        run = lambda: ra.ra_rank_share_zigzag(qz, kz, vz, w.P, rr, True, Oz, lz)  # noqa: E731
        warm(torch, run)
        ms = sorted(per_launch_ms(torch, run, reps))[reps // 2]
        f = ra.ra_share_flops_zigzag(w.B, w.N, w.P, rr, w.Hq, w.d, True)
        rows = parity_rows(w, 2 * c, w.seed + 700 + rr, n_random=32)
        o_ref, l_ref = oracle.rank_share_zigzag(ql, x["k"], x["v"], w.P, rr, True, rows=rows, nthreads=threads)
        par = compare(Oz, lz, rows, o_ref, l_ref, 1e-2, 1e-3, True)
        zz[f"rank{rr}"] = {"ms": round(ms, 4), "tflops": round(f / ms / 1e9, 3), "parity_sample": par}
        zin[rr] = (qz, Oz, lz)
    slow_contig = max(c0, mean_ms)
    slow_zz = max(v["ms"] for v in zz.values())
    log(f"load balance: contiguous rank 0 {c0:.3f} ms, rank {r} {mean_ms:.3f} ms; load-balanced "
        + ", ".join(f"{k} {v['ms']:.3f} ms ({v['tflops']:.0f} TFLOP/s, parity {v['parity_sample']['pass']})"
                    for k, v in zz.items()) + f"; slowest rank {slow_contig / slow_zz:.2f}x faster")
    out = {"contiguous_ms": {"rank0": round(c0, 4), f"rank{r}": round(mean_ms, 4)}, "zigzag": zz,
           "zigzag_inputs": f"whole-sequence Q, K, V drawn with seed {w.seed + 100}; each rank's own rows",
           "slowest_rank_speedup": round(slow_contig / slow_zz, 3)}
    return out, (kz, vz, zin)


def backward(w, r, qd, kd, vd, flop, ra, torch, zig, reps: int = 5):
    """ra_rank_share_bwd on the same share (bf16 only): the algorithmic FLOP
    of the backward is 2.5x the forward's (five products per visible pair:
    S, dP, dV, dQ, dK, against two).  With the load-balanced inputs also
    ra_rank_share_zigzag_bwd of the first and last rank on their own rows,
    O and LSE."""
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

    warm(torch, run)
    ms = sorted(per_launch_ms(torch, run, reps))[reps // 2]
    bf = 2.5 * flop
    log(f"backward (prep + dQ + dK/dV): {ms:.3f} ms -> {bf / ms / 1e9:.1f} TFLOP/s "
        f"({100 * bf / ms / 1e9 / PEAK_BF16_TFLOPS:.1f} % of peak)")
    out = {"ms": round(ms, 4), "flop": bf, "tflops": round(bf / ms / 1e9, 3),
           "frac_of_peak": round(bf / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
    if zig is not None:
        kz, vz, zin = zig
        dkz = torch.empty(kz.shape, dtype=torch.float32, device=dev)
        dvz = torch.empty(kz.shape, dtype=torch.float32, device=dev)
        zz = {}
        for rz, (qz, Oz, lz) in zin.items():
            doz = torch.randn(qz.shape, generator=g, device=dev).to(torch.bfloat16)
            dqz = torch.empty(qz.shape, dtype=torch.float32, device=dev)
            dez = torch.empty(lz.shape, dtype=torch.float32, device=dev)
            runz = lambda: ra.ra_rank_share_zigzag_bwd(qz, kz, vz, Oz, lz, doz, w.P, rz, True, dqz, dkz, dvz,  # noqa
                                                       dez)
            warm(torch, runz)
            mz = sorted(per_launch_ms(torch, runz, reps))[reps // 2]
            fz = 2.5 * ra.ra_share_flops_zigzag(w.B, w.N, w.P, rz, w.Hq, w.d, True)
            zz[f"rank{rz}"] = {"ms": round(mz, 4), "tflops": round(fz / mz / 1e9, 3)}
        log("load-balanced backward: " + ", ".join(f"{k} {v['ms']:.3f} ms ({v['tflops']:.0f} TFLOP/s)"
                                                   for k, v in zz.items()))
        out["zigzag"] = zz
    return out


def cpu_baseline(w, x, O_gpu, lse_gpu, target_s: float):
    """The fp64 oracle (plain C, one thread per core this process may run
    on) on a seeded random sample of the headline share's rows, sized to
    about target_s seconds from a short probe.  Returns the baseline and
    the parity of the same rows."""
    import numpy as np
    import torch

    import oracle

    affinity = len(os.sched_getaffinity(0))
    threads = affinity
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
    probe = sample(4 * threads)
    t0 = time.perf_counter()
    oracle.rank_share(q64, k64, v64, w.P, r, w.causal, rows=probe, nthreads=threads)
    dt = time.perf_counter() - t0
    n = int(max(4 * threads, min(400000, len(probe) * target_s / max(dt, 1e-3))))
    rows = sample(n)
    log(f"cpu baseline: oracle on {n} sampled rows with {threads} threads ({affinity} cores in the affinity set)")
    t0 = time.perf_counter()
    o_ref, l_ref = oracle.rank_share(q64, k64, v64, w.P, r, w.causal, rows=rows, nthreads=threads)
    dt = time.perf_counter() - t0
    flops = row_flops(rows)
    parity = compare(O_gpu, lse_gpu, rows, o_ref, l_ref, 1e-2, 1e-3, O_gpu.dtype == torch.bfloat16)
    # every row of the share, at the same rate (extrapolated, not run)
    pos_all = np.arange(w.nq, dtype=np.float64) + r * w.nq
    vis_all = np.minimum(pos_all + 1, w.N) if w.causal else np.full(w.nq, float(w.N))
    share_flops = 4.0 * w.d * w.B * w.Hq * float(vis_all.sum())
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "affinity_cores": affinity,
            "kind": "oracle",
            "sample": f"{n} random (b, h, i) rows of the same share, each against all its visible "
                      f"keys in ring order; {flops:.3e} FLOP in {dt:.2f} s (fp64, plain C, {threads} threads)",
            "extrapolated_share_s": round(share_flops / (flops / dt), 1), "cpu": cpu_model()}
    return base, parity


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the headline share only (no other workloads, state kernels, stepwise, "
                         "load-balance or backward measurements), so that a profiler's per-kernel summary "
                         "covers the timed launches alone")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: libringattn has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    import oracle
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

    threads = len(os.sched_getaffinity(0))
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

    # The input draws leave the GPU idle at its lowest clock; untimed
    # back-to-back steps for WARM_SECONDS bring it to the clock it holds
    # under this load before the W warm-up steps and the K timed ones.
    log(f"clock warm-up {WARM_SECONDS} s, then warmup {args.warmup}")
    warm_launches = warm(torch, step, WARM_SECONDS)
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
    per = [a.elapsed_time(b) for a, b in ev]
    km = summary(per)
    mean_ms = km["mean"]
    ms_per_step = wall * 1e3 / args.steps
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (mean_ms * 1e-3) / 1e12
    log(f"{w.name}: {ms_per_step:.3f} ms/step, kernel mean {mean_ms:.3f} ms "
        f"(median {km['median']:.3f}, min {km['min']:.3f}) -> {achieved:.1f} TFLOP/s")

    if args.no_extras:
        clock = {"recorded": False, "why": "not sampled with --no-extras (its launches would join a profiler's "
                                           "per-kernel summary)"}
    else:
        clock = ClockSampler(torch).sample_during(torch, step, 2.5)
    if clock.get("recorded"):
        log(f"engine clock under load: median {clock['gfxclk_mhz']['median']} MHz "
            f"({clock['gfxclk_mhz']['min']}..{clock['gfxclk_mhz']['max']})")
    else:
        log(f"engine clock not recorded: {clock.get('why')}")

    out = {
        "metric": METRIC,
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "clock_warmup": {"seconds": WARM_SECONDS, "launches": warm_launches},
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "N": w.N,
                   "P": w.P, "rank": r, "causal": w.causal, "q_block": w.nq, "input": w.dist,
                   "seed": w.seed},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "flop_per_step": flop,
        "kernel_ms": km,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(w.name)},
        "clock": clock,
        "inputs_sha256": {t: inputs.sha256(xq[t])[:16] for t in "qkv"},
    }
    if not args.no_extras:
        out["stepwise"] = stepwise(w, r, qd, kd, vd, flop, ra, torch)
        out.update(state_kernels(w, torch, ra))
        balance, zig = load_balance(w, r, qd, kd, vd, mean_ms, ra, torch, inputs, oracle, threads)
        out["load_balance"] = balance
        out["backward"] = backward(w, r, qd, kd, vd, flop, ra, torch, zig)
        del zig
        torch.cuda.empty_cache()
    if not args.no_extras:
        # every workload, each with its own inputs, timing and parity sample
        configs = {}
        for cw in workloads.ALL:
            configs[cw.name] = run_config(cw, 10, 2, torch, ra, inputs, oracle, threads)
            configs[cw.name]["headline"] = cw.name == w.name
        out["configs"] = configs
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
