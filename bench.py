#!/usr/bin/env python3
"""Benchmark of the TN half-precision GEMM on one MI355X.

One step = one ``mi_hgemm_run`` over the workload's synthetic operands (already
resident in HBM), through the library's normal dispatch (or a forced instance with
``--kernel``, for per-instance counter runs).  By default the
operands rotate over enough copies that every call reads A and B from HBM
rather than from the 256 MiB MALL ("cold"); ``--warm`` reuses one set.

The int8 variant (int8 operands, exact int32 result) is measured the same way
with ``--workload i8_square`` or ``i8_llm_MxNxK`` (TOP/s against the int8 MFMA
peak).

``--server`` measures the server mode instead (requests of the tiny problem
arriving at a target QPS, and the highest rate sustained), with the native load
generator ``mi_hgemm_serve`` against rocBLAS on the same operands.

Prints ONE JSON line: throughput (TFLOP/s over the timed steps), the roofline
of the dominant kernel (its per-launch duration from HIP events recorded on the
launch stream inside the timed region), and the CPU oracle timed on a bounded
sample of the same product on the host cores.

    python bench.py [--steps K] [--warmup W] [--workload square|tiny|small|llm_MxNxK]
                    [--workload i8_square|i8_llm_MxNxK]
                    [--mnk M_N_K] [--warm] [--no-cpu-baseline] [--all-configs OUT.jsonl]
                    [--kernel NAME [--group-m G] [--xcd-remap X] [--split-k S]]
                    [--sweep OUT.jsonl [--sweep-count N]]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HGEMM TFLOPS and µs/call per (M,N,K) on 1 MI355X; % of roofline"
METRIC_I8 = "IGEMM (int8 in, int32 out) TOPS and µs/call per (M,N,K) on 1 MI355X; % of roofline"
PEAK_MFMA_TFLOPS = 2516.6    # dense fp16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk/CU
PEAK_MFMA_I8_TOPS = 5033.2   # dense int8 MFMA: 256 CU x 2.4 GHz x 8192 OP/clk/CU
PEAK_HBM_GBS = 8000.0        # HBM3E
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="square")
    ap.add_argument("--mnk", default=None, help="custom shape M_N_K (randn/sqrt(K) inputs)")
    ap.add_argument("--warm", action="store_true", help="reuse one operand set (MALL-resident)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the live MFMA / HBM ceiling probes (libmi_ceiling)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--all-configs", default=None,
                    help="also time every named workload and write JSON lines here")
    ap.add_argument("--kernel", default=None,
                    help="force this compiled instance (by name) instead of the dispatcher's choice")
    ap.add_argument("--group-m", type=int, default=1, help="raster group height with --kernel")
    ap.add_argument("--xcd-remap", type=int, default=0, choices=(0, 1), help="XCD remap with --kernel")
    ap.add_argument("--split-k", type=int, default=1, help="K split with --kernel")
    ap.add_argument("--sweep", default=None, metavar="OUT.jsonl",
                    help="time the seeded 1000-shape sweep (device time, cold) against torch")
    ap.add_argument("--sweep-count", type=int, default=1000, help="first N problems of the sweep")
    ap.add_argument("--server", action="store_true",
                    help="server-mode QPS of the tiny problem (64, 4096, 64) instead")
    ap.add_argument("--target-qps", type=float, default=100.0, help="arrival rate with --server")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (to scale "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def source_digest() -> str:
    """Digest of the device sources' code (comments and blank lines removed)."""
    from dense_fp16_gemm_hgemm_amd.provenance import source_digest as digest
    return digest()


def load_traffic(kernel: str, workload: str, group_m: int, xcd_remap: int, split_k: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none, it was taken on other kernel sources, or with another
    raster or K split (both change the traffic)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_digest") != source_digest():
        return None
    try:
        if (int(vals["group_m"]), int(vals["xcd_remap"]), int(vals["split_k"])) != \
                (group_m, xcd_remap, split_k):
            return None
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def problem_for(name, mnk):
    from dense_fp16_gemm_hgemm_amd import inputs
    if mnk:
        M, N, K = (int(x) for x in mnk.split("_"))
        s = 1.0 / math.sqrt(K)
        return inputs.Problem(f"mnk_{M}x{N}x{K}", M, N, K, "randn", s, s, 7)
    if name == "square":
        return inputs.square()
    if name == "i8_square":
        return inputs.i8_square()
    for p in inputs.i8_llm():
        if p.name == name:
            return p
    if name == "tiny":
        return inputs.tiny()
    if name == "small":
        return inputs.small(False)
    for p in inputs.llm():
        if p.name == name or p.name == "llm_" + name.replace("llm_", ""):
            return p
    raise SystemExit(f"unknown workload {name!r}")


class Workload:
    """Device operand sets for one problem (copies of one seeded draw)."""

    def __init__(self, p, cold: bool, operands=None):
        import torch
        from dense_fp16_gemm_hgemm_amd import inputs
        self.p = p
        dev = torch.device("cuda", 0)
        if operands is None:
            A, Bt = inputs.make(p)
            self.A_host, self.Bt_host = A, Bt
            a = torch.from_numpy(A).to(dev)
            b = torch.from_numpy(Bt).to(dev)
        else:                      # device operands drawn by the caller
            self.A_host = self.Bt_host = None
            a, b = operands
        set_bytes = p.min_bytes
        nsets = 1
        if cold:
            nsets = max(2, math.ceil(2.2 * MALL_BYTES / max(set_bytes, 1)))
            nsets = min(nsets, 2048)
        self.sets = []
        for s in range(nsets):
            aa = a if s == 0 else a.clone()
            bb = b if s == 0 else b.clone()
            cc = torch.empty((p.M, p.N), dtype=torch.int32 if p.kind == "i8" else torch.float16,
                             device=dev)
            self.sets.append((aa, bb, cc))
        torch.cuda.synchronize()


def time_steps(run, wl, steps, warmup):
    """Warm up, then time exactly `steps` launches of run(a, b, c) bracketed by
    synchronisations.  Returns (ms per step, mean per-launch ms from event pairs,
    wall s, per-launch ms)."""
    import torch
    sets = wl.sets
    n = len(sets)
    for i in range(warmup):
        a, b, c = sets[i % n]
        run(a, b, c)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(steps):
        a, b, c = sets[i % n]
        ev[i][0].record(stream)
        run(a, b, c)
        ev[i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    per = [e0.elapsed_time(e1) for e0, e1 in ev]
    return total_ms / steps, statistics.fmean(per), wall, per


def roofline(p, launch_ms, kernel, workload, raster=(1, 0, 1)):
    flops, nbytes = p.flops, p.min_bytes
    t = launch_ms * 1e-3
    ai = flops / nbytes
    i8 = p.kind == "i8"
    mfma_peak = PEAK_MFMA_I8_TOPS if i8 else PEAK_MFMA_TFLOPS
    ridge = mfma_peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if ai >= ridge:
        achieved, peak, bound = flops / t / 1e12, mfma_peak, "mfma"
        unit = "TOP/s" if i8 else "TFLOP/s"
    else:
        achieved, peak, unit, bound = nbytes / t / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": load_traffic(kernel, workload, *raster),
            "algorithmic_flops": flops, "algorithmic_bytes": nbytes}


def practical_ceiling(roof, p):
    """libmi_ceiling's live measurement beside the published peak: for an
    MFMA-bound launch the MFMA-only rate on random fp16 (int8 work is compared
    at twice that rate, the int8 MFMA doing twice the operations per cycle),
    for an HBM-bound one the streaming read rate."""
    from dense_fp16_gemm_hgemm_amd import ceiling
    m = ceiling.measure()
    if roof["bound"] == "mfma":
        ceil = m["mfma_tflops"] * (2 if p.kind == "i8" else 1)
        unit = roof["unit"]
    else:
        ceil, unit = m["hbm_read_gbs"], "GB/s"
    m.update({"value": ceil, "unit": unit, "frac": round(roof["achieved"] / ceil, 4)})
    return m


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


SINGLE_CORE_SNIPPET = r"""
import json, sys, time
import numpy as np
sys.path.insert(0, {root!r})
import oracle
from dense_fp16_gemm_hgemm_amd import inputs
p = inputs.Problem("single_core", {rows}, {N}, {K}, {kind!r}, {a_scale!r}, {b_scale!r}, {seed})
A, Bt = inputs.make(p)
orc = oracle.default()
orc.set_num_threads(1)
f = orc.igemm_tn if p.kind == "i8" else orc.hgemm_tn
f(A[:1], Bt[:64])
t0 = time.perf_counter()
f(A, Bt)
t = time.perf_counter() - t0
print(json.dumps({{"threads": orc.num_threads(), "seconds": t, "flop": 2.0 * p.M * p.N * p.K}}))
"""


def single_core_oracle(p, target_s=3.0):
    """The oracle on one host core (one OpenMP thread, set through the oracle
    library itself, in a child process that never touches the GPU), on the
    first rows of the same problem; "threads" is what the library reports."""
    import subprocess
    rows = max(1, min(p.M, int(target_s * 4e9 / (2 * p.N * p.K))))
    code = SINGLE_CORE_SNIPPET.format(root=ROOT, rows=rows, N=p.N, K=p.K, kind=p.kind,
                                      a_scale=p.a_scale, b_scale=p.b_scale, seed=p.seed)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    try:
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                           timeout=120)
        d = json.loads(r.stdout.strip().splitlines()[-1])
    except Exception as e:  # reported, never fatal to the bench line
        return {"error": str(e)[:200]}
    return {"value": round(d["flop"] / d["seconds"] / 1e12, 6), "threads": d["threads"],
            "seconds": round(d["seconds"], 3),
            "sample": f"{rows}x{p.N}x{p.K} ({rows} rows of the workload, same distribution and seed)"}


def cpu_baseline(p, A, Bt, gpu_c, target_s):
    """The oracle, as it is, on rows 0..R-1 of the product; R sized to ~target_s."""
    import numpy as np

    import oracle
    orc = oracle.default()
    i8 = p.kind == "i8"

    def rows(R):
        r = np.repeat(np.arange(R, dtype=np.int64), p.N)
        c = np.tile(np.arange(p.N, dtype=np.int64), R)
        t0 = time.perf_counter()
        vals = (orc.igemm_tn_entries if i8 else orc.hgemm_tn_entries)(A, Bt, r, c)
        return time.perf_counter() - t0, vals.reshape(R, p.N)

    rows(1)                                   # first call starts the oracle's threads
    R0 = max(1, min(p.M, int(2e9 / (2 * p.N * p.K))))
    t0, _ = rows(R0)
    R = max(1, min(p.M, int(R0 * target_s / max(t0, 1e-6))))
    t, vals = rows(R)
    if t < 0.6 * target_s and R < p.M:          # one correction if the estimate was short
        R = max(1, min(p.M, int(R * target_s / max(t, 1e-6))))
        t, vals = rows(R)
    flop = 2.0 * R * p.N * p.K
    # the sample doubles as a parity check of the timed GPU output (exact for int8)
    if i8:
        ok = bool(np.array_equal(gpu_c[:R], vals))
    else:
        g = gpu_c[:R].astype(np.float64)
        r64 = vals.astype(np.float64)
        fin = np.isfinite(r64)
        bound = 1e-3 * np.abs(r64[fin]).max() + 2e-3 * np.abs(r64[fin])
        ok = bool(np.all(np.abs(g[fin] - r64[fin]) <= bound))
    return {"value": round(flop / t / 1e12, 6), "unit": "TOP/s" if i8 else "TFLOP/s",
            "cores": orc.num_threads(), "cpu_model": cpu_model(),
            "kind": "oracle", "seconds": round(t, 3),
            "sample": f"rows 0..{R - 1} of C ({R}x{p.N} outputs, K={p.K}) of {p.name}",
            "sample_parity": "ok" if ok else "FAIL"}


def torch_call(p):
    """The vendor library's call for the problem: torch.matmul, or torch._int_mm
    for int8 (hipBLASLt; it needs M > 16)."""
    import torch
    if p.kind == "i8":
        if p.M <= 16:
            return None
        return lambda a, b, c: torch._int_mm(a, b.t(), out=c)
    return lambda a, b, c: torch.matmul(a, b.t(), out=c)


def torch_matmul_context(wl, steps=20):
    """The vendor BLAS on the same operands, as context only."""
    import torch
    fn = torch_call(wl.p)
    if fn is None:
        return None, None
    a, b, c = wl.sets[0]
    for _ in range(3):
        fn(a, b, c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        a, b, c = wl.sets[i % len(wl.sets)]
        fn(a, b, c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return round(wl.p.flops / (ms * 1e-3) / 1e12, 2), round(ms * 1e3, 2)


def graph_us(fn, wl, reps):
    """Device time per call: `reps` calls of fn(a, b, c), rotating over the
    workload's operand sets, captured in one graph and replayed."""
    import torch
    sets = wl.sets
    fn(*sets[0])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(reps):
                fn(*sets[i % len(sets)])
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del g
    return us


def measure(lib, p, steps, warmup, cold, with_torch=False, force=None, device_time=False,
            operands=None):
    """force: None (the library's dispatch) or (kernel name, group_m, xcd_remap, split_k)."""
    wl = Workload(p, cold, operands)
    a, b, c = wl.sets[0]
    if force is None:
        kernel, gm, xcd, sk = lib.plan(a, b, c)
        run = lib.run_i8 if p.kind == "i8" else lib.run
    else:
        kernel, gm, xcd, sk = force

        def run(a, b, c):
            lib.run_kernel(kernel, a, b, c, group_m=gm, xcd_remap=xcd, split_k=sk)
    ms, launch_ms, wall, per = time_steps(run, wl, steps, warmup)
    q = statistics.quantiles(per, n=4) if len(per) >= 2 else [per[0]] * 3
    rec = {"workload": p.name, "M": p.M, "N": p.N, "K": p.K, "kernel": kernel, "group_m": gm,
           "xcd_remap": xcd, "split_k": sk, "cache": "cold" if cold else "warm", "sets": len(wl.sets),
           "ms_per_step": ms, "us_per_call": round(launch_ms * 1e3, 3),
           "us_per_call_median": round(statistics.median(per) * 1e3, 3),
           "us_per_call_iqr": [round(q[0] * 1e3, 3), round(q[2] * 1e3, 3)],
           "tflops": round(p.flops / (ms * 1e-3) / 1e12, 3), "wall_s": wall,
           "roofline": roofline(p, launch_ms, kernel, p.name, (gm, xcd, sk))}
    if with_torch:
        rec["torch_matmul_tflops"], rec["torch_matmul_us"] = torch_matmul_context(wl)
    if device_time:
        # the stream figures above include the host's launch path, which exceeds
        # the kernel for small shapes; graph replay gives the device time
        reps = min(2048, max(len(wl.sets), 20, int(20000 / max(launch_ms * 1e3, 1.0))))
        dus = graph_us(run, wl, reps)
        rec["device_us_per_call"] = round(dus, 3)
        rec["device_tflops"] = round(p.flops / (dus * 1e-6) / 1e12, 3)
        rec["device_roofline"] = roofline(p, dus * 1e-3, kernel, p.name, (gm, xcd, sk))
        tm = torch_call(p) if with_torch else None
        if tm is not None:
            rec["torch_device_us_per_call"] = round(graph_us(tm, wl, reps), 3)
    return rec, wl


def sweep_main(args, lib):
    """The seeded shape sweep (each of M, N, K = 2^U{6..13}, the stand-in for the
    pages' 1000 configurations): per problem, the device time per call (graph
    replay over cold operand copies) through the library's dispatch, its
    roofline fraction, and torch.matmul's device time on the same operands.
    The operands have the sweep's distribution (randn/sqrt(K) in binary16) but
    are drawn on the device with torch's generator, seeded with the problem's
    seed: the numpy draws of the recipe take minutes at this volume, and the
    timing depends on the distribution, not on the particular values (the
    sweep's parity is tested on the recipe's own draws).  Writes one JSON line
    per problem to args.sweep and prints a summary line."""
    import torch
    from dense_fp16_gemm_hgemm_amd import inputs
    dev = torch.device("cuda", 0)
    probs = inputs.sweep()[: args.sweep_count]
    recs = []
    t0 = time.perf_counter()
    with open(args.sweep, "w") as f:
        for i, p in enumerate(probs):
            g = torch.Generator(device=dev).manual_seed(p.seed)
            a = (torch.randn(p.M, p.K, device=dev, generator=g) * p.a_scale).half()
            b = (torch.randn(p.N, p.K, device=dev, generator=g) * p.b_scale).half()
            rec, wl = measure(lib, p, 10, 3, True, with_torch=True, device_time=True,
                              operands=(a, b))
            rec["operands"] = "torch.randn on the device, seeded with the problem's seed"
            f.write(json.dumps(rec) + "\n")
            f.flush()
            recs.append(rec)
            del wl, a, b
            torch.cuda.empty_cache()
            if (i + 1) % 25 == 0 or i + 1 == len(probs):
                print(f"# sweep {i + 1}/{len(probs)} ({time.perf_counter() - t0:.0f} s)",
                      file=sys.stderr, flush=True)
    fr = [r["device_roofline"]["frac"] for r in recs]
    ok = [r["device_roofline"]["frac"] >= (0.7 if r["device_roofline"]["bound"] == "mfma" else 0.6)
          for r in recs]
    sp = [r["torch_device_us_per_call"] / r["device_us_per_call"] for r in recs
          if r.get("torch_device_us_per_call")]
    gmean = lambda v: math.exp(statistics.fmean(math.log(max(x, 1e-12)) for x in v))
    by_bound = {}
    for r, o in zip(recs, ok):
        d = by_bound.setdefault(r["device_roofline"]["bound"], {"problems": 0, "meet_target": 0, "fracs": []})
        d["problems"] += 1
        d["meet_target"] += int(o)
        d["fracs"].append(r["device_roofline"]["frac"])
    for d in by_bound.values():
        d["geomean_frac"] = round(gmean(d.pop("fracs")), 4)
    kernels = {}
    for r in recs:
        kernels[r["kernel"]] = kernels.get(r["kernel"], 0) + 1
    summary = {
        "sweep_problems": len(recs), "cache": "cold", "timing": "device (graph replay)",
        "meet_target": sum(ok), "meet_target_rate": round(sum(ok) / len(recs), 4),
        "target": "roofline frac >= 0.7 (MFMA-bound) or >= 0.6 (HBM-bound)",
        "geomean_frac": round(gmean(fr), 4), "by_bound": by_bound,
        "geomean_speedup_vs_torch": round(gmean(sp), 4),
        "faster_than_torch": sum(1 for x in sp if x > 1.0),
        "speedup_vs_torch_min": round(min(sp), 3), "speedup_vs_torch_max": round(max(sp), 3),
        "kernels": dict(sorted(kernels.items(), key=lambda kv: -kv[1])),
        "seconds": round(time.perf_counter() - t0, 1), "source_digest": source_digest(),
    }
    print(json.dumps(summary), flush=True)


def server_cpu_baseline(mnk, target_s):
    """The oracle serving requests of the same problem back to back on the host
    cores: requests per second over ~target_s."""
    import numpy as np

    import oracle
    from dense_fp16_gemm_hgemm_amd import inputs
    orc = oracle.default()
    M, N, K = (int(x) for x in mnk.split("_"))
    A, Bt = inputs.make(inputs.Problem("server", M, N, K, "randn", 1 / math.sqrt(K),
                                       1 / math.sqrt(K), 1))
    orc.hgemm_tn(A, Bt)                                   # starts the oracle's threads
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < target_s:
        orc.hgemm_tn(A, Bt)
        n += 1
    t = time.perf_counter() - t0
    return {"value": round(n / t, 3), "unit": "requests/s", "cores": orc.num_threads(),
            "kind": "oracle", "seconds": round(t, 3),
            "sample": f"{n} requests of {M}x{N}x{K}, served back to back"}


def server_main(args):
    """Server mode: Poisson arrivals at the target rate, and the highest
    sustained rate (back to back, 8 in flight), for the library and rocBLAS.
    Runs the load generator as a child process before this process touches the
    GPU."""
    from dense_fp16_gemm_hgemm_amd import server_mode
    mnk = args.mnk or "64_4096_64"
    runs = {}
    for backend in ("mi_hgemm", "rocblas"):
        runs[backend] = {
            "target": server_mode.run(mnk, "poisson", args.target_qps,
                                      requests=max(50, int(args.target_qps * 5)), backend=backend),
            "saturation": server_mode.run(mnk, "closed", requests=max(args.steps, 1) * 200,
                                          depth=8, backend=backend),
        }
    # the floor of this harness: one empty kernel and its event per request
    runs["launch"] = {"saturation": server_mode.run(mnk, "closed", requests=max(args.steps, 1) * 200,
                                                    depth=8, backend="launch")}
    ours, vend = runs["mi_hgemm"], runs["rocblas"]
    sat = ours["saturation"]["achieved_qps"]
    # both at 80% of our sustained rate: latency under a heavy but stable load
    for backend in ("mi_hgemm", "rocblas"):
        runs[backend]["load80"] = server_mode.run(mnk, "poisson", 0.8 * sat, requests=20000,
                                                  backend=backend)
    M, N, K = (int(x) for x in mnk.split("_"))
    out = {
        "metric": "server-mode QPS of the (64,4096,64) HGEMM on 1 MI355X (sustained, 8 in flight)",
        "value": round(sat, 1),
        "unit": "requests/s",
        "n_gpus": 1,
        "steps": max(args.steps, 1) * 200,
        "warmup": 64,
        "ms_per_step": round(1e3 / sat, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": f"server_{M}x{N}x{K}", "M": M, "N": N, "K": K,
                   "target_qps": args.target_qps, "dispatch": "library",
                   "parallelism": "none (1 GPU)"},
        "server": runs,
        "context": {"rocblas_sustained_qps": vend["saturation"]["achieved_qps"],
                    "ours_over_rocblas": round(sat / vend["saturation"]["achieved_qps"], 3),
                    "empty_kernel_sustained_qps": runs["launch"]["saturation"]["achieved_qps"],
                    "issue_us_mean": {b: runs[b]["saturation"].get("issue_us", {}).get("mean")
                                      for b in ("mi_hgemm", "rocblas", "launch")}},
        "roofline": None,
        "cpu_baseline": None if args.no_cpu_baseline else server_cpu_baseline(mnk, args.cpu_seconds),
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1",
                          "n_gpus_requested": args.gpus}), flush=True)
        sys.exit(2)
    if args.server:
        server_main(args)
        return
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 2, dtype=torch.float16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return
    import dense_fp16_gemm_hgemm_amd as mh
    lib = mh.Hgemm()
    cold = not args.warm
    if args.sweep:
        sweep_main(args, lib)
        lib.close()
        return

    if args.all_configs:
        from dense_fp16_gemm_hgemm_amd import inputs
        with open(args.all_configs, "w") as f:
            for p in inputs.all_named() + inputs.i8_llm() + [inputs.i8_square()]:
                if p.kind not in ("randn", "i8"):
                    continue
                for c in (True, False):
                    rec, _ = measure(lib, p, max(20, args.steps // 2), 5, c, with_torch=True,
                                     device_time=True)
                    f.write(json.dumps(rec) + "\n")
                    f.flush()
                    print(f"# {p.name} {rec['cache']}: device {rec['device_us_per_call']} us "
                          f"({rec['kernel']} s{rec['split_k']}) torch {rec.get('torch_device_us_per_call')} us; "
                          f"stream {rec['us_per_call']} us, torch {rec['torch_matmul_us']} us",
                          file=sys.stderr, flush=True)
                torch.cuda.empty_cache()

    p = problem_for(args.workload, args.mnk)
    force = None
    if args.kernel:
        force = (args.kernel, args.group_m, args.xcd_remap, args.split_k)
    rec, wl = measure(lib, p, args.steps, args.warmup, cold, with_torch=True, force=force)
    i8 = p.kind == "i8"
    out = {
        "metric": METRIC_I8 if i8 else METRIC,
        "value": rec["tflops"],
        "unit": "TOP/s" if i8 else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(rec["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8" if i8 else "fp16",
        "data": "synthetic",
        "config": {"workload": p.name, "M": p.M, "N": p.N, "K": p.K, "layout": "TN",
                   "accumulate": "int32" if i8 else "fp32",
                   "inputs": (f"int8 uniform seed {p.seed}" if i8 else
                              f"{p.kind} a*{p.a_scale:.6g} b*{p.b_scale:.6g} seed {p.seed}"),
                   "cache": rec["cache"], "operand_sets": rec["sets"], "kernel": rec["kernel"],
                   "group_m": rec["group_m"], "xcd_remap": rec["xcd_remap"],
                   "split_k": rec["split_k"], "dispatch": "forced" if args.kernel else "library",
                   "us_per_call": rec["us_per_call"], "us_per_call_median": rec["us_per_call_median"],
                   "us_per_call_iqr": rec["us_per_call_iqr"],
                   "parallelism": "none (1 GPU)"},
        "roofline": rec["roofline"],
        "cpu_baseline": None,
        "context": {("torch_int_mm_tops" if i8 else "torch_matmul_tflops"): rec["torch_matmul_tflops"],
                    ("torch_int_mm_us" if i8 else "torch_matmul_us"): rec["torch_matmul_us"],
                    "source_digest": source_digest()},
    }
    if not args.kernel and p.name == "square_8192":
        # Beside the large square, the (128, 2048, 128) case that one page quotes
        # its H100 figure on: launch-bound at a few microseconds, so its device
        # time (graph replay) is the figure that describes the kernel.
        from dense_fp16_gemm_hgemm_amd import inputs
        ps = inputs.small(False)
        rs, _ = measure(lib, ps, 40, 5, True, with_torch=True, device_time=True)
        out["context"][ps.name] = {
            "kernel": rs["kernel"], "cache": rs["cache"], "us_per_call": rs["us_per_call"],
            "device_us_per_call": rs["device_us_per_call"], "device_tflops": rs["device_tflops"],
            "device_roofline_frac": rs["device_roofline"]["frac"],
            "device_roofline_bound": rs["device_roofline"]["bound"],
            "torch_device_us_per_call": rs.get("torch_device_us_per_call")}
        torch.cuda.empty_cache()
    if not args.no_ceiling:
        # the chip's practical ceilings, measured now (after the timed region):
        # MFMA-only on random operands with the clock under that load, and the
        # streaming HBM read rate; the kernel's rate as a fraction of each
        out["roofline"]["practical_ceiling"] = practical_ceiling(out["roofline"], p)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        gpu_c = wl.sets[(args.steps - 1) % len(wl.sets)][2].cpu().numpy()
        out["cpu_baseline"] = cpu_baseline(p, wl.A_host, wl.Bt_host, gpu_c, args.cpu_seconds)
        out["cpu_baseline"]["single_core"] = single_core_oracle(p)
    lib.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
