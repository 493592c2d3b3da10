"""Binding and sweep driver of libmi_overlap, the gfx950 load/compute overlap
micro-benchmark (operation and modes: ``include/mi_overlap.h``).

"B-08. Hopper TMA：从单线程 Bulk Copy 到吞吐墙" (lqnn.cn) §5 sweeps FMA
iterations per element and reports each mode's time and its speedup over the
synchronous cooperative load, as a CSV and a plot; §5.1 gives the expected
shape (prefetch > 1 at low intensity, all modes -> 1 at high intensity).
This module does the same for gfx950's ways of filling LDS:

    python -m dense_fp16_gemm_hgemm_amd.overlap [--n FLOATS] [--tiles-per-block T]
        [--iters 0,1,2,4,...] [--reps R] [--out DIR]

writes DIR/overlap_sweep.csv (and overlap_sweep.png when matplotlib is present)
and prints the table.  Timing: each (mode, fma_iters) point is the median of R
launches, each between two HIP events on the launch stream.
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import os
import statistics
import sys

import torch  # imported first so that both use one HIP runtime

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmi_overlap.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python dense_fp16_gemm_hgemm_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)
_lib.mi_overlap_run.restype = ctypes.c_int
_lib.mi_overlap_run.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                                ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)]
_lib.mi_overlap_tile_floats.restype = ctypes.c_int
_lib.mi_overlap_block_threads.restype = ctypes.c_int

MI_OVERLAP_SYNC, MI_OVERLAP_DIRECT, MI_OVERLAP_PIPE2, MI_OVERLAP_REG2 = 0, 1, 2, 3
MODES = {"sync": MI_OVERLAP_SYNC, "direct": MI_OVERLAP_DIRECT, "pipe2": MI_OVERLAP_PIPE2,
         "reg2": MI_OVERLAP_REG2}
TILE = _lib.mi_overlap_tile_floats()
THREADS = _lib.mi_overlap_block_threads()
ALPHA = 1.0 - 2.0 ** -11   # the chain y <- alpha y + beta settles at 0.5: no overflow
BETA = 2.0 ** -12


def mi_overlap_run(mode, x_ptr, out_ptr, n, tiles_per_block, fma_iters, alpha, beta,
                   stream=None):
    """The C ABI call; returns (status, hip_error)."""
    err = ctypes.c_int(0)
    st = _lib.mi_overlap_run(mode, x_ptr, out_ptr, n, tiles_per_block, fma_iters, alpha, beta,
                             stream, ctypes.byref(err))
    return st, err.value


def run(mode, x: torch.Tensor, out: torch.Tensor, tiles_per_block: int, fma_iters: int,
        alpha: float = ALPHA, beta: float = BETA, stream=None) -> torch.Tensor:
    """out = the FMA chain of x, staged through LDS the way `mode` says."""
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    for t, name in ((x, "x"), (out, "out")):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor")
    if x.numel() != out.numel():
        raise ValueError("x and out must have the same size")
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    st, err = mi_overlap_run(m, x.data_ptr(), out.data_ptr(), x.numel(), tiles_per_block,
                             fma_iters, alpha, beta, stream.cuda_stream)
    if st != 0:
        raise RuntimeError(f"mi_overlap_run failed: status {st}, hip error {err}")
    return out


def sweep(n: int, tiles_per_block: int, iters_list, reps: int = 20, seed: int = 0):
    """Rows of (fma_iters, {mode: median ms}) over the modes."""
    dev = torch.device("cuda", 0)
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = (torch.rand(n, generator=g, dtype=torch.float32) * 2 - 1).to(dev)
    out = torch.empty_like(x)
    rows = []
    for k in iters_list:
        times = {}
        for name in MODES:
            for _ in range(3):
                run(name, x, out, tiles_per_block, k)
            torch.cuda.synchronize()
            ms = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                run(name, x, out, tiles_per_block, k)
                e1.record()
                e1.synchronize()
                ms.append(e0.elapsed_time(e1))
            times[name] = statistics.median(ms)
        rows.append((k, times))
        print(f"fma_iters {k:4d}: " + "  ".join(f"{m} {t * 1e3:9.1f} us" for m, t in times.items())
              + "  speedup " + " ".join(f"{m} {times['sync'] / t:.3f}" for m, t in times.items()
                                       if m != "sync"), flush=True)
    return rows


def write_csv(rows, path):
    names = list(MODES)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["fma_iters"] + [f"{m}_ms" for m in names] +
                   [f"speedup_{m}" for m in names if m != "sync"])
        for k, t in rows:
            w.writerow([k] + [f"{t[m]:.6f}" for m in names] +
                       [f"{t['sync'] / t[m]:.4f}" for m in names if m != "sync"])


def write_plot(rows, path):
    try:
        import matplotlib
        matplotlib.use("Agg")
        import matplotlib.pyplot as plt
    except ImportError:
        return False
    ks = [max(k, 0.5) for k, _ in rows]
    fig, ax = plt.subplots(figsize=(6, 4))
    for m in MODES:
        if m == "sync":
            continue
        ax.plot(ks, [t["sync"] / t[m] for _, t in rows], marker="o", label=m)
    ax.axhline(1.0, color="gray", lw=0.8)
    ax.set_xscale("log", base=2)
    ax.set_xlabel("FMA iterations per element")
    ax.set_ylabel("speedup over sync (VGPR-staged, no overlap)")
    ax.set_title("gfx950 load/compute overlap")
    ax.legend()
    fig.tight_layout()
    fig.savefig(path, dpi=120)
    return True


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--n", type=int, default=1 << 26, help="floats (default 2^26 = 256 MiB)")
    ap.add_argument("--tiles-per-block", type=int, default=256)
    ap.add_argument("--iters", default="0,1,2,4,8,16,32,64,128,256,512,1024")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--out", default=".")
    a = ap.parse_args(argv)
    if not torch.cuda.is_available():
        raise SystemExit("the overlap micro-benchmark needs a GPU")
    torch.cuda.set_device(0)
    print(f"n {a.n} floats ({a.n * 4 / 2 ** 20:.0f} MiB), tiles of {TILE} floats, "
          f"{a.tiles_per_block} tiles per workgroup, {a.n // (TILE * a.tiles_per_block)} workgroups",
          flush=True)
    rows = sweep(a.n, a.tiles_per_block, [int(s) for s in a.iters.split(",")], a.reps)
    os.makedirs(a.out, exist_ok=True)
    write_csv(rows, os.path.join(a.out, "overlap_sweep.csv"))
    write_plot(rows, os.path.join(a.out, "overlap_sweep.png"))


if __name__ == "__main__":
    sys.exit(main())
