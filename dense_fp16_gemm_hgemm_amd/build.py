"""Build libmi_hgemm.so in-tree with hipcc for gfx950.

Every ``csrc/*.hip`` file is compiled for ``--offload-arch=gfx950`` and every
``csrc/*.cpp`` file as host C++, in parallel, into ``_build/``; the objects are
linked into ``dense_fp16_gemm_hgemm_amd/libmi_hgemm.so``.  Packed fp32 VALU
instructions are disabled for all device code.

It also builds ``dense_fp16_gemm_hgemm_amd/libmi_overlap.so`` (the load/compute
overlap micro-benchmark, ``overlap/overlap.hip``),
``dense_fp16_gemm_hgemm_amd/libmi_ceiling.so`` (the MFMA, copy and HBM read
ceilings, ``ceiling/ceiling.hip``) and, where rocBLAS is
installed, ``dense_fp16_gemm_hgemm_amd/mi_hgemm_serve``, the server-mode load
generator (``serve/serve_bench.cpp``), linked against the library (found beside
it at run time) and rocBLAS (the vendor backend it compares with).  Without
rocBLAS the load generator is skipped with a note and the build still succeeds
(its tests then skip).

Usage: ``python dense_fp16_gemm_hgemm_amd/build.py`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libmi_hgemm.so")
OVERLAP_SRC = os.path.join(PKG, "overlap", "overlap.hip")
OVERLAP_PATH = os.path.join(PKG, "libmi_overlap.so")
CEILING_SRC = os.path.join(PKG, "ceiling", "ceiling.hip")
CEILING_PATH = os.path.join(PKG, "libmi_ceiling.so")
SERVE_SRC = os.path.join(PKG, "serve", "serve_bench.cpp")
SERVE_PATH = os.path.join(PKG, "mi_hgemm_serve")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCBLAS_HEADER = "/opt/rocm/include/rocblas/rocblas.h"
ROCBLAS_LIB = "/opt/rocm/lib/librocblas.so*"
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]
# The kernels index their accumulator and fragment arrays with loop counters
# that must become constants: every such loop is marked for full unrolling,
# and the threshold is raised so that the largest (64 MFMAs per half trip)
# are unrolled too instead of leaving the arrays in scratch memory.
DEVICE = ["--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-pragma-unroll-threshold=1000000",
          "-Wno-unused-command-line-argument"]


def _compile_cmds():
    cmds = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmds.append((src, obj, [HIPCC, *COMMON, *DEVICE, "-c", src, "-o", obj]))
    for src in sorted(glob.glob(os.path.join(CSRC, "*.cpp"))):
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmds.append((src, obj, [HIPCC, *COMMON, *DEVICE, "-x", "hip", "-c", src, "-o", obj]))
    return cmds


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    t0 = time.time()
    cmds = _compile_cmds()
    procs = []
    for src, obj, cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature flag; that note is harmless
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append(src)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    link = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp,
            *[obj for _, obj, _ in cmds], "-ldl"]
    subprocess.run(link, check=True)
    os.replace(tmp, LIB_PATH)
    tmp = OVERLAP_PATH + ".tmp%d" % os.getpid()
    # Every inner loop starts on a 64-byte boundary.  The modes' FMA loops are
    # the same nine instructions; left where the compiler put them, two of the
    # four straddled three 32-byte fetch blocks instead of two, and ran 1.15-1.22x
    # slower at high arithmetic intensity for that reason alone.
    r = subprocess.run([HIPCC, *COMMON, *DEVICE, "-falign-loops=64", "-shared", OVERLAP_SRC, "-o", tmp],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        print(r.stdout.decode(errors="replace"), file=sys.stderr)
        raise RuntimeError("hipcc failed for " + OVERLAP_SRC)
    os.replace(tmp, OVERLAP_PATH)
    # the MFMA probe's chains stay in their registers (no accumulator copies
    # between rounds) only with the VGPR form of the MFMA
    tmp = CEILING_PATH + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, *COMMON, *DEVICE, "-mllvm", "-amdgpu-mfma-vgpr-form", "-shared",
                        CEILING_SRC, "-o", tmp], stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        print(r.stdout.decode(errors="replace"), file=sys.stderr)
        raise RuntimeError("hipcc failed for " + CEILING_SRC)
    os.replace(tmp, CEILING_PATH)
    if not (os.path.exists(ROCBLAS_HEADER) and glob.glob(ROCBLAS_LIB)):
        print(f"note: rocBLAS not found ({ROCBLAS_HEADER}); the server-mode load generator "
              "(which compares with it) is not built", file=sys.stderr)
        if verbose:
            print(f"built {LIB_PATH} in {time.time() - t0:.1f}s", flush=True)
        return LIB_PATH
    tmp = SERVE_PATH + ".tmp%d" % os.getpid()
    serve = [HIPCC, *COMMON, *DEVICE, "-x", "hip", SERVE_SRC, "-x", "none", "-o", tmp,
             "-L", PKG, "-lmi_hgemm", "-L/opt/rocm/lib", "-lrocblas",
             "-Wl,-rpath,$ORIGIN", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(serve, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        print(r.stdout.decode(errors="replace"), file=sys.stderr)
        raise RuntimeError("hipcc failed for " + SERVE_SRC)
    os.replace(tmp, SERVE_PATH)
    if verbose:
        print(f"built {LIB_PATH} in {time.time() - t0:.1f}s", flush=True)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
