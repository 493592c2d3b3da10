"""Server-mode throughput of the library: the ``mi_hgemm_serve`` load generator.

"RL驱动CUDA L2 GEMM内核自动调优：A100/H100 tile size与融合优化" (blog.hotdry.top,
2025-12-05), 集成步骤, evaluates a kernel offline and as a server at a target
QPS (100 in its example, on the (64, 4096, 64) problem) and compares the QPS
with the vendor library's.  ``mi_hgemm_serve`` (built from
``serve/serve_bench.cpp`` by ``build.py``) generates that load natively: Poisson
arrivals at a target rate, or back-to-back requests with a bounded number in
flight, served in order on one HIP stream, through ``mi_hgemm_run`` or through
rocBLAS on the same operands.  This module runs it as a child process and
returns its JSON record.

    python -m dense_fp16_gemm_hgemm_amd.server_mode [--mnk 64_4096_64] [--qps 100]
        [--mode poisson|closed] [--requests N] [--depth D] [--backend mi_hgemm|rocblas]
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys

BINARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mi_hgemm_serve")


def run(mnk: str = "64_4096_64", mode: str = "poisson", qps: float = 100.0,
        requests: int = 1000, depth: int = 8, sets: int = 64, seed: int = 1,
        backend: str = "mi_hgemm", dump: str | None = None, timeout: float = 300.0) -> dict:
    """Run one server-mode measurement; returns the load generator's record."""
    if not os.path.exists(BINARY):
        raise FileNotFoundError(f"{BINARY} is not built: run `python dense_fp16_gemm_hgemm_amd/build.py`")
    cmd = [BINARY, "--mnk", mnk, "--mode", mode, "--qps", repr(float(qps)),
           "--requests", str(requests), "--depth", str(depth), "--sets", str(sets),
           "--seed", str(seed), "--backend", backend]
    if dump:
        cmd += ["--dump", dump]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, timeout=timeout)
    if r.returncode != 0:
        raise RuntimeError(f"mi_hgemm_serve failed ({r.returncode}): {r.stderr.decode(errors='replace')}")
    lines = [ln for ln in r.stdout.decode().splitlines() if ln.startswith("{")]
    return json.loads(lines[-1])


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--mnk", default="64_4096_64")
    ap.add_argument("--mode", default="poisson", choices=("poisson", "closed"))
    ap.add_argument("--qps", type=float, default=100.0)
    ap.add_argument("--requests", type=int, default=1000)
    ap.add_argument("--depth", type=int, default=8)
    ap.add_argument("--sets", type=int, default=64)
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--backend", default="mi_hgemm", choices=("mi_hgemm", "rocblas", "launch"))
    a = ap.parse_args(argv)
    print(json.dumps(run(a.mnk, a.mode, a.qps, a.requests, a.depth, a.sets, a.seed, a.backend)),
          flush=True)


if __name__ == "__main__":
    sys.exit(main())
