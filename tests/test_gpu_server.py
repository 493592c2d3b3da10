"""Server mode: the native load generator (mi_hgemm_serve) serves GEMM requests
through the library (and through rocBLAS, the vendor backend it compares with);
the requests' results must match the oracle, and the reported rates and
latencies must be consistent.  The load generator runs as a child process."""
import os

import numpy as np
import pytest

import oracle
from parity import check_tolerance

pytestmark = pytest.mark.gpu

server_mode = pytest.importorskip("dense_fp16_gemm_hgemm_amd.server_mode")

if not os.path.exists(server_mode.BINARY):
    pytest.skip("mi_hgemm_serve is not built", allow_module_level=True)


def load(d, name, shape):
    return np.fromfile(os.path.join(d, name), dtype=np.float16).reshape(shape)


@pytest.mark.parametrize("backend", ["mi_hgemm", "rocblas"])
@pytest.mark.parametrize("mnk", ["64_4096_64", "100_300_136"])
def test_served_results_match_the_oracle(tmp_path, backend, mnk):
    M, N, K = (int(x) for x in mnk.split("_"))
    print(f"serve {backend} {mnk}", flush=True)
    rec = server_mode.run(mnk, "poisson", qps=2000.0, requests=200, sets=4, backend=backend,
                          dump=str(tmp_path))
    A = load(tmp_path, "A.bin", (M, K))
    Bt = load(tmp_path, "B.bin", (N, K))
    C = load(tmp_path, "C.bin", (M, N))
    check_tolerance(C, oracle.hgemm_tn(A, Bt), f"served {backend} {mnk}")
    assert rec["requests"] == 200 and rec["backend"] == backend
    lat = rec["latency_us"]
    assert 0 < lat["p50"] <= lat["p90"] <= lat["p99"] <= lat["max"]


def test_target_rate_is_met():
    """At 100 requests/s the server keeps up: the achieved rate tracks the
    offered one and no request waits long."""
    print("serve poisson 100 qps", flush=True)
    rec = server_mode.run("64_4096_64", "poisson", qps=100.0, requests=100)
    assert abs(rec["achieved_qps"] - rec["offered_qps"]) <= 0.1 * rec["offered_qps"]
    assert rec["latency_us"]["p99"] < 5000.0


def test_closed_loop_sustains_far_more_than_the_target():
    print("serve closed depth 8", flush=True)
    rec = server_mode.run("64_4096_64", "closed", requests=5000, depth=8)
    assert rec["achieved_qps"] > 10000.0, rec
