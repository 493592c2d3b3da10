"""GPU parity over the problems of the shape sweep, through the library's
dispatch (the shipped table's own entry for each grid shape).

By default every fifth problem (200 of the 1000); with MI_HGEMM_SWEEP_ALL=1
all 1000 (about 3 minutes on one MI355X with 16 host cores, most of it the
recipe's numpy draws of the operands).  Problems of at most 2^33
multiply-adds are compared element by element with the oracle's full product;
the larger ones on every element of the last row and the last column (the
ragged tails), the four corners and 4096 random entries.  Beside these,
test_gpu_parity.py checks 40 sweep problems and test_gpu_full_size.py the
largest sweep problem of every instance the dispatcher picks, every element.
"""
import os
import sys

import pytest
import torch

import oracle
from parity import check_tolerance, sample_indices

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

mh = pytest.importorskip("dense_fp16_gemm_hgemm_amd")
from dense_fp16_gemm_hgemm_amd import inputs  # noqa: E402

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
STRIDE = 1 if os.environ.get("MI_HGEMM_SWEEP_ALL") == "1" else 5

DEV = torch.device("cuda", 0)
FULL_MACS = 1 << 33


@pytest.fixture(scope="module")
def lib():
    h = mh.Hgemm()
    yield h
    h.close()


@pytest.mark.parametrize("p", inputs.sweep(1000)[::STRIDE], ids=lambda p: p.name)
def test_sweep_problem(lib, p):
    A, Bt = inputs.make(p)
    dA = torch.from_numpy(A).to(DEV)
    dB = torch.from_numpy(Bt).to(DEV)
    plan = lib.plan(dA, dB)
    print(f"{p.name}: {plan}", flush=True)
    sys.stdout.flush()
    got = lib.run(dA, dB).cpu().numpy()
    if p.M * p.N * p.K <= FULL_MACS:
        check_tolerance(got, oracle.hgemm_tn(A, Bt), f"{p.name} {plan[0]}")
    else:
        r, c = sample_indices(p.M, p.N, 4096, seed=p.seed)
        check_tolerance(got[r, c], oracle.hgemm_tn_entries(A, Bt, r, c), f"{p.name} {plan[0]}")
