"""GPU parity at the benchmark's full sizes: every element of C against the oracle.

The large configurations are run through the library's own dispatch -- the
launch configuration the benchmark times -- and compared with the oracle's full
product, element by element: random operands within the tolerance of
tests/parity.py, integer operands U{-4..4} bit for bit (every partial sum is an
integer below 2^24 in magnitude, so fp32 accumulation is exact and both sides
round the same value once).  The oracle takes about 16 s for 8192^3 on 16 host
cores.

The shape sweep is covered by kernel: the shipped table and the built-in rules
map the 1000 sweep problems onto a handful of instances, and for each instance
the largest sweep problem it serves is checked in full.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from parity import check_bitexact, check_tolerance

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

mh = pytest.importorskip("dense_fp16_gemm_hgemm_amd")
from dense_fp16_gemm_hgemm_amd import inputs  # noqa: E402

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda", 0)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    h = mh.Hgemm()
    yield h
    h.close()


def run_full(lib, A, Bt):
    """C through the library's dispatch, the plan it used."""
    dA = torch.from_numpy(A).to(DEV)
    dB = torch.from_numpy(Bt).to(DEV)
    plan = lib.plan(dA, dB)
    out = lib.run(dA, dB)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    del dA, dB, out
    return got, plan


def test_square_8192_every_element_randn(lib):
    p = inputs.square()
    A, Bt = inputs.make(p)
    got, plan = run_full(lib, A, Bt)
    log(f"{p.name}: {plan}; oracle over all {p.M * p.N} outputs")
    check_tolerance(got, oracle.hgemm_tn(A, Bt), f"{p.name} {plan[0]}")


def test_square_8192_every_element_integer(lib):
    p = inputs.Problem("square_int_8192", 8192, 8192, 8192, "int", seed=61)
    A, Bt = inputs.make(p)
    got, plan = run_full(lib, A, Bt)
    log(f"{p.name}: {plan}; oracle over all {p.M * p.N} outputs")
    check_bitexact(got, oracle.hgemm_tn(A, Bt), f"{p.name} {plan[0]}")


LLM_LARGE = [p for p in inputs.llm() if p.M >= 256]


@pytest.mark.parametrize("p", LLM_LARGE, ids=lambda p: p.name)
def test_llm_every_element(lib, p):
    A, Bt = inputs.make(p)
    got, plan = run_full(lib, A, Bt)
    log(f"{p.name}: {plan}")
    check_tolerance(got, oracle.hgemm_tn(A, Bt), f"{p.name} {plan[0]}")


def sweep_largest_per_kernel():
    """For every instance the dispatcher picks over the 1000 sweep problems,
    the largest problem (by FLOPs) it is picked for.  Planned on an inspection
    handle with the shipped table and fake, 16-byte aligned addresses (contiguous
    operands are in the 16-byte class)."""
    st, h = mh.mi_hgemm_create_ex(None, mh.MI_HGEMM_CREATE_NO_DEVICE)
    assert st in (mh.MI_HGEMM_OK, mh.MI_HGEMM_WARN_TABLE_DEFAULTS)
    names = mh.kernel_names()
    base = 0x7F0000000000
    best = {}
    try:
        for p in inputs.sweep(1000):
            r = mh.mi_hgemm_plan(h, p.M, p.N, p.K, base, p.K, base + (1 << 36), p.K,
                                 base + (2 << 36), p.N)
            assert r[0] == mh.MI_HGEMM_OK
            k = names[r[1]]
            if k not in best or p.flops > best[k].flops:
                best[k] = p
    finally:
        mh.mi_hgemm_destroy(h)
    return sorted(best.values(), key=lambda p: p.flops)


@pytest.mark.parametrize("p", sweep_largest_per_kernel(), ids=lambda p: p.name)
def test_sweep_largest_problem_of_each_kernel(lib, p):
    A, Bt = inputs.make(p)
    got, plan = run_full(lib, A, Bt)
    log(f"{p.name}: {plan}")
    check_tolerance(got, oracle.hgemm_tn(A, Bt), f"{p.name} {plan[0]}")
