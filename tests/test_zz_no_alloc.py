"""mi_hgemm_run_noalloc, the entry point that allocates nothing, against
mi_hgemm_run, through the C ABI.

Both entry points take the same dispatch; the no-allocation one keeps split-K
partial tiles and counters in the library's static device array instead of the
handle's workspace.  The shapes below are ones whose plan splits K, so the
array is what the launches actually use.  Integer operands must give the same
bits (fp32 sums of small integers are exact, whatever the split); random
operands must agree within the tolerance of tests/parity.py.  Two calls in a
row, the second on a smaller problem, check that the array's leftover partials
and counters from one call do not leak into the next.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from parity import check_bitexact, check_tolerance

pytestmark = pytest.mark.gpu

mh = pytest.importorskip("dense_fp16_gemm_hgemm_amd")
from dense_fp16_gemm_hgemm_amd import inputs  # noqa: E402

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda", 0)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def operands(M, N, K, kind, seed):
    s = 1.0 / np.sqrt(K)
    A, Bt = inputs.make(inputs.Problem(f"noalloc_{M}x{N}x{K}", M, N, K, kind, s, s, seed))
    return A, Bt


def call(fn, h, dA, dB, out):
    M, K = dA.shape
    N = dB.shape[0]
    st = fn(h, M, N, K, dA.data_ptr(), dA.stride(0), dB.data_ptr(), dB.stride(0),
            out.data_ptr(), out.stride(0), mh.MI_HGEMM_LAYOUT_TN,
            torch.cuda.current_stream().cuda_stream)
    assert st == mh.MI_HGEMM_OK, mh.mi_hgemm_status_string(st)


@pytest.fixture(scope="module")
def lib():
    h = mh.Hgemm()
    yield h
    h.close()


# first call larger than the second: 256x4096x11008 splits K four ways over 64
# tiles of 128x128 (exactly the array's 16 MiB of partials), 64x4096x4096 four
# ways over 64 tiles of 64x64
SHAPES = [(256, 4096, 11008), (64, 4096, 4096)]


@pytest.mark.parametrize("kind", ["int", "randn"])
def test_noalloc_matches_run_two_calls(lib, kind):
    for i, (M, N, K) in enumerate(SHAPES):
        log(f"noalloc {kind} {M}x{N}x{K}")
        A, Bt = operands(M, N, K, kind, seed=11 + i)
        dA, dB = torch.from_numpy(A).to(DEV), torch.from_numpy(Bt).to(DEV)
        plan = lib.plan(dA, dB)
        assert plan[3] > 1, f"{M}x{N}x{K} was meant to split K: {plan}"
        ref = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        out = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        call(mh.mi_hgemm_run, lib.handle, dA, dB, ref)
        call(mh.mi_hgemm_run_noalloc, lib.handle, dA, dB, out)
        torch.cuda.synchronize()
        got, want = out.cpu().numpy(), ref.cpu().numpy()
        what = f"noalloc {kind} {M}x{N}x{K} ({plan[0]} split {plan[3]})"
        if kind == "int":
            check_bitexact(got, want, what)
            if i == len(SHAPES) - 1:
                check_bitexact(got, oracle.hgemm_tn(A, Bt), what + " vs oracle")
        else:
            check_tolerance(got, want, what)
            if i == len(SHAPES) - 1:
                check_tolerance(got, oracle.hgemm_tn(A, Bt), what + " vs oracle")


def test_noalloc_split_beyond_the_array_is_reduced(tmp_path):
    """A table entry whose split needs 32 MiB of partials (64 tiles x 8 slices
    of 128x128 fp32) runs from the 16 MiB array with a smaller split, and still
    gives mi_hgemm_run's bits on integer operands."""
    M, N, K = 256, 4096, 8192
    table = tmp_path / "split8.tsv"
    table.write_text(f"gfx950 {M} {N} {K} TN a16 ktile_128x128_w2x4_k128_s3b2_sc 1 0 1.0 8\n")
    h = mh.Hgemm(str(table))
    try:
        A, Bt = operands(M, N, K, "int", seed=23)
        dA, dB = torch.from_numpy(A).to(DEV), torch.from_numpy(Bt).to(DEV)
        assert h.plan(dA, dB) == ("ktile_128x128_w2x4_k128_s3b2_sc", 1, 0, 8)
        ref = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        out = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        log(f"noalloc reduced split {M}x{N}x{K}")
        call(mh.mi_hgemm_run, h.handle, dA, dB, ref)
        call(mh.mi_hgemm_run_noalloc, h.handle, dA, dB, out)
        torch.cuda.synchronize()
        check_bitexact(out.cpu().numpy(), ref.cpu().numpy(), "reduced split")
    finally:
        h.close()


def test_noalloc_allocates_no_device_memory(lib):
    """With every tensor allocated beforehand, repeated calls leave the
    device's free memory unchanged."""
    M, N, K = 64, 4096, 4096
    A, Bt = operands(M, N, K, "randn", seed=31)
    dA, dB = torch.from_numpy(A).to(DEV), torch.from_numpy(Bt).to(DEV)
    out = torch.empty((M, N), dtype=torch.float16, device=DEV)
    call(mh.mi_hgemm_run_noalloc, lib.handle, dA, dB, out)  # first launch of these kernels
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info(DEV)
    for _ in range(20):
        call(mh.mi_hgemm_run_noalloc, lib.handle, dA, dB, out)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info(DEV)
    assert free1 == free0, f"free device memory changed by {free0 - free1} bytes"


def test_noalloc_edges_and_errors(lib):
    h = lib.handle
    A = torch.empty((5, 0), dtype=torch.float16, device=DEV)
    Bt = torch.empty((7, 0), dtype=torch.float16, device=DEV)
    out = torch.full((5, 7), float("nan"), dtype=torch.float16, device=DEV)
    st = mh.mi_hgemm_run_noalloc(h, 5, 7, 0, A.data_ptr(), 1, Bt.data_ptr(), 1, out.data_ptr(), 7)
    assert st == mh.MI_HGEMM_OK
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), np.zeros((5, 7), np.uint16))
    assert mh.mi_hgemm_run_noalloc(h, 0, 7, 4, 0, 4, 0, 4, 0, 7) == mh.MI_HGEMM_OK
    assert mh.mi_hgemm_run_noalloc(h, 4, 4, 4, 0, 4, 0, 4, 0, 4) == mh.MI_HGEMM_ERR_INVALID_ARG
    assert mh.mi_hgemm_run_noalloc(None, 4, 4, 4, 0, 4, 0, 4, 0, 4) == \
        mh.MI_HGEMM_ERR_INVALID_ARG
    assert mh.mi_hgemm_run_noalloc(h, 4, 4, 4, 16, 3, 4096, 4, 8192, 4) == \
        mh.MI_HGEMM_ERR_INVALID_ARG
