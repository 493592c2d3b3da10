"""GPU parity of the int8 variant (int8 operands, exact int32 result), through
the C ABI, against the CPU oracle's exact integer GEMM.

Every comparison is exact equality: the sums are integers well inside int32
(|sum| <= 16384 K < 2^31 for K <= 131071), so any correct summation order gives
the same bits.  Sizes the oracle finishes in seconds are compared element by
element; the full benchmark sizes on sampled elements (corners, the last row
and column, and random entries).
"""
import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

mh = pytest.importorskip("dense_fp16_gemm_hgemm_amd")
from dense_fp16_gemm_hgemm_amd import inputs  # noqa: E402

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda", 0)
NAMES = mh.kernel_names()
I8_KIDX = [i for i, n in enumerate(NAMES) if n.startswith("i8_")]
SENTINEL = -1234567


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    h = mh.Hgemm()
    yield h
    h.close()


def gpu(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def padded_out(M, N, extra=0):
    """int32 C with ldc rounded up to a multiple of 4 (16 bytes) plus `extra`,
    filled with a sentinel so that stray writes show."""
    ldc = (N + 3) // 4 * 4 + extra
    full = torch.full((max(M, 1), ldc), SENTINEL, dtype=torch.int32, device=DEV)
    return full, full[:M, :N]


def problem(M, N, K, seed):
    return inputs.make(inputs.Problem(f"i8_{M}x{N}x{K}", M, N, K, "i8", seed=seed))


def check_exact(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    bad = np.flatnonzero(got.ravel() != want.ravel())
    if bad.size:
        t = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {got.size} elements differ; first flat "
                             f"index {t}: gpu {got.ravel()[t]} vs oracle {want.ravel()[t]}")


def check_padding(full, M, N, what):
    f = host(full)
    assert np.all(f[:M, N:] == SENTINEL), f"{what}: C's row padding was written"


# K a multiple of 16 (the int8 16-byte class), ragged against every tile and K step
SHAPES = [(64, 64, 128), (100, 130, 144), (17, 33, 48), (256, 256, 512), (300, 520, 1008),
          (1, 8, 16), (16, 4096, 256), (64, 200, 2064), (257, 129, 4112)]


@pytest.fixture(scope="module")
def cases():
    out = {}
    for (M, N, K) in SHAPES:
        A, Bt = problem(M, N, K, seed=M * 5 + N * 3 + K)
        out[(M, N, K)] = (A, Bt, oracle.igemm_tn(A, Bt))
    return out


@pytest.mark.parametrize("kidx", I8_KIDX, ids=[NAMES[i] for i in I8_KIDX])
def test_i8_every_instance_small_shapes(lib, cases, kidx):
    name = NAMES[kidx]
    for (M, N, K), (A, Bt, ref) in cases.items():
        for gm, xcd in ((1, 0), (8, 1)):
            what = f"{name} {M}x{N}x{K} raster=({gm},{xcd})"
            log(what)
            full, out = padded_out(M, N)
            lib.run_kernel(kidx, gpu(A), gpu(Bt), out, group_m=gm, xcd_remap=xcd)
            check_exact(host(out), ref, what)
            check_padding(full, M, N, what)


SPLIT_KIDX = [i for i in I8_KIDX if NAMES[i].startswith("i8_ktile")]


@pytest.mark.parametrize("kidx", SPLIT_KIDX, ids=[NAMES[i] for i in SPLIT_KIDX])
def test_i8_split_k_exact(lib, kidx):
    name = NAMES[kidx]
    for (M, N, K) in ((64, 256, 4096), (16, 512, 8192), (100, 300, 2064)):
        A, Bt = problem(M, N, K, seed=K + M)
        ref = oracle.igemm_tn(A, Bt)
        dA, dB = gpu(A), gpu(Bt)
        for sk in (2, 4, 8):
            what = f"{name} {M}x{N}x{K} split {sk}"
            log(what)
            full, out = padded_out(M, N)
            lib.run_kernel(kidx, dA, dB, out, split_k=sk)
            check_exact(host(out), ref, what)
            # a second launch right after: partials and counters start fresh
            full2, out2 = padded_out(M, N)
            lib.run_kernel(kidx, dA, dB, out2, split_k=sk)
            check_exact(host(out2), ref, what + " (second launch)")


@pytest.mark.parametrize("p", inputs.i8_llm(), ids=lambda p: p.name)
def test_i8_llm_shapes_dispatch(lib, p):
    A, Bt = inputs.make(p)
    log(f"{p.name} plan {lib.plan(gpu(A[:1]), gpu(Bt[:1]))}")
    got = host(lib.run_i8(gpu(A), gpu(Bt)))
    check_exact(got, oracle.igemm_tn(A, Bt), p.name)


@pytest.mark.slow
def test_i8_square_8192_every_element(lib):
    """The int8 8192^3 problem the benchmark times, every element exact."""
    p = inputs.i8_square()
    A, Bt = inputs.make(p)
    dA, dB = gpu(A), gpu(Bt)
    log(f"{p.name} plan {lib.plan(dA, dB)}")
    got = host(lib.run_i8(dA, dB))
    del dA, dB
    check_exact(got, oracle.igemm_tn(A, Bt), p.name)


def test_i8_misaligned_operands_take_the_elementwise_instance(lib):
    generic = NAMES.index("i8_generic_64x64_w2x2_m16")
    rng = np.random.default_rng(5)
    for (M, N, K, pad_a, pad_b, off) in ((33, 47, 77, 0, 0, 0), (64, 64, 64, 3, 0, 0),
                                         (40, 36, 1, 0, 0, 0), (64, 64, 64, 0, 0, 1)):
        Abig = rng.integers(-128, 128, size=(M, K + pad_a)).astype(np.int8)
        Bbig = rng.integers(-128, 128, size=(N, K + pad_b)).astype(np.int8)
        A, Bt = Abig[:, :K], Bbig[:, :K]
        ref = oracle.igemm_tn(A, Bt)
        dA = gpu(Abig)[:, :K]
        dB = gpu(Bbig)[:, :K]
        full = torch.full((M * (N + 1) + 8,), SENTINEL, dtype=torch.int32, device=DEV)
        out = full[off:off + M * N].view(M, N)
        what = f"{M}x{N}x{K} pad_a {pad_a} C offset {off}"
        log(what)
        assert NAMES.index(lib.plan(dA, dB, out)[0]) == generic, what
        lib.run_i8(dA, dB, out)
        check_exact(host(out), ref, what)
        f = host(full)
        assert np.all(f[:off] == SENTINEL) and np.all(f[off + M * N:] == SENTINEL), what


def test_i8_k_zero_and_empty(lib):
    full, out = padded_out(5, 7)
    lib.run_i8(torch.zeros((5, 0), dtype=torch.int8, device=DEV),
               torch.zeros((7, 0), dtype=torch.int8, device=DEV), out)
    assert np.all(host(out) == 0)
    check_padding(full, 5, 7, "K = 0")
    e = lib.run_i8(torch.zeros((0, 16), dtype=torch.int8, device=DEV),
                   torch.zeros((9, 16), dtype=torch.int8, device=DEV))
    assert tuple(e.shape) == (0, 9)


def test_i8_extreme_values_near_the_int32_limit(lib):
    """(-128)(-128) summed over K = 131056 (the largest multiple of 16 allowed)
    is 2147221504, and (-128)(127) over K gives the most negative sum; the
    vector and the element-wise paths both reach them exactly."""
    K = 131056
    A = torch.full((16, K), -128, dtype=torch.int8, device=DEV)
    Bt = torch.full((16, K), -128, dtype=torch.int8, device=DEV)
    Bt[8:] = 127
    want = np.empty((16, 16), np.int64)
    want[:, :8] = 16384 * K
    want[:, 8:] = -128 * 127 * K
    log(f"extremes plan {lib.plan(A, Bt)}")
    check_exact(host(lib.run_i8(A, Bt)), want, "dispatch")
    for name in ("i8_generic_64x64_w2x2_m16", "i8_ktile_16x64_w1x4_k512_s3"):
        log(f"extremes {name}")
        check_exact(host(lib.run_kernel(name, A, Bt)), want, name)
    with pytest.raises(mh.HgemmError):
        z = torch.zeros((4, 131072), dtype=torch.int8, device=DEV)
        lib.run_i8(z, z)


def test_i8_tuner_builds_a_table_entry(tmp_path):
    h = mh.Hgemm(table_path=str(tmp_path / "none.tsv"))
    try:
        M, N, K = 128, 512, 1024
        log("tune int8 128x512x1024")
        h.tune(M, N, K, mh.MI_HGEMM_TUNE_HEURISTIC | mh.MI_HGEMM_TUNE_INT8)
        assert h.table_size() == 1
        A, Bt = problem(M, N, K, seed=3)
        name, g, x, s = h.plan(gpu(A), gpu(Bt))
        assert name.startswith("i8_"), name
        check_exact(host(h.run_i8(gpu(A), gpu(Bt))), oracle.igemm_tn(A, Bt), f"tuned {name}")
        out = tmp_path / "t.tsv"
        h.save_table(str(out))
        assert " i8a16 " in out.read_text()
    finally:
        h.close()
