"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Every case draws seeded inputs from dense_fp16_gemm_hgemm_amd.inputs, runs the
GPU library, copies C back and compares with the oracle (tests/parity.py for
the rules), element by element.  The full benchmark sizes are compared in full
in tests/test_gpu_full_size.py; the sampled variants here (8192^3 and the
M >= 256 projection shapes on a few thousand entries) are the quick form.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from parity import check_bitexact, check_tolerance, sample_indices

pytestmark = pytest.mark.gpu

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


def gpu(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def padded_out(M, N):
    """C with ldc rounded up to a multiple of 8 (the 16-byte class), NaN-filled."""
    ldc = (N + 7) // 8 * 8
    return torch.full((M, ldc), float("nan"), dtype=torch.float16, device=DEV)[:, :N]


def rand_problem(M, N, K, kind="randn", seed=0, scale=None):
    s = (1.0 / np.sqrt(K)) if scale is None else scale
    p = inputs.Problem(f"case_{M}x{N}x{K}", M, N, K, kind, s, s, seed)
    return inputs.make(p)


SMALL_SHAPES = [(64, 64, 64), (100, 130, 72), (17, 33, 40), (256, 256, 512), (300, 520, 1000),
                (1, 8, 8), (16, 4096, 256), (64, 200, 2048)]


@pytest.fixture(scope="module")
def small_cases():
    cases = {}
    for (M, N, K) in SMALL_SHAPES:
        for kind in ("randn", "int"):
            A, Bt = rand_problem(M, N, K, kind, seed=M * 7 + N * 3 + K)
            cases[(M, N, K, kind)] = (A, Bt, oracle.hgemm_tn(A, Bt))
    return cases


# fp16 instances (the int8 ones are covered by test_gpu_int8.py)
F16_KIDX = [i for i, n in enumerate(mh.kernel_names()) if not n.startswith("i8_")]


@pytest.mark.parametrize("kidx", F16_KIDX, ids=[mh.kernel_names()[i] for i in F16_KIDX])
def test_every_instance_small_shapes(lib, small_cases, kidx):
    name = mh.kernel_names()[kidx]
    rasters = [(1, 0), (8, 1), (3, 1)] if name.startswith("tile_") else [(1, 0)]
    for (M, N, K, kind), (A, Bt, ref) in small_cases.items():
        dA, dB = gpu(A), gpu(Bt)
        for gm, xcd in rasters:
            log(f"{name} {M}x{N}x{K} {kind} raster=({gm},{xcd})")
            out = padded_out(M, N)
            lib.run_kernel(kidx, dA, dB, out, group_m=gm, xcd_remap=xcd)
            got = host(out)
            what = f"{name} {M}x{N}x{K} {kind} raster=({gm},{xcd})"
            if kind == "int":
                check_bitexact(got, ref, what)
            else:
                check_tolerance(got, ref, what)


LARGE_VARIANTS = [n for n in mh.kernel_names() if n.startswith("d2tile3p_") or n.endswith("_sc")]


@pytest.mark.parametrize("kernel", LARGE_VARIANTS)
@pytest.mark.parametrize("M,N,K,kind", [(4400, 4400, 200, "int"), (8192, 4352, 64, "randn"),
                                        (4352, 4400, 1000, "randn")])
def test_persistent_grid_walks_every_tile(lib, kernel, M, N, K, kind):
    """The persistent instance launches one workgroup per CU, and each walks
    several output tiles.  These shapes have 289-544 tiles of 256x256 against
    256 CUs, with ragged edges in M, N and K (200, 1000 are not multiples of
    64), so most workgroups carry a second or third tile through the
    prologue-overlapped transition.  The same shapes check the instances that
    stage C through LDS ("_sc") over many tiles and ragged edges.  Checked in
    full against the oracle."""
    A, Bt = rand_problem(M, N, K, kind, seed=M + N + K)
    log(f"persistent {kernel} {M}x{N}x{K} {kind}")
    full = padded_out(M, N)
    got = host(lib.run_kernel(kernel, gpu(A), gpu(Bt), full, group_m=4, xcd_remap=1))
    ref = oracle.hgemm_tn(A, Bt)
    if kind == "int":
        check_bitexact(got, ref, f"{kernel} {M}x{N}x{K}")
    else:
        check_tolerance(got, ref, f"{kernel} {M}x{N}x{K}")
    again = host(lib.run_kernel(kernel, gpu(A), gpu(Bt), padded_out(M, N), group_m=4, xcd_remap=1))
    assert np.array_equal(got.view(np.uint16), again.view(np.uint16)), "repeat differs"


def test_tiny_config_full(lib):
    p = inputs.tiny()
    A, Bt = inputs.make(p)
    log(f"{p.name}")
    got = host(lib.run(gpu(A), gpu(Bt)))
    check_tolerance(got, oracle.hgemm_tn(A, Bt), p.name)


@pytest.mark.parametrize("integer", [False, True], ids=["randn", "int"])
def test_small_config_full(lib, integer):
    p = inputs.small(integer)
    A, Bt = inputs.make(p)
    log(f"{p.name}")
    got = host(lib.run(gpu(A), gpu(Bt)))
    ref = oracle.hgemm_tn(A, Bt)
    if integer:
        check_bitexact(got, ref, p.name)
    else:
        check_tolerance(got, ref, p.name)


@pytest.mark.parametrize("p", inputs.llm(), ids=lambda p: p.name)
def test_llm_configs(lib, p):
    A, Bt = inputs.make(p)
    log(f"{p.name}")
    got = host(lib.run(gpu(A), gpu(Bt)))
    if p.M <= 64:
        check_tolerance(got, oracle.hgemm_tn(A, Bt), p.name)
    else:
        r, c = sample_indices(p.M, p.N, 4096, seed=p.seed)
        check_tolerance(got[r, c], oracle.hgemm_tn_entries(A, Bt, r, c), p.name)


@pytest.mark.slow
def test_square_8192_sampled(lib):
    p = inputs.square()
    A, Bt = inputs.make(p)
    log(f"{p.name}")
    got = host(lib.run(gpu(A), gpu(Bt)))
    r, c = sample_indices(p.M, p.N, 8192, seed=6)
    check_tolerance(got[r, c], oracle.hgemm_tn_entries(A, Bt, r, c), p.name)


INT_SHAPES = [(64, 4096, 64), (128, 2048, 128), (16, 4096, 4096), (64, 11008, 4096),
              (256, 4096, 11008), (1024, 14336, 4096), (8192, 8192, 8192)]


@pytest.mark.parametrize("shape", INT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_integer_variant_bitexact_every_config_shape(lib, shape):
    """U{-4..4} inputs: every partial sum is an integer below 2^24 in magnitude,
    so fp32 accumulation is exact and the result must equal the oracle bit for bit."""
    M, N, K = shape
    A, Bt = rand_problem(M, N, K, "int", seed=3 + M + N + K)
    log(f"int {M}x{N}x{K}")
    got = host(lib.run(gpu(A), gpu(Bt)))
    if M * N * K < 8192 ** 3:
        check_bitexact(got, oracle.hgemm_tn(A, Bt), f"int {shape}")
    else:   # every element of 8192^3 in tests/test_gpu_full_size.py
        r, c = sample_indices(M, N, 4096, seed=M)
        check_bitexact(got[r, c], oracle.hgemm_tn_entries(A, Bt, r, c), f"int {shape}")


@pytest.mark.parametrize("kind,M", [("identity", 128), ("identity", 256), ("perm", 128),
                                    ("perm", 256)])
def test_identity_and_permutation_bitexact(lib, kind, M):
    p = inputs.Problem(f"{kind}{M}", M, 2048, M, kind, seed=M)
    A, Bt = inputs.make(p)
    log(p.name)
    got = host(lib.run(gpu(A), gpu(Bt)))
    check_bitexact(got, oracle.hgemm_tn(A, Bt), p.name)


def test_k_zero_writes_zeros(lib):
    A = torch.empty((5, 0), dtype=torch.float16, device=DEV)
    Bt = torch.empty((7, 0), dtype=torch.float16, device=DEV)
    out = torch.full((5, 7), float("nan"), dtype=torch.float16, device=DEV)
    lib.run(A, Bt, out)
    got = host(out)
    assert np.array_equal(got.view(np.uint16), np.zeros((5, 7), np.uint16))


def test_empty_output_is_a_no_op(lib):
    A = torch.ones((0, 16), dtype=torch.float16, device=DEV)
    Bt = torch.ones((8, 16), dtype=torch.float16, device=DEV)
    assert lib.run(A, Bt).shape == (0, 8)


@pytest.mark.parametrize("M,N,K,pad_a,pad_b,pad_c,off", [
    (1, 1, 1, 0, 0, 0, 0),
    (33, 45, 70, 5, 3, 1, 0),      # K not a multiple of 8 and odd leading dims: element-wise path
    (64, 64, 64, 0, 0, 0, 1),      # operands offset by one element: misaligned
    (96, 130, 136, 8, 16, 6, 0),   # padded, aligned ld; N tail not a multiple of 4 in C
    (128, 128, 4104, 0, 0, 0, 0),  # K tail beyond a 64-multiple
    (48, 1000, 8, 0, 0, 0, 0),     # minimal K for the vector path
])
def test_edge_shapes_and_layouts(lib, M, N, K, pad_a, pad_b, pad_c, off):
    A, Bt = rand_problem(M, N, K, "randn", seed=K)
    ref = oracle.hgemm_tn(A, Bt)
    log(f"edge {M}x{N}x{K} pads=({pad_a},{pad_b},{pad_c}) off={off}")
    bigA = torch.zeros(M * (K + pad_a) + off + 8, dtype=torch.float16, device=DEV)
    bigB = torch.zeros(N * (K + pad_b) + off + 8, dtype=torch.float16, device=DEV)
    bigC = torch.full((M * (N + pad_c) + off + 8,), 7.0, dtype=torch.float16, device=DEV)
    dA = bigA[off:off + M * (K + pad_a)].view(M, K + pad_a)[:, :K]
    dB = bigB[off:off + N * (K + pad_b)].view(N, K + pad_b)[:, :K]
    dC = bigC[off:off + M * (N + pad_c)].view(M, N + pad_c)[:, :N]
    dA.copy_(gpu(A))
    dB.copy_(gpu(Bt))
    lib.run(dA, dB, dC)
    got = host(dC)
    check_tolerance(got, ref, f"edge {M}x{N}x{K}")
    full = host(bigC)
    mask = np.ones(full.shape, bool)
    view = np.arange(full.size)[off:off + M * (N + pad_c)].reshape(M, N + pad_c)[:, :N]
    mask[view.ravel()] = False
    assert np.all(full[mask] == np.float16(7.0)), "elements outside C were written"


def test_integer_ragged_bitexact_all_paths(lib):
    A, Bt = rand_problem(77, 93, 200, "int", seed=5)
    ref = oracle.hgemm_tn(A, Bt)
    for kidx in F16_KIDX:
        name = mh.kernel_names()[kidx]
        log(f"ragged int {name}")
        got = host(lib.run_kernel(kidx, gpu(A), gpu(Bt), padded_out(77, 93)))
        check_bitexact(got, ref, name)


def test_subnormal_inputs(lib):
    rng = np.random.default_rng(21)
    A = (rng.standard_normal((128, 512)) * 1e-4).astype(np.float16)   # many subnormal
    Bt = (rng.standard_normal((256, 512)) * 3.0).astype(np.float16)
    assert np.count_nonzero(np.abs(A) < 2.0 ** -14) > 1000
    got = host(lib.run(gpu(A), gpu(Bt)))
    check_tolerance(got, oracle.hgemm_tn(A, Bt), "subnormal inputs")


def _all_subnormal_bt(N, K):
    """Bt (N x K) holding every nonzero binary16 subnormal pattern -- 0x0001..0x03FF
    and 0x8001..0x83FF, 2046 of them -- once forwards and once backwards, zeros
    after that."""
    pats = np.concatenate([np.arange(0x0001, 0x0400), np.arange(0x8001, 0x8400)]).astype(np.uint16)
    assert N * K >= 2 * pats.size
    flat = np.zeros(N * K, np.uint16)
    flat[:pats.size] = pats
    flat[pats.size:2 * pats.size] = pats[::-1]
    return flat.reshape(N, K).view(np.float16)


@pytest.mark.parametrize("kidx", F16_KIDX, ids=[mh.kernel_names()[i] for i in F16_KIDX])
def test_subnormals_bitexact_every_instance(lib, kidx):
    """Whether the matrix cores keep binary16 subnormals, answered bit for bit.

    (a) A = I: C = B, so every subnormal input must come out unchanged
        (subnormal in, subnormal out: a flush of either shows as 0);
    (b) A = 1024 I: C = 1024 B, normal results of subnormal inputs (a flush of
        the inputs shows as 0);
    (c) normal inputs whose sums are subnormal: A, B = U{-4..4} * 2^-12 with
        K = 56, so every partial sum is a multiple of 2^-24 below 1024 * 2^-24
        in magnitude, exact in fp32 and in binary16 (a flush of the fp32 ->
        binary16 conversion shows as 0).
    Every product and sum is exact, so the oracle's single rounding and the
    GPU's must agree bit for bit."""
    name = mh.kernel_names()[kidx]
    K = 64
    Bt = _all_subnormal_bt(64, K)
    cases = []
    for scale in (1.0, 1024.0):
        A = (np.eye(K) * scale).astype(np.float16)
        cases.append((f"A={scale:g}*I", A, Bt))
    rng = np.random.default_rng(77)
    A3 = (rng.integers(-4, 5, (64, 56)) * 2.0 ** -12).astype(np.float16)
    B3 = (rng.integers(-4, 5, (72, 56)) * 2.0 ** -12).astype(np.float16)
    cases.append(("subnormal sums", A3, B3))
    for what, A, B in cases:
        log(f"subnormal {name} {what}")
        ref = oracle.hgemm_tn(A, B)
        if what == "A=1*I":
            assert np.array_equal(ref.view(np.uint16), B.T.view(np.uint16))
        if what == "subnormal sums":
            assert np.count_nonzero(np.abs(ref) < 2.0 ** -14) > ref.size // 2
        got = host(lib.run_kernel(kidx, gpu(A), gpu(B), padded_out(A.shape[0], B.shape[0])))
        check_bitexact(got, ref, f"{name} {what}")


STAGED_C = [n for n in mh.kernel_names() if n.endswith("_sc") or n.startswith("d2tile3p_")]


@pytest.mark.parametrize("kernel", STAGED_C)
@pytest.mark.parametrize("K", [64, 200], ids=["K64_nt_stores", "K200_cached_stores"])
def test_staged_c_leaves_padding_untouched(lib, kernel, K):
    """The instances that stage C through LDS (and the persistent grid) write
    whole 16-byte row chunks.  With N a multiple of 8, ldc = N + 8 and a ragged
    M, every element outside the M x N block -- the padding columns [N, ldc) of
    each row and the rows after M -- keeps its sentinel value.  K <= 128 takes
    the non-temporal stores, K > 128 the cached ones."""
    M, N = 300, 520
    ldc = N + 8
    A, Bt = rand_problem(M, N, K, "int", seed=K + M)
    buf = torch.full((M + 3, ldc), 7.0, dtype=torch.float16, device=DEV)
    out = buf[:M, :N]
    log(f"staged C padding {kernel} {M}x{N}x{K} ldc={ldc}")
    lib.run_kernel(kernel, gpu(A), gpu(Bt), out, group_m=4, xcd_remap=1)
    full = host(buf)
    check_bitexact(full[:M, :N], oracle.hgemm_tn(A, Bt), f"{kernel} K={K}")
    assert np.all(full[:M, N:] == np.float16(7.0)), "padding columns were written"
    assert np.all(full[M:] == np.float16(7.0)), "rows past M were written"


def test_overflow_to_infinity(lib):
    A = np.full((64, 64), 64.0, dtype=np.float16)
    Bt = np.full((64, 64), 32.0, dtype=np.float16)    # 64*64*32 = 131072 > 65504
    Bt[1::2] = -Bt[1::2]
    got = host(lib.run(gpu(A), gpu(Bt)))
    check_bitexact(got, oracle.hgemm_tn(A, Bt), "overflow")


def test_deterministic(lib):
    A, Bt = rand_problem(512, 1024, 2048, "randn", seed=9)
    dA, dB = gpu(A), gpu(Bt)
    first = host(lib.run(dA, dB)).view(np.uint16).copy()
    for _ in range(3):
        assert np.array_equal(host(lib.run(dA, dB)).view(np.uint16), first)


def test_runs_on_a_side_stream(lib):
    A, Bt = rand_problem(256, 384, 512, "int", seed=11)
    ref = oracle.hgemm_tn(A, Bt)
    s = torch.cuda.Stream()
    dA, dB = gpu(A), gpu(Bt)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = lib.run(dA, dB, stream=s)
    s.synchronize()
    check_bitexact(out.cpu().numpy(), ref, "side stream")


def test_invalid_arguments_raise(lib):
    A = torch.ones((4, 8), dtype=torch.float16, device=DEV)
    Bt = torch.ones((4, 8), dtype=torch.float16, device=DEV)
    st = mh.mi_hgemm_run(lib.handle, 4, 4, 8, A.data_ptr(), 4, Bt.data_ptr(), 8,
                         torch.empty(16, dtype=torch.float16, device=DEV).data_ptr(), 4)
    assert st == mh.MI_HGEMM_ERR_INVALID_ARG   # lda < K
    st = mh.mi_hgemm_run(lib.handle, 4, 4, 8, A.data_ptr(), 8, Bt.data_ptr(), 8,
                         A.data_ptr(), 4)
    assert st == mh.MI_HGEMM_ERR_INVALID_ARG   # C overlaps A
    with pytest.raises(mh.HgemmError) as ei:
        lib.tune(64, 64, 60)                   # K % 8 != 0: nothing to tune
    assert ei.value.status == mh.MI_HGEMM_ERR_UNSUPPORTED
    # the binding checks tensors before anything reaches the C ABI
    with pytest.raises(ValueError):
        lib.run(A, Bt, out=torch.empty((4, 4), dtype=torch.float16))       # out on the host
    with pytest.raises(ValueError):
        lib.run(A, Bt[:, :4].contiguous())                                # K mismatch
    with pytest.raises(TypeError):
        lib.run(A, Bt, out=torch.empty((4, 4), dtype=torch.float32, device=DEV))


def test_tuner_builds_a_table_entry(tmp_path):
    table = tmp_path / "tuned.tsv"
    h = mh.Hgemm(str(table))
    assert h.create_status == mh.MI_HGEMM_WARN_TABLE_DEFAULTS
    log("tune 192x640x320")
    h.tune(192, 640, 320, mh.MI_HGEMM_TUNE_EXHAUSTIVE | mh.MI_HGEMM_TUNE_PERSIST)
    assert h.table_size() == 1
    lines = [ln for ln in table.read_text().splitlines() if not ln.startswith("#")]
    assert len(lines) == 1 and lines[0].startswith("gfx950 192 640 320 TN a16 ")
    A, Bt = rand_problem(192, 640, 320, "randn", seed=4)
    dA, dB = gpu(A), gpu(Bt)
    name, _, _, _ = h.plan(dA, dB)
    assert name == lines[0].split()[6]
    check_tolerance(host(h.run(dA, dB)), oracle.hgemm_tn(A, Bt), "tuned")
    h2 = mh.Hgemm(str(table))
    assert h2.create_status == mh.MI_HGEMM_OK and h2.table_size() == 1
    h.close()
    h2.close()


SPLIT_CASES = [(256, 512, 4096, 2), (256, 512, 4096, 4), (200, 300, 2560, 3), (128, 256, 1000, 4),
               (64, 128, 8192, 8), (256, 4096, 4096, 4)]
SPLIT_KERNELS = ["dtile_128x128_w2x2_m16_s4", "dtile_256x128_w2x2_m16_s4",
                 "dtile_128x256_w2x2_m16_s4", "skinny_1x4_w4_u2", "skinny_2x2_w4_u4",
                 "skinny_4x1_w8_u2", "ktile_16x64_w1x4_k256_s3", "ktile_64x64_w2x2_k128_s3",
                 "ktile_128x128_w2x2_k128_s2", "ktile_128x128_w2x4_k128_s3b2",
                 "ktile_16x64_w1x4_k256_s3_nt", "ktile_64x64_w2x2_k128_s3_nt",
                 "ktile_128x128_w2x4_k128_s3b2_noxor", "ktile_128x128_w2x4_k128_s3b2_sc",
                 "ktile_64x64_w2x2_k128_s3b3_sc", "pp2tile_256x256_w8_m16_sc_sk",
                 "pp2tile_256x128_w8_m16_sc_sk"]


@pytest.mark.parametrize("kernel", SPLIT_KERNELS)
@pytest.mark.parametrize("M,N,K,sk", SPLIT_CASES, ids=lambda v: str(v))
def test_split_k_integer_bitexact(lib, kernel, M, N, K, sk):
    """Split-K sums fp32 partial tiles; on integer inputs every partial and
    total is exact, so the result must equal the oracle bit for bit."""
    A, Bt = rand_problem(M, N, K, "int", seed=M + N + K + sk)
    log(f"split-K {kernel} {M}x{N}x{K} s={sk}")
    got = host(lib.run_kernel(kernel, gpu(A), gpu(Bt), padded_out(M, N), split_k=sk))
    if M * N * K <= 256 * 512 * 4096:
        check_bitexact(got, oracle.hgemm_tn(A, Bt), f"split {sk}")
    else:
        r, c = sample_indices(M, N, 4096, seed=sk)
        check_bitexact(got[r, c], oracle.hgemm_tn_entries(A, Bt, r, c), f"split {sk}")


@pytest.mark.parametrize("kernel", SPLIT_KERNELS)
def test_split_k_back_to_back_fresh_partials(lib, kernel):
    """Consecutive launches of one geometry reuse the same workspace slots and
    counters.  With different inputs each launch must read the partials of
    its own slices, not those the previous launch left behind."""
    M, N, K, sk = 256, 1024, 4096, 4
    probs = [rand_problem(M, N, K, "int", seed=s) for s in (11, 12, 13)]
    outs = [padded_out(M, N) for _ in probs]
    dev = [(gpu(A), gpu(Bt)) for A, Bt in probs]
    log(f"split-K back-to-back {kernel} {M}x{N}x{K} s={sk}")
    for (dA, dB), out in zip(dev, outs):   # no synchronisation in between
        lib.run_kernel(kernel, dA, dB, out, split_k=sk)
    for i, ((A, Bt), out) in enumerate(zip(probs, outs)):
        check_bitexact(host(out), oracle.hgemm_tn(A, Bt), f"launch {i}")


def test_split_k_dispatch_randn_deterministic(tmp_path):
    """The built-in dispatch (no table) splits K for 64x4096x11008; results are
    within tolerance and identical over repeated launches (fixed summation
    order, counters reset)."""
    p = inputs.llm()[6]          # M = 64, (N, K) = (4096, 11008)
    assert (p.M, p.N, p.K) == (64, 4096, 11008)
    A, Bt = inputs.make(p)
    dA, dB = gpu(A), gpu(Bt)
    h = mh.Hgemm(table_path=str(tmp_path / "absent.tsv"))
    try:
        name, _, _, sk = h.plan(dA, dB)
        log(f"dispatch {p.name}: {name} split {sk}")
        assert sk > 1
        first = host(h.run(dA, dB))
        for _ in range(3):
            assert np.array_equal(host(h.run(dA, dB)).view(np.uint16), first.view(np.uint16))
    finally:
        h.close()
    r, c = sample_indices(p.M, p.N, 4096, seed=1)
    check_tolerance(first[r, c], oracle.hgemm_tn_entries(A, Bt, r, c), p.name)


# --- the shape sweep and maximum sizes -------------------------------------------------------

def _sweep_sample():
    """Every 10th problem of the 1000-problem sweep whose operands stay below 2^26
    elements each (the seeded generator then runs in seconds), 40 at most."""
    out = []
    for i, p in enumerate(inputs.sweep(1000)):
        if i % 10 == 0 and p.M * p.K <= (1 << 26) and p.N * p.K <= (1 << 26):
            out.append(p)
    return out[:40]


@pytest.mark.parametrize("p", _sweep_sample(), ids=lambda p: p.name)
def test_shape_sweep_sample(lib, p):
    """Sweep problems through the dispatcher (table, nearest entry or heuristic,
    whichever the shape reaches): every element within tolerance."""
    A, Bt = inputs.make(p)
    dA, dB = gpu(A), gpu(Bt)
    log(f"sweep {p.name}: {lib.plan(dA, dB)}")
    got = host(lib.run(dA, dB))
    check_tolerance(got, oracle.hgemm_tn(A, Bt), p.name)


@pytest.mark.parametrize("M,N,K", [(1000, 3000, 520), (100, 7000, 4104), (5000, 304, 3000),
                                   (70, 9000, 1504), (600, 600, 6000), (3000, 3000, 200),
                                   (3000, 200, 3000), (48, 11000, 700)])
def test_off_grid_shapes_through_dispatch(lib, M, N, K):
    """Shapes between the tuned grid's points run the nearest tuned shape's
    configuration (or the built-in rules when none is within a factor of two):
    every element within tolerance, with ragged tails in M, N and K."""
    A, Bt = rand_problem(M, N, K, "randn", seed=M + 3 * N + 7 * K)
    dA, dB = gpu(A), gpu(Bt)
    log(f"off-grid {M}x{N}x{K}: {lib.plan(dA, dB)}")
    check_tolerance(host(lib.run(dA, dB)), oracle.hgemm_tn(A, Bt), f"off-grid {M}x{N}x{K}")


@pytest.mark.parametrize("M,N", [(128, 256), (64, 64)])
def test_long_k_integer_bitexact(lib, M, N):
    """K = 65536: every partial sum of small integers is exact in fp32 (|sum| <
    2^24), so the dispatcher's result (split K or not) equals the oracle's bit
    for bit, rounding of large sums to fp16 included."""
    K = 65536
    A, Bt = rand_problem(M, N, K, "int", seed=M + N)
    log(f"long K {M}x{N}x{K}: {lib.plan(gpu(A), gpu(Bt))}")
    got = host(lib.run(gpu(A), gpu(Bt)))
    check_bitexact(got, oracle.hgemm_tn(A, Bt), "K=65536")


@pytest.mark.parametrize("ld,vector", [(1 << 21, True), ((1 << 21) + 8, False)])
def test_leading_dimension_at_the_vector_limit(lib, ld, vector):
    """lda = ldb = 2^21 is the largest leading dimension of the vector path;
    one more multiple of 8 falls back to the element-wise instance.  Both give
    the oracle's result (integer inputs, bit-exact)."""
    M, N, K = 16, 64, 256
    A, Bt = rand_problem(M, N, K, "int", seed=ld % 97)
    a = torch.zeros((M, ld), dtype=torch.float16, device=DEV)
    b = torch.zeros((N, ld), dtype=torch.float16, device=DEV)
    a[:, :K] = gpu(A)
    b[:, :K] = gpu(Bt)
    av, bv = a[:, :K], b[:, :K]
    name = lib.plan(av, bv)[0]
    log(f"ld {ld}: {name}")
    assert (name != mh.kernel_names()[0]) == vector
    got = host(lib.run(av, bv))
    check_bitexact(got, oracle.hgemm_tn(A, Bt), f"ld={ld}")
