"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises ``AssertionError``
when the oracle disagrees with what the pages, the IEEE binary16 format or the
mathematics fix.  ``test_oracle_pins.py`` runs them on the real oracle and
``test_oracle_mutants.py`` runs them on copies with planted mistakes, each of
which must fail at least one pin.

Independent sources used here (none is the oracle's own code):
  * numpy's float16 <-> float64 casts (exhaustive over bit patterns),
  * ``fractions.Fraction`` exact sums and a binary16 rounding written below
    from the IEEE definition,
  * hand-worked cases in ``tests/golden/`` and textbook binary16 encodings,
  * closed forms (identity, permutation, small-integer inputs against an int64
    matmul), numpy's float64 matmul, and metamorphic identities.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ helpers --

def exact_to_f16_bits(q: Fraction) -> int:
    """Round an exact rational to binary16, ties to even (IEEE 754 binary16).

    Zero maps to +0 (an exactly cancelling sum started from +0 is +0)."""
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = -q if q < 0 else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(1, 1 << 24) if e < -14 else Fraction(2) ** (e - 10)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    if e < -14:
        return sign | fl                      # fl <= 1024; 1024 is the smallest normal
    if fl == 2048:
        fl, e = 1024, e + 1
    if e > 15:
        return sign | 0x7C00
    return sign | ((e + 15) << 10) | (fl - 1024)


def bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x).view(np.uint16)


def zero_sign_folded(b: np.ndarray) -> np.ndarray:
    """Bit patterns with -0 (0x8000) folded onto +0."""
    b = np.array(b, dtype=np.uint16, copy=True)
    b[b == 0x8000] = 0
    return b


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    g = zero_sign_folded(bits(got) if got.dtype == np.float16 else got)
    w = zero_sign_folded(bits(want) if want.dtype == np.float16 else want)
    bad = np.flatnonzero(g.ravel() != w.ravel())
    assert bad.size == 0, (f"{what}: {bad.size} mismatches, first at flat index "
                           f"{bad[0]}: got 0x{g.ravel()[bad[0]]:04X} want 0x{w.ravel()[bad[0]]:04X}")


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in binary16 steps between two finite float16 arrays."""
    def ordered(x):
        u = bits(x).astype(np.int32)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a) - ordered(b))


def random_finite_f16(rng, shape, exp_lo=0, exp_hi=30) -> np.ndarray:
    """Random finite binary16 values: uniform sign, exponent field in
    [exp_lo, exp_hi] and fraction; exponent field 0 gives zero/subnormals."""
    sign = rng.integers(0, 2, size=shape, dtype=np.uint16) << 15
    expo = rng.integers(exp_lo, exp_hi + 1, size=shape, dtype=np.uint16) << 10
    frac = rng.integers(0, 1024, size=shape, dtype=np.uint16)
    return (sign | expo | frac).astype(np.uint16).view(np.float16)


def load_golden_cases():
    cases = []
    cur = None
    with open(os.path.join(GOLDEN, "handworked_tn_hgemm.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tok = line.split()
            if tok[0] == "case":
                cur = {"name": tok[1], "M": int(tok[2]), "N": int(tok[3]),
                       "K": int(tok[4]), "A": [], "Bt": [], "C": []}
            elif tok[0] in ("A", "Bt"):
                cur[tok[0]].append([float(t) for t in tok[1:]])
            elif tok[0] == "C":
                cur["C"].append([int(t, 16) for t in tok[1:]])
            elif tok[0] == "end":
                M, N, K = cur["M"], cur["N"], cur["K"]
                A = np.array(cur["A"], dtype=np.float64).reshape(M, K)
                Bt = np.array(cur["Bt"], dtype=np.float64).reshape(N, K)
                cur["A"] = A.astype(np.float16)
                cur["Bt"] = Bt.astype(np.float16)
                # every listed operand value must be exact in binary16
                assert np.array_equal(cur["A"].astype(np.float64), A), cur["name"]
                assert np.array_equal(cur["Bt"].astype(np.float64), Bt), cur["name"]
                cur["C"] = np.array(cur["C"], dtype=np.uint16).reshape(M, N)
                cases.append(cur)
                cur = None
    return cases


def load_golden_encodings():
    out = []
    with open(os.path.join(GOLDEN, "binary16_encodings.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            v, b = line.split()
            out.append((float(v), int(b, 16)))
    return out


# --------------------------------------------------------------------- pins --

def pin_decode_exhaustive(orc):
    """Decoder agrees with numpy's float16 -> float64 on all 65536 patterns."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_to_f64(allbits)
    want = allbits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "NaN patterns differ"
    assert np.array_equal(got[~nan], want[~nan]), "decoded values differ"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), "zero signs differ"


def pin_encode_exhaustive(orc):
    """Encoder agrees with numpy's float64 -> float16 on every finite binary16
    value, every midpoint between neighbours and one binary64 ulp either side."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = allbits.view(np.float16).astype(np.float64)
    fin = np.isfinite(vals)
    assert np.array_equal(orc.f64_to_f16(vals[fin]), allbits[fin]), "round trip"
    pos = np.sort(np.unique(vals[fin & (vals >= 0)]))
    pos = np.append(pos, 65536.0)                     # the overflow neighbour
    mids = (pos[:-1] + pos[1:]) / 2.0                 # exact in binary64
    probes = np.concatenate([mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)])
    probes = np.concatenate([probes, -probes,
                             [1e-300, -1e-300, 5e-324, 1e300, -1e300, 70000.0, np.inf, -np.inf]])
    with np.errstate(over="ignore"):
        want = probes.astype(np.float16).view(np.uint16)
    got = orc.f64_to_f16(probes)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} encodings differ, e.g. {probes[bad[0]]!r}: " \
                          f"0x{got[bad[0]]:04X} vs 0x{want[bad[0]]:04X}"
    n = orc.f64_to_f16(np.array([np.nan, -np.nan]))
    assert all((x & 0x7C00) == 0x7C00 and (x & 0x3FF) for x in n), "NaN not kept"


def pin_encoding_golden(orc):
    """Textbook binary16 encodings and named boundary cases."""
    for v, b in load_golden_encodings():
        assert orc.f64_to_f16(np.array([v]))[0] == b, f"encode {v}"
        d = orc.f16_to_f64(np.array([b], dtype=np.uint16))[0]
        assert d == v and np.signbit(d) == np.signbit(v), f"decode 0x{b:04X}"
    named = {65504.0: 0x7BFF, 65519.99: 0x7BFF, 65520.0: 0x7C00,
             2.0 ** -24: 0x0001, 2.0 ** -25: 0x0000, 3 * 2.0 ** -26: 0x0001,
             1 + 2.0 ** -11: 0x3C00, 1 + 3 * 2.0 ** -11: 0x3C02,
             2.0 ** -14 - 2.0 ** -25: 0x0400, -(2.0 ** -25): 0x8000}
    for v, b in named.items():
        got = int(orc.f64_to_f16(np.array([v]))[0])
        assert got == b, f"named case {v!r}: 0x{got:04X} vs 0x{b:04X}"


def pin_handworked_golden(orc):
    """Hand-worked GEMM cases from tests/golden/handworked_tn_hgemm.txt."""
    for c in load_golden_cases():
        got = orc.hgemm_tn(c["A"], c["Bt"])
        assert np.array_equal(bits(got), c["C"]), \
            f"{c['name']}: got {bits(got)} want {c['C']}"


def pin_bruteforce_fraction(orc, trials: int = 60):
    """Tiny random GEMMs against exact rational sums rounded once.

    Operand exponents are limited to [2^-6, 2^8) so every partial sum is exact
    in binary64 (products keep 22 significant bits within a 2^-33..2^17 window);
    the oracle must then equal the exactly rounded sum bit for bit."""
    rng = np.random.default_rng(12345)
    for _ in range(trials):
        M, N, K = (int(x) for x in rng.integers(1, 7, size=3))
        A = random_finite_f16(rng, (M, K), 9, 22)
        Bt = random_finite_f16(rng, (N, K), 9, 22)
        A[rng.random((M, K)) < 0.1] = 0.0
        got = bits(orc.hgemm_tn(A, Bt))
        Aq = [[Fraction(float(x)) for x in r] for r in A]
        Bq = [[Fraction(float(x)) for x in r] for r in Bt]
        for i in range(M):
            for j in range(N):
                s = sum((Aq[i][k] * Bq[j][k] for k in range(K)), Fraction(0))
                want = exact_to_f16_bits(s)
                g = int(got[i, j])
                assert (g if g != 0x8000 else 0) == want, \
                    f"({M},{N},{K}) element ({i},{j}): 0x{g:04X} vs exact 0x{want:04X}"


def pin_identity(orc):
    """A = I (M = K): C is the logical K x N matrix B, C[i][j] = Bt[j][i]."""
    rng = np.random.default_rng(7)
    K, N = 48, 37
    Bt = random_finite_f16(rng, (N, K), 0, 30)          # subnormals to 65504
    C = orc.hgemm_tn(np.eye(K, dtype=np.float16), Bt)
    assert_bits_equal(C, Bt.T.copy(), "identity on the left")


def pin_identity_right(orc):
    """B = I (N = K): C = A."""
    rng = np.random.default_rng(8)
    M, K = 29, 40
    A = random_finite_f16(rng, (M, K), 0, 30)
    C = orc.hgemm_tn(A, np.eye(K, dtype=np.float16))
    assert_bits_equal(C, A, "identity on the right")


def pin_permutation(orc):
    """A a permutation matrix: C[i][j] = Bt[j][perm[i]]."""
    rng = np.random.default_rng(9)
    K, N = 64, 50
    perm = rng.permutation(K)
    A = np.zeros((K, K), dtype=np.float16)
    A[np.arange(K), perm] = 1.0
    Bt = random_finite_f16(rng, (N, K), 1, 29)
    C = orc.hgemm_tn(A, Bt)
    assert_bits_equal(C, Bt.T[perm, :].copy(), "permutation")


def pin_small_integer(orc):
    """Small-integer inputs equal an int64 matmul rounded once to binary16."""
    rng = np.random.default_rng(10)
    for (M, N, K) in ((33, 47, 130), (16, 24, 1000)):
        Ai = rng.integers(-4, 5, size=(M, K))
        Bi = rng.integers(-4, 5, size=(N, K))
        want = (Ai @ Bi.T).astype(np.float64).astype(np.float16)
        got = orc.hgemm_tn(Ai.astype(np.float16), Bi.astype(np.float16))
        assert_bits_equal(got, want, f"integers {M}x{N}x{K}")


def pin_numpy_crosscheck(orc):
    """numpy's float64 matmul, rounded to binary16, differs at most by one
    binary16 step and only rarely (near-ties, a different summation order)."""
    rng = np.random.default_rng(11)
    for (M, N, K) in ((37, 53, 301), (64, 64, 1024)):
        A = rng.standard_normal((M, K)).astype(np.float16)
        Bt = rng.standard_normal((N, K)).astype(np.float16)
        want = (A.astype(np.float64) @ Bt.astype(np.float64).T).astype(np.float16)
        got = orc.hgemm_tn(A, Bt)
        d = ulp_distance(got, want)
        assert d.max() <= 1, f"{M}x{N}x{K}: {d.max()} binary16 steps"
        assert np.count_nonzero(d) <= max(2, d.size // 1000), \
            f"{M}x{N}x{K}: {np.count_nonzero(d)} one-step differences"


def pin_metamorphic(orc):
    """Negating A negates C; scaling A by 2^3 scales C by 2^3 (normal range);
    swapping the operands' roles transposes C exactly."""
    rng = np.random.default_rng(12)
    M, N, K = 23, 31, 77
    A = rng.standard_normal((M, K)).astype(np.float16)
    Bt = rng.standard_normal((N, K)).astype(np.float16)
    C = orc.hgemm_tn(A, Bt)
    assert_bits_equal(orc.hgemm_tn(-A, Bt), -C, "negation")
    C8 = orc.hgemm_tn(A * np.float16(8), Bt).astype(np.float64)
    ok = (np.abs(C.astype(np.float64)) >= 2.0 ** -10) & (np.abs(C.astype(np.float64)) < 8000)
    assert np.array_equal(C8[ok], 8 * C.astype(np.float64)[ok]), "scaling by 2^3"
    assert_bits_equal(orc.hgemm_tn(Bt, A), C.T.copy(), "swapped roles")


def pin_strides(orc):
    """Padded leading dimensions give the contiguous result; C's padding is untouched."""
    rng = np.random.default_rng(13)
    M, N, K = 19, 26, 45
    Abig = rng.standard_normal((M, K + 5)).astype(np.float16)
    Bbig = rng.standard_normal((N, K + 3)).astype(np.float16)
    A, Bt = Abig[:, :K], Bbig[:, :K]
    want = orc.hgemm_tn(np.ascontiguousarray(A), np.ascontiguousarray(Bt))
    Cbig = np.full((M, N + 7), 1234.0, dtype=np.float16)
    orc.hgemm_tn(A, Bt, Cbig[:, :N])
    assert_bits_equal(Cbig[:, :N], want, "strided")
    assert np.all(Cbig[:, N:] == np.float16(1234.0)), "padding of C was written"


def pin_entries(orc):
    """Selected elements equal the full product; returned sums round to them."""
    rng = np.random.default_rng(14)
    M, N, K = 40, 70, 200
    A = rng.standard_normal((M, K)).astype(np.float16)
    Bt = rng.standard_normal((N, K)).astype(np.float16)
    full = orc.hgemm_tn(A, Bt)
    r = rng.integers(0, M, 300)
    c = rng.integers(0, N, 300)
    vals, sums = orc.hgemm_tn_entries(A, Bt, r, c, return_sums=True)
    assert_bits_equal(vals, full[r, c], "entries")
    assert_bits_equal(sums.astype(np.float16), full[r, c], "entry sums")


def pin_empty(orc):
    """Empty extents: M = 0 or N = 0 give empty C; K = 0 gives +0 everywhere."""
    z = np.zeros((0, 5), dtype=np.float16)
    assert orc.hgemm_tn(z, np.ones((3, 5), np.float16)).shape == (0, 3)
    assert orc.hgemm_tn(np.ones((3, 5), np.float16), z).shape == (3, 0)
    C = orc.hgemm_tn(np.zeros((4, 0), np.float16), np.zeros((6, 0), np.float16))
    assert np.array_equal(bits(C), np.zeros((4, 6), np.uint16))


# ------------------------------------------------------------ int8 variant --

def pin_i8_bruteforce(orc, trials: int = 80):
    """Tiny random int8 GEMMs (extremes -128 and 127 over-represented) against
    sums of Python integers."""
    rng = np.random.default_rng(21)
    for _ in range(trials):
        M, N, K = (int(x) for x in rng.integers(1, 7, size=3))
        A = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
        Bt = rng.integers(-128, 128, size=(N, K)).astype(np.int8)
        A[rng.random((M, K)) < 0.2] = -128
        Bt[rng.random((N, K)) < 0.2] = 127
        got = orc.igemm_tn(A, Bt)
        for i in range(M):
            for j in range(N):
                want = sum(int(A[i, k]) * int(Bt[j, k]) for k in range(K))
                assert int(got[i, j]) == want, f"({M},{N},{K}) ({i},{j}): {got[i, j]} vs {want}"


def pin_i8_closed_forms(orc):
    """All -128: every element is 16384 K; A = I: C = B; A a permutation:
    C[i][j] = Bt[j][perm[i]]; a column of ones sums the row of the other operand."""
    K, N = 96, 40
    A = np.full((5, K), -128, np.int8)
    Bt = np.full((7, K), -128, np.int8)
    assert np.all(orc.igemm_tn(A, Bt) == 16384 * K), "all -128"
    rng = np.random.default_rng(22)
    Bt = rng.integers(-128, 128, size=(N, K)).astype(np.int8)
    C = orc.igemm_tn(np.eye(K, dtype=np.int8), Bt)
    assert np.array_equal(C, Bt.T.astype(np.int32)), "identity"
    perm = rng.permutation(K)
    P = np.zeros((K, K), np.int8)
    P[np.arange(K), perm] = 1
    assert np.array_equal(orc.igemm_tn(P, Bt), Bt.T[perm, :].astype(np.int32)), "permutation"
    ones = np.ones((1, K), np.int8)
    assert np.array_equal(orc.igemm_tn(ones, Bt)[0], Bt.astype(np.int64).sum(axis=1)), "row sums"


def pin_i8_int32_limit(orc):
    """The largest sum, 16384 K with every product (-128)(-128): K = 131071 fits
    int32 (2147467264), K = 131072 reaches 2^31 and is reported."""
    A = np.full((1, 131071), -128, np.int8)
    assert int(orc.igemm_tn(A, A)[0, 0]) == 2147467264, "K = 131071"
    A = np.full((1, 131072), -128, np.int8)
    try:
        orc.igemm_tn(A, A)
    except OverflowError:
        pass
    else:
        raise AssertionError("a sum of 2^31 was not reported")
    B = np.full((1, 131072), 127, np.int8)
    assert int(orc.igemm_tn(A, B)[0, 0]) == -128 * 127 * 131072, "negative side fits"


def pin_i8_numpy_and_metamorphic(orc):
    """numpy's int64 matmul gives the same integers; swapping the operands
    transposes C; negating A (no -128 present) negates C."""
    rng = np.random.default_rng(23)
    M, N, K = 45, 61, 517
    A = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    Bt = rng.integers(-128, 128, size=(N, K)).astype(np.int8)
    C = orc.igemm_tn(A, Bt)
    assert np.array_equal(C, A.astype(np.int64) @ Bt.astype(np.int64).T), "numpy int64"
    assert np.array_equal(orc.igemm_tn(Bt, A), C.T), "swapped roles"
    assert np.array_equal(orc.igemm_tn(-A, Bt), -C), "negation"


def pin_i8_strides_entries_empty(orc):
    """Padded operands give the contiguous result and leave C's padding alone;
    selected entries equal the full product; empty extents; K = 0 gives 0."""
    rng = np.random.default_rng(24)
    M, N, K = 21, 33, 70
    Abig = rng.integers(-128, 128, size=(M, K + 9)).astype(np.int8)
    Bbig = rng.integers(-128, 128, size=(N, K + 2)).astype(np.int8)
    want = orc.igemm_tn(np.ascontiguousarray(Abig[:, :K]), np.ascontiguousarray(Bbig[:, :K]))
    Cbig = np.full((M, N + 5), 777, np.int32)
    orc.igemm_tn(Abig[:, :K], Bbig[:, :K], Cbig[:, :N])
    assert np.array_equal(Cbig[:, :N], want), "strided"
    assert np.all(Cbig[:, N:] == 777), "padding of C was written"
    r = rng.integers(0, M, 200)
    c = rng.integers(0, N, 200)
    assert np.array_equal(orc.igemm_tn_entries(Abig[:, :K], Bbig[:, :K], r, c), want[r, c]), \
        "entries"
    assert orc.igemm_tn(np.zeros((0, 4), np.int8), np.ones((3, 4), np.int8)).shape == (0, 3)
    assert np.array_equal(orc.igemm_tn(np.zeros((4, 0), np.int8), np.zeros((6, 0), np.int8)),
                          np.zeros((4, 6), np.int32)), "K = 0"


# ------------------------------------------------- overlap micro-benchmark --

def exact_to_f32(q: Fraction) -> float:
    """Round an exact rational to binary32, ties to even (IEEE 754 binary32),
    normal range only (the pins below stay there)."""
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert -126 <= e <= 127, "outside the normal binary32 range"
    scaled = a / Fraction(2) ** (e - 23)          # in [2^23, 2^24)
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return sign * float(Fraction(m) * Fraction(2) ** (e - 23))


def pin_fma_chain_bruteforce(orc):
    """Random binary32 inputs, constants and step counts: each step is the exact
    product-plus-addend rounded once to binary32 (a fused multiply-add)."""
    rng = np.random.default_rng(31)
    fused_differs = False
    for trial in range(40):
        x = (rng.uniform(-1, 1, 16) * 2.0 ** rng.integers(-8, 8, 16)).astype(np.float32)
        alpha = np.float32(rng.uniform(0.5, 1.5))
        beta = np.float32(rng.uniform(-1, 1))
        iters = int(rng.integers(1, 9))
        got = orc.fma_chain(x, iters, float(alpha), float(beta))
        for i in range(x.size):
            y = float(x[i])
            for _ in range(iters):
                y = exact_to_f32(Fraction(y) * Fraction(float(alpha)) + Fraction(float(beta)))
            assert float(got[i]) == y, f"trial {trial} element {i}: {got[i]!r} vs exact {y!r}"
            # the same steps with two roundings (multiply, then add) differ somewhere
            z = np.float32(x[i])
            for _ in range(iters):
                z = np.float32(np.float32(z * alpha) + beta)
            fused_differs |= bool(z != np.float32(y))
    assert fused_differs, "no case separates fused from unfused steps; the pin is too weak"


def pin_fma_chain_closed_forms(orc):
    """Zero steps and (alpha, beta) = (1, 0) leave x unchanged; (2, 0) multiplies
    by 2^k exactly; (0.5, 0.25) on dyadic inputs is exact: y_k = x/2^k + (1 - 2^-k)/2."""
    rng = np.random.default_rng(32)
    x = rng.uniform(-4, 4, 1000).astype(np.float32)
    assert np.array_equal(orc.fma_chain(x, 0, 0.3, 0.7).view(np.uint32), x.view(np.uint32))
    assert np.array_equal(orc.fma_chain(x, 17, 1.0, 0.0).view(np.uint32), x.view(np.uint32))
    assert np.array_equal(orc.fma_chain(x, 5, 2.0, 0.0), x * np.float32(32.0))
    xd = (rng.integers(-1024, 1024, 1000) / 256.0).astype(np.float32)
    for k in (1, 3, 6):
        want = xd.astype(np.float64) / 2 ** k + (1 - 2.0 ** -k) / 2
        assert np.array_equal(orc.fma_chain(xd, k, 0.5, 0.25).astype(np.float64), want), k


ALL_PINS = [
    pin_decode_exhaustive, pin_encode_exhaustive, pin_encoding_golden,
    pin_handworked_golden, pin_bruteforce_fraction, pin_identity, pin_identity_right,
    pin_permutation, pin_small_integer, pin_numpy_crosscheck, pin_metamorphic,
    pin_strides, pin_entries, pin_empty,
    pin_i8_bruteforce, pin_i8_closed_forms, pin_i8_int32_limit, pin_i8_numpy_and_metamorphic,
    pin_i8_strides_entries_empty, pin_fma_chain_bruteforce, pin_fma_chain_closed_forms,
]
