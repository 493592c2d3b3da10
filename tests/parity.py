"""Comparison rules between the GPU path and the CPU oracle.

Bit-exact (integer, identity and permutation inputs, where fp32 accumulation
is exact and both sides round the same value once): equal binary16 patterns,
+0 and -0 counted equal (accumulators start at +0 on both sides).

Tolerance (random inputs), per element and in aggregate, with ref the oracle's
binary16 result taken as float64:
    |gpu - ref| <= 1e-3 * max|ref| + 2e-3 * |ref|
    ||gpu - ref||_F / ||ref||_F <= 1e-3
Infinite and NaN reference values must be matched exactly.  When only sampled
elements are compared, max|ref| and the norms are taken over the sample.
"""
from __future__ import annotations

import numpy as np

ABS_REL = 1e-3     # times max|ref|
ELEM_REL = 2e-3    # times |ref|
FROB_REL = 1e-3


def f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float16).view(np.uint16)


def check_bitexact(got: np.ndarray, want: np.ndarray, what: str = ""):
    g = f16_bits(got).copy()
    w = f16_bits(want).copy()
    g[g == 0x8000] = 0
    w[w == 0x8000] = 0
    bad = np.flatnonzero(g.ravel() != w.ravel())
    if bad.size:
        t = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {g.size} elements differ; first flat index "
                             f"{t}: gpu 0x{g.ravel()[t]:04X} ({got.ravel()[t]}) vs oracle "
                             f"0x{w.ravel()[t]:04X} ({want.ravel()[t]})")


def check_tolerance(got: np.ndarray, want: np.ndarray, what: str = ""):
    g = np.asarray(got, dtype=np.float16).astype(np.float64).ravel()
    r = np.asarray(want, dtype=np.float16).astype(np.float64).ravel()
    nonfinite = ~np.isfinite(r)
    if nonfinite.any():
        rn, gn = r[nonfinite], g[nonfinite]
        nan = np.isnan(rn)
        assert np.all(np.isnan(gn[nan])), f"{what}: oracle NaN not matched"
        assert np.array_equal(gn[~nan], rn[~nan]), f"{what}: oracle infinity not matched"
    fin = ~nonfinite
    g, r = g[fin], r[fin]
    assert np.all(np.isfinite(g)), f"{what}: GPU produced non-finite values where the oracle did not"
    if r.size == 0:
        return
    bound = ABS_REL * np.max(np.abs(r)) + ELEM_REL * np.abs(r)
    err = np.abs(g - r)
    worst = int(np.argmax(err - bound))
    assert np.all(err <= bound), (f"{what}: element bound exceeded at {worst}: gpu {g[worst]} "
                                  f"oracle {r[worst]} err {err[worst]:.3e} bound {bound[worst]:.3e}")
    nr = np.linalg.norm(r)
    if nr > 0:
        frob = np.linalg.norm(g - r) / nr
        assert frob <= FROB_REL, f"{what}: Frobenius relative error {frob:.3e} > {FROB_REL}"


def sample_indices(M: int, N: int, count: int, seed: int = 0):
    """Random (row, col) pairs plus the four corners and the last row and column
    (the ragged tails), as int64 arrays."""
    rng = np.random.default_rng(seed)
    r = [rng.integers(0, M, count), np.array([0, 0, M - 1, M - 1]), np.full(N, M - 1),
         np.arange(M)]
    c = [rng.integers(0, N, count), np.array([0, N - 1, 0, N - 1]), np.arange(N), np.full(M, N - 1)]
    return np.concatenate(r).astype(np.int64), np.concatenate(c).astype(np.int64)
