"""Seeded synthetic inputs for the TN half-precision GEMM.

This module only draws and casts random numbers; it holds none of the GEMM's
arithmetic, so both the GPU path and the CPU oracle may take their inputs from it.

Every operand is produced as binary16 by drawing binary64 values with numpy's
``default_rng(seed)`` (PCG64), scaling them, and casting with ``astype(float16)``
(round to nearest even).  A is drawn first, then B.  B is returned in its
storage form ``Bt`` (N rows of K halves = the column-major K x N matrix).

Workload families (the shapes and value distributions the benchmark names):
  * ``tiny``   (64, 4096, 64), randn * 1.0, seed 1
  * ``small``  (128, 2048, 128), randn * 1.0, seed 2; integer variant U{-4..4}, seed 3
  * ``sweep``  1000 problems, M, N, K each 2^U{6..13} (list seed 4), problem i
               seed 1000 + i, randn / sqrt(K)
  * ``llm``    M in {16, 64, 256, 1024} x (N, K) in {(4096, 4096), (11008, 4096),
               (4096, 11008), (14336, 4096)}; activations A = randn, weights
               B = randn * 0.02; problem index t uses seed 5 + t
  * ``square`` (8192, 8192, 8192), randn / sqrt(8192), seed 6

The int8 variant's operands (``kind="i8"``) are int8 uniform over [-128, 127],
drawn with ``rng.integers`` (A first, then B); ``i8_square`` is the 8192^3
problem with seed 7 and ``i8_llm`` the LLM shapes with seeds 40 + t.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

LLM_M = (16, 64, 256, 1024)
LLM_NK = ((4096, 4096), (11008, 4096), (4096, 11008), (14336, 4096))


@dataclasses.dataclass(frozen=True)
class Problem:
    """One GEMM problem: shape, value recipe and seed."""
    name: str
    M: int
    N: int
    K: int
    kind: str = "randn"      # "randn" | "int" | "identity" | "perm" | "i8"
    a_scale: float = 1.0
    b_scale: float = 1.0
    seed: int = 0

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def min_bytes(self) -> int:
        """A and B read once, C written once (beta = 0): binary16, or int8
        operands and an int32 result."""
        if self.kind == "i8":
            return self.M * self.K + self.N * self.K + 4 * self.M * self.N
        return 2 * (self.M * self.K + self.N * self.K + self.M * self.N)


def randn_f16(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float64)
    if scale != 1.0:
        x *= scale
    return x.astype(np.float16)


def int_f16(rng: np.random.Generator, shape, lo: int = -4, hi: int = 4) -> np.ndarray:
    """Uniform integers in [lo, hi] inclusive, stored exactly as binary16."""
    return rng.integers(lo, hi + 1, size=shape).astype(np.float16)


def int8_uniform(rng: np.random.Generator, shape) -> np.ndarray:
    """int8 values, every one of the 256 equally likely."""
    return rng.integers(-128, 128, size=shape).astype(np.int8)


def make(p: Problem) -> tuple[np.ndarray, np.ndarray]:
    """Materialise (A[M,K], Bt[N,K]) as contiguous float16 (int8 for kind "i8") arrays."""
    rng = np.random.default_rng(p.seed)
    if p.kind == "i8":
        A = int8_uniform(rng, (p.M, p.K))
        Bt = int8_uniform(rng, (p.N, p.K))
    elif p.kind == "randn":
        A = randn_f16(rng, (p.M, p.K), p.a_scale)
        Bt = randn_f16(rng, (p.N, p.K), p.b_scale)
    elif p.kind == "int":
        A = int_f16(rng, (p.M, p.K))
        Bt = int_f16(rng, (p.N, p.K))
    elif p.kind == "identity":
        # A = I (M == K); B random integers so every output value is distinct-ish.
        if p.M != p.K:
            raise ValueError("identity needs M == K")
        A = np.eye(p.M, dtype=np.float16)
        Bt = int_f16(rng, (p.N, p.K), -1000, 1000)
    elif p.kind == "perm":
        if p.M != p.K:
            raise ValueError("perm needs M == K")
        perm = rng.permutation(p.M)
        A = np.zeros((p.M, p.K), dtype=np.float16)
        A[np.arange(p.M), perm] = 1.0
        Bt = randn_f16(rng, (p.N, p.K), 1.0)
    else:
        raise ValueError(f"unknown kind {p.kind!r}")
    return A, Bt


def tiny() -> Problem:
    return Problem("tiny_64x4096x64", 64, 4096, 64, "randn", 1.0, 1.0, 1)


def small(integer: bool = False) -> Problem:
    if integer:
        return Problem("small_int_128x2048x128", 128, 2048, 128, "int", seed=3)
    return Problem("small_128x2048x128", 128, 2048, 128, "randn", 1.0, 1.0, 2)


def square(n: int = 8192) -> Problem:
    s = 1.0 / math.sqrt(n)
    return Problem(f"square_{n}", n, n, n, "randn", s, s, 6)


def llm() -> list[Problem]:
    out = []
    t = 0
    for m in LLM_M:
        for n, k in LLM_NK:
            out.append(Problem(f"llm_{m}x{n}x{k}", m, n, k, "randn", 1.0, 0.02, 5 + t))
            t += 1
    return out


def sweep(count: int = 1000) -> list[Problem]:
    rng = np.random.default_rng(4)
    e = rng.integers(6, 14, size=(count, 3))
    out = []
    for i in range(count):
        m, n, k = (1 << int(x) for x in e[i])
        s = 1.0 / math.sqrt(k)
        out.append(Problem(f"sweep{i}_{m}x{n}x{k}", m, n, k, "randn", s, s, 1000 + i))
    return out


def i8_square(n: int = 8192) -> Problem:
    return Problem(f"i8_square_{n}", n, n, n, "i8", seed=7)


def i8_llm() -> list[Problem]:
    out = []
    t = 0
    for m in LLM_M:
        for n, k in LLM_NK:
            out.append(Problem(f"i8_llm_{m}x{n}x{k}", m, n, k, "i8", seed=40 + t))
            t += 1
    return out


def all_named() -> list[Problem]:
    """Every distinct benchmark problem except the 1000-problem sweep."""
    return [tiny(), small(False), small(True)] + llm() + [square()]
