"""CPU oracle for the TN half-precision GEMM.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never import it, and the two share no code.

The arithmetic lives in ``ref_hgemm.c`` (plain C, binary64 accumulation in index
order, one round-to-nearest-even to binary16); this module only compiles it with
gcc and marshals numpy arrays through ctypes.  The operation follows
"RL驱动CUDA L2 GEMM内核自动调优：A100/H100 tile size与融合优化" (blog.hotdry.top),
正文 paragraphs 1 and 3: a half-precision GEMM with row-major A and column-major
B ("TN").  With B column-major K x N, its storage is N rows of K halves, i.e. the
``Bt`` array below, and ``C = A @ Bt.T``.

``igemm_tn`` is the int8 variant: the exact integer sum of int8 products,
stored as int32 (the INT8 mode of the same page's 正文 paragraph 3; the page
leaves the result type open and the exact int32 sum is the reading taken).

``fma_chain`` is the arithmetic of the load/compute overlap micro-benchmark:
every element after ``fma_iters`` steps of ``y = fmaf(y, alpha, beta)``, one
binary32 rounding per step ("B-08. Hopper TMA：从单线程 Bulk Copy 到吞吐墙"
(lqnn.cn) §5, the FMA-iterations intensity knob).

Parity pins for every function here live in ``tests/test_oracle_pins.py``; no
function of the oracle is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "ref_hgemm.c")
LIB_PATH = os.path.join(_HERE, "libref_hgemm.so")
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC"]


def compile_source(src: str, out: str) -> str:
    """Compile an oracle C source file into a shared library at ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile ``ref_hgemm.c`` into ``oracle/libref_hgemm.so`` when stale."""
    if force or not os.path.exists(LIB_PATH) or (
        os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE)
    ):
        compile_source(SOURCE, LIB_PATH)
    return LIB_PATH


def _as_rows(x: np.ndarray, name: str, dtype=np.float16) -> tuple[np.ndarray, int]:
    """(array, leading dimension in elements) for a 2-D array of ``dtype`` whose
    rows may be padded (row stride >= row length) but whose elements are unit-stride."""
    if x.ndim != 2:
        raise ValueError(f"{name} must be 2-D")
    if x.dtype != dtype:
        raise TypeError(f"{name} must be {np.dtype(dtype).name}, got {x.dtype}")
    es = x.itemsize
    rows, cols = x.shape
    if rows <= 1:
        return x if x.flags.c_contiguous else np.ascontiguousarray(x), max(cols, 1)
    if (cols > 1 and x.strides[1] != es) or x.strides[0] % es or x.strides[0] // es < cols:
        x = np.ascontiguousarray(x)
    return x, int(x.strides[0] // es)


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, lib_path: str | None = None):
        if lib_path is None:
            lib_path = build()
        lib = ctypes.CDLL(lib_path)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.ref_f16_to_f64.restype = ctypes.c_double
        lib.ref_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.ref_f64_to_f16.restype = ctypes.c_uint16
        lib.ref_f64_to_f16.argtypes = [ctypes.c_double]
        lib.ref_f16_to_f64_array.argtypes = [p, p, i64]
        lib.ref_f64_to_f16_array.argtypes = [p, p, i64]
        lib.ref_hgemm_tn.restype = ctypes.c_int
        lib.ref_hgemm_tn.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64]
        lib.ref_hgemm_tn_entries.restype = ctypes.c_int
        lib.ref_hgemm_tn_entries.argtypes = [i64, i64, i64, p, i64, p, i64,
                                             i64, p, p, p, p]
        lib.ref_igemm_tn.restype = ctypes.c_int
        lib.ref_igemm_tn.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64]
        lib.ref_igemm_tn_entries.restype = ctypes.c_int
        lib.ref_igemm_tn_entries.argtypes = [i64, i64, i64, p, i64, p, i64, i64, p, p, p]
        lib.ref_fma_chain.restype = ctypes.c_int
        lib.ref_fma_chain.argtypes = [p, p, i64, ctypes.c_int32, ctypes.c_float, ctypes.c_float]
        lib.ref_num_threads.restype = ctypes.c_int
        lib.ref_set_num_threads.restype = None
        lib.ref_set_num_threads.argtypes = [ctypes.c_int]
        self.lib = lib
        self.path = lib_path

    def f16_to_f64(self, bits: np.ndarray) -> np.ndarray:
        """Decode binary16 bit patterns (uint16) exactly to float64."""
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, dtype=np.float64)
        self.lib.ref_f16_to_f64_array(bits.ctypes.data, out.ctypes.data, bits.size)
        return out

    def f64_to_f16(self, x: np.ndarray) -> np.ndarray:
        """Round float64 values to binary16, ties to even; returns uint16 bit patterns."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.ref_f64_to_f16_array(x.ctypes.data, out.ctypes.data, x.size)
        return out

    def hgemm_tn(self, A: np.ndarray, Bt: np.ndarray,
                 C: np.ndarray | None = None) -> np.ndarray:
        """C[M,N] = fp16_rne(A[M,K] @ Bt[N,K].T), summed in binary64 in k order.

        ``A``/``Bt`` are float16 with unit-stride rows (row padding allowed).
        A given ``C`` (float16, unit-stride rows, possibly a padded view) is
        written in place; elements outside the M x N block are not touched.
        """
        A, lda = _as_rows(A, "A")
        Bt, ldb = _as_rows(Bt, "Bt")
        M, K = A.shape
        N, K2 = Bt.shape
        if K != K2:
            raise ValueError(f"K mismatch: A has {K}, Bt has {K2}")
        if C is None:
            C = np.empty((M, N), dtype=np.float16)
        if M == 0 or N == 0:
            if C.shape != (M, N):
                raise ValueError("C must have shape (M, N)")
            return C
        if C.shape != (M, N) or C.dtype != np.float16 or (N > 1 and C.strides[1] != 2):
            raise ValueError("C must be a float16 (M, N) array with unit-stride rows")
        ldc = C.strides[0] // 2 if M > 1 else max(N, 1)
        rc = self.lib.ref_hgemm_tn(M, N, K, A.ctypes.data, lda, Bt.ctypes.data, ldb,
                                   C.ctypes.data, ldc)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return C

    def hgemm_tn_entries(self, A: np.ndarray, Bt: np.ndarray, rows, cols,
                         return_sums: bool = False):
        """Elements (rows[t], cols[t]) of ``hgemm_tn(A, Bt)`` as float16; with
        ``return_sums`` also the unrounded binary64 sums."""
        A, lda = _as_rows(A, "A")
        Bt, ldb = _as_rows(Bt, "Bt")
        M, K = A.shape
        N, K2 = Bt.shape
        if K != K2:
            raise ValueError(f"K mismatch: A has {K}, Bt has {K2}")
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if rows.shape != cols.shape:
            raise ValueError("rows and cols must have the same shape")
        out = np.empty(rows.shape, dtype=np.uint16)
        sums = np.empty(rows.shape, dtype=np.float64) if return_sums else None
        rc = self.lib.ref_hgemm_tn_entries(
            M, N, K, A.ctypes.data, lda, Bt.ctypes.data, ldb, rows.size,
            rows.ctypes.data, cols.ctypes.data, out.ctypes.data,
            sums.ctypes.data if sums is not None else None)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        vals = out.view(np.float16)
        return (vals, sums) if return_sums else vals

    def igemm_tn(self, A: np.ndarray, Bt: np.ndarray,
                 C: np.ndarray | None = None) -> np.ndarray:
        """C[M,N] = A[M,K] @ Bt[N,K].T for int8 operands, exact, as int32.

        Raises OverflowError when a sum does not fit int32.  A given ``C``
        (int32, unit-stride rows, possibly a padded view) is written in place.
        """
        A, lda = _as_rows(A, "A", np.int8)
        Bt, ldb = _as_rows(Bt, "Bt", np.int8)
        M, K = A.shape
        N, K2 = Bt.shape
        if K != K2:
            raise ValueError(f"K mismatch: A has {K}, Bt has {K2}")
        if C is None:
            C = np.empty((M, N), dtype=np.int32)
        if M == 0 or N == 0:
            if C.shape != (M, N):
                raise ValueError("C must have shape (M, N)")
            return C
        if C.shape != (M, N) or C.dtype != np.int32 or (N > 1 and C.strides[1] != 4):
            raise ValueError("C must be an int32 (M, N) array with unit-stride rows")
        ldc = C.strides[0] // 4 if M > 1 else max(N, 1)
        rc = self.lib.ref_igemm_tn(M, N, K, A.ctypes.data, lda, Bt.ctypes.data, ldb,
                                   C.ctypes.data, ldc)
        if rc == -2:
            raise OverflowError("an int8 dot product does not fit int32")
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return C

    def igemm_tn_entries(self, A: np.ndarray, Bt: np.ndarray, rows, cols) -> np.ndarray:
        """Elements (rows[t], cols[t]) of ``igemm_tn(A, Bt)`` as int32."""
        A, lda = _as_rows(A, "A", np.int8)
        Bt, ldb = _as_rows(Bt, "Bt", np.int8)
        M, K = A.shape
        N, K2 = Bt.shape
        if K != K2:
            raise ValueError(f"K mismatch: A has {K}, Bt has {K2}")
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if rows.shape != cols.shape:
            raise ValueError("rows and cols must have the same shape")
        out = np.empty(rows.shape, dtype=np.int32)
        rc = self.lib.ref_igemm_tn_entries(M, N, K, A.ctypes.data, lda, Bt.ctypes.data, ldb,
                                           rows.size, rows.ctypes.data, cols.ctypes.data,
                                           out.ctypes.data)
        if rc == -2:
            raise OverflowError("an int8 dot product does not fit int32")
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return out

    def fma_chain(self, x: np.ndarray, fma_iters: int, alpha: float, beta: float) -> np.ndarray:
        """Each element after ``fma_iters`` steps of y = fmaf(y, alpha, beta) (binary32)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty_like(x)
        rc = self.lib.ref_fma_chain(x.ctypes.data, out.ctypes.data, x.size, int(fma_iters),
                                    float(alpha), float(beta))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return out

    def num_threads(self) -> int:
        """OpenMP threads the oracle's parallel loops use."""
        return int(self.lib.ref_num_threads())

    def set_num_threads(self, n: int) -> None:
        """Threads of the oracle's later parallel loops (n >= 1)."""
        if n < 1:
            raise ValueError("n must be at least 1")
        self.lib.ref_set_num_threads(int(n))


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def f16_to_f64(bits):
    return default().f16_to_f64(bits)


def f64_to_f16(x):
    return default().f64_to_f16(x)


def hgemm_tn(A, Bt, C=None):
    return default().hgemm_tn(A, Bt, C)


def hgemm_tn_entries(A, Bt, rows, cols, return_sums=False):
    return default().hgemm_tn_entries(A, Bt, rows, cols, return_sums)


def igemm_tn(A, Bt, C=None):
    return default().igemm_tn(A, Bt, C)


def igemm_tn_entries(A, Bt, rows, cols):
    return default().igemm_tn_entries(A, Bt, rows, cols)


def fma_chain(x, fma_iters, alpha, beta):
    return default().fma_chain(x, fma_iters, alpha, beta)


def num_threads():
    return default().num_threads()
