"""Python binding of libmi_hgemm, the TN half-precision GEMM for MI355X (gfx950).

``C[M,N] = fp16_rne(A[M,K] @ Bt[N,K].T)`` with fp32 accumulation, where ``Bt``
is the storage of the column-major K x N operand B (torch's ``nn.Linear``
weight layout).  Every step runs in the HIP kernels of ``libmi_hgemm.so``; this
module only marshals arguments: torch supplies device memory and the stream.

Two layers:
  * ``mi_hgemm_*`` functions with the C ABI's names and arguments (see
    ``include/mi_hgemm.h``), returning the status code (and out-values);
  * ``Hgemm``, a handle wrapper taking torch tensors and raising ``HgemmError``.

Importing fails loudly when the library has not been built
(``python dense_fp16_gemm_hgemm_amd/build.py``); there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch  # imported before the library so both use one HIP runtime

__all__ = [
    "MI_HGEMM_OK", "MI_HGEMM_ERR_INVALID_ARG", "MI_HGEMM_ERR_UNSUPPORTED",
    "MI_HGEMM_ERR_NO_DEVICE", "MI_HGEMM_ERR_HIP", "MI_HGEMM_ERR_IO",
    "MI_HGEMM_WARN_TABLE_DEFAULTS", "MI_HGEMM_LAYOUT_TN", "MI_HGEMM_CREATE_NO_DEVICE",
    "MI_HGEMM_TUNE_EXHAUSTIVE", "MI_HGEMM_TUNE_HEURISTIC", "MI_HGEMM_TUNE_PERSIST",
    "MI_HGEMM_TUNE_INT8", "mi_hgemm_run_i8", "mi_hgemm_plan_i8", "igemm",
    "HgemmError", "Hgemm", "hgemm", "kernel_names", "LIB_PATH",
    "mi_hgemm_create", "mi_hgemm_create_ex", "mi_hgemm_destroy", "mi_hgemm_run",
    "mi_hgemm_run_kernel", "mi_hgemm_plan", "mi_hgemm_tune", "mi_hgemm_status_string",
    "mi_hgemm_last_hip_error", "mi_hgemm_kernel_count", "mi_hgemm_kernel_name",
    "mi_hgemm_table_size", "mi_hgemm_table_save", "mi_hgemm_run_noalloc",
]

MI_HGEMM_OK = 0
MI_HGEMM_ERR_INVALID_ARG = 1
MI_HGEMM_ERR_UNSUPPORTED = 2
MI_HGEMM_ERR_NO_DEVICE = 3
MI_HGEMM_ERR_HIP = 4
MI_HGEMM_ERR_IO = 5
MI_HGEMM_WARN_TABLE_DEFAULTS = 6
MI_HGEMM_LAYOUT_TN = 0
MI_HGEMM_CREATE_NO_DEVICE = 1
MI_HGEMM_TUNE_EXHAUSTIVE = 1
MI_HGEMM_TUNE_HEURISTIC = 2
MI_HGEMM_TUNE_PERSIST = 4
MI_HGEMM_TUNE_INT8 = 8

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmi_hgemm.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python dense_fp16_gemm_hgemm_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

_i64, _i32, _u32, _p = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)


def _sig(name, restype, *argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)
    return f


_create = _sig("mi_hgemm_create", ctypes.c_int, ctypes.POINTER(_p), ctypes.c_char_p)
_create_ex = _sig("mi_hgemm_create_ex", ctypes.c_int, ctypes.POINTER(_p), ctypes.c_char_p, _u32)
_destroy = _sig("mi_hgemm_destroy", ctypes.c_int, _p)
_run = _sig("mi_hgemm_run", ctypes.c_int, _p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64,
            ctypes.c_int, _p)
_run_kernel = _sig("mi_hgemm_run_kernel", ctypes.c_int, _p, _i32, _i32, _i32, _i32, _i64, _i64,
                   _i64, _p, _i64, _p, _i64, _p, _i64, ctypes.c_int, _p)
_plan = _sig("mi_hgemm_plan", ctypes.c_int, _p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64,
             ctypes.c_int, _I32P, _I32P, _I32P, _I32P)
_run_noalloc = _sig("mi_hgemm_run_noalloc", ctypes.c_int, _p, _i64, _i64, _i64, _p, _i64, _p,
                    _i64, _p, _i64, ctypes.c_int, _p)
_run_i8 = _sig("mi_hgemm_run_i8", ctypes.c_int, _p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p,
               _i64, ctypes.c_int, _p)
_plan_i8 = _sig("mi_hgemm_plan_i8", ctypes.c_int, _p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p,
                _i64, ctypes.c_int, _I32P, _I32P, _I32P, _I32P)
_tune = _sig("mi_hgemm_tune", ctypes.c_int, _p, _i64, _i64, _i64, ctypes.c_int, _p, _u32)
_status_string = _sig("mi_hgemm_status_string", ctypes.c_char_p, ctypes.c_int)
_last_hip_error = _sig("mi_hgemm_last_hip_error", ctypes.c_int, _p)
_kernel_count = _sig("mi_hgemm_kernel_count", ctypes.c_int)
_kernel_name = _sig("mi_hgemm_kernel_name", ctypes.c_char_p, ctypes.c_int)
_table_size = _sig("mi_hgemm_table_size", ctypes.c_int, _p)
_table_save = _sig("mi_hgemm_table_save", ctypes.c_int, _p, ctypes.c_char_p)


def _cstr(s):
    return None if s is None else os.fsencode(s)


# ------------------------------------------------------- C-ABI mirrors --

def mi_hgemm_create(table_path=None):
    """-> (status, handle or None)"""
    h = _p()
    st = _create(ctypes.byref(h), _cstr(table_path))
    return st, h.value


def mi_hgemm_create_ex(table_path=None, flags=0):
    """-> (status, handle or None)"""
    h = _p()
    st = _create_ex(ctypes.byref(h), _cstr(table_path), flags)
    return st, h.value


def mi_hgemm_destroy(h):
    return _destroy(h)


def mi_hgemm_run(h, M, N, K, A, lda, B, ldb, C, ldc, layout=MI_HGEMM_LAYOUT_TN, stream=None):
    return _run(h, M, N, K, A, lda, B, ldb, C, ldc, layout, stream)


def mi_hgemm_run_noalloc(h, M, N, K, A, lda, B, ldb, C, ldc, layout=MI_HGEMM_LAYOUT_TN,
                         stream=None):
    return _run_noalloc(h, M, N, K, A, lda, B, ldb, C, ldc, layout, stream)


def mi_hgemm_run_i8(h, M, N, K, A, lda, B, ldb, C, ldc, layout=MI_HGEMM_LAYOUT_TN, stream=None):
    return _run_i8(h, M, N, K, A, lda, B, ldb, C, ldc, layout, stream)


def mi_hgemm_run_kernel(h, kernel_index, group_m, xcd_remap, split_k, M, N, K, A, lda, B, ldb,
                        C, ldc, layout=MI_HGEMM_LAYOUT_TN, stream=None):
    return _run_kernel(h, kernel_index, group_m, xcd_remap, split_k, M, N, K, A, lda, B, ldb, C,
                       ldc, layout, stream)


def mi_hgemm_plan(h, M, N, K, A, lda, B, ldb, C, ldc, layout=MI_HGEMM_LAYOUT_TN):
    """-> (status, kernel_index, group_m, xcd_remap, split_k)"""
    k, g, x, s = ctypes.c_int32(-2), ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    st = _plan(h, M, N, K, A, lda, B, ldb, C, ldc, layout, ctypes.byref(k), ctypes.byref(g),
               ctypes.byref(x), ctypes.byref(s))
    return st, k.value, g.value, x.value, s.value


def mi_hgemm_plan_i8(h, M, N, K, A, lda, B, ldb, C, ldc, layout=MI_HGEMM_LAYOUT_TN):
    """-> (status, kernel_index, group_m, xcd_remap, split_k)"""
    k, g, x, s = ctypes.c_int32(-2), ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    st = _plan_i8(h, M, N, K, A, lda, B, ldb, C, ldc, layout, ctypes.byref(k), ctypes.byref(g),
                  ctypes.byref(x), ctypes.byref(s))
    return st, k.value, g.value, x.value, s.value


def mi_hgemm_tune(h, M, N, K, layout=MI_HGEMM_LAYOUT_TN, stream=None,
                  flags=MI_HGEMM_TUNE_EXHAUSTIVE):
    return _tune(h, M, N, K, layout, stream, flags)


def mi_hgemm_status_string(status):
    return _status_string(status).decode()


def mi_hgemm_last_hip_error(h):
    return _last_hip_error(h)


def mi_hgemm_kernel_count():
    return _kernel_count()


def mi_hgemm_kernel_name(index):
    s = _kernel_name(index)
    return None if s is None else s.decode()


def mi_hgemm_table_size(h):
    return _table_size(h)


def mi_hgemm_table_save(h, path):
    return _table_save(h, _cstr(path))


def kernel_names() -> list[str]:
    return [mi_hgemm_kernel_name(i) for i in range(mi_hgemm_kernel_count())]


# ------------------------------------------------------- torch wrapper --

class HgemmError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: {mi_hgemm_status_string(status)}" if what
                         else mi_hgemm_status_string(status))


def _check(st, what, allow=(MI_HGEMM_OK,)):
    if st not in allow:
        raise HgemmError(st, what)
    return st


def _operand(x: torch.Tensor, name: str, dtype=torch.float16) -> int:
    """Leading dimension (elements) of a 2-D GPU tensor of ``dtype`` with unit-stride rows."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    if x.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {x.dtype}")
    if not x.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    rows, cols = x.shape
    if cols > 1 and x.stride(1) != 1:
        raise ValueError(f"{name} must have unit-stride rows")
    if rows <= 1:
        return max(cols, 1)
    return x.stride(0)


def _stream_ptr(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)


class Hgemm:
    """A library handle.  ``run(A, Bt)`` returns ``A @ Bt.T`` computed by the HIP kernels."""

    def __init__(self, table_path=None, inspect_only: bool = False):
        flags = MI_HGEMM_CREATE_NO_DEVICE if inspect_only else 0
        st, h = mi_hgemm_create_ex(table_path, flags)
        _check(st, "mi_hgemm_create", (MI_HGEMM_OK, MI_HGEMM_WARN_TABLE_DEFAULTS))
        self.handle = h
        self.create_status = st

    def close(self):
        if self.handle:
            mi_hgemm_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _args(self, A, Bt, out):
        """int8 A and Bt select the int8 variant (int32 result), else fp16."""
        i8 = isinstance(A, torch.Tensor) and A.dtype == torch.int8
        in_t, out_t = (torch.int8, torch.int32) if i8 else (torch.float16, torch.float16)
        lda, ldb = _operand(A, "A", in_t), _operand(Bt, "Bt", in_t)
        M, K = A.shape
        N, K2 = Bt.shape
        if K != K2:
            raise ValueError(f"K mismatch: A has {K}, Bt has {K2}")
        if A.device != Bt.device:
            raise ValueError("A and Bt must be on the same device")
        if out is None:
            out = torch.empty((M, N), dtype=out_t, device=A.device)
        elif tuple(out.shape) != (M, N):
            raise ValueError(f"out must have shape {(M, N)}")
        ldc = _operand(out, "out", out_t)
        if out.device != A.device:
            raise ValueError("out must be on the operands' device")
        return M, N, K, lda, ldb, ldc, out

    def run(self, A: torch.Tensor, Bt: torch.Tensor, out: torch.Tensor | None = None,
            stream=None) -> torch.Tensor:
        if A.dtype != torch.float16:
            raise TypeError(f"A must be torch.float16 (int8 operands: run_i8), got {A.dtype}")
        M, N, K, lda, ldb, ldc, out = self._args(A, Bt, out)
        st = mi_hgemm_run(self.handle, M, N, K, A.data_ptr(), lda, Bt.data_ptr(), ldb,
                          out.data_ptr(), ldc, MI_HGEMM_LAYOUT_TN, _stream_ptr(stream, A.device))
        _check(st, "mi_hgemm_run")
        return out

    def run_i8(self, A: torch.Tensor, Bt: torch.Tensor, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
        """``A @ Bt.T`` for int8 A [M, K] and Bt [N, K], exact, as int32 [M, N]."""
        if A.dtype != torch.int8:
            raise TypeError(f"A must be torch.int8, got {A.dtype}")
        M, N, K, lda, ldb, ldc, out = self._args(A, Bt, out)
        st = mi_hgemm_run_i8(self.handle, M, N, K, A.data_ptr(), lda, Bt.data_ptr(), ldb,
                             out.data_ptr(), ldc, MI_HGEMM_LAYOUT_TN,
                             _stream_ptr(stream, A.device))
        _check(st, "mi_hgemm_run_i8")
        return out

    def run_kernel(self, kernel, A, Bt, out=None, group_m=1, xcd_remap=0, split_k=1,
                   stream=None):
        idx = kernel if isinstance(kernel, int) else kernel_names().index(kernel)
        # the C ABI takes the element type from the instance: operands of the
        # other type would be read and written with the wrong element size
        name = mi_hgemm_kernel_name(idx)
        if name is not None and name.startswith("i8_") != (A.dtype == torch.int8):
            raise TypeError(f"instance {name} does not take {A.dtype} operands")
        M, N, K, lda, ldb, ldc, out = self._args(A, Bt, out)
        st = mi_hgemm_run_kernel(self.handle, idx, group_m, xcd_remap, split_k, M, N, K,
                                 A.data_ptr(), lda, Bt.data_ptr(), ldb, out.data_ptr(), ldc,
                                 MI_HGEMM_LAYOUT_TN, _stream_ptr(stream, A.device))
        _check(st, "mi_hgemm_run_kernel")
        return out

    def plan(self, A, Bt, out=None):
        """-> (kernel name or None, group_m, xcd_remap, split_k) that ``run`` (or
        ``run_i8``, for int8 operands) would use."""
        M, N, K, lda, ldb, ldc, out = self._args(A, Bt, out)
        fn = mi_hgemm_plan_i8 if A.dtype == torch.int8 else mi_hgemm_plan
        st, k, g, x, s = fn(self.handle, M, N, K, A.data_ptr(), lda, Bt.data_ptr(),
                            ldb, out.data_ptr(), ldc)
        _check(st, "mi_hgemm_plan")
        return (mi_hgemm_kernel_name(k) if k >= 0 else None), g, x, s

    def tune(self, M, N, K, flags=MI_HGEMM_TUNE_EXHAUSTIVE, stream=None):
        dev = torch.device("cuda", torch.cuda.current_device())
        _check(mi_hgemm_tune(self.handle, M, N, K, MI_HGEMM_LAYOUT_TN,
                             _stream_ptr(stream, dev), flags), "mi_hgemm_tune")

    def table_size(self):
        return mi_hgemm_table_size(self.handle)

    def save_table(self, path):
        _check(mi_hgemm_table_save(self.handle, path), "mi_hgemm_table_save")

    def last_hip_error(self):
        return mi_hgemm_last_hip_error(self.handle)


_default_handle: Hgemm | None = None


def hgemm(A: torch.Tensor, Bt: torch.Tensor, out: torch.Tensor | None = None,
          stream=None) -> torch.Tensor:
    """``A @ Bt.T`` in fp16 with fp32 accumulation, on a process-wide handle."""
    global _default_handle
    if _default_handle is None:
        _default_handle = Hgemm()
    return _default_handle.run(A, Bt, out, stream)


def igemm(A: torch.Tensor, Bt: torch.Tensor, out: torch.Tensor | None = None,
          stream=None) -> torch.Tensor:
    """``A @ Bt.T`` for int8 operands, exact int32 result, on a process-wide handle."""
    global _default_handle
    if _default_handle is None:
        _default_handle = Hgemm()
    return _default_handle.run_i8(A, Bt, out, stream)
