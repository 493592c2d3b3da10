"""libmi_overlap without a GPU: it loads, exports what include/mi_overlap.h
declares, and rejects invalid arguments before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi_overlap.h")
LIB = os.path.join(ROOT, "dense_fp16_gemm_hgemm_amd", "libmi_overlap.so")

if not os.path.exists(LIB):
    pytest.skip("libmi_overlap.so is not built", allow_module_level=True)


def declared():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER, encoding="utf-8").read(), flags=re.S)
    return sorted(set(re.findall(r"\b(mi_overlap_\w+)\s*\(", text)))


def lib():
    L = ctypes.CDLL(LIB)
    L.mi_overlap_run.restype = ctypes.c_int
    L.mi_overlap_run.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                                 ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)]
    return L


def test_exports_every_declared_symbol():
    L = ctypes.CDLL(LIB)
    names = declared()
    assert "mi_overlap_run" in names
    assert [n for n in names if not hasattr(L, n)] == []
    assert L.mi_overlap_tile_floats() == 1024 and L.mi_overlap_block_threads() == 256


def test_invalid_arguments_are_rejected_before_launch():
    L = lib()
    X, O = 0x7F0000000000, 0x7F1000000000       # fake device addresses, never touched
    err = ctypes.c_int(7)

    def run(mode=0, x=X, o=O, n=4096, tpb=4, it=1):
        return L.mi_overlap_run(mode, x, o, n, tpb, it, 1.0, 0.0, None, ctypes.byref(err))
    assert run(mode=4) == 1 and run(mode=-1) == 1
    assert run(x=0) == 1 and run(o=0) == 1
    assert run(x=X + 4) == 1                      # not 16-byte aligned
    assert run(n=4096 + 1024) == 1                # not a multiple of 1024 * tiles_per_block
    assert run(n=0) == 1 and run(tpb=0) == 1 and run(it=-1) == 1
    assert run(o=X + 1024) == 1                   # overlapping
    assert run(n=1 << 30, tpb=1) == 1             # 4 GiB: beyond 32-bit buffer offsets
    assert err.value == 0
