"""libmi_ceiling loads and exports what include/mi_ceiling.h declares; argument
errors are refused before anything is launched (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi_ceiling.h")
LIB = os.path.join(ROOT, "dense_fp16_gemm_hgemm_amd", "libmi_ceiling.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmi_ceiling.so is not built")


def test_exports_every_declared_function():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER, encoding="utf-8").read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(mi_ceiling_\w+)\s*\(", text)))
    assert names == ["mi_ceiling_copy_lds", "mi_ceiling_copy_lds_cycle", "mi_ceiling_mfma",
                     "mi_ceiling_read"]
    lib = ctypes.CDLL(LIB)
    assert all(hasattr(lib, n) for n in names)


def test_argument_errors_need_no_device():
    lib = ctypes.CDLL(LIB)
    p = ctypes.c_void_p
    lib.mi_ceiling_read.argtypes = [p, ctypes.c_int64, ctypes.c_int32, p, p, p]
    lib.mi_ceiling_copy_lds.argtypes = [p, ctypes.c_int64, ctypes.c_int32, p, p, p]
    lib.mi_ceiling_mfma.argtypes = [p, ctypes.c_int32, ctypes.c_int32, p, p, p, p]
    fake = 0x7F0000000000
    assert lib.mi_ceiling_read(None, 4096, 1, fake, None, None) == 1
    assert lib.mi_ceiling_read(fake, 4095, 1, fake, None, None) == 1
    assert lib.mi_ceiling_read(fake + 4, 4096, 1, fake, None, None) == 1
    assert lib.mi_ceiling_copy_lds(fake, 65536, 2, fake, None, None) == 1
    lib.mi_ceiling_copy_lds_cycle.argtypes = [p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, p, p, p]
    assert lib.mi_ceiling_copy_lds_cycle(fake, 65536, 1, 0, fake, None, None) == 1
    assert lib.mi_ceiling_copy_lds_cycle(fake, 65536 + 16, 1, 1, fake, None, None) == 1
    assert lib.mi_ceiling_copy_lds_cycle(fake, 65536, 0, 1, fake, None, None) == 1
    assert lib.mi_ceiling_mfma(fake, 0, 1, fake, None, None, None) == 1
    assert lib.mi_ceiling_mfma(fake, 1, 0, fake, None, None, None) == 1
    assert lib.mi_ceiling_mfma(fake, 1, 1, fake, fake + 4, None, None) == 1
