"""Binding of libmi_ceiling: the practical MFMA, global -> LDS copy (from HBM
and from L2) and HBM read ceilings of one MI355X, measured live (operation and exact results:
``include/mi_ceiling.h``).

``measure()`` runs the three probes on the current device and returns their
rates, the clock under MFMA load and the ratio of the MFMA rate to the
published peak; the benchmark reports them beside each roofline as practical
denominators.

    python -m dense_fp16_gemm_hgemm_amd.ceiling     # prints one JSON line
"""
from __future__ import annotations

import ctypes
import json
import os

import torch  # imported first so that both use one HIP runtime

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmi_ceiling.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python dense_fp16_gemm_hgemm_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)
_p, _i32, _i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
_IP = ctypes.POINTER(ctypes.c_int)
_lib.mi_ceiling_mfma.restype = ctypes.c_int
_lib.mi_ceiling_mfma.argtypes = [_p, _i32, _i32, _p, _p, _p, _IP]
_lib.mi_ceiling_copy_lds.restype = ctypes.c_int
_lib.mi_ceiling_copy_lds.argtypes = [_p, _i64, _i32, _p, _p, _IP]
_lib.mi_ceiling_copy_lds_cycle.restype = ctypes.c_int
_lib.mi_ceiling_copy_lds_cycle.argtypes = [_p, _i64, _i32, _i32, _p, _p, _IP]
_lib.mi_ceiling_read.restype = ctypes.c_int
_lib.mi_ceiling_read.argtypes = [_p, _i64, _i32, _p, _p, _IP]

NACC = 8           # MFMA chains per wave
SETS = 64          # operand sets
FRAG_HALVES = SETS * NACC * 2 * 512
FLOP_PER_MFMA = 2 * 16 * 16 * 32
TRIP = 65536       # bytes per workgroup and copy trip
PEAK_MFMA_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0


class CeilingError(RuntimeError):
    pass


def _check(st, err, what):
    if st != 0:
        raise CeilingError(f"{what}: status {st}, hipError {err.value}")


def _stream(stream):
    return (torch.cuda.current_stream() if stream is None else stream).cuda_stream


def mfma(frags: torch.Tensor, workgroups: int, iters: int, out: torch.Tensor | None = None,
         clocks: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """out[(wave * 8 + j) * 64 + lane, 0:4] = iters MFMAs of operand pair j (see the header)."""
    if frags.dtype != torch.float16 or frags.numel() < FRAG_HALVES or not frags.is_cuda:
        raise ValueError(f"frags must be a GPU float16 tensor of at least {FRAG_HALVES} halves")
    if out is None:
        out = torch.empty((workgroups * 4 * NACC * 64, 4), dtype=torch.float32, device=frags.device)
    err = ctypes.c_int(0)
    st = _lib.mi_ceiling_mfma(frags.data_ptr(), workgroups, iters, out.data_ptr(),
                              None if clocks is None else clocks.data_ptr(), _stream(stream),
                              ctypes.byref(err))
    _check(st, err, "mi_ceiling_mfma")
    return out


def copy_lds(src: torch.Tensor, workgroups: int, out: torch.Tensor | None = None,
             stream=None) -> torch.Tensor:
    """out[g] = XOR of the 32-bit words of workgroup g's share of src, copied through LDS."""
    if out is None:
        out = torch.empty(workgroups, dtype=torch.int32, device=src.device)
    err = ctypes.c_int(0)
    st = _lib.mi_ceiling_copy_lds(src.data_ptr(), src.numel() * src.element_size(), workgroups,
                                  out.data_ptr(), _stream(stream), ctypes.byref(err))
    _check(st, err, "mi_ceiling_copy_lds")
    return out


def copy_lds_cycle(src: torch.Tensor, workgroups: int, trips: int, out: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """out[g] = XOR of the 32-bit words of 64 KiB trips (g + t) mod T, t < trips, of src."""
    if out is None:
        out = torch.empty(workgroups, dtype=torch.int32, device=src.device)
    err = ctypes.c_int(0)
    st = _lib.mi_ceiling_copy_lds_cycle(src.data_ptr(), src.numel() * src.element_size(), workgroups,
                                        trips, out.data_ptr(), _stream(stream), ctypes.byref(err))
    _check(st, err, "mi_ceiling_copy_lds_cycle")
    return out


def read(src: torch.Tensor, workgroups: int, out: torch.Tensor | None = None,
         stream=None) -> torch.Tensor:
    """out[g] = XOR of the 32-bit words of workgroup g's share of src, read into registers."""
    if out is None:
        out = torch.empty(workgroups, dtype=torch.int32, device=src.device)
    err = ctypes.c_int(0)
    st = _lib.mi_ceiling_read(src.data_ptr(), src.numel() * src.element_size(), workgroups,
                              out.data_ptr(), _stream(stream), ctypes.byref(err))
    _check(st, err, "mi_ceiling_read")
    return out


def _time_ms(fn, reps):
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(reps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def measure(device=None, mfma_iters: int = 4096, read_mib: int = 1024, copy_mib: int = 512) -> dict:
    """The three practical ceilings on `device` (default: the current one):
    MFMA-only TFLOP/s on random-mantissa operands (as the GEMM sees them; the
    clock depends on the data) with the measured shader clock, the global ->
    LDS copy rate, the rate at which one CU copies from L2 into its LDS, and
    the streaming HBM read rate of a buffer four times the 256 MiB MALL."""
    dev = torch.device("cuda", torch.cuda.current_device() if device is None else device)
    g = torch.Generator(device=dev).manual_seed(1)
    frags = (torch.rand(FRAG_HALVES, device=dev, generator=g) * 2 - 1).half()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    wgs = 2 * cus  # two waves per SIMD
    out = torch.empty((wgs * 4 * NACC * 64, 4), dtype=torch.float32, device=dev)
    clocks = torch.zeros(4, dtype=torch.int64, device=dev)
    ms = _time_ms(lambda: mfma(frags, wgs, mfma_iters, out, clocks), 5)
    flops = wgs * 4 * NACC * mfma_iters * FLOP_PER_MFMA
    c = clocks.cpu().tolist()
    clock_ghz = (c[2] - c[0]) / ((c[3] - c[1]) / 1e8) / 1e9 if c[3] > c[1] else None
    mfma_tflops = flops / (ms * 1e-3) / 1e12

    cbytes = copy_mib << 20
    cwgs = cus * 4
    cbytes -= cbytes % (cwgs * TRIP)
    src = torch.empty(cbytes // 4, dtype=torch.int32, device=dev)
    src.random_(generator=g)
    cout = torch.empty(cwgs, dtype=torch.int32, device=dev)
    cms = _time_ms(lambda: copy_lds(src, cwgs, cout), 5)
    del src

    # per-CU feed from L2: one 4-wave workgroup per CU cycling through 2 MiB
    small = torch.empty((2 << 20) // 4, dtype=torch.int32, device=dev)
    small.random_(generator=g)
    l2trips = 256
    lout = torch.empty(cus, dtype=torch.int32, device=dev)
    lms = _time_ms(lambda: copy_lds_cycle(small, cus, l2trips, lout), 5)
    lbytes = cus * l2trips * TRIP
    del small

    rbytes = read_mib << 20
    rwgs = cus * 8
    rbytes -= rbytes % (rwgs * 4096)
    big = torch.empty(rbytes // 4, dtype=torch.int32, device=dev)
    big.random_(generator=g)
    rout = torch.empty(rwgs, dtype=torch.int32, device=dev)
    rms = _time_ms(lambda: read(big, rwgs, rout), 5)
    del big
    return {
        "mfma_tflops": round(mfma_tflops, 1),
        "mfma_frac_of_peak": round(mfma_tflops / PEAK_MFMA_TFLOPS, 4),
        "clock_ghz_under_mfma": None if clock_ghz is None else round(clock_ghz, 3),
        "copy_lds_gbs": round(cbytes / (cms * 1e-3) / 1e9, 1),
        "copy_lds_l2_gbs_per_cu": round(lbytes / (lms * 1e-3) / 1e9 / cus, 1),
        "hbm_read_gbs": round(rbytes / (rms * 1e-3) / 1e9, 1),
        "hbm_read_frac_of_peak": round(rbytes / (rms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "probes": (f"MFMA: {wgs} workgroups x 4 waves x {NACC} chains x {mfma_iters} "
                   f"v_mfma_f32_16x16x32_f16 on random fp16; copy: {cbytes >> 20} MiB through LDS "
                   f"by {cwgs} workgroups; L2 copy: {cus} workgroups x {l2trips} trips of 64 KiB "
                   f"cycling through 2 MiB; read: {rbytes >> 20} MiB by {rwgs} workgroups"),
    }


if __name__ == "__main__":
    print(json.dumps(measure()), flush=True)
