"""The practical-ceiling probes (include/mi_ceiling.h) compute exact results:
the MFMA probe's accumulators are `iters` times the 16 x 16 block product of
its integer operands in the MFMA operand layout, and the copy and read probes
return the XOR of every 32-bit word of each workgroup's share.  Both are
checked here against numpy; then the probes are timed once and their rates
must be plausible for one MI355X."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

ce = pytest.importorskip("dense_fp16_gemm_hgemm_amd.ceiling")

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda", 0)


def expected_mfma(frags: np.ndarray, wave: int, iters: int) -> np.ndarray:
    """[8, 64, 4]: for chain j, lane l, value v of wave `wave`.  Lane l supplies
    row l % 16 of the first operand X (16 x 32) and column l % 16 of the second
    Y (32 x 16), elements 8 (l // 16) .. +7 of the reduction; lane l's value v
    is D[4 (l // 16) + v][l % 16] of D = X Y."""
    s = wave % ce.SETS
    out = np.zeros((ce.NACC, 64, 4), np.int64)
    lane = np.arange(64)
    for j in range(ce.NACC):
        a = frags[((s * ce.NACC + j) * 2) * 512:][:512].reshape(64, 8).astype(np.int64)
        b = frags[((s * ce.NACC + j) * 2 + 1) * 512:][:512].reshape(64, 8).astype(np.int64)
        X = np.zeros((16, 32), np.int64)
        Y = np.zeros((32, 16), np.int64)
        for l in range(64):
            X[l % 16, 8 * (l // 16):8 * (l // 16) + 8] = a[l]
            Y[8 * (l // 16):8 * (l // 16) + 8, l % 16] = b[l]
        D = X @ Y
        for v in range(4):
            out[j, :, v] = D[4 * (lane // 16) + v, lane % 16] * iters
    return out


def test_mfma_probe_exact():
    rng = np.random.default_rng(3)
    frags = rng.integers(-3, 4, ce.FRAG_HALVES).astype(np.float16)
    wgs, iters = 20, 37           # 80 waves: sets wrap around; iters not a multiple of 16
    d = torch.from_numpy(frags).to(DEV)
    clocks = torch.zeros(4, dtype=torch.int64, device=DEV)
    out = ce.mfma(d, wgs, iters, clocks=clocks)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(wgs * 4, ce.NACC, 64, 4)
    for w in (0, 1, 63, 64, 79):
        want = expected_mfma(frags.view(np.float16).astype(np.float64).astype(np.int64), w, iters)
        assert np.array_equal(got[w].astype(np.int64), want), f"wave {w}"
    c = clocks.cpu().numpy()
    assert c[2] > c[0] and c[3] > c[1], c


@pytest.mark.parametrize("probe,unit", [("copy_lds", 65536), ("read", 4096)])
def test_checksum_probes_exact(probe, unit):
    wgs = 7
    nbytes = wgs * unit * 3
    rng = np.random.default_rng(5)
    host = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    out = getattr(ce, probe)(src, wgs)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(host.reshape(wgs, -1), axis=1)
    assert np.array_equal(got, want)


def test_copy_cycle_probe_exact():
    ntrips, wgs, trips = 5, 9, 7      # workgroups wrap around the buffer; trips > ntrips
    rng = np.random.default_rng(8)
    host = rng.integers(0, 2 ** 32, ntrips * 65536 // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    out = ce.copy_lds_cycle(src, wgs, trips)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    per_trip = np.bitwise_xor.reduce(host.reshape(ntrips, -1), axis=1)
    want = np.array([np.bitwise_xor.reduce(per_trip[[(g + t) % ntrips for t in range(trips)]])
                     for g in range(wgs)], dtype=np.uint32)
    assert np.array_equal(got, want)


def test_invalid_arguments():
    src = torch.zeros(1024, dtype=torch.int32, device=DEV)
    with pytest.raises(ce.CeilingError):
        ce.copy_lds(src, 3)          # 4 KiB is not a multiple of 3 x 64 KiB
    with pytest.raises(ce.CeilingError):
        ce.read(src[1:], 1)          # misaligned
    with pytest.raises(ValueError):
        ce.mfma(torch.zeros(16, dtype=torch.float16, device=DEV), 1, 1)


def test_measured_ceilings_are_plausible():
    m = ce.measure()
    print(m)
    assert 300 < m["mfma_tflops"] <= ce.PEAK_MFMA_TFLOPS * 1.02
    assert m["clock_ghz_under_mfma"] is None or 0.5 < m["clock_ghz_under_mfma"] < 3.0
    assert 1000 < m["hbm_read_gbs"] < 9000
    assert m["copy_lds_gbs"] > 1000
    assert 5 < m["copy_lds_l2_gbs_per_cu"] < 200
