"""GPU parity of the overlap micro-benchmark: every mode, tile count and FMA
step count gives exactly the oracle's binary32 FMA chain (fused multiply-add is
correctly rounded on both sides, so the comparison is bit for bit)."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

ov = pytest.importorskip("dense_fp16_gemm_hgemm_amd.overlap")

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda", 0)


def inputs(n, seed):
    rng = np.random.default_rng(seed)
    return rng.uniform(-1, 1, n).astype(np.float32)


@pytest.mark.parametrize("mode", list(ov.MODES))
def test_modes_match_the_oracle(mode):
    for tpb, blocks, iters in ((1, 3, 0), (3, 5, 1), (16, 7, 7), (4, 300, 64)):
        n = ov.TILE * tpb * blocks
        x = inputs(n, seed=tpb * 31 + iters)
        print(f"overlap {mode} tpb {tpb} blocks {blocks} iters {iters}", flush=True)
        dx = torch.from_numpy(x).to(DEV)
        out = torch.full_like(dx, float("nan"))
        ov.run(mode, dx, out, tpb, iters)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        want = oracle.fma_chain(x, iters, ov.ALPHA, ov.BETA)
        bad = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
        assert bad.size == 0, (f"{mode} tpb {tpb} iters {iters}: {bad.size} differ, first {bad[0]}: "
                               f"{got[bad[0]]!r} vs {want[bad[0]]!r}")


def test_full_size_sampled():
    """The sweep's default size (2^26 floats, 256 tiles per workgroup), sampled."""
    n, tpb, iters = 1 << 26, 256, 3
    rng = np.random.default_rng(5)
    x = rng.uniform(-1, 1, n).astype(np.float32)
    dx = torch.from_numpy(x).to(DEV)
    idx = np.concatenate([rng.integers(0, n, 20000), np.arange(2048), np.arange(n - 2048, n)])
    want = oracle.fma_chain(x[idx], iters, ov.ALPHA, ov.BETA)
    for mode in ov.MODES:
        print(f"overlap full {mode}", flush=True)
        out = torch.full_like(dx, float("nan"))
        ov.run(mode, dx, out, tpb, iters)
        torch.cuda.synchronize()
        got = out.cpu().numpy()[idx]
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), mode
