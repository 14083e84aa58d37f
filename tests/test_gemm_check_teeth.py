"""The GEMM parity bound (|y - y_ref| <= 1e-5 sum|terms|) has teeth on the narrow-scale
operands the GPU tests also use: on the CPU, every single-block fault a kernel could make (one
scale byte read one off, one block's 16 code bytes taken from another block) moves some
output of the oracle's own product beyond the bound.  With the wide scale range many such
faults stay inside it, which is why the GPU GEMM cases run in both ranges."""
import numpy as np

import workloads as wl

NARROW, WIDE = (125, 130), (110, 145)


def detected(orc, scales, trials=24, S=8, N=1024, out=32, seed=5):
    lo, hi = scales
    xq, xe = wl.random_mxfp4(S, N, seed=(seed, 1), scale_lo=lo, scale_hi=hi)
    wq, we = wl.random_mxfp4(out, N, seed=(seed, 2), scale_lo=lo, scale_hi=hi)
    y, t = orc.gemm(xq, xe, wq, we)
    rng = np.random.default_rng(seed)
    hits = []
    for i in range(trials):
        r, b = int(rng.integers(S)), int(rng.integers(N // 32))
        xe2, xq2 = xe.copy(), xq.copy()
        if i % 2 == 0:
            xe2[r, b] = int(xe2[r, b]) + (1 if xe2[r, b] < hi - 1 else -1)   # scale byte off by one
        else:
            b2 = (b + 1 + int(rng.integers(N // 32 - 1))) % (N // 32)     # another block's codes
            xq2[r, 16 * b:16 * b + 16] = xq[r, 16 * b2:16 * b2 + 16]
        y2, _ = orc.gemm(xq2, xe2, wq, we)
        hits.append(bool(np.any(np.abs(y2 - y) > 1e-5 * t)))
    return np.array(hits)


def test_narrow_scales_detect_every_single_block_fault(orc):
    assert detected(orc, NARROW).all()


def test_wide_scales_let_single_block_faults_through(orc):
    assert not detected(orc, WIDE).all()
