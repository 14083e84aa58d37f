"""GPU tests of the GEMM epilogue variants (bf16 output, bf16 residual): against the oracle's
exact product plus the residual within the bound the epilogue's arithmetic implies, and, bit
for bit, against its own definition applied to the same kernel's fp32 output
(round(fp32(acc + residual)))."""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import ORACLE_THREADS, to_tiled_scales, u8_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bq():
    import torch
    import w4a4_batq_quantize_amd as bq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bq.lib()
    return bq


def bf16_rne(a32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite values)."""
    u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def run(bq, xq, xe, wq, we, tiled, w4a8, out_dtype, residual_bits):
    import torch
    if tiled:
        xe, we = to_tiled_scales(xe), to_tiled_scales(we)
    res = None
    if residual_bits is not None:
        res = torch.from_numpy(residual_bits.view(np.int16)).cuda().view(torch.bfloat16)
    y = bq.gemm_out(u8_to_device(xq), u8_to_device(xe), u8_to_device(wq), u8_to_device(we),
                    out_dtype=out_dtype, residual=res,
                    layout=bq.SCALES_MFMA_TILED if tiled else bq.SCALES_ROW_MAJOR, w4a8=w4a8)
    torch.cuda.synchronize()
    if out_dtype == torch.bfloat16:
        return y.view(torch.int16).cpu().numpy().view(np.uint16)
    return y.cpu().numpy()


CASES = [
    # (S, N, out, tiled, w4a8): producer/consumer, row-major DMA, generic (N % 256 != 0),
    # few-token, ragged out (not a multiple of 4), and the W4A8 kernels
    (200, 4096, 300, True, False),
    (130, 2048, 256, False, False),
    (70, 4192, 130, True, False),
    (17, 4096, 200, True, False),
    (33, 512, 258, False, False),
    (150, 2048, 260, True, True),
    (20, 1024, 300, True, True),
    # at most 16 tokens: the 16-row few-token kernel, both layouts and both token formats
    (5, 4096, 258, True, False),
    (3, 2048, 130, False, False),
    (7, 1024, 300, True, True),
    (2, 512, 66, False, True),
]


@pytest.mark.parametrize("S,N,out,tiled,w4a8", CASES)
def test_epilogue_bf16_and_residual(bq, orc, S, N, out, tiled, w4a8):
    import torch
    seed = (71, S, N, out, int(w4a8))
    if w4a8:
        xq, xe = wl.random_mxfp8(S, N, seed=seed, scale_lo=120, scale_hi=134)
    else:
        xq, xe = wl.random_mxfp4(S, N, seed=seed, scale_lo=120, scale_hi=134)
    wq, we = wl.random_mxfp4(out, N, seed=seed + (1,), scale_lo=120, scale_hi=134)
    rng = np.random.default_rng(S * 7 + out)
    res_bits = wl.f32_to_bf16_bits(rng.standard_normal((S, out)).astype(np.float32) * 8)
    res64 = bf16_to_f64(res_bits)

    y32 = run(bq, xq, xe, wq, we, tiled, w4a8, torch.float32, None)
    gemm = orc.gemm_w4a8 if w4a8 else orc.gemm
    y_ref, t_ref = gemm(xq, xe, wq, we, nthreads=ORACLE_THREADS)
    rel = 1e-5
    what = f"S={S} N={N} out={out} tiled={tiled} w4a8={w4a8}"

    for dtype, res in ((torch.bfloat16, None), (torch.bfloat16, res_bits),
                       (torch.float32, res_bits)):
        got = run(bq, xq, xe, wq, we, tiled, w4a8, dtype, res)
        pre = y32 if res is None else (y32 + bf16_to_f64(res).astype(np.float32)).astype(np.float32)
        exact = y_ref + (0 if res is None else res64)
        # (1) against the oracle: accumulation bound + one fp32 add (+ bf16 rounding)
        if dtype == torch.bfloat16:
            g = bf16_to_f64(got)
            bound = rel * t_ref + 2.0 ** -8 * (np.abs(exact) + rel * t_ref) + 2.0 ** -24 * np.abs(exact)
        else:
            g = got.astype(np.float64)
            bound = rel * t_ref + 2.0 ** -23 * (np.abs(exact) + rel * t_ref)
        bad = np.argwhere(np.abs(g - exact) > bound * 1.0001 + 1e-30)
        assert bad.size == 0, f"{what} {dtype} res={res is not None}: {len(bad)} beyond bound"
        # (2) the epilogue's definition on the same kernel's fp32 accumulation, bit for bit
        if dtype == torch.bfloat16:
            assert np.array_equal(got, bf16_rne(pre)), f"{what}: bf16 epilogue"
        else:
            assert np.array_equal(got.view(np.uint32), pre.view(np.uint32)), f"{what}: residual"


def test_epilogue_zero_k_gives_the_residual(bq):
    import torch
    S, out = 5, 12
    res = (torch.arange(S * out, dtype=torch.float32, device="cuda").reshape(S, out) / 8
           ).to(torch.bfloat16)
    x = torch.empty((S, 0), dtype=torch.uint8, device="cuda")
    w = torch.empty((out, 0), dtype=torch.uint8, device="cuda")
    y = bq.gemm_out(x, x, w, w, out_dtype=torch.bfloat16, residual=res)
    assert torch.equal(y, res)
