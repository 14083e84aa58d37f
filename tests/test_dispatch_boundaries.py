"""GPU parity on both sides of every kernel-choice boundary of the few-token GEMMs and the
one-call layers: the 16-row kernel's rounds rule (out = 4096 / 4112 at k = 384) and its K
limit (k = 512 / 520), 16 / 17 and 64 / 65 tokens, the token-halves grid (out = 4096 / 4128
at 33..64 tokens), the one-kernel layer's 16-row / 32-row split (S k = 1536 / 1568) and the
W4A8 layer's one-kernel limit (S k = 768 / 784).  Every case against the oracle within the
GEMM's accumulation bound, 1e-5 of sum|terms| (W4A8 included)."""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import (ORACLE_THREADS, assert_gemm_close, bf16_to_device, f32_to_device,
                            to_host, to_tiled_scales, u8_to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bq():
    import torch
    import w4a4_batq_quantize_amd as bq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bq.lib()
    return bq


GEMM_CASES = [
    (8, 12288, 4096), (8, 12288, 4112),      # 16-row kernel: one round / two (32-row)
    (16, 16384, 64), (16, 16640, 64),        # k = 512 (16-row) / 520 (32-row)
    (17, 2048, 300),                         # one-column 32-row kernel
    (40, 2048, 4096), (40, 2048, 4128),      # token halves / two-column kernel
    (64, 1024, 96), (65, 1024, 96),          # few-token / tiled kernels
]


# scale bytes of the random operands: 35 octaves, or 5 (every block then matters to every
# output at the 1e-5 sum|terms| bound)
SCALES = {"wide": (110, 145), "narrow": (125, 130)}


@pytest.mark.parametrize("scales", list(SCALES))
@pytest.mark.parametrize("w4a8", [False, True])
@pytest.mark.parametrize("S,N,out", GEMM_CASES)
def test_gemm_dispatch_boundaries(bq, orc, S, N, out, w4a8, scales):
    import torch
    seed = (121, S, N, out, int(w4a8))
    lo, hi = SCALES[scales]
    xq, xe = (wl.random_mxfp8 if w4a8 else wl.random_mxfp4)(S, N, seed=seed, scale_lo=lo,
                                                           scale_hi=hi)
    wq, we = wl.random_mxfp4(out, N, seed=seed + (1,), scale_lo=lo, scale_hi=hi)
    print(f"[dispatch gemm] S={S} N={N} out={out} w4a8={w4a8} scales={scales}", flush=True)
    f = bq.gemm_w4a8 if w4a8 else bq.gemm_w4a4
    y = f(u8_to_device(xq), u8_to_device(to_tiled_scales(xe)), u8_to_device(wq),
          u8_to_device(to_tiled_scales(we)), layout=bq.SCALES_MFMA_TILED)
    torch.cuda.synchronize()
    y = to_host(y)
    what = f"S={S} N={N} out={out} w4a8={w4a8} scales={scales}"
    if w4a8:
        y_ref, t_ref = orc.gemm_w4a8(xq, xe, wq, we, nthreads=ORACLE_THREADS)
        assert_gemm_close(y, y_ref, t_ref, what=what)
    else:
        y_ref, t_ref = orc.gemm(xq, xe, wq, we, nthreads=ORACLE_THREADS)
        assert_gemm_close(y, y_ref, t_ref, what=what)


def layer_inputs(bq, L, layout):
    wq, we = bq.prepare_weight(f32_to_device(L.W), L.A, L.B, layout=layout)
    return (bf16_to_device(L.x_bits), f32_to_device(L.A), f32_to_device(L.B),
            f32_to_device(bq.clip_ratios(L.alpha_min)),
            f32_to_device(bq.clip_ratios(L.alpha_max)), wq, we)


def call_raw(bq, fn, S, N, out, x, A, B, r1, r2, wq, we, layout):
    """The C entry with no workspace: the one-kernel path, which must accept the shape."""
    import torch
    y = torch.empty((S, out), dtype=torch.float32, device="cuda")
    st = fn(x.data_ptr(), S, N, x.stride(0), A.data_ptr(), B.data_ptr(), r1.data_ptr(),
            r2.data_ptr(), wq.data_ptr(), we.data_ptr(), out, y.data_ptr(), 0, 0,
            layout=layout, stream=torch.cuda.current_stream().cuda_stream)
    assert st == 0, bq.status_string(st)
    torch.cuda.synchronize()
    return to_host(y)


@pytest.mark.parametrize("S,N,out", [
    (3, 16384, 100),            # S k = 1536: 16-row one-kernel layer
    (4, 12544, 100),            # S k = 1568: 32-row one-kernel layer
])
def test_linear_one_kernel_split(bq, orc, S, N, out):
    L = wl.make_layer(wl.custom("bnd", S, N, out, seed=(122, S, N, out)))
    T = bq.SCALES_MFMA_TILED
    args = layer_inputs(bq, L, T)
    print(f"[dispatch linear] S={S} N={N} out={out}", flush=True)
    y = call_raw(bq, bq.linear_w4a4_raw, S, N, out, *args, T)
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    xq, xe = orc.quantize_act(L.x_bits, L.A, L.B, rmin, rmax, nthreads=ORACLE_THREADS)
    wq, we = orc.prepare_weight(L.W, L.A, L.B, nthreads=ORACLE_THREADS)
    y_ref, t_ref = orc.gemm(xq, xe, wq, we, nthreads=ORACLE_THREADS)
    assert_gemm_close(y, y_ref, t_ref, what=f"linear S={S} N={N} out={out}")


def test_linear8_one_kernel_limit(bq, orc):
    """S k = 768 runs as one kernel with no workspace; S k = 784 needs the workspace."""
    import torch
    T = bq.SCALES_MFMA_TILED
    L = wl.make_layer(wl.custom("bnd8", 2, 12288, 64, seed=123))
    y = call_raw(bq, bq.linear_w4a8_raw, 2, 12288, 64, *layer_inputs(bq, L, T), T)
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    xq8, xe = orc.quantize_act_fp8(L.x_bits, L.A, L.B, rmin, rmax, nthreads=ORACLE_THREADS)
    wq, we = orc.prepare_weight(L.W, L.A, L.B, nthreads=ORACLE_THREADS)
    y_ref, t_ref = orc.gemm_w4a8(xq8, xe, wq, we, nthreads=ORACLE_THREADS)
    assert_gemm_close(y, y_ref, t_ref, what="w4a8 S k = 768")
    L2 = wl.make_layer(wl.custom("bnd8b", 2, 12544, 64, seed=124))
    x, A, B, r1, r2, wq2, we2 = layer_inputs(bq, L2, T)
    y2 = torch.empty((2, 64), dtype=torch.float32, device="cuda")
    st = bq.linear_w4a8_raw(x.data_ptr(), 2, 12544, 12544, A.data_ptr(), B.data_ptr(),
                            r1.data_ptr(), r2.data_ptr(), wq2.data_ptr(), we2.data_ptr(), 64,
                            y2.data_ptr(), 0, 0, layout=T)
    assert bq._binding.STATUS[st] == "BATQ_ERR_NULL", bq.status_string(st)   # workspace needed
