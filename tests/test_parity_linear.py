"""GPU parity of batq_linear_w4a4 and batq_linear_w4a8, the linear layer in one call: for 1..4
tokens one kernel (the few-token GEMM encoding the token rows itself), otherwise quantiser +
GEMM through the caller's workspace; against the oracle's quantisation, weight preparation
and fp64 product within the GEMM's accumulation bound (1e-5 * sum|terms|, W4A8 included)."""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import (ORACLE_THREADS, assert_gemm_close, bf16_to_device, f32_to_device,
                            to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bq():
    import torch
    import w4a4_batq_quantize_amd as bq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bq.lib()
    return bq


def run_linear(bq, L, layout, ldx=None, workspace=True):
    """batq_linear_w4a4 on the layer; workspace=False calls the C entry with no workspace,
    which takes the one-kernel path; workspace=True passes one and lets the library
    choose."""
    import torch
    S, N = L.x_bits.shape
    wq, we = bq.prepare_weight(f32_to_device(L.W), L.A, L.B, layout=layout)
    if ldx is not None and ldx != N:
        wide = np.zeros((S, ldx), dtype=np.uint16)
        wide[:, :N] = L.x_bits
        wide[:, N:] = 0x7FC0                       # NaN padding: must never be read
        x = bf16_to_device(wide)[:, :N]
    else:
        x = bf16_to_device(L.x_bits)
    A, B = f32_to_device(L.A), f32_to_device(L.B)
    r1 = f32_to_device(bq.clip_ratios(L.alpha_min))
    r2 = f32_to_device(bq.clip_ratios(L.alpha_max))
    if workspace:
        # the caller's workspace: the library chooses between the one kernel and two calls
        xq = torch.empty((S, N // 2), dtype=torch.uint8, device="cuda")
        xe = torch.empty((bq.scale_bytes(S, N, layout),), dtype=torch.uint8, device="cuda")
        y = bq.linear_w4a4(x, A, B, r1, r2, wq, we, layout=layout, workspace=(xq, xe))
    else:
        out = wq.shape[0]
        y = torch.empty((S, out), dtype=torch.float32, device="cuda")
        st = bq.linear_w4a4_raw(x.data_ptr(), S, N, x.stride(0), A.data_ptr(), B.data_ptr(),
                                r1.data_ptr(), r2.data_ptr(), wq.data_ptr(), we.data_ptr(), out,
                                y.data_ptr(), 0, 0, layout=layout,
                                stream=torch.cuda.current_stream().cuda_stream)
        assert st == 0, bq.status_string(st)
    torch.cuda.synchronize()
    return to_host(y)


def oracle_linear(orc, L):
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    xq, xe = orc.quantize_act(L.x_bits, L.A, L.B, rmin, rmax, nthreads=ORACLE_THREADS)
    wq, we = orc.prepare_weight(L.W, L.A, L.B, nthreads=ORACLE_THREADS)
    return orc.gemm(xq, xe, wq, we, nthreads=ORACLE_THREADS)


@pytest.mark.parametrize("tiled", [True, False])
@pytest.mark.parametrize("S,N,out,ldx", [
    (1, 256, 33, None),         # one stage, ragged out
    (1, 12288, 4096, None),     # decode shape
    (2, 4096, 300, 4104),       # strided rows
    (3, 16384, 130, None),      # k = 512, the largest row of the one-kernel path
    (4, 2048, 4096, None),
    (4, 8192, 64, 8200),
])
def test_linear_one_kernel(bq, orc, S, N, out, ldx, tiled):
    L = wl.make_layer(wl.custom("lin", S, N, out, seed=(101, S, N, out),
                                outliers=("channels_uniform", 8, 20.0, 100.0)))
    layout = bq.SCALES_MFMA_TILED if tiled else bq.SCALES_ROW_MAJOR
    print(f"[linear one-kernel] S={S} N={N} out={out} tiled={tiled}", flush=True)
    y = run_linear(bq, L, layout, ldx=ldx, workspace=False)
    y_ref, t_ref = oracle_linear(orc, L)
    assert_gemm_close(y, y_ref, t_ref, what=f"S={S} N={N} out={out} tiled={tiled}")


@pytest.mark.parametrize("tiled", [True, False])
@pytest.mark.parametrize("S,N,out", [
    (1, 4096, 12288),           # decode gate/up shape: 768 workgroups, 8 waves, 1 stage each
    (3, 16384, 4112),           # 257 workgroups: 8 waves with 8 stages each (k = 512)
    (1, 12288, 4112),           # 8 waves with 6 stages each (k = 384)
])
def test_linear_one_kernel_eight_waves(bq, orc, S, N, out, tiled):
    """The one-kernel layer takes 16 waves when one round of 16-row workgroups covers out
    (ceil(out/16) <= 256 CUs) and 8 otherwise: these shapes are on the 8-wave side, with no
    workspace, across the per-wave stage counts."""
    L = wl.make_layer(wl.custom("lin8w", S, N, out, seed=(105, S, N, out)))
    layout = bq.SCALES_MFMA_TILED if tiled else bq.SCALES_ROW_MAJOR
    print(f"[linear one-kernel 8 waves] S={S} N={N} out={out} tiled={tiled}", flush=True)
    y = run_linear(bq, L, layout, workspace=False)
    y_ref, t_ref = oracle_linear(orc, L)
    assert_gemm_close(y, y_ref, t_ref, what=f"8 waves S={S} N={N} out={out} tiled={tiled}")


def test_linear_workspace_one_kernel_wide_out(bq, orc):
    """With a workspace, S = 1, N = 4096, out = 12288 still takes the one kernel (S k
    ceil(out/16) = 98304 is within the rule) on its 8-wave side."""
    L = wl.make_layer(wl.custom("lin8ws", 1, 4096, 12288, seed=106))
    y = run_linear(bq, L, bq.SCALES_MFMA_TILED, workspace=True)
    y_ref, t_ref = oracle_linear(orc, L)
    assert_gemm_close(y, y_ref, t_ref, what="workspace one kernel out=12288")


@pytest.mark.parametrize("S,N,out", [
    (5, 4096, 96),              # more tokens than the one-kernel path takes
    (2, 16640, 64),             # k = 520 > 512
    (3, 96, 40),                # k = 3: not a multiple of 8
])
def test_linear_two_steps(bq, orc, S, N, out):
    L = wl.make_layer(wl.custom("lin2", S, N, out, seed=(102, S, N, out)))
    y = run_linear(bq, L, bq.SCALES_MFMA_TILED)
    y_ref, t_ref = oracle_linear(orc, L)
    assert_gemm_close(y, y_ref, t_ref, what=f"two steps S={S} N={N} out={out}")


@pytest.mark.parametrize("S,N,out", [
    (1, 4096, 96), (3, 16384, 64),        # one kernel
    (5, 4096, 96), (16, 1024, 130),       # one kernel for more than 4 tokens (small S k)
    (4, 12288, 2064), (2, 16384, 6200),   # two calls: S k ceil(out/16) beyond 196608
    (8, 4096, 4096),                      # two calls: S k ceil(out/16) = 262144
])
def test_linear_with_workspace_either_path(bq, orc, S, N, out):
    """With a workspace the library picks a path by shape (the one kernel, or the two calls
    when the token encoding all its workgroups repeat grows large): the result is the
    oracle's within the bound either way."""
    L = wl.make_layer(wl.custom("lin4", S, N, out, seed=(104, S, N, out)))
    y = run_linear(bq, L, bq.SCALES_MFMA_TILED, workspace=True)
    y_ref, t_ref = oracle_linear(orc, L)
    assert_gemm_close(y, y_ref, t_ref, what=f"workspace S={S} N={N} out={out}")


def test_linear_one_kernel_matches_two_calls(bq):
    """Same codes as batq_quantize_act (the quantiser's own arithmetic): the one-kernel output
    and the two-call output differ only by the GEMM's fp32 summation order."""
    import torch
    L = wl.make_layer(wl.custom("lin3", 4, 4096, 512, seed=103))
    T = bq.SCALES_MFMA_TILED
    wq, we = bq.prepare_weight(f32_to_device(L.W), L.A, L.B, layout=T)
    args = (bf16_to_device(L.x_bits), f32_to_device(L.A), f32_to_device(L.B),
            f32_to_device(bq.clip_ratios(L.alpha_min)), f32_to_device(bq.clip_ratios(L.alpha_max)))
    y1 = bq.linear_w4a4(*args, wq, we, layout=T)
    xq, xe = bq.quantize_act(*args, layout=T)
    y2 = bq.gemm_w4a4(xq, xe, wq, we, layout=T)
    torch.cuda.synchronize()
    a, b = to_host(y1).astype(np.float64), to_host(y2).astype(np.float64)
    assert np.max(np.abs(a - b) / (np.abs(b) + 1e-3)) < 1e-4
    # deterministic
    y3 = bq.linear_w4a4(*args, wq, we, layout=T)
    torch.cuda.synchronize()
    assert torch.equal(y1, y3)


# ----------------------------------------------------------------------------------------
# W4A8: MXFP8 token rows
# ----------------------------------------------------------------------------------------

def run_linear8(bq, L, layout, workspace=True):
    import torch
    S, N = L.x_bits.shape
    wq, we = bq.prepare_weight(f32_to_device(L.W), L.A, L.B, layout=layout)
    x = bf16_to_device(L.x_bits)
    A, B = f32_to_device(L.A), f32_to_device(L.B)
    r1 = f32_to_device(bq.clip_ratios(L.alpha_min))
    r2 = f32_to_device(bq.clip_ratios(L.alpha_max))
    if workspace:
        y = bq.linear_w4a8(x, A, B, r1, r2, wq, we, layout=layout)
    else:
        out = wq.shape[0]
        y = torch.empty((S, out), dtype=torch.float32, device="cuda")
        st = bq.linear_w4a8_raw(x.data_ptr(), S, N, x.stride(0), A.data_ptr(), B.data_ptr(),
                                r1.data_ptr(), r2.data_ptr(), wq.data_ptr(), we.data_ptr(), out,
                                y.data_ptr(), 0, 0, layout=layout,
                                stream=torch.cuda.current_stream().cuda_stream)
        assert st == 0, bq.status_string(st)
    torch.cuda.synchronize()
    return to_host(y)


def check_linear8(orc, L, y, what):
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    xq8, xe = orc.quantize_act_fp8(L.x_bits, L.A, L.B, rmin, rmax, nthreads=ORACLE_THREADS)
    wq, we = orc.prepare_weight(L.W, L.A, L.B, nthreads=ORACLE_THREADS)
    y_ref, t_ref = orc.gemm_w4a8(xq8, xe, wq, we, nthreads=ORACLE_THREADS)
    assert_gemm_close(y, y_ref, t_ref, what=what)


@pytest.mark.parametrize("tiled", [True, False])
@pytest.mark.parametrize("S,N,out", [
    (1, 256, 33),               # one stage, ragged out
    (1, 16384, 4100),           # k = 512 (S k = 512)
    (2, 12288, 300),            # S k = 768, the largest the one kernel takes
    (3, 8192, 130),
    (4, 6144, 4096),            # S k = 768
])
def test_linear8_one_kernel(bq, orc, S, N, out, tiled):
    L = wl.make_layer(wl.custom("lin8", S, N, out, seed=(111, S, N, out),
                                outliers=("channels_uniform", 8, 20.0, 100.0)))
    layout = bq.SCALES_MFMA_TILED if tiled else bq.SCALES_ROW_MAJOR
    print(f"[linear8 one-kernel] S={S} N={N} out={out} tiled={tiled}", flush=True)
    y = run_linear8(bq, L, layout, workspace=False)
    check_linear8(orc, L, y, f"w4a8 one kernel S={S} N={N} out={out} tiled={tiled}")


@pytest.mark.parametrize("S,N,out", [
    (5, 4096, 96),              # more tokens than the one kernel takes
    (4, 8192, 64),              # S k = 1024 > 768
    (4, 4096, 12300),           # one kernel, the workspace unused
    (1, 2048, 40),
])
def test_linear8_with_workspace(bq, orc, S, N, out):
    L = wl.make_layer(wl.custom("lin8w", S, N, out, seed=(112, S, N, out)))
    y = run_linear8(bq, L, bq.SCALES_MFMA_TILED, workspace=True)
    check_linear8(orc, L, y, f"w4a8 workspace S={S} N={N} out={out}")

