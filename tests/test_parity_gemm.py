"""GPU parity of the W4A4 scaled-MFMA GEMM against the oracle's fp64 reference:
|y_gpu - y_ref| <= 1e-5 * sum|terms| for every checked output."""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import (ORACLE_THREADS, assert_gemm_close, bf16_to_device,
                            f32_to_device, to_host, u8_to_device)

pytestmark = pytest.mark.gpu

# Scale bytes of the random operands: "wide" spans 35 octaves per operand (the sum |terms| of
# an output is then set by its few largest-scale blocks), "narrow" 5 octaves, so that every
# block's contribution is far above the 1e-5 sum|terms| bound and a misread code fragment or
# scale byte anywhere shows.
SCALES = {"wide": (110, 145), "narrow": (125, 130)}


@pytest.fixture(scope="module")
def bq():
    import torch
    import w4a4_batq_quantize_amd as bq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bq.lib()
    return bq


def gpu_gemm(bq, xq, xe, wq, we):
    import torch
    y = bq.gemm_w4a4(u8_to_device(xq), u8_to_device(xe), u8_to_device(wq), u8_to_device(we))
    torch.cuda.synchronize()
    return to_host(y)


@pytest.mark.parametrize("scales", list(SCALES))
@pytest.mark.parametrize("S,N,out", [
    (1, 32, 1), (3, 96, 5), (17, 4096, 100), (129, 4192, 300), (200, 256, 257),
    (64, 12288, 64), (128, 4096, 128), (256, 1024, 384), (300, 640, 20),
    # few tokens (weight-streaming path): ragged out, one and two token columns, K ranges
    # shorter than the number of waves splitting K
    (45, 2048, 77), (64, 256, 33), (1, 8192, 4100), (32, 512, 96), (33, 1536, 1),
])
def test_gemm_random_operands_ragged(bq, orc, S, N, out, scales):
    lo, hi = SCALES[scales]
    xq, xe = wl.random_mxfp4(S, N, seed=(7, S, N, out), scale_lo=lo, scale_hi=hi)
    wq, we = wl.random_mxfp4(out, N, seed=(8, S, N, out), scale_lo=lo, scale_hi=hi)
    y = gpu_gemm(bq, xq, xe, wq, we)
    y_ref, t_ref = orc.gemm(xq, xe, wq, we, nthreads=ORACLE_THREADS)
    assert_gemm_close(y, y_ref, t_ref, what=f"S={S} N={N} out={out} scales={scales}")


@pytest.mark.parametrize("scales", list(SCALES))
@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("S,N,out", [
    # at most 16 tokens: the 16-row kernel (one K stage over eight waves; the longest K it
    # takes, k = 512, with ragged out; a full round of workgroups; three rounds) and, past
    # its dispatch rule, the 32-row kernel with the same token count (k = 384, out = 6144)
    (1, 256, 17), (16, 256, 40), (2, 16384, 4100), (16, 4096, 4096), (1, 2048, 12290),
    (9, 8192, 700), (5, 12288, 6144),
    # 33..64 tokens: two token halves per 32-row tile (out <= 4096) or the two-column kernel
    (40, 2048, 4100), (64, 1024, 4096), (33, 1024, 4200), (64, 512, 8200),
])
def test_gemm_few_tokens_both_layouts(bq, orc, S, N, out, tiled, scales):
    import torch
    from tests.gpu_util import to_tiled_scales
    lo, hi = SCALES[scales]
    xq, xe = wl.random_mxfp4(S, N, seed=(77, S, N, out), scale_lo=lo, scale_hi=hi)
    wq, we = wl.random_mxfp4(out, N, seed=(78, S, N, out), scale_lo=lo, scale_hi=hi)
    if tiled:
        xe_d, we_d = to_tiled_scales(xe), to_tiled_scales(we)
    else:
        xe_d, we_d = xe, we
    print(f"[gemm few tokens] S={S} N={N} out={out} tiled={tiled} scales={scales}", flush=True)
    y = bq.gemm_w4a4(u8_to_device(xq), u8_to_device(xe_d), u8_to_device(wq), u8_to_device(we_d),
                     layout=bq.SCALES_MFMA_TILED if tiled else bq.SCALES_ROW_MAJOR)
    torch.cuda.synchronize()
    y_ref, t_ref = orc.gemm(xq, xe, wq, we, nthreads=ORACLE_THREADS)
    assert_gemm_close(to_host(y), y_ref, t_ref,
                      what=f"S={S} N={N} out={out} tiled={tiled} scales={scales}")


def test_gemm_zero_k_writes_zeros(bq):
    import torch
    y = torch.full((5, 7), 3.0, device="cuda")
    e = torch.empty((5, 0), dtype=torch.uint8, device="cuda")
    w = torch.empty((7, 0), dtype=torch.uint8, device="cuda")
    bq.gemm_w4a4(e, e, w, w, y=y)
    assert torch.all(y == 0).item()


def test_gemm_deterministic(bq):
    xq, xe = wl.random_mxfp4(512, 4096, seed=1)
    wq, we = wl.random_mxfp4(1024, 4096, seed=2)
    y1 = gpu_gemm(bq, xq, xe, wq, we)
    y2 = gpu_gemm(bq, xq, xe, wq, we)
    assert np.array_equal(y1, y2)


def sample_rows(S):
    if S <= 64:
        return np.arange(S)
    return np.unique(np.array([0, 1, 127, 128, 255, 256, S // 2, S - 2, S - 1] +
                              list(range(0, S, max(1, S // 8)))))


@pytest.mark.parametrize("name", ["tiny", "q_proj", "gate_up", "down_proj",
                                  "sweep_s1_n12288", "sweep_s8_n4096", "sweep_s64_n12288",
                                  "sweep_s16384_n4096"])
def test_linear_end_to_end(bq, orc, name):
    """Seeded layer -> HIP quantise + HIP weight prep + HIP GEMM, against the oracle's own
    quantisation, weight preparation and fp64 GEMM on sampled token rows (every output
    column of those rows)."""
    import torch
    L = wl.make_layer(name)
    S, N, out = L.cfg.S, L.cfg.N, L.cfg.out
    print(f"[linear] {name} S={S} N={N} out={out}", flush=True)
    wq, we = bq.prepare_weight(f32_to_device(L.W), L.A, L.B)
    y = bq.linear_w4a4(bf16_to_device(L.x_bits), f32_to_device(L.A), f32_to_device(L.B),
                       f32_to_device(bq.clip_ratios(L.alpha_min)),
                       f32_to_device(bq.clip_ratios(L.alpha_max)), wq, we)
    torch.cuda.synchronize()
    y = to_host(y)
    rows = sample_rows(S)
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    xq_ref, xe_ref = orc.quantize_act(L.x_bits[rows], L.A, L.B, rmin, rmax,
                                      nthreads=ORACLE_THREADS)
    wq_ref, we_ref = orc.prepare_weight(L.W, L.A, L.B, nthreads=ORACLE_THREADS)
    y_ref, t_ref = orc.gemm(xq_ref, xe_ref, wq_ref, we_ref, nthreads=ORACLE_THREADS)
    assert_gemm_close(y[rows], y_ref, t_ref, what=name)


# ----------------------------------------------------------------------------------------
# MFMA-tiled scale layout (padding bytes are E8M0 NaN: any use would poison a result)
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("scales", list(SCALES))
@pytest.mark.parametrize("S,N,out", [
    (1, 32, 1), (17, 4096, 100), (129, 4192, 300), (64, 12288, 64), (128, 4096, 128),
    (256, 1024, 384), (300, 2048, 520), (33, 256, 36),
    (50, 1024, 130), (2, 512, 31), (63, 4096, 64),
])
def test_gemm_random_operands_tiled_scales(bq, orc, S, N, out, scales):
    import torch
    from tests.gpu_util import to_tiled_scales
    lo, hi = SCALES[scales]
    xq, xe = wl.random_mxfp4(S, N, seed=(17, S, N, out), scale_lo=lo, scale_hi=hi)
    wq, we = wl.random_mxfp4(out, N, seed=(18, S, N, out), scale_lo=lo, scale_hi=hi)
    y = bq.gemm_w4a4(u8_to_device(xq), u8_to_device(to_tiled_scales(xe)), u8_to_device(wq),
                     u8_to_device(to_tiled_scales(we)), layout=bq.SCALES_MFMA_TILED)
    torch.cuda.synchronize()
    y_ref, t_ref = orc.gemm(xq, xe, wq, we, nthreads=ORACLE_THREADS)
    assert_gemm_close(to_host(y), y_ref, t_ref, what=f"tiled S={S} N={N} out={out} {scales}")


@pytest.mark.parametrize("name", ["q_proj", "gate_up", "down_proj", "sweep_s1_n12288",
                                  "sweep_s16384_n12288"])
def test_linear_end_to_end_tiled_scales(bq, orc, name):
    import torch
    L = wl.make_layer(name)
    S, N, out = L.cfg.S, L.cfg.N, L.cfg.out
    print(f"[linear tiled] {name} S={S} N={N} out={out}", flush=True)
    T = bq.SCALES_MFMA_TILED
    wq, we = bq.prepare_weight(f32_to_device(L.W), L.A, L.B, layout=T)
    y = bq.linear_w4a4(bf16_to_device(L.x_bits), f32_to_device(L.A), f32_to_device(L.B),
                       f32_to_device(bq.clip_ratios(L.alpha_min)),
                       f32_to_device(bq.clip_ratios(L.alpha_max)), wq, we, layout=T)
    torch.cuda.synchronize()
    y = to_host(y)
    rows = sample_rows(S)
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    xq_ref, xe_ref = orc.quantize_act(L.x_bits[rows], L.A, L.B, rmin, rmax,
                                      nthreads=ORACLE_THREADS)
    wq_ref, we_ref = orc.prepare_weight(L.W, L.A, L.B, nthreads=ORACLE_THREADS)
    y_ref, t_ref = orc.gemm(xq_ref, xe_ref, wq_ref, we_ref, nthreads=ORACLE_THREADS)
    assert_gemm_close(y[rows], y_ref, t_ref, what=f"{name} tiled")


# ----------------------------------------------------------------------------------------
# persistent 256 x 256 big-tile kernel (MFMA-tiled scales, N % 1024 == 0, >= 512 tiles)
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("scales", list(SCALES))
@pytest.mark.parametrize("S,N,out", [
    (8192, 4096, 4096),          # exactly 512 tiles: two per workgroup
    (4133, 1024, 8292),          # ragged tokens and outputs (17 x 33 tiles), K = 8 stages
    (16384, 2048, 8192),         # 2048 tiles: eight per workgroup
    (2048, 3072, 24576 + 40),    # gate/up-like, ragged out, K = 24 stages
])
def test_gemm_big_tiles(bq, orc, S, N, out, scales):
    """Sampled token rows (every output of each) against the oracle: the rows at every tile
    edge, the ragged tail and a spread through the middle."""
    import torch
    from tests.gpu_util import to_tiled_scales
    lo, hi = SCALES[scales]
    xq, xe = wl.random_mxfp4(S, N, seed=(91, S, N, out), scale_lo=lo, scale_hi=hi)
    wq, we = wl.random_mxfp4(out, N, seed=(92, S, N, out), scale_lo=lo, scale_hi=hi)
    print(f"[gemm big tiles] S={S} N={N} out={out} scales={scales}", flush=True)
    y = bq.gemm_w4a4(u8_to_device(xq), u8_to_device(to_tiled_scales(xe)), u8_to_device(wq),
                     u8_to_device(to_tiled_scales(we)), layout=bq.SCALES_MFMA_TILED)
    torch.cuda.synchronize()
    y = to_host(y)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 255, 256, 257, S // 2, S - 2, S - 1],
                                     np.arange(13, S, max(1, S // 24))]))
    rows = rows[rows < S]
    y_ref, t_ref = orc.gemm(xq, xe, wq, we, rows=rows, nthreads=ORACLE_THREADS)
    assert_gemm_close(y[rows], y_ref, t_ref, what=f"big S={S} N={N} out={out} {scales}")
