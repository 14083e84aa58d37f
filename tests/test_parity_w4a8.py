"""GPU parity of the W4A8 setting (MXFP8 E4M3 activations against the MXFP4 weights)
against the CPU oracle on the same seeded inputs: activation codes and scales bit for bit,
and the W4A8 product within 1e-5 of sum|terms| of the oracle's exact fp64 product, the bound
of the W4A4 GEMM.  The product's operands are dequantised to bf16 on the GPU, which is exact
for activation scale bytes 9..246 (every random operand here uses 110..144); a case whose
sum has a large product and many small ones in each group of 8 K positions checks that the
small ones are kept (the scaled MFMA with an E4M3 operand drops them)."""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import (ORACLE_THREADS, assert_fp8_codes_equal, assert_gemm_close,
                            bf16_to_device,
                            f32_to_device, from_tiled_scales, to_host, to_tiled_scales,
                            u8_to_device)

W4A8_REL = 1e-5

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bq():
    import torch
    import w4a4_batq_quantize_amd as bq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bq.lib()
    return bq


def run_act8(bq, L, ldx=None, layout=0):
    import torch
    S, N = L.x_bits.shape
    if ldx is not None and ldx != N:
        wide = np.zeros((S, ldx), dtype=np.uint16)
        wide[:, :N] = L.x_bits
        wide[:, N:] = 0x7FC0                       # NaN padding: must never be read
        x = bf16_to_device(wide)[:, :N]
    else:
        x = bf16_to_device(L.x_bits)
    q, e = bq.quantize_act_mxfp8(x, f32_to_device(L.A), f32_to_device(L.B),
                                 f32_to_device(bq.clip_ratios(L.alpha_min)),
                                 f32_to_device(bq.clip_ratios(L.alpha_max)), layout=layout)
    torch.cuda.synchronize()
    q, e = to_host(q), to_host(e)
    if layout == bq.SCALES_MFMA_TILED:
        e = from_tiled_scales(e, S, N // 32)
    return q, e


def oracle_act8(orc, L):
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    q, e = orc.quantize_act_fp8(L.x_bits, L.A, L.B, rmin, rmax, nthreads=ORACLE_THREADS)
    # exact zeros of the clipped values (the transform and clip are those of the MXFP4 path)
    _, _, _, yc = orc.quantize_act(L.x_bits, L.A, L.B, rmin, rmax, debug=True,
                                   nthreads=ORACLE_THREADS)
    return q, e, yc == 0


@pytest.mark.parametrize("name", ["tiny", "q_proj", "down_proj", "sweep_s1_n12288",
                                  "sweep_s64_n4096"])
def test_act8_parity(bq, orc, name):
    L = wl.make_layer(name, with_weight=False)
    print(f"[act8 parity] {name} S={L.cfg.S} N={L.cfg.N}", flush=True)
    q, e = run_act8(bq, L)
    q_ref, e_ref, zero = oracle_act8(orc, L)
    assert_fp8_codes_equal(q, e, q_ref, e_ref, zero, what=name)
    # random activations reach E4M3 saturation (|y| / 2^(e-127) beyond 448) somewhere
    assert np.any((q_ref & 0x7F) == 0x7E)


@pytest.mark.parametrize("name", ["tiny", "down_proj", "sweep_s8_n4096"])
def test_act8_parity_tiled_scales(bq, orc, name):
    L = wl.make_layer(name, with_weight=False)
    q, e = run_act8(bq, L, layout=bq.SCALES_MFMA_TILED)
    q_ref, e_ref, zero = oracle_act8(orc, L)
    assert_fp8_codes_equal(q, e, q_ref, e_ref, zero, what=f"{name} tiled")


@pytest.mark.parametrize("S,N,ldx,seed", [
    (1, 32, 32, 1), (3, 96, 104, 2), (37, 4192, 4256, 3), (130, 2048, 2048, 4),
    (5, 64 * 32 * 3 + 32, 6208, 5),
    (2047, 4096, 4104, 6), (4099, 8224, 8232, 7),   # row-group kernels, ragged tails
])
def test_act8_parity_ragged_and_strided(bq, orc, S, N, ldx, seed):
    L = wl.make_layer(wl.custom("ragged", S, N, 8, seed=seed), with_weight=False)
    q, e = run_act8(bq, L, ldx=ldx)
    q_ref, e_ref, zero = oracle_act8(orc, L)
    assert_fp8_codes_equal(q, e, q_ref, e_ref, zero, what=f"S={S} N={N} ldx={ldx}")


def test_act8_parity_edge_blocks(bq, orc):
    """Identity factors, no clipping (r = 1), hand-built blocks: all zero, bf16 subnormals
    (scale clamped at 0), tiny normals, a block whose amax is just below the next power of
    two (saturation at 448 of the largest elements), exact powers of two, a single spike,
    alternating signs."""
    k = 8
    L = wl.make_layer(wl.custom("edge8", 6, 32 * k, 8, seed=98), with_weight=False)
    L.A = np.eye(8, dtype=np.float32)
    L.B = np.tile(np.eye(4, dtype=np.float32), (k, 1, 1))
    L.alpha_min = np.full(k, 40.0, dtype=np.float32)         # sigmoid rounds to 1
    L.alpha_max = np.full(k, 40.0, dtype=np.float32)
    rng = np.random.default_rng(6)
    f = lambda v: wl.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))
    x = L.x_bits.copy()
    x[0, 0:32] = 0
    x[0, 32:64] = rng.integers(1, 0x80, 32) | (rng.integers(0, 2, 32) << 15)
    x[1, 0:32] = f(rng.standard_normal(32) * 1e-37)
    x[1, 32:64] = f(np.linspace(-1.99, 1.99, 32))              # amax 1.99: top values saturate
    x[2, 0:32] = f(2.0 ** np.arange(-16, 16))                  # powers of two
    x[2, 32:64] = f(-(2.0 ** np.arange(90, 122)))
    x[3, 0:32] = f(np.where(np.arange(32) == 17, 1e4, 1e-3))
    x[3, 32:64] = f(np.where(np.arange(32) % 2 == 0, 1.0, -1.0))
    L.x_bits = x
    q, e = run_act8(bq, L)
    q_ref, e_ref, zero = oracle_act8(orc, L)
    assert_fp8_codes_equal(q, e, q_ref, e_ref, zero, what="edge8")
    assert e_ref[0, 1] == 0 and np.any(q_ref[0, 32:64] & 0x7F)
    assert np.sum((q_ref[1, 32:64] & 0x7F) == 0x7E) >= 2


# ----------------------------------------------------------------------------------------
# W4A8 GEMM
# ----------------------------------------------------------------------------------------

def gpu_gemm8(bq, xq8, xe, wq, we, tiled=False):
    import torch
    if tiled:
        xe, we = to_tiled_scales(xe), to_tiled_scales(we)
    y = bq.gemm_w4a8(u8_to_device(xq8), u8_to_device(xe), u8_to_device(wq), u8_to_device(we),
                     layout=bq.SCALES_MFMA_TILED if tiled else bq.SCALES_ROW_MAJOR)
    torch.cuda.synchronize()
    return to_host(y)


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("S,N,out", [
    (1, 256, 1), (3, 256, 5), (17, 4096, 100), (129, 4352, 300), (200, 256, 257),
    (64, 12288, 64), (128, 4096, 128), (256, 1024, 384), (300, 768, 20), (45, 2048, 77),
    (260, 512, 515),
    # few tokens (weight-streaming kernel): one and two token columns, ragged out, K ranges
    # shorter than the number of waves splitting K
    (33, 1280, 1), (2, 512, 31), (63, 4096, 64), (1, 8192, 4100), (64, 256, 33),
    (32, 512, 96), (40, 2048, 77),
])
def test_gemm8_random_operands_ragged(bq, orc, S, N, out, tiled):
    xq8, xe = wl.random_mxfp8(S, N, seed=(27, S, N, out))
    wq, we = wl.random_mxfp4(out, N, seed=(28, S, N, out))
    y = gpu_gemm8(bq, xq8, xe, wq, we, tiled)
    what = f"w4a8 S={S} N={N} out={out} tiled={tiled}"
    y_ref, t_ref = orc.gemm_w4a8(xq8, xe, wq, we, nthreads=ORACLE_THREADS)
    assert_gemm_close(y, y_ref, t_ref, rel=W4A8_REL, what=what)


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("S,N,out", [
    # at most 16 tokens: the 16-row kernel with E4M3 token fragments (one K stage; k = 512
    # with ragged out; a full round) and, past its dispatch rule, the 32-row kernel
    (1, 256, 17), (16, 4096, 1000), (3, 16384, 4100), (8, 12288, 6144), (4, 4096, 12300),
    # 33..64 tokens: two token halves per tile (out <= 4096) or the two-column kernel
    (40, 2048, 4096), (64, 1024, 300), (33, 1024, 4200),
])
def test_gemm8_few_tokens(bq, orc, S, N, out, tiled):
    xq8, xe = wl.random_mxfp8(S, N, seed=(79, S, N, out))
    wq, we = wl.random_mxfp4(out, N, seed=(80, S, N, out))
    print(f"[gemm8 few tokens] S={S} N={N} out={out} tiled={tiled}", flush=True)
    y = gpu_gemm8(bq, xq8, xe, wq, we, tiled)
    what = f"w4a8 few tokens S={S} N={N} out={out} tiled={tiled}"
    y_ref, t_ref = orc.gemm_w4a8(xq8, xe, wq, we, nthreads=ORACLE_THREADS)
    assert_gemm_close(y, y_ref, t_ref, rel=W4A8_REL, what=what)


@pytest.mark.parametrize("S,N,out", [(33, 1024, 70), (130, 2048, 260)])
def test_gemm8_narrow_scales(bq, orc, S, N, out):
    """Scales within a factor 32 of each other: every block contributes to every output, so
    a block dropped or misread anywhere shows."""
    xq8, xe = wl.random_mxfp8(S, N, seed=(29, S), scale_lo=125, scale_hi=130)
    wq, we = wl.random_mxfp4(out, N, seed=(30, S), scale_lo=125, scale_hi=130)
    for tiled in (False, True):
        y = gpu_gemm8(bq, xq8, xe, wq, we, tiled)
        y_ref, t_ref = orc.gemm_w4a8(xq8, xe, wq, we, nthreads=ORACLE_THREADS)
        assert_gemm_close(y, y_ref, t_ref, rel=W4A8_REL, what=f"narrow tiled={tiled}")


# E4M3 codes: 448 (the largest value) and 2^-6 (the smallest normal); E2M1 code of 1.0
E4M3_448, E4M3_2M6, E2M1_ONE = 0x7E, 0x08, 0x2


def small_products_operands(S, out, N=256):
    """Every token row: block 0 holds 448 and 31 times 2^-6, the other blocks zeros; every
    weight is 1.0; all scale bytes 127.  Each output is 448 + 31 * 2^-6 = 448.484375, exact
    in fp32 at every partial sum; products 2^-6 sit 14 octaves below 448 in every group of
    8 K positions of block 0."""
    xq8 = np.zeros((S, N), dtype=np.uint8)
    xq8[:, 0] = E4M3_448
    xq8[:, 1:32] = E4M3_2M6
    xe = np.full((S, N // 32), 127, dtype=np.uint8)
    wq = np.full((out, N // 2), E2M1_ONE | (E2M1_ONE << 4), dtype=np.uint8)
    we = np.full((out, N // 32), 127, dtype=np.uint8)
    return xq8, xe, wq, we


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("S,out", [(1, 64), (12, 4096), (17, 300), (40, 96), (64, 4096),
                                   (100, 300)])
def test_gemm8_small_products_are_kept(bq, orc, S, out, tiled):
    """Each W4A8 GEMM kernel (16-row and 32-row few-token kernels, the tiled kernel) keeps
    products far below the largest of their group: the exact sum, not 448.375 (what the
    scaled MFMA with an E4M3 operand returns here)."""
    xq8, xe, wq, we = small_products_operands(S, out)
    print(f"[gemm8 small products] S={S} out={out} tiled={tiled}", flush=True)
    y = gpu_gemm8(bq, xq8, xe, wq, we, tiled)
    y_ref, t_ref = orc.gemm_w4a8(xq8, xe, wq, we)
    assert np.all(y_ref == 448.0 + 31 * 2.0 ** -6)
    assert_gemm_close(y, y_ref, t_ref, rel=W4A8_REL, what=f"small products S={S} out={out}")
    assert np.array_equal(y.astype(np.float64), y_ref)


@pytest.mark.parametrize("S", [1, 4, 100])
def test_linear_w4a8_small_products_are_kept(bq, orc, S):
    """The same sum through the W4A8 layer (one kernel for S <= 4, quantiser + GEMM above):
    identity factors and unit clip ratios, so the MXFP8 quantiser encodes 448 and 2^-6
    exactly (scale byte 127), and weights of 1.0."""
    import torch
    N, out = 256, 64
    k = N // 32
    x = np.zeros((S, N), dtype=np.float32)
    x[:, 0] = 448.0
    x[:, 1:32] = 2.0 ** -6
    x_bits = wl.f32_to_bf16_bits(x)
    A = np.eye(8, dtype=np.float32)
    B = np.tile(np.eye(4, dtype=np.float32), (k, 1, 1))
    r = np.ones(k, dtype=np.float32)
    W = np.ones((out, N), dtype=np.float32)
    T = bq.SCALES_MFMA_TILED
    wq, we = bq.prepare_weight(f32_to_device(W), A, B, layout=T)
    y = bq.linear_w4a8(bf16_to_device(x_bits), f32_to_device(A), f32_to_device(B),
                       f32_to_device(r), f32_to_device(r), wq, we, layout=T)
    torch.cuda.synchronize()
    y = to_host(y).astype(np.float64)
    xq, xe = orc.quantize_act_fp8(x_bits, A, B, r, r)
    wq_ref, we_ref = orc.prepare_weight(W, A, B)
    y_ref, _ = orc.gemm_w4a8(xq, xe, wq_ref, we_ref)
    assert np.all(y_ref == 448.0 + 31 * 2.0 ** -6)
    assert np.array_equal(y, y_ref), f"S={S}: gpu {np.unique(y)[:4]}"


def test_gemm8_zero_k_writes_zeros(bq):
    import torch
    y = torch.full((5, 7), 3.0, device="cuda")
    x = torch.empty((5, 0), dtype=torch.uint8, device="cuda")
    w = torch.empty((7, 0), dtype=torch.uint8, device="cuda")
    bq.gemm_w4a8(x, x, w, w, y=y)
    assert torch.all(y == 0).item()


def test_gemm8_deterministic(bq):
    xq8, xe = wl.random_mxfp8(512, 4096, seed=1)
    wq, we = wl.random_mxfp4(1024, 4096, seed=2)
    assert np.array_equal(gpu_gemm8(bq, xq8, xe, wq, we), gpu_gemm8(bq, xq8, xe, wq, we))


def sample_rows(S):
    if S <= 64:
        return np.arange(S)
    return np.unique(np.array([0, 1, 127, 128, 255, 256, S // 2, S - 2, S - 1] +
                              list(range(0, S, max(1, S // 8)))))


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("name", ["tiny", "q_proj", "down_proj", "sweep_s1_n12288",
                                  "sweep_s8_n4096", "sweep_s16384_n12288"])
def test_linear_w4a8_end_to_end(bq, orc, name, tiled):
    """Seeded layer -> HIP weight prep + batq_linear_w4a8 (one kernel for the one-token
    decode layer, else HIP MXFP8 quantise + HIP W4A8 GEMM), against the oracle's MXFP8
    quantisation, weight preparation and fp64 W4A8 product on sampled token rows (every
    output column of those rows)."""
    import torch
    L = wl.make_layer(name)
    S, N, out = L.cfg.S, L.cfg.N, L.cfg.out
    print(f"[linear w4a8] {name} S={S} N={N} out={out} tiled={tiled}", flush=True)
    lay = bq.SCALES_MFMA_TILED if tiled else bq.SCALES_ROW_MAJOR
    wq, we = bq.prepare_weight(f32_to_device(L.W), L.A, L.B, layout=lay)
    y = bq.linear_w4a8(bf16_to_device(L.x_bits), f32_to_device(L.A), f32_to_device(L.B),
                       f32_to_device(bq.clip_ratios(L.alpha_min)),
                       f32_to_device(bq.clip_ratios(L.alpha_max)), wq, we, layout=lay)
    torch.cuda.synchronize()
    y = to_host(y)
    rows = sample_rows(S)
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    xq_ref, xe_ref = orc.quantize_act_fp8(L.x_bits[rows], L.A, L.B, rmin, rmax,
                                          nthreads=ORACLE_THREADS)
    wq_ref, we_ref = orc.prepare_weight(L.W, L.A, L.B, nthreads=ORACLE_THREADS)
    y_ref, t_ref = orc.gemm_w4a8(xq_ref, xe_ref, wq_ref, we_ref, nthreads=ORACLE_THREADS)
    assert_gemm_close(y[rows], y_ref, t_ref, rel=W4A8_REL, what=f"w4a8 {name} tiled={tiled}")
