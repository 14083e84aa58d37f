"""GPU parity of the RMSNorm-fused activation quantiser against the oracle on the same seeded
inputs: codes and scales bit for bit (the scale r and every normalised element are part of
the contract, so any difference in the sum order, the square root or the division shows)."""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import (ORACLE_THREADS, assert_codes_equal, bf16_to_device,
                            f32_to_device, from_tiled_scales, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bq():
    import torch
    import w4a4_batq_quantize_amd as bq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bq.lib()
    return bq


def gamma_for(N, seed):
    rng = np.random.default_rng(seed)
    return (1 + 0.1 * rng.standard_normal(N)).astype(np.float32)


def run(bq, L, gamma, eps, ldx=None, layout=0):
    import torch
    S, N = L.x_bits.shape
    if ldx is not None and ldx != N:
        wide = np.zeros((S, ldx), dtype=np.uint16)
        wide[:, :N] = L.x_bits
        wide[:, N:] = 0x7FC0                       # NaN padding: must never be read
        x = bf16_to_device(wide)[:, :N]
    else:
        x = bf16_to_device(L.x_bits)
    q, e = bq.quantize_act_rmsnorm(x, f32_to_device(gamma), eps, f32_to_device(L.A),
                                   f32_to_device(L.B), f32_to_device(bq.clip_ratios(L.alpha_min)),
                                   f32_to_device(bq.clip_ratios(L.alpha_max)), layout=layout)
    torch.cuda.synchronize()
    q, e = to_host(q), to_host(e)
    if layout == bq.SCALES_MFMA_TILED:
        e = from_tiled_scales(e, S, N // 32)
    return q, e


def oracle(orc, L, gamma, eps):
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    q, e = orc.quantize_act_rmsnorm(L.x_bits, gamma, eps, L.A, L.B, rmin, rmax)
    xh, _ = orc.rmsnorm(L.x_bits, gamma, eps)
    _, _, v = orc.clip_quantize_f32(orc.transform_f32(xh, L.A, L.B), rmin, rmax, debug=True)
    return q, e, v == 0


@pytest.mark.parametrize("name", ["tiny", "q_proj", "down_proj", "sweep_s1_n12288",
                                  "sweep_s64_n4096"])
def test_rmsnorm_quantize_parity(bq, orc, name):
    L = wl.make_layer(name, with_weight=False)
    gamma = gamma_for(L.cfg.N, 81)
    print(f"[rmsnorm parity] {name} S={L.cfg.S} N={L.cfg.N}", flush=True)
    q, e = run(bq, L, gamma, 1e-6)
    q_ref, e_ref, zero = oracle(orc, L, gamma, 1e-6)
    assert_codes_equal(q, e, q_ref, e_ref, zero, what=name)


@pytest.mark.parametrize("S,N,ldx,seed", [
    (3, 32, 32, 1),            # one block: the tree is empty
    (5, 96, 104, 2),           # k = 3: padded to 4
    (37, 4192, 4256, 3),       # k = 131: padded to 256, both threads' blocks in use
    (20, 16384, 16384, 4),     # k = 512, the largest row
    (130, 2048, 2048, 5),
])
def test_rmsnorm_quantize_ragged_strided_and_tiled(bq, orc, S, N, ldx, seed):
    L = wl.make_layer(wl.custom("rms-ragged", S, N, 8, seed=seed), with_weight=False)
    gamma = gamma_for(N, seed + 100)
    q_ref, e_ref, zero = oracle(orc, L, gamma, 1e-5)
    for layout in (bq.SCALES_ROW_MAJOR, bq.SCALES_MFMA_TILED):
        q, e = run(bq, L, gamma, 1e-5, ldx=ldx, layout=layout)
        assert_codes_equal(q, e, q_ref, e_ref, zero, what=f"S={S} N={N} layout={layout}")


def test_rmsnorm_quantize_edge_rows(bq, orc):
    """A zero row (scale 1/sqrt(eps)), a constant row, rows of very large and very small
    magnitude, a single spike, and eps = 0."""
    L = wl.make_layer(wl.custom("rms-edge", 6, 512, 8, seed=6), with_weight=False)
    f = lambda v: wl.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))
    x = L.x_bits.copy()
    x[0] = 0
    x[1] = f(np.full(512, 3.0))
    x[2] = f(np.random.default_rng(7).standard_normal(512) * 1e15)
    x[3] = f(np.random.default_rng(8).standard_normal(512) * 1e-15)
    x[4] = f(np.where(np.arange(512) == 100, 1e4, 1e-2))
    L.x_bits = x
    gamma = gamma_for(512, 9)
    for eps in (1e-6, 2.0 ** -20):
        q, e = run(bq, L, gamma, eps)
        q_ref, e_ref, zero = oracle(orc, L, gamma, eps)
        assert_codes_equal(q, e, q_ref, e_ref, zero, what=f"edge eps={eps}")
    L.x_bits = x[1:]                                  # eps = 0 needs a nonzero row
    q, e = run(bq, L, gamma, 0.0)
    q_ref, e_ref, zero = oracle(orc, L, gamma, 0.0)
    assert_codes_equal(q, e, q_ref, e_ref, zero, what="edge eps=0")


@pytest.mark.parametrize("squares,T_halving,T_sequential", [
    ([2 ** 24, 1, 1, 1, 1, 1, 1, 1], 2 ** 24 + 6, 2 ** 24),
    ([2 ** 24, 1, 1, 1, 1, 1], 2 ** 24 + 4, 2 ** 24),
])
def test_rmsnorm_block_sum_order_on_gpu(bq, orc, squares, T_halving, T_sequential):
    """The rows of the oracle's order pin (block sums of squares whose fp32 total depends on
    the order of the additions), with identity factors and unit ratios, and gamma of one
    element set so that its code is 4 under the halving order's scale r and 6 under the
    sequential order's: the code then shows which order the kernel used."""
    import torch
    k = len(squares)
    N = 32 * k
    x = np.zeros((1, N), dtype=np.float32)
    for b, sq in enumerate(squares):
        x[0, 32 * b] = np.sqrt(sq)
    f = np.float32
    r_h = f(1) / np.sqrt(f(T_halving) / f(N))
    r_s = f(1) / np.sqrt(f(T_sequential) / f(N))
    # gamma for element 32 (x = 1, alone in its block, so its scaled value lies in [4, 8)):
    # the fp32 nearest to 5 / r_h, nudged until r_h * gamma rounds to exactly 5 (a tie,
    # which rounds to the even code: value 4) while r_s * gamma rounds above 5 (value 6)
    g = f(5.0 / float(r_h))
    for _ in range(8):
        if f(r_h * g) == f(5) and f(r_s * g) > f(5):
            break
        g = np.nextafter(g, f(np.inf) if f(r_h * g) < f(5) else f(0))
    assert f(r_h * g) == f(5) and f(r_s * g) > f(5), "no separating gamma"
    gamma = np.ones(N, np.float32)
    gamma[32] = g
    L = wl.make_layer(wl.custom("rms-order", 1, N, 8, seed=10), with_weight=False)
    L.x_bits = wl.f32_to_bf16_bits(x)
    L.A = np.eye(8, dtype=np.float32)
    L.B = np.tile(np.eye(4, dtype=np.float32), (k, 1, 1))
    L.alpha_min = L.alpha_max = np.full(k, 30.0, np.float32)     # sigmoid(30) = 1 in fp32
    q, e = run(bq, L, gamma, 0.0)
    q_ref, e_ref, zero = oracle(orc, L, gamma, 0.0)
    assert (q_ref[0, 16] & 0xF) == 6                            # value 4 (the halving order)
    assert_codes_equal(q, e, q_ref, e_ref, zero, what=f"rmsnorm order k={k}")
