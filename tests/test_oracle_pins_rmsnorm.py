"""CPU pins of the oracle's RMSNorm prologue (its arithmetic contract is stated in
oracle/batq_oracle.c, orc_rmsnorm_f32): properties the definition must satisfy, checked
against float64 and exact scaling identities rather than a retyped formula."""
import numpy as np
import pytest

import workloads as wl


def bf16(a):
    return wl.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


@pytest.mark.parametrize("N", [32, 96, 4096, 4192, 12288])
def test_scale_within_a_few_ulp_of_float64(orc, N):
    rng = np.random.default_rng(N)
    x = bf16(rng.standard_normal((6, N)) * np.array([1, 10, 0.01, 300, 1e-3, 5])[:, None])
    gamma = (1 + 0.1 * rng.standard_normal(N)).astype(np.float32)
    eps = 1e-6
    xh, r = orc.rmsnorm(x, gamma, eps)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    r64 = 1.0 / np.sqrt((xf ** 2).sum(axis=1) / N + eps)
    k = N // 32
    tol = (40 + np.ceil(np.log2(max(k, 1)))) * 2.0 ** -24
    assert np.all(np.abs(r / r64 - 1) <= tol)
    ref = xf * r64[:, None] * gamma.astype(np.float64)[None, :]
    assert np.all(np.abs(xh - ref) <= (tol + 3 * 2.0 ** -24) * np.abs(ref) + 1e-38)


def test_power_of_two_input_scale_cancels_exactly(orc):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 1024)).astype(np.float32)
    gamma = (1 + 0.1 * rng.standard_normal(1024)).astype(np.float32)
    a, _ = orc.rmsnorm(bf16(x), gamma, 0.0)
    for m in (-20, -3, 4, 30):
        b, _ = orc.rmsnorm(bf16(x * 2.0 ** m), gamma, 0.0)
        assert np.array_equal(a, b), m


def test_gamma_scales_the_output_exactly(orc):
    rng = np.random.default_rng(2)
    x = bf16(rng.standard_normal((3, 512)))
    gamma = (1 + 0.1 * rng.standard_normal(512)).astype(np.float32)
    a, ra = orc.rmsnorm(x, gamma, 1e-5)
    b, rb = orc.rmsnorm(x, gamma * 4, 1e-5)
    assert np.array_equal(ra, rb) and np.array_equal(b, 4 * a)


def test_mean_is_over_n_and_eps_inside_the_root(orc):
    # constant rows: with eps = 0 the scale is exactly 1 for any block count, including
    # k = 3 and 5 where the power-of-two padding of the block sums must add only zeros
    for N in (96, 160, 4096):
        xh, r = orc.rmsnorm(bf16(np.ones((1, N))), np.full(N, 3.0, np.float32), 0.0)
        assert r[0] == 1.0 and np.all(xh == 3.0)
        xh, r = orc.rmsnorm(bf16(np.full((1, N), 4.0)), np.ones(N, np.float32), 0.0)
        assert r[0] == 0.25 and np.all(xh == 1.0)
    # a zero row: r = 1/sqrt(eps) exactly for eps = 2^-20, output zeros
    xh, r = orc.rmsnorm(bf16(np.zeros((1, 64))), np.ones(64, np.float32), 2.0 ** -20)
    assert r[0] == 2.0 ** 10 and np.all(xh == 0)


def test_fused_quantiser_is_rmsnorm_then_the_pinned_quantiser(orc):
    L = wl.make_layer(wl.custom("rms-pin", 9, 416, 8, seed=3), with_weight=False)
    rng = np.random.default_rng(4)
    gamma = (1 + 0.2 * rng.standard_normal(416)).astype(np.float32)
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    q, e = orc.quantize_act_rmsnorm(L.x_bits, gamma, 1e-6, L.A, L.B, rmin, rmax)
    xh, _ = orc.rmsnorm(L.x_bits, gamma, 1e-6)
    q2, e2 = orc.clip_quantize_f32(orc.transform_f32(xh, L.A, L.B), rmin, rmax)
    assert np.array_equal(q, q2) and np.array_equal(e, e2)


@pytest.mark.parametrize("squares,T_halving,T_sequential", [
    # block sums of squares chosen so that fp32 rounding depends on the order of the additions
    # (2^24 + 1 is a tie between 2^24 and 2^24 + 2 and rounds to the even 2^24; 2^24 + 3 a
    # tie between 2^24 + 2 and 2^24 + 4, which is the even one):
    #   halving (t[b] += t[b + h], h = K/2 .. 1), eight blocks:
    #     h=4: 2^24+1 -> 2^24, 2, 2, 2;  h=2: 2^24+2, 4;  h=1: 2^24+6
    #   sequential: every +1 onto 2^24 is a tie that rounds back to 2^24
    ([2 ** 24, 1, 1, 1, 1, 1, 1, 1], 2 ** 24 + 6, 2 ** 24),
    # six blocks, padded to eight with zero sums:
    #     h=4: 2^24+1 -> 2^24, 1+1 = 2, 1, 1;  h=2: 2^24+1 -> 2^24, 3;  h=1: 2^24+3 -> 2^24+4
    ([2 ** 24, 1, 1, 1, 1, 1], 2 ** 24 + 4, 2 ** 24),
])
def test_block_sums_are_added_by_halving(orc, squares, T_halving, T_sequential):
    """The order in which the per-block sums of squares are added is part of the stated
    arithmetic (halving over the zero-padded power-of-two count).  Rows whose sum rounds
    differently under another order pin it: the expected scale is worked out by hand from
    the sum above, then through fp32 division, square root and reciprocal (IEEE, correctly
    rounded: numpy's float32 operations)."""
    k = len(squares)
    N = 32 * k
    x = np.zeros((1, N), dtype=np.float32)
    for b, sq in enumerate(squares):
        x[0, 32 * b] = np.sqrt(sq)                   # one element per block: 2^12 or 1
    _, r = orc.rmsnorm(bf16(x), np.ones(N, np.float32), 0.0)
    f = np.float32
    expect = f(1) / np.sqrt(f(T_halving) / f(N))
    other = f(1) / np.sqrt(f(T_sequential) / f(N))
    assert expect != other
    assert r[0] == expect
