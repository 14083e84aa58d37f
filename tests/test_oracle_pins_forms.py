"""CPU pins of the oracle's transform forms (thelatestinai listing, Table 1): a full 32x32
P_i per block ("w/o decomposition") and the naive Kronecker P_i = B_i (x) A_i with a private
A_i, next to GPK's P_i = B_i (x) A.  Each pin is checked against mathematics the oracle does
not share: exact arithmetic on dyadic inputs, a float64 matvec with its error bound, the
textbook fast Walsh-Hadamard transform, and exact rational inverses."""
from fractions import Fraction

import numpy as np
import pytest

import workloads as wl

FORM_GPK, FORM_KRONECKER, FORM_FULL = 0, 1, 2


def dyadic(rng, shape, lo=-16, hi=17, den=8):
    """Small dyadic rationals n/den: every product and partial sum below stays exact."""
    return (rng.integers(lo, hi, size=shape) / den).astype(np.float32)


def kron_blocks(B, A):
    """P_i = B_i (x) A_i with (B (x) A)[8r'+c', 8r+c] = B[r'][r] A[c'][c]."""
    k = B.shape[0]
    A = np.broadcast_to(A, (k, 8, 8)) if A.ndim == 2 else A
    return np.stack([np.kron(B[i].astype(np.float64), A[i].astype(np.float64))
                     for i in range(k)]).astype(np.float32)


def test_full_form_of_a_kronecker_product_equals_the_gpk_reshape(orc):
    rng = np.random.default_rng(1)
    k = 6
    x = rng.integers(-8, 9, size=(5, 32 * k)).astype(np.float32)
    A = dyadic(rng, (8, 8))
    B = dyadic(rng, (k, 4, 4))
    P = kron_blocks(B, A)
    y_full = orc.transform_form_f32(x, FORM_FULL, P, None)
    y_gpk = orc.transform_form_f32(x, FORM_GPK, A, B)
    y64 = np.concatenate([x[:, 32 * i:32 * i + 32].astype(np.float64) @ P[i].astype(np.float64)
                          for i in range(k)], axis=1)
    assert np.array_equal(y_full, y_gpk)
    assert np.array_equal(y_full.astype(np.float64), y64)
    # the GPK entry point of the original path agrees too
    assert np.array_equal(orc.transform_f32(x, A, B), y_gpk)


def test_kronecker_form_uses_each_blocks_own_a(orc):
    rng = np.random.default_rng(2)
    k = 5
    x = rng.integers(-8, 9, size=(4, 32 * k)).astype(np.float32)
    A = dyadic(rng, (k, 8, 8))
    B = dyadic(rng, (k, 4, 4))
    y_kron = orc.transform_form_f32(x, FORM_KRONECKER, A, B)
    y_full = orc.transform_form_f32(x, FORM_FULL, kron_blocks(B, A), None)
    assert np.array_equal(y_kron, y_full)
    # a shared A (every A_i equal) is GPK
    A0 = np.broadcast_to(A[0], (k, 8, 8)).copy()
    assert np.array_equal(orc.transform_form_f32(x, FORM_KRONECKER, A0, B),
                          orc.transform_form_f32(x, FORM_GPK, A[0], B))


def test_full_form_within_the_fp32_chain_bound_of_float64(orc):
    rng = np.random.default_rng(3)
    k = 4
    x = rng.standard_normal((16, 32 * k)).astype(np.float32) * 3
    P = (np.eye(32) + 0.3 * rng.standard_normal((k, 32, 32))).astype(np.float32)
    y = orc.transform_form_f32(x, FORM_FULL, P, None).astype(np.float64)
    for i in range(k):
        xb = x[:, 32 * i:32 * i + 32].astype(np.float64)
        exact = xb @ P[i].astype(np.float64)
        bound = 33 * 2.0 ** -24 * (np.abs(xb) @ np.abs(P[i].astype(np.float64)))
        err = np.abs(y[:, 32 * i:32 * i + 32] - exact)
        assert np.all(err <= bound)
        assert err.max() > 0                      # really fp32, not float64


def fwht(v):
    """Textbook unnormalised fast Walsh-Hadamard transform (natural order)."""
    v = list(v)
    h = 1
    while h < len(v):
        for i in range(0, len(v), 2 * h):
            for j in range(i, i + h):
                a, b = v[j], v[j + h]
                v[j], v[j + h] = a + b, a - b
        h *= 2
    return v


def test_full_form_with_sylvester_h32_is_the_walsh_hadamard_transform(orc):
    H = np.array([[1.0]])
    for _ in range(5):
        H = np.block([[H, H], [H, -H]])
    rng = np.random.default_rng(4)
    x = rng.integers(-100, 101, size=(3, 64)).astype(np.float32)
    y = orc.transform_form_f32(x, FORM_FULL, np.stack([H, H]).astype(np.float32), None)
    for r in range(3):
        for i in range(2):
            assert y[r, 32 * i:32 * i + 32].tolist() == fwht(x[r, 32 * i:32 * i + 32].tolist())


def test_identity_factors_reduce_to_plain_mxfp4(orc):
    L = wl.make_layer(wl.custom("forms-id", 7, 256, 8, seed=5), with_weight=False)
    k = 8
    ones = np.ones(k, dtype=np.float32)
    xf = wl.bf16_bits_to_f32(L.x_bits)
    q0, e0 = orc.clip_quantize_f32(xf, ones, ones)
    eye32 = np.broadcast_to(np.eye(32, dtype=np.float32), (k, 32, 32)).copy()
    eye8 = np.broadcast_to(np.eye(8, dtype=np.float32), (k, 8, 8)).copy()
    eye4 = np.broadcast_to(np.eye(4, dtype=np.float32), (k, 4, 4)).copy()
    for form, F0, F1 in ((FORM_FULL, eye32, None), (FORM_KRONECKER, eye8, eye4)):
        q, e = orc.quantize_act_form(L.x_bits, form, F0, F1, ones, ones)
        assert np.array_equal(q, q0) and np.array_equal(e, e0)


def test_form_dispatch_of_gpk_matches_the_original_entry_points(orc):
    L = wl.make_layer(wl.custom("forms-gpk", 9, 256, 12, seed=6))
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    q0, e0 = orc.quantize_act(L.x_bits, L.A, L.B, rmin, rmax)
    q1, e1 = orc.quantize_act_form(L.x_bits, FORM_GPK, L.A, L.B, rmin, rmax)
    assert np.array_equal(q0, q1) and np.array_equal(e0, e1)
    w0 = orc.prepare_weight(L.W, L.A, L.B)
    w1 = orc.prepare_weight_form(L.W, FORM_GPK, L.A, L.B)
    assert all(np.array_equal(a, b) for a, b in zip(w0, w1))


def test_full_inverse_is_exact_and_rounded_once(orc):
    rng = np.random.default_rng(7)
    P = (np.eye(32) + 0.1 * rng.standard_normal((32, 32))).astype(np.float32)
    inv = orc.exact_inverse(P)
    Pf = [[Fraction(float(v)) for v in row] for row in P]
    for i in range(32):
        for j in range(32):
            assert sum(inv[i][m] * Pf[m][j] for m in range(32)) == (1 if i == j else 0)
    G0, G1 = orc.weight_factors_form(FORM_FULL, P[None], None, 1)
    assert G1 is None
    # transposed, and each entry the nearest fp32 to the exact entry
    for i in range(0, 32, 7):
        for j in range(0, 32, 5):
            exact = inv[j][i]
            got = Fraction(float(G0[0, i, j]))
            nxt = np.nextafter(G0[0, i, j], np.float32(np.inf), dtype=np.float32)
            prv = np.nextafter(G0[0, i, j], np.float32(-np.inf), dtype=np.float32)
            assert abs(got - exact) <= abs(Fraction(float(nxt)) - exact)
            assert abs(got - exact) <= abs(Fraction(float(prv)) - exact)


@pytest.mark.parametrize("form", [FORM_KRONECKER, FORM_FULL])
def test_weight_side_keeps_x_w_transpose_invariant(orc, form):
    """(x P)(W P^-T)^T = x W^T: the transformed activations against the transformed weights
    (float64 product of the fp32 transforms) reproduce the plain product; a transposed or
    inverted-the-wrong-way factor breaks it by O(1)."""
    rng = np.random.default_rng(8 + form)
    k = 3
    x = rng.standard_normal((6, 32 * k)).astype(np.float32)
    W = rng.standard_normal((10, 32 * k)).astype(np.float32)
    if form == FORM_FULL:
        F0 = (np.eye(32) + 0.1 * rng.standard_normal((k, 32, 32))).astype(np.float32)
        F1 = None
    else:
        F0 = (np.eye(8) + 0.1 * rng.standard_normal((k, 8, 8))).astype(np.float32)
        F1 = (np.eye(4) + 0.1 * rng.standard_normal((k, 4, 4))).astype(np.float32)
    G0, G1 = orc.weight_factors_form(form, F0, F1, k)
    xa = orc.transform_form_f32(x, form, F0, F1).astype(np.float64)
    wa = orc.transform_form_f32(W, form, G0, G1).astype(np.float64)
    ref = x.astype(np.float64) @ W.astype(np.float64).T
    scale = np.abs(x).astype(np.float64) @ np.abs(W).astype(np.float64).T
    assert np.all(np.abs(xa @ wa.T - ref) <= 1e-5 * scale)
