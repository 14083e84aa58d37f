"""Pins of the CPU oracle against what the pages and the mathematics fix (CPU only).

Each test states its check in a formulation of its own (closed forms, the explicit
Kronecker product, a textbook Walsh-Hadamard transform, exact rationals, exhaustive
enumeration), so that a dropped term, a wrong sign or index or a transposed operand in the
oracle fails at least one of them.
"""
import json
import math
import os
from concurrent.futures import ThreadPoolExecutor
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f32bits(v) -> int:
    return int(np.array(v, dtype=np.float32).view(np.uint32))


def dyadic(rng, shape, num=8):
    """Entries k/8 with |k| <= num: every fp32 product and short sum of them is exact."""
    return (rng.integers(-num, num + 1, size=shape) / 8.0).astype(np.float32)


# E2M1 rounding written as bit-pattern thresholds: the magnitude code is the number of
# midpoints passed; a value exactly on a midpoint goes to the even code, so the comparison
# is strict where the lower neighbour is even and inclusive where the upper one is.
E2M1_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
_THRESH = [(0.25, "gt"), (0.75, "ge"), (1.25, "gt"), (1.75, "ge"), (2.5, "gt"), (3.5, "ge"),
           (5.0, "gt")]


def expected_e2m1_codes(u: np.ndarray) -> np.ndarray:
    u = u.astype(np.uint32, copy=False)
    mag = u & np.uint32(0x7FFFFFFF)
    code = np.zeros(u.shape, dtype=np.uint8)
    for val, op in _THRESH:
        b = np.uint32(f32bits(val))
        code += (mag > b) if op == "gt" else (mag >= b)
    code |= ((u >> np.uint32(31)).astype(np.uint8) << np.uint8(3))
    code[mag >= np.uint32(0x7F800000)] = 0xFF
    return code


def nearest_even_code_exact(v: float) -> int:
    """Definition by brute force: nearest E2M1 value by exact rational distance, ties to the
    even magnitude code, sign copied."""
    a = abs(Fraction(v))
    d = [abs(a - Fraction(g)) for g in E2M1_GRID]
    best = min(d)
    cands = [c for c in range(8) if d[c] == best]
    c = cands[0] if len(cands) == 1 else next(c for c in cands if c % 2 == 0)
    return (8 if math.copysign(1.0, v) < 0 else 0) | c


def plain_mxfp4(x: np.ndarray):
    """Plain MXFP4 round-to-nearest of fp32 rows (no transform, no clip), written here
    independently of the oracle: OCP MX scale exponent floor(log2 amax) - 2 clamped to
    [-127, 127], values divided by the scale, E2M1 by the threshold table."""
    rows, N = x.shape
    xb = x.reshape(rows, N // 32, 32).astype(np.float64)
    amax = np.abs(xb).max(-1)
    _, ex = np.frexp(amax)
    sexp = np.clip(ex - 1 - 2, -127, 127)
    byte = np.where(amax > 0, sexp + 127, 0).astype(np.int64)
    v = xb / np.ldexp(1.0, byte - 127)[..., None]
    codes = expected_e2m1_codes(v.astype(np.float32).view(np.uint32)).reshape(rows, N)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return q, byte.astype(np.uint8)


def zero_sign_equal(q_a, q_b, exact_zero_mask):
    """Codes equal, except that a code whose pre-rounding value is exactly +-0 may differ
    in its sign bit."""
    ca = np.stack([q_a & 0xF, q_a >> 4], -1).reshape(q_a.shape[0], -1)
    cb = np.stack([q_b & 0xF, q_b >> 4], -1).reshape(q_b.shape[0], -1)
    diff = ca != cb
    ok_zero = exact_zero_mask & ((ca & 7) == 0) & ((cb & 7) == 0)
    return not np.any(diff & ~ok_zero)


# ----------------------------------------------------------------------------------------
# P1  reshape form == explicit 32x32 Kronecker matvec
# ----------------------------------------------------------------------------------------

def test_p1_reshape_equals_kron_matvec_exactly_on_dyadic_inputs(orc):
    rng = np.random.default_rng(11)
    k, rows = 6, 5
    A = dyadic(rng, (8, 8))
    B = dyadic(rng, (k, 4, 4))
    x = dyadic(rng, (rows, 32 * k))
    y = orc.transform_f32(x, A, B)
    for i in range(k):
        P = np.kron(B[i].astype(np.float64), A.astype(np.float64))
        ref = x[:, 32 * i:32 * i + 32].astype(np.float64) @ P
        assert np.array_equal(y[:, 32 * i:32 * i + 32].astype(np.float64), ref)


def test_p1_reshape_vs_kron_matvec_random_within_fp32_chain_bound(orc):
    rng = np.random.default_rng(12)
    k, rows = 8, 9
    A = (np.eye(8) + 0.3 * rng.standard_normal((8, 8))).astype(np.float32)
    B = (np.eye(4) + 0.3 * rng.standard_normal((k, 4, 4))).astype(np.float32)
    x = (rng.standard_normal((rows, 32 * k)) * 3).astype(np.float32)
    y = orc.transform_f32(x, A, B).astype(np.float64)
    for i in range(k):
        P = np.kron(B[i].astype(np.float64), A.astype(np.float64))
        xb = x[:, 32 * i:32 * i + 32].astype(np.float64)
        ref = xb @ P
        T = np.abs(xb) @ np.abs(P)
        # 8-term then 4-term fp32 chains: |error| <= ~12 u sum|terms|, u = 2^-24
        assert np.all(np.abs(y[:, 32 * i:32 * i + 32] - ref) <= 2e-6 * T)
        # and the transform is not the identity (the check has teeth)
        assert np.max(np.abs(ref - xb)) > 0.1


# ----------------------------------------------------------------------------------------
# P2  GPK structure and Table 1 counts
# ----------------------------------------------------------------------------------------

def test_p2_table1_parameter_counts():
    g = json.load(open(os.path.join(GOLDEN, "table1_gpk_params.json")))
    N, gs, g1, g2 = g["N"], g["g"], g["g1"], g["g2"]
    k = N // gs
    assert g1 * g2 == gs
    p = g["params"]
    assert g1 ** 2 + k * g2 ** 2 == p["gpk"] == 2112
    assert N * gs == p["wo_decomposition"]
    assert k * (g1 ** 2 + g2 ** 2) == p["naive_kronecker"]
    assert 2 * N == p["flatquant_kronecker"]
    r = g["reduction_percent"]
    assert round(100 * (1 - p["gpk"] / p["wo_decomposition"]), 1) == r["vs_wo_decomposition"]
    assert round(100 * (1 - p["gpk"] / p["flatquant_kronecker"])) == r["vs_flatquant"]
    assert round(100 * (1 - p["gpk"] / p["naive_kronecker"])) == r["vs_naive_kronecker"]
    # the configs' own counts
    assert 8 ** 2 + (256 // 32) * 16 == 192
    assert 8 ** 2 + (12288 // 32) * 16 == 6208


def test_p2_oracle_transform_is_block_diagonal_kron_with_shared_A(orc):
    """Probing the oracle's transform with unit vectors at N=4096 recovers P itself: it is
    block-diagonal with 32x32 blocks B_i (x) A, so its parameters are A's 64 entries and
    the 16 entries of each of the 128 B_i: g1^2 + k g2^2 = 2,112."""
    rng = np.random.default_rng(21)
    N = 4096
    k = N // 32
    A = (np.eye(8) + 0.2 * rng.standard_normal((8, 8))).astype(np.float32)
    B = (np.eye(4) + 0.2 * rng.standard_normal((k, 4, 4))).astype(np.float32)
    P = orc.transform_f32(np.eye(N, dtype=np.float32), A, B)   # row j = e_j P
    blk = np.arange(N) // 32
    off = blk[:, None] != blk[None, :]
    assert not np.any(P[off])
    for i in range(k):
        ref = np.kron(B[i].astype(np.float64), A.astype(np.float64)).astype(np.float32)
        assert np.array_equal(P[32 * i:32 * i + 32, 32 * i:32 * i + 32], ref)
    assert A.size + B.size == 2112


# ----------------------------------------------------------------------------------------
# P3  E2M1 and E8M0
# ----------------------------------------------------------------------------------------

def test_p3_threshold_table_is_nearest_ties_to_even():
    """The threshold table used below is the definition 'nearest E2M1 value, ties to the
    even code, saturate at 6', checked by exact brute force around every midpoint."""
    pts = [0.0, -0.0, 1e-45, -1e-45, 6.0, 7.0, 100.0, 3.0e38, -3.0e38]
    for m in [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] + E2M1_GRID:
        f = np.float32(m)
        for s in range(-3, 4):
            pts.append(float(np.nextafter(f, np.float32(np.inf * np.sign(s))) if s else f))
            g = f
            for _ in range(abs(s)):
                g = np.nextafter(g, np.float32(np.inf if s > 0 else -np.inf))
            pts.append(float(g))
    pts += [-p for p in pts]
    u = np.array(pts, dtype=np.float32).view(np.uint32)
    exp = expected_e2m1_codes(u)
    for p, c in zip(pts, exp):
        assert c == nearest_even_code_exact(p), (p, c)


def test_p3_e2m1_exhaustive_all_fp32_patterns(orc):
    """Every one of the 2^32 fp32 bit patterns (non-finite ones are marked 0xFF)."""
    chunk = 1 << 26

    def run(t):
        start = t * chunk
        got = orc.e2m1_round_bits(start, chunk)
        u = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
        exp = expected_e2m1_codes(u)
        bad = np.flatnonzero(got != exp)
        return None if bad.size == 0 else (start + int(bad[0]), int(got[bad[0]]), int(exp[bad[0]]))

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(run, range((1 << 32) // chunk)))
    fails = [r for r in results if r is not None]
    assert not fails, fails[:4]


def test_p3_e2m1_values_and_e8m0_scale_table(orc):
    # all 16 codes decode to {+-0, +-0.5, ..., +-6}; all 255 finite scale bytes to 2^(b-127)
    codes = np.arange(16, dtype=np.uint8)
    q = np.zeros((255, 16), dtype=np.uint8)
    q[:, :8] = codes[0::2] | (codes[1::2] << 4)
    e = np.arange(255, dtype=np.uint8).reshape(255, 1)
    dq = orc.dequant(q, e)
    vals = np.array(E2M1_GRID + [-g for g in E2M1_GRID])
    for b in range(255):
        assert np.array_equal(dq[b, :16], vals * 2.0 ** (b - 127))
        assert np.all(dq[b, 16:] == 0)


def test_p3_e8m0_rule_matches_exponent_field_form(orc):
    """Oracle scale (floor(log2 amax) - 2, clamped, via frexp) equals max(E - 2, 0) where E
    is the biased exponent field of fp32 amax, for every exponent field and several
    mantissas, including subnormal amax and zero."""
    amax, exp = [0.0], [0]
    for E in range(0, 255):
        for m in (0, 1, 0x2AAAAA, 0x400000, 0x7FFFFF):
            if E == 0 and m == 0:
                continue
            u = np.uint32((E << 23) | m)
            amax.append(float(u.view(np.float32)))
            exp.append(max(E - 2, 0))
    got = orc.e8m0_scale(np.array(amax, dtype=np.float32))
    assert np.array_equal(got, np.array(exp, dtype=np.uint8))
    # floor(log2) by integer arithmetic on the exact rational value, for normal amax
    for a, g in zip(amax[1:50:3] + amax[300::97], got[1:50:3].tolist() + got[300::97].tolist()):
        fr = Fraction(a)
        fl = fr.numerator.bit_length() - fr.denominator.bit_length()
        if Fraction(2) ** fl > fr:
            fl -= 1
        assert g == min(max(fl - 2, -127), 127) + 127


# ----------------------------------------------------------------------------------------
# P4  identity factors + unit clip ratios == plain MXFP4 RTN
# ----------------------------------------------------------------------------------------

def test_p4_identity_transform_and_saturated_clip_reduce_to_plain_mxfp4(orc):
    cfg = wl.custom("p4", 40, 512, 32, seed=123)
    L = wl.make_layer(cfg, with_weight=False)
    k = cfg.k
    r = orc.clip_ratio(np.full(k, 30.0, dtype=np.float32))
    assert np.all(r == 1.0)
    A = np.eye(8, dtype=np.float32)
    B = np.tile(np.eye(4, dtype=np.float32), (k, 1, 1))
    q, e, v, yc = orc.quantize_act(L.x_bits, A, B, r, r, debug=True)
    x = wl.bf16_bits_to_f32(L.x_bits)
    q_ref, e_ref = plain_mxfp4(x)
    assert np.array_equal(e, e_ref)
    assert zero_sign_equal(q, q_ref, x == 0)


def test_p4_identity_weight_prep_is_plain_mxfp4_of_fp32_weights(orc):
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((24, 320)) * 0.02).astype(np.float32)
    W[3, 7] = 1.5    # an outlier
    k = 10
    A = np.eye(8, dtype=np.float32)
    B = np.tile(np.eye(4, dtype=np.float32), (k, 1, 1))
    q, e = orc.prepare_weight(W, A, B)
    q_ref, e_ref = plain_mxfp4(W)
    assert np.array_equal(e, e_ref)
    assert zero_sign_equal(q, q_ref, W == 0)


# ----------------------------------------------------------------------------------------
# P5  Hadamard factors give the block Walsh-Hadamard transform
# ----------------------------------------------------------------------------------------

def sylvester(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def fwht(x):
    """Textbook in-place fast Walsh-Hadamard transform (natural order) on the last axis."""
    x = np.array(x, dtype=np.float64)
    h = 1
    n = x.shape[-1]
    while h < n:
        for i in range(0, n, 2 * h):
            a = x[..., i:i + h].copy()
            b = x[..., i + h:i + 2 * h].copy()
            x[..., i:i + h] = a + b
            x[..., i + h:i + 2 * h] = a - b
        h *= 2
    return x


def test_p5_hadamard_factors_give_block_walsh_hadamard(orc):
    assert np.array_equal(np.kron(sylvester(4), sylvester(8)), sylvester(32))
    rng = np.random.default_rng(3)
    k, rows = 4, 6
    x = rng.integers(-100, 101, size=(rows, 32 * k)).astype(np.float32)
    A = sylvester(8).astype(np.float32)
    B = np.tile(sylvester(4).astype(np.float32), (k, 1, 1))
    y = orc.transform_f32(x, A, B)
    ref = fwht(x.reshape(rows, k, 32)).reshape(rows, 32 * k)
    assert np.array_equal(y.astype(np.float64), ref)


# ----------------------------------------------------------------------------------------
# P6  clipping
# ----------------------------------------------------------------------------------------

def test_p6_clip_matches_numpy_clamp_of_transform_output(orc):
    cfg = wl.custom("p6", 33, 384, 16, seed=77)
    L = wl.make_layer(cfg, with_weight=False)
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    assert not np.array_equal(rmin, rmax)
    q, e, v, yc = orc.quantize_act(L.x_bits, L.A, L.B, rmin, rmax, debug=True)
    y = orc.transform_f32(wl.bf16_bits_to_f32(L.x_bits), L.A, L.B)
    yb = y.reshape(cfg.S, cfg.k, 32)
    lo = (rmin[None, :] * yb.min(-1)).astype(np.float32)      # fp32 products, RNE
    hi = (rmax[None, :] * yb.max(-1)).astype(np.float32)
    ref = np.minimum(np.maximum(yb, lo[..., None]), hi[..., None])
    assert np.array_equal(yc.reshape(cfg.S, cfg.k, 32), ref)
    assert np.all(ref >= lo[..., None]) and np.all(ref <= hi[..., None])
    # clipping is active on these inputs (sigmoid(~2) ~ 0.88)
    assert np.mean(ref != yb) > 0.01
    # largest |clipped| equals max(|clamp(min)|, |clamp(max)|)
    cm = np.minimum(np.maximum(yb.min(-1), lo), hi)
    cM = np.minimum(np.maximum(yb.max(-1), lo), hi)
    assert np.array_equal(np.abs(ref).max(-1), np.maximum(np.abs(cm), np.abs(cM)))


def test_p6_unit_ratio_is_a_no_op_and_lo_above_hi_gives_hi(orc):
    rng = np.random.default_rng(8)
    y = rng.standard_normal((4, 64)).astype(np.float32)
    one = np.ones(2, dtype=np.float32)
    q1, e1 = orc.clip_quantize_f32(y, one, one, clip=True)
    q0, e0 = orc.clip_quantize_f32(y, clip=False)
    assert np.array_equal(q1, q0) and np.array_equal(e1, e0)
    # an all-positive block with r_min * min > r_max * max: every element becomes hi
    yb = np.linspace(10.0, 11.0, 32, dtype=np.float32)[None, :]
    rmin = np.array([0.99], dtype=np.float32)
    rmax = np.array([0.5], dtype=np.float32)
    q, e, v = orc.clip_quantize_f32(yb, rmin, rmax, clip=True, debug=True)
    hi = np.float32(rmax[0] * np.float32(11.0))
    assert np.float32(rmin[0] * np.float32(10.0)) > hi
    assert np.array_equal(v[0].astype(np.float64) * 2.0 ** (int(e[0, 0]) - 127),
                          np.full(32, float(hi)))


# ----------------------------------------------------------------------------------------
# P7  offline weight side: exact inverses and the direction of P^-1
# ----------------------------------------------------------------------------------------

def test_p7_round_fraction_f32_is_correct_rounding(orc):
    rng = np.random.default_rng(9)
    d = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000),
                        rng.standard_normal(200) * 1e-42])
    for v in d.tolist():
        assert orc.round_fraction_f32(Fraction(v)) == float(np.float32(v))
    one = Fraction(1)
    assert orc.round_fraction_f32(one + Fraction(1, 2 ** 24)) == 1.0              # tie -> even
    assert orc.round_fraction_f32(one + Fraction(3, 2 ** 24)) == 1.0 + 2.0 ** -22  # tie -> even
    assert orc.round_fraction_f32(Fraction(1, 2 ** 150)) == 0.0                     # subnormal tie
    assert orc.round_fraction_f32(Fraction(3, 2 ** 150)) == 2.0 ** -148
    assert orc.round_fraction_f32(-Fraction(1, 3)) == float(np.float32(-1 / 3))


def test_p7_exact_inverse(orc):
    rng = np.random.default_rng(10)
    for n in (4, 8):
        for _ in range(5):
            M = (np.eye(n) + 0.1 * rng.standard_normal((n, n))).astype(np.float32)
            inv = orc.exact_inverse(M)
            Mf = [[Fraction(float(v)) for v in row] for row in M]
            prod = [[sum(Mf[i][t] * inv[t][j] for t in range(n)) for j in range(n)]
                    for i in range(n)]
            assert all(prod[i][j] == (1 if i == j else 0) for i in range(n) for j in range(n))
            inv32 = orc.exact_inverse_f32(M)
            ref = np.linalg.inv(M.astype(np.float64)).astype(np.float32)
            assert np.max(np.abs(inv32.view(np.int32) - ref.view(np.int32))) <= 1
    with pytest.raises(ZeroDivisionError):
        orc.exact_inverse(np.array([[1, 2], [2, 4]], dtype=np.float32))


def test_p7_weight_side_transform_undoes_activation_side(orc):
    """(X P)(W P^-T)^T = X W^T up to fp32 rounding; a transposed or un-inverted factor
    leaves errors of order 0.1."""
    rng = np.random.default_rng(13)
    S, N, out = 6, 128, 5
    k = N // 32
    A = (np.eye(8) + 0.2 * rng.standard_normal((8, 8))).astype(np.float32)
    B = (np.eye(4) + 0.2 * rng.standard_normal((k, 4, 4))).astype(np.float32)
    X = rng.standard_normal((S, N)).astype(np.float32)
    W = rng.standard_normal((out, N)).astype(np.float32)
    Ai, Bi = orc.weight_factors(A, B)
    XT = orc.transform_f32(X, A, B).astype(np.float64)
    WT = orc.transform_f32(W, Ai, Bi).astype(np.float64)
    lhs = XT @ WT.T
    rhs = X.astype(np.float64) @ W.astype(np.float64).T
    T = np.abs(XT) @ np.abs(WT).T
    assert np.all(np.abs(lhs - rhs) <= 1e-5 * T)
    # teeth: the un-transposed inverse does not undo the transform
    Ai_wrong = np.ascontiguousarray(Ai.T)
    WT_wrong = orc.transform_f32(W, Ai_wrong, Bi).astype(np.float64)
    assert np.max(np.abs(XT @ WT_wrong.T - rhs) / T) > 1e-2


# ----------------------------------------------------------------------------------------
# P8  GEMM reference against exact rational arithmetic
# ----------------------------------------------------------------------------------------

TWICE_E2M1 = [0, 1, 2, 3, 4, 6, 8, 12]   # 2 x E2M1 magnitudes are integers


def exact_value(code, ebyte):
    m = Fraction(TWICE_E2M1[code & 7], 2) * Fraction(2) ** (int(ebyte) - 127)
    return -m if code & 8 else m


@pytest.mark.parametrize("S,N,out", [(3, 32, 5), (5, 64, 7), (2, 96, 3)])
def test_p8_gemm_reference_vs_exact_rationals(orc, S, N, out):
    rng = np.random.default_rng(S * 100 + N + out)
    xq = rng.integers(0, 256, size=(S, N // 2), dtype=np.uint8)
    wq = rng.integers(0, 256, size=(out, N // 2), dtype=np.uint8)
    xe = rng.integers(100, 150, size=(S, N // 32), dtype=np.uint8)
    we = rng.integers(100, 150, size=(out, N // 32), dtype=np.uint8)
    y, t = orc.gemm(xq, xe, wq, we)

    def codes(q):
        return np.stack([q & 0xF, q >> 4], -1).reshape(q.shape[0], -1)

    xc, wc = codes(xq), codes(wq)
    for s in range(S):
        for o in range(out):
            terms = [exact_value(xc[s, n], xe[s, n // 32]) * exact_value(wc[o, n], we[o, n // 32])
                     for n in range(N)]
            ex = sum(terms, Fraction(0))
            ab = sum((abs(v) for v in terms), Fraction(0))
            assert abs(Fraction(y[s, o]) - ex) <= Fraction(N, 2 ** 52) * ab
            assert abs(Fraction(t[s, o]) - ab) <= Fraction(N, 2 ** 52) * ab
    # selecting rows/columns gives the same numbers
    ys, ts = orc.gemm(xq, xe, wq, we, rows=[S - 1, 0], cols=[out - 1, 1])
    assert np.array_equal(ys, y[[S - 1, 0]][:, [out - 1, 1]])


# ----------------------------------------------------------------------------------------
# P9  values after division by the scale, before rounding
# ----------------------------------------------------------------------------------------

def test_p9_scaled_values_and_codes_are_consistent(orc):
    L = wl.make_layer("tiny", with_weight=False)
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    q, e, v, yc = orc.quantize_act(L.x_bits, L.A, L.B, rmin, rmax, debug=True)
    S, N = L.x_bits.shape
    scale = np.ldexp(1.0, e.astype(np.int64) - 127).repeat(32, axis=1)
    assert np.array_equal(v.astype(np.float64) * scale, yc.astype(np.float64))
    # for blocks whose scale is not clamped, max |v| lies in [4, 8)
    vb = np.abs(v.reshape(S, N // 32, 32)).max(-1)
    assert np.all((vb >= 4) & (vb < 8))
    codes = np.stack([q & 0xF, q >> 4], -1).reshape(S, N)
    assert np.array_equal(codes, expected_e2m1_codes(v.view(np.uint32)))


def test_quantize_act_honours_row_stride(orc):
    L = wl.make_layer(wl.custom("ld", 7, 128, 8, seed=4), with_weight=False)
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    q, e = orc.quantize_act(L.x_bits, L.A, L.B, rmin, rmax)
    wide = np.zeros((7, 160), dtype=np.uint16)
    wide[:, :128] = L.x_bits
    wide[:, 128:] = 0x7F80     # +inf padding must never be read
    q2, e2 = orc.quantize_act(wide, L.A, L.B, rmin, rmax, ldx=160)
    assert np.array_equal(q, q2) and np.array_equal(e, e2)


# ----------------------------------------------------------------------------------------
# clip ratios: sigmoid of the logits
# ----------------------------------------------------------------------------------------

def test_clip_ratio_is_sigmoid_rounded_to_fp32(orc):
    getcontext().prec = 50
    rng = np.random.default_rng(1)
    alpha = np.concatenate([rng.normal(2.0, 0.5, 300), rng.normal(0, 8, 300),
                            [0.0, 30.0, -30.0, 17.0]]).astype(np.float32)
    r = orc.clip_ratio(alpha)
    for a, got in zip(alpha.tolist(), r.tolist()):
        exact = Decimal(1) / (Decimal(1) + (-Decimal(a)).exp())
        assert got == float(np.float32(float(exact))), a
    assert r[-4] == 0.5 and r[-3] == 1.0
