"""Pins of the oracle's W4A8 pieces (MXFP8 activations, E4M3 elements) on the CPU.

The W4A8 setting runs the same transform and clip as W4A4 and encodes the activations as
MXFP8: E4M3 elements (OCP FP8 without infinities, largest value 448) sharing one E8M0 scale
per 32 (gist.science summary section 4 and the daily-arxiv results bullet name W4A8KV16).
Each check below is written in a formulation of its own: the E4M3 value table from its
bit-field definition with exact rationals, the rounding as integer arithmetic on the fp32
bit pattern (exhaustive over whole binades, every midpoint in every binade and the
saturation range), the scale rule from the exponent field, plain MXFP8 of untransformed
data, and the W4A8 product against exact rationals.
"""
from concurrent.futures import ThreadPoolExecutor
from fractions import Fraction

import numpy as np
import pytest

import workloads as wl


def e4m3_table():
    """The 127 finite E4M3 magnitudes from the bit fields: code 8E + m."""
    vals = []
    for c in range(127):
        E, m = c >> 3, c & 7
        vals.append(Fraction(m, 8) * Fraction(1, 2 ** 6) if E == 0
                    else (1 + Fraction(m, 8)) * Fraction(2) ** (E - 7))
    return vals


def e4m3_codes_from_bits(u: np.ndarray) -> np.ndarray:
    """E4M3 round-to-nearest-even with saturation at 448, computed with integer arithmetic
    on fp32 bit patterns u (finite values only)."""
    u = u.astype(np.uint64)
    sign = ((u >> 31) & 1).astype(np.uint8) << 7
    ef = ((u >> 23) & 0xFF).astype(np.int64)
    mant = (u & 0x7FFFFF).astype(np.int64)
    m24 = np.where(ef > 0, mant | (1 << 23), mant)        # significand, 24 bits
    e2 = np.where(ef > 0, ef - 127, -126)                  # value = m24 * 2^(e2 - 23)
    code = np.zeros(u.shape, dtype=np.int64)
    # normal E4M3 range (value >= 2^-6): keep 4 significant bits
    nrm = e2 >= -6
    sh = 20
    q = m24 >> sh
    rem = m24 & ((1 << sh) - 1)
    up = (rem > (1 << (sh - 1))) | ((rem == (1 << (sh - 1))) & ((q & 1) == 1))
    q = q + up
    e_n = e2 + (q >> 4)                                    # carry into the exponent
    q = np.where(q >> 4 == 1, 8, q)                        # 16 -> 8 (1.000 of next binade)
    cn = ((e_n + 7) << 3) | (q - 8)
    code = np.where(nrm, cn, code)
    # below 2^-6: multiples of 2^-9, i.e. value * 2^9 = m24 * 2^(e2 - 14) rounded to an integer
    sub = ~nrm
    shs = np.clip(14 - e2, 0, 62)
    qs = np.where(shs >= 40, 0, m24 >> np.minimum(shs, 40))
    rems = np.where(shs >= 40, m24, m24 & ((np.int64(1) << np.minimum(shs, 40)) - 1))
    halfs = np.where(shs >= 40, np.int64(1) << 39, np.int64(1) << np.maximum(np.minimum(shs, 40) - 1, 0))
    ups = np.where(shs >= 40, False, (rems > halfs) | ((rems == halfs) & ((qs & 1) == 1)))
    code = np.where(sub, qs + ups, code)                   # 8 -> 0x08, the smallest normal
    code = np.minimum(code, 0x7E)                          # saturate at 448
    return (code.astype(np.uint8) | sign)


def f32_from_bits(u):
    return np.asarray(u, dtype=np.uint32).view(np.float32)


# ----------------------------------------------------------------------------------------
# E4M3 element format
# ----------------------------------------------------------------------------------------

def test_e4m3_value_table_from_bit_fields(orc):
    table = e4m3_table()
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]                  # NaN patterns excluded
    vals = orc.e4m3_value(codes)
    for c, v in zip(codes, vals):
        ref = table[c & 0x7F]
        assert Fraction(v) == (-ref if c & 0x80 else ref), hex(c)
    assert table[126] == 448 and table[1] == Fraction(1, 512) and table[8] == Fraction(1, 64)
    assert all(table[i] < table[i + 1] for i in range(126))


def test_e4m3_rounding_exhaustive_over_binades(orc):
    """Every fp32 pattern of [1, 2), [256, 512), of the whole E4M3 subnormal range and of the
    fp32 subnormals; the rounding is scale-free from binade to binade in the normal range,
    the midpoints of every binade are checked in the next test."""
    ranges = [(f32bits_of(1.0), f32bits_of(2.0)), (f32bits_of(256.0), f32bits_of(512.0)),
              (f32bits_of(2.0 ** -12), f32bits_of(2.0 ** -5)), (0, 1 << 23)]
    chunk = 1 << 21

    def check(lo):
        def run(start):
            n = min(chunk, hi - start)
            u = np.arange(start, start + n, dtype=np.uint64).astype(np.uint32)
            for sgn in (0, 0x80000000):
                uu = u | np.uint32(sgn)
                got = orc.e4m3_round(f32_from_bits(uu))
                exp = e4m3_codes_from_bits(uu)
                bad = np.nonzero(got != exp)[0]
                assert bad.size == 0, (hex(int(uu[bad[0]])), hex(int(got[bad[0]])),
                                       hex(int(exp[bad[0]])))
        return run

    for lo, hi in ranges:
        with ThreadPoolExecutor(8) as ex:
            list(ex.map(check(lo), range(lo, hi, chunk)))


def f32bits_of(x):
    return int(np.array(x, dtype=np.float32).view(np.uint32))


def test_e4m3_midpoints_ties_and_saturation(orc):
    table = [float(v) for v in e4m3_table()]
    pts, want = [], []
    for i in range(126):
        a, b = table[i], table[i + 1]
        mid = (a + b) / 2                                  # exact in fp32 here
        even = i if i % 2 == 0 else i + 1
        pts += [mid, np.nextafter(np.float32(mid), np.float32(0)),
                np.nextafter(np.float32(mid), np.float32(1e9)), a, b]
        want += [even, i, i + 1, i, i + 1]
    for v in [448.0, 448.5, 463.9, 464.0, 480.0, 500.0, 511.9, 1e4, 3e38]:
        pts.append(v)
        want.append(126)
    v = np.array(pts, dtype=np.float32)
    assert np.array_equal(orc.e4m3_round(v), np.array(want, dtype=np.uint8))
    assert np.array_equal(orc.e4m3_round(-v), np.array(want, dtype=np.uint8) | 0x80)
    assert np.array_equal(e4m3_codes_from_bits(v.view(np.uint32)), np.array(want, dtype=np.uint8))
    assert orc.e4m3_round(np.array([-0.0], dtype=np.float32))[0] == 0x80


def test_e4m3_random_patterns_all_exponents(orc):
    rng = np.random.default_rng(41)
    u = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    f = f32_from_bits(u)
    u = u[np.isfinite(f)]
    assert np.array_equal(orc.e4m3_round(f32_from_bits(u)), e4m3_codes_from_bits(u))


# ----------------------------------------------------------------------------------------
# MXFP8 scale rule and the plain reduction
# ----------------------------------------------------------------------------------------

def test_mxfp8_scale_is_exponent_minus_8(orc):
    rng = np.random.default_rng(42)
    amax = np.abs(rng.standard_normal(100_000) * 10.0 ** rng.uniform(-40, 38, 100_000))
    amax = np.concatenate([amax.astype(np.float32),
                           np.float32([0.0, 1e-45, 2.0 ** -126, 1.0, 255.99, 256.0, 3e38])])
    e = orc.e8m0_scale_fp8(amax).astype(np.int64)
    fe = ((amax.view(np.uint32) >> 23) & 0xFF).astype(np.int64)
    nz = amax > 0
    # normal amax: the E8M0 byte is the fp32 exponent field minus 8 (clamped at 0)
    normal = fe > 0
    assert np.array_equal(e[normal], np.maximum(fe[normal] - 8, 0))
    assert np.all(e[~nz] == 0)
    # and amax / scale lies in [256, 512) wherever the scale is not clamped
    ok = normal & (fe - 8 > 0)
    ratio = amax[ok].astype(np.float64) / np.ldexp(1.0, e[ok] - 127)
    assert np.all((ratio >= 256) & (ratio < 512))


def test_mxfp8_scale_is_mxfp4_scale_minus_6(orc):
    """Same amax, E4M3's largest exponent 8 against E2M1's 2."""
    rng = np.random.default_rng(43)
    amax = (np.abs(rng.standard_normal(10000)) * 1e3).astype(np.float32)
    assert np.array_equal(orc.e8m0_scale_fp8(amax).astype(int),
                          orc.e8m0_scale(amax).astype(int) - 6)


def plain_mxfp8(x):
    """MXFP8 of untransformed data in a formulation of its own (exponent field, bit-level
    rounding)."""
    rows, N = x.shape
    xb = x.reshape(rows, N // 32, 32).astype(np.float32)
    amax = np.abs(xb).max(-1)
    fe = ((amax.view(np.uint32) >> 23) & 0xFF).astype(np.int64)
    e = np.where(amax > 0, np.maximum(fe - 8, 0), 0).astype(np.uint8)
    v = (xb.astype(np.float64) / np.ldexp(1.0, e.astype(np.int64) - 127)[..., None])
    v32 = v.astype(np.float32)
    assert np.array_equal(v32.astype(np.float64), v)      # the division is exact here
    codes = e4m3_codes_from_bits(v32.view(np.uint32)).reshape(rows, N)
    return codes, e


def test_identity_transform_and_unit_ratios_reduce_to_plain_mxfp8(orc):
    cfg = wl.custom("fp8", 40, 512, 32, seed=321)
    L = wl.make_layer(cfg, with_weight=False)
    k = cfg.k
    r = np.ones(k, dtype=np.float32)
    A = np.eye(8, dtype=np.float32)
    B = np.tile(np.eye(4, dtype=np.float32), (k, 1, 1))
    q, e = orc.quantize_act_fp8(L.x_bits, A, B, r, r)
    x = wl.bf16_bits_to_f32(L.x_bits)
    q_ref, e_ref = plain_mxfp8(x)
    assert np.array_equal(e, e_ref)
    # an exactly-zero input may carry either sign
    diff = q != q_ref
    assert np.all(x[diff] == 0) and np.all((q[diff] & 0x7F) == 0)


def test_fp8_path_clips_like_the_fp4_path(orc):
    """The MXFP8 codes dequantise to the clipped transform output within half an E4M3 step,
    and the two paths' scales differ by exactly 6 (same clip, same amax)."""
    L = wl.make_layer("tiny", with_weight=False)
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    q4, e4, v4, yc = orc.quantize_act(L.x_bits, L.A, L.B, rmin, rmax, debug=True)
    q8, e8 = orc.quantize_act_fp8(L.x_bits, L.A, L.B, rmin, rmax)
    assert np.array_equal(e8.astype(int), e4.astype(int) - 6)
    d = orc.dequant_fp8(q8, e8)
    y = yc.astype(np.float64)
    scale = np.ldexp(1.0, e8.astype(np.int64) - 127).repeat(32, axis=1)
    # E4M3 step at |y|: 2^(floor(log2 |y/scale|) - 3) (>= 2^-9) times the scale
    v = np.abs(y) / scale
    sat = v > 448                                          # saturates to the largest value
    assert np.array_equal(d[sat], np.sign(y[sat]) * 448 * scale[sat])
    step = np.ldexp(1.0, np.maximum(np.floor(np.log2(np.maximum(v, 1e-300))), -6).astype(int) - 3)
    assert np.all(np.abs(d - y)[~sat] <= (0.5 * step * scale)[~sat])
    assert np.all(v < 512) and np.all(v.reshape(v.shape[0], -1, 32).max(-1) >= 256)


# ----------------------------------------------------------------------------------------
# W4A8 product against exact rationals
# ----------------------------------------------------------------------------------------

TWICE_E2M1 = [0, 1, 2, 3, 4, 6, 8, 12]


@pytest.mark.parametrize("S,N,out", [(3, 32, 5), (4, 64, 3)])
def test_w4a8_gemm_reference_vs_exact_rationals(orc, S, N, out):
    rng = np.random.default_rng(S * 10 + N + out)
    table = e4m3_table()
    xq8 = rng.integers(0, 256, size=(S, N), dtype=np.uint8)
    xq8[(xq8 & 0x7F) == 0x7F] = 0x7E                        # no NaN codes
    wq = rng.integers(0, 256, size=(out, N // 2), dtype=np.uint8)
    xe = rng.integers(110, 140, size=(S, N // 32), dtype=np.uint8)
    we = rng.integers(110, 140, size=(out, N // 32), dtype=np.uint8)
    y, t = orc.gemm_w4a8(xq8, xe, wq, we)
    wc = np.stack([wq & 0xF, wq >> 4], -1).reshape(out, N)
    for s in range(S):
        for o in range(out):
            terms = []
            for n in range(N):
                xv = table[xq8[s, n] & 0x7F] * Fraction(2) ** (int(xe[s, n // 32]) - 127)
                xv = -xv if xq8[s, n] & 0x80 else xv
                wv = Fraction(TWICE_E2M1[wc[o, n] & 7], 2) * Fraction(2) ** (int(we[o, n // 32]) - 127)
                wv = -wv if wc[o, n] & 8 else wv
                terms.append(xv * wv)
            ex = sum(terms, Fraction(0))
            ab = sum((abs(v) for v in terms), Fraction(0))
            assert abs(Fraction(y[s, o]) - ex) <= Fraction(N, 2 ** 52) * ab
            assert abs(Fraction(t[s, o]) - ab) <= Fraction(N, 2 ** 52) * ab
