"""CPU pins of the oracle's KV-cache functions (W4A8KV8 / W4A8KV4): the slot-mapped cache
quantiser against the pinned row quantisers, the attention-score invariance
q P^-T (k P)^T = q k^T with grouped query heads, the recovery of attention outputs by P^-1,
and bf16 rounding against a rint-based formulation."""
import numpy as np
import pytest

import workloads as wl


@pytest.mark.parametrize("fmt", [4, 8])
def test_slot_mapped_cache_is_the_row_quantiser_written_at_the_slots(orc, fmt):
    L = wl.make_layer(wl.custom("kv-pin", 12, 256, 8, seed=21), with_weight=False)
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    if fmt == 4:
        q_ref, e_ref = orc.quantize_act(L.x_bits, L.A, L.B, rmin, rmax)
    else:
        q_ref, e_ref = orc.quantize_act_fp8(L.x_bits, L.A, L.B, rmin, rmax)
    slots = np.array([7, 0, 19, -1, 3, 11, -1, 2, 18, 5, 9, 1])
    cq = np.full((20, q_ref.shape[1]), 0xAB, dtype=np.uint8)
    ce = np.full((20, 8), 0xCD, dtype=np.uint8)
    orc.quantize_kv(L.x_bits, slots, fmt, L.A, L.B, rmin, rmax, cq, ce)
    for t, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(cq[s], q_ref[t]) and np.array_equal(ce[s], e_ref[t])
    untouched = sorted(set(range(20)) - set(int(s) for s in slots))
    assert np.all(cq[untouched] == 0xAB) and np.all(ce[untouched] == 0xCD)


def test_attention_scores_are_invariant_with_grouped_query_heads(orc):
    rng = np.random.default_rng(22)
    T, Hkv, group, D = 9, 2, 2, 128
    Hq, kd = Hkv * group, D // 32
    A = (np.eye(8) + 0.1 * rng.standard_normal((8, 8))).astype(np.float32)
    B = (np.eye(4) + 0.1 * rng.standard_normal((Hkv * kd, 4, 4))).astype(np.float32)
    kx = rng.standard_normal((T, Hkv * D)).astype(np.float32)
    qx = rng.standard_normal((T, Hq * D)).astype(np.float32)
    Ai, Bi = orc.weight_factors(A, B)                 # (A^-1)^T, (B_i^-1)^T
    # query head h uses the factors of kv head h // group
    Bq = np.concatenate([Bi[(h // group) * kd:(h // group + 1) * kd] for h in range(Hq)])
    kt = orc.transform_rows(kx, A, B).astype(np.float64)
    qt = orc.transform_rows(qx, Ai, Bq).astype(np.float64)
    for h in range(Hq):
        g = h // group
        qs, ks = slice(h * D, (h + 1) * D), slice(g * D, (g + 1) * D)
        s_ref = qx[:, qs].astype(np.float64) @ kx[:, ks].astype(np.float64).T
        scale = np.abs(qx[:, qs]).astype(np.float64) @ np.abs(kx[:, ks]).astype(np.float64).T
        assert np.all(np.abs(qt[:, qs] @ kt[:, ks].T - s_ref) <= 1e-5 * scale)
    # the factors of the wrong kv head break it
    wrong = orc.transform_rows(qx, Ai, np.concatenate([Bi[::-1]] * group))
    s0 = qx[:, :D].astype(np.float64) @ kx[:, :D].astype(np.float64).T
    assert np.max(np.abs(wrong[:, :D].astype(np.float64) @ kt[:, :D].T - s0)) > 1e-2


def test_value_rows_come_back_through_p_inverse(orc):
    rng = np.random.default_rng(23)
    A = (np.eye(8) + 0.1 * rng.standard_normal((8, 8))).astype(np.float32)
    B = (np.eye(4) + 0.1 * rng.standard_normal((8, 4, 4))).astype(np.float32)
    v = rng.standard_normal((11, 256)).astype(np.float32)
    Ai_t, Bi_t = orc.weight_factors(A, B)
    Ainv = np.ascontiguousarray(Ai_t.T)
    Binv = np.ascontiguousarray(np.transpose(Bi_t, (0, 2, 1)))
    back = orc.transform_rows(orc.transform_rows(v, A, B), Ainv, Binv)
    assert np.all(np.abs(back - v) <= 1e-5 * (np.abs(v).max(axis=1, keepdims=True) + 1))
    # bf16 input path equals the fp32 path on bf16-representable values
    vb = wl.f32_to_bf16_bits(v)
    assert np.array_equal(orc.transform_rows(vb, A, B, x_is_bf16_bits=True),
                          orc.transform_rows(wl.bf16_bits_to_f32(vb), A, B))


def test_bf16_rounding_is_nearest_ties_to_even(orc):
    rng = np.random.default_rng(24)
    bits = np.concatenate([
        rng.integers(0, 0x7F7F0000, size=200000, dtype=np.uint64),
        (rng.integers(0, 0x7F7F, size=20000, dtype=np.uint64) << 16) | 0x8000,   # exact ties
        np.arange(0, 0x30000, dtype=np.uint64),                                   # subnormals
    ]).astype(np.uint32)
    bits = np.concatenate([bits, bits | 0x80000000])
    v = bits.view(np.float32)
    got = orc.f32_to_bf16(v)
    # independent formulation: np.rint (ties to even) on the significand scaled to bf16's 8
    # bits, and on the fixed 2^-133 grid below the smallest normal
    x = v.astype(np.float64)
    m, e = np.frexp(x)                                # x = m 2^e, 0.5 <= |m| < 1
    nearest = np.where(np.abs(x) < 2.0 ** -126, np.rint(x * 2.0 ** 133) * 2.0 ** -133,
                       np.ldexp(np.rint(m * 256.0) / 256.0, e))
    want = (nearest.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    # keep the sign of values that round to zero
    want = np.where(nearest == 0, (bits >> 16).astype(np.uint16) & 0x8000, want)
    assert np.array_equal(got, want)
    # and it is exact on values that bf16 holds
    held = bits & 0xFFFF0000
    assert np.array_equal(orc.f32_to_bf16(held.view(np.float32)), (held >> 16).astype(np.uint16))
