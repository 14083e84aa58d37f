"""GPU parity of the KV-cache calls (W4A8KV8 / W4A8KV4 settings) against the oracle on the
same seeded inputs: the slot-mapped cache write (every cache row bit for bit, written rows and
untouched ones), the transform of rows without quantisation (fp32 bit for bit, bf16 as the
oracle's rounding of it), and the dequantisation of cache rows (exact)."""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import (ORACLE_THREADS, assert_codes_equal, assert_fp8_codes_equal,
                            bf16_to_device, f32_to_device, to_host, u8_to_device)

pytestmark = pytest.mark.gpu

SENT_Q, SENT_E = 0xAB, 0xCD


@pytest.fixture(scope="module")
def bq():
    import torch
    import w4a4_batq_quantize_amd as bq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bq.lib()
    return bq


def code_cols(fmt, N):
    return N // 2 if fmt == 4 else N


def run_kv(bq, L, slots, fmt, num_slots, ldx=None):
    import torch
    T, N = L.x_bits.shape
    if ldx is not None and ldx != N:
        wide = np.zeros((T, ldx), dtype=np.uint16)
        wide[:, :N] = L.x_bits
        wide[:, N:] = 0x7FC0                       # NaN padding: must never be read
        x = bf16_to_device(wide)[:, :N]
    else:
        x = bf16_to_device(L.x_bits)
    cq = torch.full((num_slots, code_cols(fmt, N)), SENT_Q, dtype=torch.uint8, device="cuda")
    ce = torch.full((num_slots, N // 32), SENT_E, dtype=torch.uint8, device="cuda")
    bq.quantize_kv(x, torch.from_numpy(slots).cuda(), fmt, f32_to_device(L.A),
                   f32_to_device(L.B), f32_to_device(bq.clip_ratios(L.alpha_min)),
                   f32_to_device(bq.clip_ratios(L.alpha_max)), cq, ce)
    torch.cuda.synchronize()
    return to_host(cq), to_host(ce)


def oracle_kv(orc, L, slots, fmt, num_slots):
    """The oracle's cache (same sentinel start) and the exact-zero mask of the clipped
    values at the cache positions.  Slots at or beyond num_slots are skips, like negative
    ones."""
    T, N = L.x_bits.shape
    s = np.where(slots < num_slots, slots, -1)
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    cq = np.full((num_slots, code_cols(fmt, N)), SENT_Q, dtype=np.uint8)
    ce = np.full((num_slots, N // 32), SENT_E, dtype=np.uint8)
    orc.quantize_kv(L.x_bits, s, fmt, L.A, L.B, rmin, rmax, cq, ce)
    _, _, _, yc = orc.quantize_act(L.x_bits, L.A, L.B, rmin, rmax, debug=True,
                                   nthreads=ORACLE_THREADS)
    zero = np.zeros((num_slots, N), dtype=bool)
    keep = s >= 0
    zero[s[keep]] = yc[keep] == 0
    return cq, ce, zero


def assert_cache_equal(fmt, cq, ce, cq_ref, ce_ref, zero, what):
    if fmt == 4:
        assert_codes_equal(cq, ce, cq_ref, ce_ref, zero, what=what)
    else:
        assert_fp8_codes_equal(cq, ce, cq_ref, ce_ref, zero, what=what)


@pytest.mark.parametrize("fmt", [4, 8])
@pytest.mark.parametrize("name,num_slots,skip", [("kv_prefill", 2048 + 301, 0.0),
                                                 ("kv_decode", 4096, 0.1)])
def test_kv_cache_parity(bq, orc, fmt, name, num_slots, skip):
    L = wl.make_layer(name, with_weight=False)
    T = L.cfg.S
    slots = wl.kv_slots(T, num_slots, seed=(61, fmt, T), skip=skip)
    print(f"[kv parity] {name} fmt={fmt} T={T} N={L.cfg.N} slots={num_slots}", flush=True)
    cq, ce = run_kv(bq, L, slots, fmt, num_slots)
    cq_ref, ce_ref, zero = oracle_kv(orc, L, slots, fmt, num_slots)
    assert_cache_equal(fmt, cq, ce, cq_ref, ce_ref, zero, what=f"{name} fmt={fmt}")
    untouched = np.setdiff1d(np.arange(num_slots), slots)
    assert untouched.size > 0
    assert np.all(cq[untouched] == SENT_Q) and np.all(ce[untouched] == SENT_E)


@pytest.mark.parametrize("fmt", [4, 8])
@pytest.mark.parametrize("T,N,ldx,num_slots,seed", [
    (1, 32, 32, 3, 1),          # one block, one token
    (5, 96, 104, 9, 2),         # k = 3, strided rows
    (37, 4192, 4256, 50, 3),    # k = 131: three block columns in the grid, ragged
    (130, 256, 256, 200, 4),    # rows over several workgroups, ragged tail
])
def test_kv_cache_ragged_strided_and_out_of_range_slots(bq, orc, fmt, T, N, ldx, num_slots,
                                                        seed):
    L = wl.make_layer(wl.custom("kv-ragged", T, N, 0, seed=seed), with_weight=False)
    slots = wl.kv_slots(T, num_slots, seed=(62, seed), skip=0.2)
    # tokens whose slot is beyond the cache are skipped, like negative slots
    rng = np.random.default_rng(seed)
    far = rng.random(T) < 0.15
    slots[far] = num_slots + rng.integers(0, 1 << 40, size=int(far.sum()))
    cq, ce = run_kv(bq, L, slots, fmt, num_slots, ldx=ldx)
    cq_ref, ce_ref, zero = oracle_kv(orc, L, slots, fmt, num_slots)
    assert_cache_equal(fmt, cq, ce, cq_ref, ce_ref, zero, what=f"T={T} N={N} fmt={fmt}")


@pytest.mark.parametrize("fmt", [4, 8])
def test_kv_cache_with_identity_slots_is_the_activation_quantiser(bq, fmt):
    """slots = 0..T-1 writes exactly what batq_quantize_act / batq_quantize_act_mxfp8 give."""
    import torch
    L = wl.make_layer("kv_decode", with_weight=False)
    T, N = L.x_bits.shape
    cq, ce = run_kv(bq, L, np.arange(T, dtype=np.int64), fmt, T)
    args = (bf16_to_device(L.x_bits), f32_to_device(L.A), f32_to_device(L.B),
            f32_to_device(bq.clip_ratios(L.alpha_min)), f32_to_device(bq.clip_ratios(L.alpha_max)))
    q, e = (bq.quantize_act if fmt == 4 else bq.quantize_act_mxfp8)(*args)
    torch.cuda.synchronize()
    assert np.array_equal(cq, to_host(q)) and np.array_equal(ce, to_host(e))


def test_kv_cache_all_tokens_skipped_and_empty(bq):
    import torch
    L = wl.make_layer(wl.custom("kv-skip", 8, 256, 0, seed=5), with_weight=False)
    cq, ce = run_kv(bq, L, np.full(8, -1, dtype=np.int64), 4, 6)
    assert np.all(cq == SENT_Q) and np.all(ce == SENT_E)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    c = torch.full((4, 128), SENT_Q, dtype=torch.uint8, device="cuda")
    e = torch.full((4, 8), SENT_E, dtype=torch.uint8, device="cuda")
    z = torch.zeros(0, dtype=torch.int64, device="cuda")
    f = f32_to_device(np.zeros(8 * 16, np.float32))
    bq.quantize_kv(x, z, 4, f32_to_device(L.A), f32_to_device(L.B), f[:8], f[:8], c, e)
    torch.cuda.synchronize()
    assert torch.all(c == SENT_Q) and torch.all(e == SENT_E)


# ---------------------------------------------------------------------------------------
# transform of rows (queries with P^-T per kv head, attention outputs with P^-1)
# ---------------------------------------------------------------------------------------

def run_transform(bq, x, A, B, x_bf16, y_bf16, ldx=None):
    """x: fp32 values (x_bf16: bf16 bit patterns) [rows, N]."""
    import torch
    rows, N = x.shape
    if ldx is not None and ldx != N:
        wide = np.zeros((rows, ldx), dtype=x.dtype)
        wide[:, :N] = x
        wide[:, N:] = 0x7FC0 if x_bf16 else np.nan
        x = wide
    xd = bf16_to_device(x) if x_bf16 else f32_to_device(x)
    xd = xd[:, :N]
    y = bq.transform_rows(xd, f32_to_device(A), f32_to_device(B),
                          out_dtype=torch.bfloat16 if y_bf16 else torch.float32)
    torch.cuda.synchronize()
    if y_bf16:
        return y.view(torch.int16).cpu().numpy().view(np.uint16)
    return y.cpu().numpy()


def check_transform(bq, orc, x, A, B, ldx=None, what=""):
    """All four input/output type pairs against the oracle: fp32 out bit for bit, bf16 out
    equal to the oracle's round-to-nearest-even of the fp32 result."""
    xb = wl.f32_to_bf16_bits(x)
    for x_bf16 in (False, True):
        ref = orc.transform_rows(xb if x_bf16 else x, A, B, x_is_bf16_bits=x_bf16)
        for y_bf16 in (False, True):
            got = run_transform(bq, xb if x_bf16 else x, A, B, x_bf16, y_bf16, ldx=ldx)
            want = orc.f32_to_bf16(ref) if y_bf16 else ref
            assert np.array_equal(got.view(np.uint16 if y_bf16 else np.uint32),
                                  want.view(np.uint16 if y_bf16 else np.uint32)), \
                f"{what} x_bf16={x_bf16} y_bf16={y_bf16}"


def test_query_transform_with_grouped_heads(bq, orc):
    """q~ = q P^-T with the factors of the kv head each of the 32 query heads attends to
    (GQA group 4), at the decode step's size."""
    Lk = wl.make_layer("kv_decode", with_weight=False)
    T, Hkv, D, group = 64, 8, 128, 4
    kd = D // 32
    Ai, Bi = orc.weight_factors(Lk.A, Lk.B)
    Bq = np.ascontiguousarray(np.concatenate(
        [Bi[(h // group) * kd:(h // group + 1) * kd] for h in range(Hkv * group)]))
    rng = np.random.default_rng(63)
    q = rng.standard_normal((T, Hkv * group * D)).astype(np.float32)
    q[:, rng.choice(q.shape[1], 6, replace=False)] *= 30
    check_transform(bq, orc, q, Ai, Bq, what="query")


def test_output_transform_with_inverse_factors(bq, orc):
    """o = o~ P^-1 (the transposed factors of P^-T) on attention outputs, strided rows."""
    L = wl.make_layer(wl.custom("kv-out", 70, 1024, 0, seed=64), with_weight=False)
    Ai_t, Bi_t = orc.weight_factors(L.A, L.B)
    Ainv = np.ascontiguousarray(Ai_t.T)
    Binv = np.ascontiguousarray(np.transpose(Bi_t, (0, 2, 1)))
    o = wl.bf16_bits_to_f32(L.x_bits)
    check_transform(bq, orc, o, Ainv, Binv, ldx=1032, what="output")


@pytest.mark.parametrize("rows,N,ldx", [(1, 32, 40), (3, 96, 104), (37, 4192, 4256),
                                        (130, 256, 256)])
def test_transform_rows_ragged(bq, orc, rows, N, ldx):
    L = wl.make_layer(wl.custom("tr-ragged", rows, N, 0, seed=rows), with_weight=False)
    x = wl.bf16_bits_to_f32(L.x_bits) * np.float32(1.0 + 1.0 / 3.0)   # not bf16-exact
    check_transform(bq, orc, x.astype(np.float32), L.A, L.B, ldx=ldx, what=f"{rows}x{N}")


# ---------------------------------------------------------------------------------------
# dequantisation of cache rows
# ---------------------------------------------------------------------------------------

def run_dequant(bq, cq, ce, fmt, index, y_bf16):
    import torch
    y = bq.dequantize_rows(u8_to_device(cq), u8_to_device(ce), fmt,
                           index=torch.from_numpy(index).cuda() if index is not None else None,
                           out_dtype=torch.bfloat16 if y_bf16 else torch.float32)
    torch.cuda.synchronize()
    if y_bf16:
        return y.view(torch.int16).cpu().numpy().view(np.uint16)
    return y.cpu().numpy()


@pytest.mark.parametrize("fmt", [4, 8])
def test_dequantize_cache_rows(bq, orc, fmt):
    """A cache written by the oracle, read back through an index with out-of-range entries
    (zero rows), and in full; exact against the oracle's fp64 decoding."""
    L = wl.make_layer("kv_decode", with_weight=False)
    T, N = L.x_bits.shape
    num_slots = 300
    slots = wl.kv_slots(T, num_slots, seed=(65, fmt))
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    if fmt == 4:
        cq, ce = wl.random_mxfp4(num_slots, N, seed=(66,), scale_lo=100, scale_hi=150)
    else:
        cq, ce = wl.random_mxfp8(num_slots, N, seed=(66,), scale_lo=100, scale_hi=150)
    ce[0, :3] = (0, 1, 254)                                   # extreme finite scales
    orc.quantize_kv(L.x_bits, slots, fmt, L.A, L.B, rmin, rmax, cq, ce)
    dq = orc.dequant if fmt == 4 else orc.dequant_fp8
    full = dq(cq, ce)
    index = np.concatenate([slots[::-1], [-1, num_slots, 1 << 40, 0]]).astype(np.int64)
    want = np.zeros((index.size, N))
    ok = (index >= 0) & (index < num_slots)
    want[ok] = full[index[ok]]
    for y_bf16 in (False, True):
        for idx, ref in ((index, want), (None, full)):
            got = run_dequant(bq, cq, ce, fmt, idx, y_bf16)
            finite = np.abs(ref) < 2.0 ** 128          # codes hold <= 4 significant bits
            if y_bf16:
                exp = orc.f32_to_bf16(np.where(finite, ref, 0).astype(np.float32))
                assert np.array_equal(got[finite], exp[finite])
                assert np.all((got[~finite] & 0x7FFF) == 0x7F80)      # overflow to inf
            else:
                assert np.array_equal(got[finite], ref[finite].astype(np.float32))
                assert np.all(np.isinf(got[~finite]))
    # NaN encodings: E8M0 0xFF and the E4M3 NaN byte
    ce2 = ce.copy()
    ce2[1, 2] = 0xFF
    got = run_dequant(bq, cq, ce2, fmt, None, False)
    assert np.all(np.isnan(got[1, 64:96]))
    if fmt == 8:
        cq2 = cq.copy()
        cq2[2, 5], cq2[2, 6] = 0x7F, 0xFF
        got = run_dequant(bq, cq2, ce, fmt, None, False)
        assert np.isnan(got[2, 5]) and np.isnan(got[2, 6])
        assert np.array_equal(np.delete(got[2], [5, 6]),
                              np.delete(full[2], [5, 6]).astype(np.float32))
