"""GPU parity on exact rounding ties of both element encodings.

The scaled value of an element is y / 2^(e-127); it is rounded to the nearest E2M1 (or E4M3)
value, ties to the even code, with saturation (thelatestinai listing, Fig. 2 caption: the
division by the scale comes before the rounding).  Random layer data almost never lands on
a tie, so these blocks are built to: with identity factors and unit clip ratios the
transformed value is the input itself, one element per block pins the scale byte (its
scaled magnitude is the format's largest value), and the other elements sit exactly on
every midpoint between neighbouring codes, one bf16 step below and above it, and in the
saturation range, with both signs.  Scale bytes 0, 1, 127 and a high one (250 for MXFP4;
246 for MXFP8, whose largest block value 448 * 2^(e-127) must stay below the fp32 range)
cover the subnormal, the smallest-normal, the ordinary and the top of the range.

Checked bit for bit against the oracle: the MXFP4 and MXFP8 quantisers (both scale
layouts), and the encoders inside the one-kernel layers, whose codes are read back through
the product with an identity weight matrix of a chosen power of two (each output then has
one nonzero term, so y is exactly the code's value, and the sums are exact).
"""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import (ORACLE_THREADS, assert_codes_equal, assert_fp8_codes_equal,
                            bf16_to_device, f32_to_device, from_tiled_scales, to_host)

pytestmark = pytest.mark.gpu

SCALE_BYTES_FP4 = [0, 1, 127, 250]
SCALE_BYTES_FP8 = [0, 1, 127, 246]
K = 8                       # blocks per row


@pytest.fixture(scope="module")
def bq():
    import torch
    import w4a4_batq_quantize_amd as bq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bq.lib()
    return bq


def bf16_exact(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float64 values; every value must be exactly representable."""
    bits = wl.f32_to_bf16_bits(v.astype(np.float32))
    back = wl.bf16_bits_to_f32(bits).astype(np.float64)
    assert np.array_equal(back, v), "tie value not exact in bf16"
    return bits


def e2m1_grid() -> np.ndarray:
    return np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e4m3_grid() -> np.ndarray:
    """Non-negative E4M3 values from the bit fields (bias 7, no infinities, 448 the top)."""
    vals = [m / 8 * 2.0 ** -6 for m in range(8)]
    vals += [(1 + m / 8) * 2.0 ** (E - 7) for E in range(1, 16) for m in range(8)
             if not (E == 15 and m == 7)]
    return np.array(vals)


def tie_values(grid: np.ndarray, sat: list) -> np.ndarray:
    """Scaled values (in units of the block scale): every midpoint of the grid, the
    saturation range and the grid points themselves."""
    mids = (grid[:-1] + grid[1:]) / 2
    return np.concatenate([mids, grid[1:], np.array(sat)])


def neighbours(bits: np.ndarray) -> np.ndarray:
    """bf16 patterns one step below and above each (non-negative, nonzero) pattern."""
    b = bits.astype(np.int64)
    return np.concatenate([b - 1, b + 1]).astype(np.uint16)


def tie_rows(e: int, fp8: bool) -> np.ndarray:
    """bf16 rows of K blocks at scale byte e: element 0 of every block pins the scale (the
    largest code value times 2^(e-127)), the rest are the tie values, their bf16 neighbours
    and their negatives, padded with zeros."""
    grid = e4m3_grid() if fp8 else e2m1_grid()
    top = 448.0 if fp8 else 6.0
    sat = [464.0, 480.0, 496.0, 510.0] if fp8 else [6.5, 7.0, 7.5, 7.875]
    scale = 2.0 ** (e - 127)
    vals = tie_values(grid, sat) * scale
    # keep only the values bf16 holds exactly (the smallest midpoints at scale bytes 0 and 1
    # fall below bf16's subnormal range)
    f32 = vals.astype(np.float32).astype(np.float64)
    keep = (f32 == vals) & (wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(f32.astype(np.float32)))
                            .astype(np.float64) == vals)
    pos = bf16_exact(vals[keep])
    pos = np.concatenate([pos, neighbours(pos[pos > 0])])
    # the pin's binade ends at 2^(floor(log2 top) + 1): larger magnitudes would raise the
    # scale byte
    limit = 2.0 ** (np.floor(np.log2(top)) + 1) * scale
    pos = pos[wl.bf16_bits_to_f32(pos).astype(np.float64) < limit]
    allv = np.concatenate([pos, pos | np.uint16(0x8000)])
    pin = bf16_exact(np.array([top * scale]))[0]
    per_block = 31
    nblk = -(-allv.size // per_block)
    rows = -(-nblk // K)
    x = np.zeros((rows, K * 32), dtype=np.uint16)
    blocks = x.reshape(rows * K, 32)
    blocks[:, 0] = pin
    flat = np.zeros(rows * K * per_block, dtype=np.uint16)
    flat[:allv.size] = allv
    blocks[:, 1:] = flat.reshape(rows * K, per_block)
    return x


def identity_layer(x_bits: np.ndarray):
    S, N = x_bits.shape
    k = N // 32
    A = np.eye(8, dtype=np.float32)
    B = np.tile(np.eye(4, dtype=np.float32), (k, 1, 1))
    r = np.ones(k, dtype=np.float32)
    return A, B, r


def test_tie_rows_are_ties():
    """The generated blocks hold what the test claims: scale bytes as chosen, and exact
    midpoints of both formats among the scaled values (checked on the host)."""
    for fp8, scale_bytes in ((False, SCALE_BYTES_FP4), (True, SCALE_BYTES_FP8)):
        for e in scale_bytes:
            x = tie_rows(e, fp8)
            v = wl.bf16_bits_to_f32(x).astype(np.float64) / 2.0 ** (e - 127)
            grid = e4m3_grid() if fp8 else e2m1_grid()
            mids = (grid[:-1] + grid[1:]) / 2
            hit = np.unique(v[np.isin(np.abs(v), mids)])
            if e >= 127:
                assert hit.size == 2 * mids.size, (fp8, e, hit.size)   # every midpoint, +-
            else:
                assert hit.size >= 14, (fp8, e, hit.size)
            top = 448.0 if fp8 else 6.0
            assert np.all(np.abs(v).reshape(-1, 32).max(1) >= top)
            assert np.all(np.abs(v).reshape(-1, 32).max(1) < 2 * 2.0 ** np.floor(np.log2(top)))
            # the saturation range is present
            assert np.any(np.abs(v) > top)


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("e", SCALE_BYTES_FP4)
def test_mxfp4_ties(bq, orc, e, tiled):
    import torch
    x = tie_rows(e, fp8=False)
    S, N = x.shape
    A, B, r = identity_layer(x)
    layout = bq.SCALES_MFMA_TILED if tiled else bq.SCALES_ROW_MAJOR
    print(f"[ties mxfp4] e={e} tiled={tiled} S={S}", flush=True)
    q, sc = bq.quantize_act(bf16_to_device(x), f32_to_device(A), f32_to_device(B),
                            f32_to_device(r), f32_to_device(r), layout=layout)
    torch.cuda.synchronize()
    q, sc = to_host(q), to_host(sc)
    if tiled:
        sc = from_tiled_scales(sc, S, N // 32)
    q_ref, e_ref, v, yc = orc.quantize_act(x, A, B, r, r, debug=True)
    assert np.all(e_ref == e)
    assert_codes_equal(q, sc, q_ref, e_ref, yc == 0, what=f"mxfp4 ties e={e}")


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("e", SCALE_BYTES_FP8)
def test_mxfp8_ties(bq, orc, e, tiled):
    import torch
    x = tie_rows(e, fp8=True)
    S, N = x.shape
    A, B, r = identity_layer(x)
    layout = bq.SCALES_MFMA_TILED if tiled else bq.SCALES_ROW_MAJOR
    print(f"[ties mxfp8] e={e} tiled={tiled} S={S}", flush=True)
    q, sc = bq.quantize_act_mxfp8(bf16_to_device(x), f32_to_device(A), f32_to_device(B),
                                  f32_to_device(r), f32_to_device(r), layout=layout)
    torch.cuda.synchronize()
    q, sc = to_host(q), to_host(sc)
    if tiled:
        sc = from_tiled_scales(sc, S, N // 32)
    q_ref, e_ref = orc.quantize_act_fp8(x, A, B, r, r)
    assert np.all(e_ref == e)
    zero = wl.bf16_bits_to_f32(x) == 0
    assert_fp8_codes_equal(q, sc, q_ref, e_ref, zero, what=f"mxfp8 ties e={e}")


def identity_weights(bq, N, e, layout):
    """W = 2^(127-e) I [N, N] prepared with identity factors: every weight row has one
    nonzero, whose code value times its scale is 2^(127-e), so y[s][o] is the code value of
    token element (s, o) exactly."""
    import torch
    W = np.eye(N, dtype=np.float32) * np.float32(2.0 ** (127 - e))
    A = np.eye(8, dtype=np.float32)
    B = np.tile(np.eye(4, dtype=np.float32), (N // 32, 1, 1))
    wq, we = bq.prepare_weight(f32_to_device(W), A, B, layout=layout)
    torch.cuda.synchronize()
    return W, wq, we


# The W4A8 product dequantises the E4M3 codes to bf16, exact for scale bytes 9..246, so the
# MXFP8 encoder is read back through it at bytes of that range (the quantiser alone is
# checked at 0, 1, 127 and 246 above); 9 puts the smallest E4M3 value on bf16's subnormals.
SCALE_BYTES_FP8_PRODUCT = [9, 10, 127, 246]


@pytest.mark.parametrize("fp8,e", [(False, e) for e in SCALE_BYTES_FP4] +
                         [(True, e) for e in SCALE_BYTES_FP8_PRODUCT])
def test_one_kernel_layer_ties(bq, orc, e, fp8):
    """The encoders inside the one-kernel layers (at most four tokens, no workspace), read
    back through an identity product: y equals the oracle's code values exactly."""
    import torch
    x_all = tie_rows(e, fp8)
    N = x_all.shape[1]
    A, B, r = identity_layer(x_all)
    T = bq.SCALES_MFMA_TILED
    W, wq, we = identity_weights(bq, N, e, T)
    wq_ref, we_ref = orc.prepare_weight(W, A, B)
    fn = bq.linear_w4a8_raw if fp8 else bq.linear_w4a4_raw
    dA, dB, dr = f32_to_device(A), f32_to_device(B), f32_to_device(r)
    for s0 in range(0, x_all.shape[0], 4):
        x = x_all[s0:s0 + 4]
        S = x.shape[0]
        print(f"[ties one-kernel] fp8={fp8} e={e} rows {s0}..{s0 + S - 1}", flush=True)
        xd = bf16_to_device(x)
        y = torch.empty((S, N), dtype=torch.float32, device="cuda")
        st = fn(xd.data_ptr(), S, N, N, dA.data_ptr(), dB.data_ptr(), dr.data_ptr(),
                dr.data_ptr(), wq.data_ptr(), we.data_ptr(), N, y.data_ptr(), 0, 0, layout=T,
                stream=torch.cuda.current_stream().cuda_stream)
        assert st == 0, bq.status_string(st)
        torch.cuda.synchronize()
        if fp8:
            xq, xe = orc.quantize_act_fp8(x, A, B, r, r)
            y_ref, _ = orc.gemm_w4a8(xq, xe, wq_ref, we_ref)
            assert np.array_equal(y_ref, orc.e4m3_value(xq))
        else:
            xq, xe = orc.quantize_act(x, A, B, r, r)
            y_ref, _ = orc.gemm(xq, xe, wq_ref, we_ref)
        yh = to_host(y).astype(np.float64)
        bad = np.argwhere(yh != y_ref)
        assert bad.size == 0, (f"fp8={fp8} e={e}: {len(bad)} outputs differ, first "
                               f"{bad[:4].tolist()} gpu {yh[tuple(bad[0])]} ref "
                               f"{y_ref[tuple(bad[0])]}")


@pytest.mark.parametrize("e", [1, 127])
def test_one_kernel_layer_ties_sixteen_tokens(bq, orc, e):
    """With a workspace and 5-16 tokens the W4A4 layer still takes the one kernel here
    (S k and the encoding work are small): its 16-token encoder on the same ties."""
    import torch
    x = tie_rows(e, fp8=False)
    x = np.concatenate([x] * (-(-12 // x.shape[0])))[:12]
    S, N = x.shape
    A, B, r = identity_layer(x)
    T = bq.SCALES_MFMA_TILED
    W, wq, we = identity_weights(bq, N, e, T)
    print(f"[ties one-kernel 12 tokens] e={e}", flush=True)
    y = bq.linear_w4a4(bf16_to_device(x), f32_to_device(A), f32_to_device(B), f32_to_device(r),
                       f32_to_device(r), wq, we, layout=T)
    torch.cuda.synchronize()
    xq, xe = orc.quantize_act(x, A, B, r, r)
    wq_ref, we_ref = orc.prepare_weight(W, A, B)
    y_ref, _ = orc.gemm(xq, xe, wq_ref, we_ref)
    assert np.array_equal(to_host(y).astype(np.float64), y_ref)
