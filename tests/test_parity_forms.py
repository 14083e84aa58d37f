"""GPU parity of the transform forms of thelatestinai listing's Table 1 (naive Kronecker with
a private A_i per block, full 32x32 P_i per block) against the oracle on the same seeded
inputs: activation and weight codes and scales bit for bit, the W4A4 product end to end
within 1e-5 * sum|terms|."""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import (ORACLE_THREADS, assert_codes_equal, assert_gemm_close,
                            bf16_to_device, f32_to_device, from_tiled_scales, to_host)

pytestmark = pytest.mark.gpu

FORMS = {"kronecker": 1, "full": 2}


@pytest.fixture(scope="module")
def bq():
    import torch
    import w4a4_batq_quantize_amd as bq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bq.lib()
    return bq


def run_act_form(bq, L, form, F0, F1, ldx=None, layout=0):
    import torch
    S, N = L.x_bits.shape
    if ldx is not None and ldx != N:
        wide = np.zeros((S, ldx), dtype=np.uint16)
        wide[:, :N] = L.x_bits
        wide[:, N:] = 0x7FC0                       # NaN padding: must never be read
        x = bf16_to_device(wide)[:, :N]
    else:
        x = bf16_to_device(L.x_bits)
    q, e = bq.quantize_act_form(x, form, f32_to_device(F0),
                                f32_to_device(F1) if F1 is not None else None,
                                f32_to_device(bq.clip_ratios(L.alpha_min)),
                                f32_to_device(bq.clip_ratios(L.alpha_max)), layout=layout)
    torch.cuda.synchronize()
    q, e = to_host(q), to_host(e)
    if layout == bq.SCALES_MFMA_TILED:
        e = from_tiled_scales(e, S, N // 32)
    return q, e


def oracle_act_form(orc, L, form, F0, F1):
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    q, e = orc.quantize_act_form(L.x_bits, form, F0, F1, rmin, rmax, nthreads=ORACLE_THREADS)
    # exact zeros of the clipped values: transform with the form, then the clip
    xf = wl.bf16_bits_to_f32(L.x_bits)
    y = orc.transform_form_f32(xf, form, F0, F1)
    k = L.cfg.k
    m = y.reshape(y.shape[0], k, 32)
    lo = np.minimum(rmin[None, :] * m.min(axis=2), rmax[None, :] * m.max(axis=2))
    hi = rmax[None, :] * m.max(axis=2)
    yc = np.minimum(np.maximum(m, lo[:, :, None]), hi[:, :, None]).reshape(y.shape)
    return q, e, yc == 0


@pytest.mark.parametrize("form_name", ["kronecker", "full"])
@pytest.mark.parametrize("name", ["tiny", "q_proj", "down_proj", "sweep_s8_n4096"])
def test_act_form_parity(bq, orc, name, form_name):
    form = FORMS[form_name]
    L = wl.make_layer(name, with_weight=False)
    F0, F1 = wl.form_factors(form, L.cfg.k, seed=(51, form, L.cfg.N))
    print(f"[act form parity] {form_name} {name} S={L.cfg.S} N={L.cfg.N}", flush=True)
    q, e = run_act_form(bq, L, form, F0, F1)
    q_ref, e_ref, zero = oracle_act_form(orc, L, form, F0, F1)
    assert_codes_equal(q, e, q_ref, e_ref, zero, what=f"{form_name} {name}")


@pytest.mark.parametrize("form_name", ["kronecker", "full"])
@pytest.mark.parametrize("S,N,ldx,seed", [(1, 32, 32, 1), (37, 4192, 4256, 3),
                                          (130, 2048, 2048, 4)])
def test_act_form_ragged_strided_and_tiled(bq, orc, S, N, ldx, seed, form_name):
    form = FORMS[form_name]
    L = wl.make_layer(wl.custom("ragged-form", S, N, 8, seed=seed), with_weight=False)
    F0, F1 = wl.form_factors(form, L.cfg.k, seed=(52, form, S, N))
    q_ref, e_ref, zero = oracle_act_form(orc, L, form, F0, F1)
    for layout in (bq.SCALES_ROW_MAJOR, bq.SCALES_MFMA_TILED):
        q, e = run_act_form(bq, L, form, F0, F1, ldx=ldx, layout=layout)
        assert_codes_equal(q, e, q_ref, e_ref, zero,
                           what=f"{form_name} S={S} N={N} ldx={ldx} layout={layout}")


def test_act_form_gpk_dispatch_and_hadamard_full_form(bq, orc):
    """The GPK form equals batq_quantize_act; the full form with the orthonormal Sylvester
    Hadamard H32 / sqrt(32) (block Hadamard, the BRQ baseline) matches the oracle."""
    L = wl.make_layer("down_proj", with_weight=False)
    k = L.cfg.k
    q0, e0 = run_act_form(bq, L, 0, L.A, L.B)
    import torch
    q1, e1 = bq.quantize_act(bf16_to_device(L.x_bits), f32_to_device(L.A), f32_to_device(L.B),
                             f32_to_device(bq.clip_ratios(L.alpha_min)),
                             f32_to_device(bq.clip_ratios(L.alpha_max)))
    torch.cuda.synchronize()
    assert np.array_equal(q0, to_host(q1)) and np.array_equal(e0, to_host(e1))
    H = np.array([[1.0]])
    for _ in range(5):
        H = np.block([[H, H], [H, -H]])
    P = np.broadcast_to((H / np.sqrt(32)).astype(np.float32), (k, 32, 32)).copy()
    q, e = run_act_form(bq, L, 2, P, None)
    q_ref, e_ref, zero = oracle_act_form(orc, L, 2, P, None)
    assert_codes_equal(q, e, q_ref, e_ref, zero, what="hadamard full form")


@pytest.mark.parametrize("form_name", ["kronecker", "full"])
@pytest.mark.parametrize("out,N", [(64, 256), (300, 512)])
def test_weight_form_parity(bq, orc, out, N, form_name):
    import torch
    form = FORMS[form_name]
    L = wl.make_layer(wl.custom("wform", 4, N, out, seed=9))
    F0, F1 = wl.form_factors(form, N // 32, seed=(53, form, N))
    wq_ref, we_ref = orc.prepare_weight_form(L.W, form, F0, F1, nthreads=ORACLE_THREADS)
    for layout in (bq.SCALES_ROW_MAJOR, bq.SCALES_MFMA_TILED):
        wq, we = bq.prepare_weight_form(f32_to_device(L.W), form, F0, F1, layout=layout)
        torch.cuda.synchronize()
        wq, we = to_host(wq), to_host(we)
        if layout == bq.SCALES_MFMA_TILED:
            we = from_tiled_scales(we, out, N // 32)
        assert_codes_equal(wq, we, wq_ref, we_ref, L.W == 0, what=f"{form_name} weights")


@pytest.mark.parametrize("form_name", ["kronecker", "full"])
def test_linear_form_end_to_end(bq, orc, form_name):
    import torch
    form = FORMS[form_name]
    L = wl.make_layer(wl.custom("e2e-form", 96, 256, 130, seed=11))
    F0, F1 = wl.form_factors(form, L.cfg.k, seed=(54, form))
    T = bq.SCALES_MFMA_TILED
    wq, we = bq.prepare_weight_form(f32_to_device(L.W), form, F0, F1, layout=T)
    x = bf16_to_device(L.x_bits)
    xq, xe = bq.quantize_act_form(x, form, f32_to_device(F0),
                                  f32_to_device(F1) if F1 is not None else None,
                                  f32_to_device(bq.clip_ratios(L.alpha_min)),
                                  f32_to_device(bq.clip_ratios(L.alpha_max)), layout=T)
    y = bq.gemm_w4a4(xq, xe, wq, we, layout=T)
    torch.cuda.synchronize()
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    xq_r, xe_r = orc.quantize_act_form(L.x_bits, form, F0, F1, rmin, rmax)
    wq_r, we_r = orc.prepare_weight_form(L.W, form, F0, F1)
    y_ref, t_ref = orc.gemm(xq_r, xe_r, wq_r, we_r, nthreads=ORACLE_THREADS)
    assert_gemm_close(to_host(y), y_ref, t_ref, what=f"{form_name} end to end")
