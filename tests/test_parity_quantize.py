"""GPU parity of the fused transform + clip + MXFP4 kernel (activation side) and of the
offline weight preparation, against the CPU oracle on the same seeded inputs.  Codes and
scales must match bit for bit."""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import (ORACLE_THREADS, assert_codes_equal, bf16_to_device,
                            f32_to_device, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bq():
    import torch
    import w4a4_batq_quantize_amd as bq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bq.lib()
    return bq


def run_act(bq, L, ldx=None, rmin=None, rmax=None):
    """HIP path on layer L; returns host (q, e)."""
    import torch
    S, N = L.x_bits.shape
    if ldx is not None and ldx != N:
        wide = np.zeros((S, ldx), dtype=np.uint16)
        wide[:, :N] = L.x_bits
        wide[:, N:] = 0x7FC0                       # NaN padding: must never be read
        x = bf16_to_device(wide)[:, :N]
    else:
        x = bf16_to_device(L.x_bits)
    rmin = bq.clip_ratios(L.alpha_min) if rmin is None else rmin
    rmax = bq.clip_ratios(L.alpha_max) if rmax is None else rmax
    q, e = bq.quantize_act(x, f32_to_device(L.A), f32_to_device(L.B), f32_to_device(rmin),
                           f32_to_device(rmax))
    torch.cuda.synchronize()
    return to_host(q), to_host(e)


def oracle_act(orc, L, rows=None, rmin=None, rmax=None):
    rmin = orc.clip_ratio(L.alpha_min) if rmin is None else rmin
    rmax = orc.clip_ratio(L.alpha_max) if rmax is None else rmax
    x = L.x_bits if rows is None else L.x_bits[rows]
    q, e, v, yc = orc.quantize_act(x, L.A, L.B, rmin, rmax, debug=True,
                                   nthreads=ORACLE_THREADS)
    return q, e, yc == 0


FULL = ["tiny", "q_proj", "gate_up", "down_proj", "sweep_s1_n12288", "sweep_s8_n12288",
        "sweep_s64_n12288", "sweep_s1_n4096", "sweep_s8_n4096", "sweep_s64_n4096"]


@pytest.mark.parametrize("name", FULL)
def test_act_parity_full(bq, orc, name):
    L = wl.make_layer(name, with_weight=False)
    print(f"[act parity] {name} S={L.cfg.S} N={L.cfg.N}", flush=True)
    q, e = run_act(bq, L)
    q_ref, e_ref, zero = oracle_act(orc, L)
    assert_codes_equal(q, e, q_ref, e_ref, zero, what=name)


@pytest.mark.parametrize("name", ["sweep_s16384_n4096", "sweep_s16384_n12288"])
def test_act_parity_prefill_sampled_rows(bq, orc, name):
    """S=16384 prefill: the GPU quantises every row; the oracle checks a spread of rows
    (both ends, every 97th, and the rows around each multiple of 4096)."""
    L = wl.make_layer(name, with_weight=False)
    S = L.cfg.S
    print(f"[act parity] {name} S={S} N={L.cfg.N} (sampled rows)", flush=True)
    q, e = run_act(bq, L)
    rows = sorted(set([0, 1, S - 2, S - 1] + list(range(0, S, 97)) +
                      [r for m in range(4096, S, 4096) for r in (m - 1, m)]))
    q_ref, e_ref, zero = oracle_act(orc, L, rows=rows)
    assert_codes_equal(q[rows], e[rows], q_ref, e_ref, zero, what=name)


@pytest.mark.parametrize("S,N,ldx,seed", [
    (1, 32, 32, 1),          # one block
    (3, 96, 104, 2),         # k=3 < one wave, padded rows
    (37, 4192, 4256, 3),     # k=131: ragged against 64-block waves, padded rows
    (130, 2048, 2048, 4),    # several rows per wave and ragged row count
    (5, 64 * 32 * 3 + 32, 6208, 5),   # k=193
    # larger shapes: many rounds of waves, ragged row counts and block counts, padded rows
    (2047, 4096, 4104, 6),
    (1025, 4160, 4160, 7),   # k=130
    (2049, 12288, 12288, 8),
    (4099, 8224, 8232, 9),   # k=257
])
def test_act_parity_ragged_and_strided(bq, orc, S, N, ldx, seed):
    L = wl.make_layer(wl.custom("ragged", S, N, 8, seed=seed), with_weight=False)
    q, e = run_act(bq, L, ldx=ldx)
    q_ref, e_ref, zero = oracle_act(orc, L)
    assert_codes_equal(q, e, q_ref, e_ref, zero, what=f"S={S} N={N} ldx={ldx}")


def edge_layer():
    """Hand-built blocks: all zero, bf16 subnormals only, huge and tiny magnitudes, one
    sign everywhere, a single spike, alternating signs; with near-identity factors."""
    k = 8
    cfg = wl.custom("edge", 6, 32 * k, 8, seed=99)
    L = wl.make_layer(cfg, with_weight=False)
    x = L.x_bits.copy()
    rng = np.random.default_rng(5)
    f = lambda v: wl.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))
    x[0, 0:32] = 0                                              # all-zero block
    x[0, 32:64] = rng.integers(1, 0x80, 32) | (rng.integers(0, 2, 32) << 15)  # subnormals
    x[1, 0:32] = f(rng.standard_normal(32) * 1e36)              # near the top of fp32
    x[1, 32:64] = f(rng.standard_normal(32) * 1e-36)            # tiny normals
    x[2, 0:32] = f(10.0 + rng.random(32))                       # one sign
    x[2, 32:64] = f(-(10.0 + rng.random(32)))
    x[3, 0:32] = f(np.where(np.arange(32) == 17, 1e4, 1e-3))    # single spike
    x[3, 32:64] = f(np.where(np.arange(32) % 2 == 0, 1.0, -1.0))
    L.x_bits = x
    return L


def test_act_parity_edge_blocks(bq, orc):
    L = edge_layer()
    q, e = run_act(bq, L)
    q_ref, e_ref, zero = oracle_act(orc, L)
    assert_codes_equal(q, e, q_ref, e_ref, zero, what="edge")
    assert e_ref[0, 1] == 0 and np.any(q_ref[0, 16:32] & 0x77)  # subnormal block gets codes


def test_act_parity_edge_blocks_identity_and_extreme_ratios(bq, orc):
    """Identity factors; per-block ratios from saturated logits (r = 1: no clipping),
    r_min near 1 with r_max small (lo > hi on one-signed blocks: everything becomes hi),
    and small ratios (heavy clipping)."""
    L = edge_layer()
    k = L.cfg.k
    L.A = np.eye(8, dtype=np.float32)
    L.B = np.tile(np.eye(4, dtype=np.float32), (k, 1, 1))
    # block 0 holds a positive-only row (lo > hi with r_min ~ 1, r_max small), block 1 a
    # negative-only row (lo > hi the other way round), block 5 has r = 1 exactly
    amin = np.array([10, -3, 10, 0.0, -3, 30, 2, 2], dtype=np.float32)
    amax = np.array([-3, 10, -3, 0.0, -3, 30, 2, 2], dtype=np.float32)
    L.alpha_min, L.alpha_max = amin, amax
    q, e = run_act(bq, L)
    q_ref, e_ref, zero = oracle_act(orc, L)
    assert_codes_equal(q, e, q_ref, e_ref, zero, what="edge-identity")


def test_act_deterministic_and_independent_of_layout(bq):
    L = wl.make_layer("down_proj", with_weight=False)
    q1, e1 = run_act(bq, L)
    q2, e2 = run_act(bq, L)
    assert np.array_equal(q1, q2) and np.array_equal(e1, e2)
    q3, e3 = run_act(bq, L, ldx=L.cfg.N + 256)
    assert np.array_equal(q1, q3) and np.array_equal(e1, e3)


def test_act_empty_is_a_no_op(bq):
    import torch
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    A = torch.eye(8, device="cuda")
    B = torch.eye(4, device="cuda").repeat(2, 1, 1).contiguous()
    r = torch.ones(2, device="cuda")
    q, e = bq.quantize_act(x, A, B, r, r)
    assert q.shape == (0, 32) and e.shape == (0, 2)


# ----------------------------------------------------------------------------------------
# offline weight preparation
# ----------------------------------------------------------------------------------------

def run_weight(bq, L):
    import torch
    wq, we = bq.prepare_weight(f32_to_device(L.W), L.A, L.B)
    torch.cuda.synchronize()
    return to_host(wq), to_host(we)


@pytest.mark.parametrize("name,rows", [("tiny", None), ("q_proj", None),
                                       ("down_proj", "sample"), ("gate_up", "sample")])
def test_weight_prep_parity(bq, orc, name, rows):
    L = wl.make_layer(name)
    print(f"[weight parity] {name} out={L.cfg.out} N={L.cfg.N}", flush=True)
    wq, we = run_weight(bq, L)
    Ai, Bi = orc.weight_factors(L.A, L.B)
    out = L.cfg.out
    sel = np.arange(out) if rows is None else np.unique(
        np.concatenate([[0, out - 1], np.arange(0, out, 61), np.arange(127, out, 128)]))
    wq_ref, we_ref = orc.quantize_weight(L.W[sel], Ai, Bi, nthreads=ORACLE_THREADS)
    assert_codes_equal(wq[sel], we[sel], wq_ref, we_ref, L.W[sel] == 0, what=name)


# ----------------------------------------------------------------------------------------
# MFMA-tiled scale layout
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "q_proj", "down_proj", "sweep_s8_n4096"])
def test_act_parity_tiled_scales(bq, orc, name):
    import torch
    from tests.gpu_util import from_tiled_scales
    L = wl.make_layer(name, with_weight=False)
    S, N = L.x_bits.shape
    q, e = bq.quantize_act(bf16_to_device(L.x_bits), f32_to_device(L.A), f32_to_device(L.B),
                           f32_to_device(bq.clip_ratios(L.alpha_min)),
                           f32_to_device(bq.clip_ratios(L.alpha_max)),
                           layout=bq.SCALES_MFMA_TILED)
    torch.cuda.synchronize()
    q_ref, e_ref, zero = oracle_act(orc, L)
    e_rm = from_tiled_scales(to_host(e), S, N // 32)
    assert_codes_equal(to_host(q), e_rm, q_ref, e_ref, zero, what=f"{name} tiled")


@pytest.mark.parametrize("S,N", [(37, 4192), (2050, 4160), (4097, 12288)])
def test_act_parity_tiled_scales_ragged(bq, orc, S, N):
    import torch
    from tests.gpu_util import from_tiled_scales
    L = wl.make_layer(wl.custom("ragged_t", S, N, 8, seed=31), with_weight=False)
    S, N = L.x_bits.shape
    q, e = bq.quantize_act(bf16_to_device(L.x_bits), f32_to_device(L.A), f32_to_device(L.B),
                           f32_to_device(bq.clip_ratios(L.alpha_min)),
                           f32_to_device(bq.clip_ratios(L.alpha_max)),
                           layout=bq.SCALES_MFMA_TILED)
    torch.cuda.synchronize()
    q_ref, e_ref, zero = oracle_act(orc, L)
    assert_codes_equal(to_host(q), from_tiled_scales(to_host(e), S, N // 32), q_ref, e_ref,
                       zero, what="ragged tiled")


@pytest.mark.parametrize("name", ["tiny", "q_proj"])
def test_weight_prep_parity_tiled_scales(bq, orc, name):
    import torch
    from tests.gpu_util import from_tiled_scales
    L = wl.make_layer(name)
    wq, we = bq.prepare_weight(f32_to_device(L.W), L.A, L.B, layout=bq.SCALES_MFMA_TILED)
    torch.cuda.synchronize()
    wq_ref, we_ref = orc.prepare_weight(L.W, L.A, L.B, nthreads=ORACLE_THREADS)
    out, N = L.W.shape
    assert_codes_equal(to_host(wq), from_tiled_scales(to_host(we), out, N // 32), wq_ref,
                       we_ref, L.W == 0, what=f"{name} weights tiled")
