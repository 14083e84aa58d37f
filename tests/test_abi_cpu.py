"""The C ABI on a host without a GPU: the library loads, exports every entry point that
include/batq.h declares, validates arguments before any HIP call, and its host-side
parameter steps agree bit for bit with the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, ALIGN, UNSUPPORTED, SINGULAR, HIP, TOO_LARGE = range(8)

# plausible, aligned device addresses; validation must fail before anything dereferences them
D = 1 << 40


@pytest.fixture(scope="module")
def bq():
    import w4a4_batq_quantize_amd as bq
    bq.lib()
    return bq


def declared_entry_points():
    src = open(os.path.join(ROOT, "include", "batq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(batq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_entry_point(bq):
    names = declared_entry_points()
    assert names == sorted(["batq_quantize_act", "batq_prepare_weight", "batq_gemm_w4a4",
                            "batq_clip_ratios", "batq_weight_factors", "batq_status_string",
                            "batq_quantize_act_mxfp8", "batq_gemm_w4a8",
                            "batq_quantize_act_form", "batq_prepare_weight_form",
                            "batq_gemm_w4a4_out", "batq_gemm_w4a8_out",
                            "batq_quantize_act_rmsnorm", "batq_quantize_kv",
                            "batq_transform_rows", "batq_dequantize_rows",
                            "batq_linear_w4a4", "batq_linear_w4a8",
                            "batq_linear_w4a4_noalloc"])
    L = ctypes.CDLL(bq.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(bq.SIGNATURES) == set(names)
    # internal symbols stay hidden
    assert not hasattr(L, "_ZN4batq15launch_quantizeEbPKvlllPKfS3_S3_S3_PhS4_P12ihipStream_t")


def test_status_strings(bq):
    for code, name in bq._binding.STATUS.items():
        assert bq.status_string(code).startswith(name)


def test_quantize_act_argument_errors(bq):
    q = bq.quantize_act_raw
    # shape
    assert q(D, -1, 64, 64, D, D, D, D, D, D) == SHAPE
    assert q(D, 4, 48, 64, D, D, D, D, D, D) == SHAPE            # N % 32
    assert q(D, 4, 64, 32, D, D, D, D, D, D) == SHAPE            # ldx < N
    assert q(D, 1 << 40, 64, 1 << 40, D, D, D, D, D, D) == SHAPE  # S * ldx overflows
    # empty inputs are no-ops that read nothing
    assert q(0, 0, 64, 64, 0, 0, 0, 0, 0, 0) == OK
    assert q(0, 5, 0, 0, 0, 0, 0, 0, 0, 0) == OK
    # null pointers
    for i in (0, 4, 5, 6, 7, 8, 9):
        args = [D, 4, 64, 64, D, D, D, D, D, D]
        args[i] = 0
        assert q(*args) == NULL, i
    # alignment
    assert q(D + 2, 4, 64, 64, D, D, D, D, D, D) == ALIGN        # x not 16-byte aligned
    assert q(D, 4, 64, 68, D, D, D, D, D, D) == ALIGN            # row stride not 16 bytes
    assert q(D, 4, 64, 64, D, D + 4, D, D, D, D) == ALIGN        # B
    assert q(D, 4, 64, 64, D, D, D, D, D + 8, D) == ALIGN        # codes
    assert q(D, 4, 64, 64, D + 2, D, D, D, D, D) == ALIGN        # A


def test_gemm_argument_errors(bq):
    g = bq.gemm_w4a4_raw
    assert g(D, D, D, D, -1, 64, 8, D) == SHAPE
    assert g(D, D, D, D, 4, 40, 8, D) == SHAPE
    assert g(D, D, D, D, 4, 64, -8, D) == SHAPE
    assert g(0, 0, 0, 0, 0, 64, 8, 0) == OK
    assert g(0, 0, 0, 0, 4, 64, 0, 0) == OK
    assert g(0, D, D, D, 4, 64, 8, D) == NULL
    assert g(D, D, D, D, 4, 64, 8, 0) == NULL
    assert g(D, D, D + 1, D, 4, 64, 8, D) == ALIGN
    assert g(D, D, D, D, 4, 64, 8, D + 4) == ALIGN
    assert g(D, D, D, D, 1 << 62, 64, 8, D) == SHAPE


def test_quantize_act_mxfp8_argument_errors(bq):
    q = bq.quantize_act_mxfp8_raw
    assert q(D, -1, 64, 64, D, D, D, D, D, D) == SHAPE
    assert q(D, 4, 48, 64, D, D, D, D, D, D) == SHAPE
    assert q(D, 4, 64, 32, D, D, D, D, D, D) == SHAPE
    assert q(0, 0, 64, 64, 0, 0, 0, 0, 0, 0) == OK
    assert q(0, 5, 0, 0, 0, 0, 0, 0, 0, 0) == OK
    for i in (0, 4, 5, 6, 7, 8, 9):
        args = [D, 4, 64, 64, D, D, D, D, D, D]
        args[i] = 0
        assert q(*args) == NULL, i
    assert q(D + 2, 4, 64, 64, D, D, D, D, D, D) == ALIGN
    assert q(D, 4, 64, 64, D, D, D, D, D + 8, D) == ALIGN        # FP8 codes
    assert q(D, 4, 64, 64, D, D, D, D, D, D, layout=7) == UNSUPPORTED


def test_gemm_w4a8_argument_errors(bq):
    g = bq.gemm_w4a8_raw
    assert g(D, D, D, D, -1, 256, 8, D) == SHAPE
    assert g(D, D, D, D, 4, 40, 8, D) == SHAPE
    assert g(0, 0, 0, 0, 0, 256, 8, 0) == OK
    assert g(0, 0, 0, 0, 4, 256, 0, 0) == OK
    assert g(0, D, D, D, 4, 256, 8, D) == NULL
    assert g(D, D, D, D, 4, 256, 8, 0) == NULL
    assert g(D, D, D + 1, D, 4, 256, 8, D) == ALIGN
    assert g(D, D + 2, D, D, 4, 256, 8, D) == ALIGN              # activation scales
    assert g(D, D, D, D, 4, 256, 8, D + 4) == ALIGN
    assert g(D, D, D, D, 4, 96, 8, D) == UNSUPPORTED               # N % 256
    assert g(D, D, D, D, 1 << 24, 256, 8, D) == UNSUPPORTED        # S * N >= 2^32
    assert g(D, D, D, D, 1 << 62, 256, 8, D) == SHAPE


def test_transform_form_argument_errors_and_singular_factors(bq):
    q = bq.quantize_act_form_raw
    G, K, F = bq.TRANSFORM_GPK, bq.TRANSFORM_KRONECKER, bq.TRANSFORM_FULL
    assert q(D, -1, 64, 64, F, D, 0, D, D, D, D) == SHAPE
    assert q(D, 4, 48, 64, K, D, D, D, D, D, D) == SHAPE
    assert q(0, 0, 64, 64, 5, 0, 0, 0, 0, 0, 0) == OK           # empty: nothing read
    assert q(D, 4, 64, 64, 5, D, D, D, D, D, D) == UNSUPPORTED   # unknown form
    assert q(D, 4, 64, 64, K, D, 0, D, D, D, D) == NULL          # Kronecker needs B
    # (every case below stops in validation: no launch with these fake pointers)
    assert q(D + 2, 4, 64, 64, F, D, 0, D, D, D, D) == ALIGN     # full form: F1 may be NULL
    assert q(D, 4, 64, 64, F, D + 4, 0, D, D, D, D) == ALIGN     # P_i must be 16-aligned
    assert q(D, 4, 64, 64, G, D + 2, D, D, D, D, D) == ALIGN     # a shared A: 4-aligned
    assert q(D, 4, 64, 64, K, D, D + 8, D, D, D, D) == ALIGN
    p = bq.prepare_weight_form_raw
    k = 2
    P = np.tile(np.eye(32, dtype=np.float32), (k, 1, 1))
    assert p(D, 4, 64, 7, P.ctypes.data, 0, D, D) == UNSUPPORTED
    assert p(D, 4, 64, K, P.ctypes.data, 0, D, D) == NULL
    assert p(D, 4, 70, F, P.ctypes.data, 0, D, D) == SHAPE
    Ps = P.copy()
    Ps[1, 5] = Ps[1, 9]
    assert p(D, 4, 64, F, Ps.ctypes.data, 0, D, D) == SINGULAR   # checked before device work
    A = np.tile(np.eye(8, dtype=np.float32), (k, 1, 1))
    A[0, 2] = 0
    B = np.tile(np.eye(4, dtype=np.float32), (k, 1, 1))
    assert p(D, 4, 64, K, A.ctypes.data, B.ctypes.data, D, D) == SINGULAR


def test_gemm_epilogue_argument_errors(bq):
    for g, n in ((bq.gemm_w4a4_out_raw, 64), (bq.gemm_w4a8_out_raw, 256)):
        assert g(D, D, D, D, -1, n, 8, D) == SHAPE
        assert g(0, 0, 0, 0, 0, n, 8, 0) == OK
        assert g(D, D, D, D, 4, n, 8, 0) == NULL
        assert g(D, D, D, D, 4, n, 8, D, 3) == UNSUPPORTED            # unknown output type
        assert g(D, D, D, D, 4, n, 8, D, 1, D + 8) == ALIGN           # residual alignment
        assert g(D, D, D, D, 4, n, 8, D + 8, 1) == ALIGN              # output alignment


def test_rmsnorm_argument_errors(bq):
    q = bq.quantize_act_rmsnorm_raw
    assert q(D, 4, 48, 64, D, 1e-6, D, D, D, D, D, D) == SHAPE
    assert q(0, 0, 64, 64, 0, 1e-6, 0, 0, 0, 0, 0, 0) == OK
    assert q(D, 4, 64, 64, 0, 1e-6, D, D, D, D, D, D) == NULL           # gamma
    assert q(D, 4, 64, 64, D + 4, 1e-6, D, D, D, D, D, D) == ALIGN      # gamma alignment
    assert q(D, 4, 64, 64, D, -1.0, D, D, D, D, D, D) == SHAPE          # eps < 0
    assert q(D, 4, 64, 64, D, float("nan"), D, D, D, D, D, D) == SHAPE
    assert q(D, 4, 32 * 513, 32 * 513 + 8, D, 1e-6, D, D, D, D, D, D) == UNSUPPORTED


def test_kv_cache_argument_errors(bq):
    kv = bq.quantize_kv_raw
    F4, F8 = bq.KV_MXFP4, bq.KV_MXFP8
    assert kv(D, 4, 48, 64, D, 10, F4, D, D, D, D, D, D) == SHAPE       # N % 32
    assert kv(D, 4, 64, 64, D, -1, F4, D, D, D, D, D, D) == SHAPE       # num_slots < 0
    assert kv(D, 4, 64, 64, D, 10, 6, D, D, D, D, D, D) == UNSUPPORTED  # unknown format
    assert kv(0, 0, 64, 64, 0, 10, F8, 0, 0, 0, 0, 0, 0) == OK          # no tokens
    assert kv(D, 4, 64, 64, 0, 10, F4, D, D, D, D, D, D) == NULL        # slots
    assert kv(D, 4, 64, 32, D, 10, F4, D, D, D, D, D, D) == SHAPE       # ldx < N
    assert kv(D, 4, 64, 64, D + 4, 10, F4, D, D, D, D, D, D) == ALIGN   # slots alignment
    assert kv(D, 4, 64, 64, D, 10, F8, D, D, D, D, D + 8, D) == ALIGN   # cache alignment
    assert kv(D, 4, 64, 68, D, 10, F4, D, D, D, D, D, D) == ALIGN       # ldx % 8
    t = bq.transform_rows_raw
    assert t(D, 0, 4, 48, 64, D, D, D, 0) == SHAPE
    assert t(D, 2, 4, 64, 64, D, D, D, 0) == UNSUPPORTED                # unknown input type
    assert t(D, 0, 4, 64, 64, D, D, D, 2) == UNSUPPORTED                # unknown output type
    assert t(0, 0, 0, 64, 64, 0, 0, 0, 0) == OK
    assert t(D, 0, 4, 64, 64, D, 0, D, 0) == NULL
    assert t(D, 0, 4, 64, 66, D, D, D, 0) == ALIGN                      # fp32 ldx % 4
    assert t(D, 1, 4, 64, 68, D, D, D, 0) == ALIGN                      # bf16 ldx % 8
    assert t(D, 0, 4, 64, 68, D, D, D + 8, 1) == ALIGN                  # output alignment
    d = bq.dequantize_rows_raw
    assert d(D, D, 4, 48, F4, 0, 4, D, 0) == SHAPE
    assert d(D, D, 4, 64, F4, 0, 5, D, 0) == SHAPE                      # rows > src without index
    assert d(D, D, 4, 64, 5, 0, 4, D, 0) == UNSUPPORTED
    assert d(D, D, 4, 64, F8, 0, 4, D, 3) == UNSUPPORTED
    assert d(0, 0, 0, 64, F4, 0, 0, 0, 0) == OK
    assert d(D, D, 4, 64, F4, 0, 4, 0, 0) == NULL                       # output
    assert d(D, D, 4, 64, F8, D + 4, 9, D, 0) == ALIGN                  # index alignment
    assert d(D + 8, D, 4, 64, F4, 0, 4, D, 1) == ALIGN                  # codes alignment


def test_linear_argument_errors(bq):
    f = bq.linear_w4a4_raw
    # (x, S, N, ldx, A, B, r_min, r_max, wq, we, out, y, xq, xe)
    assert f(D, 4, 48, 64, D, D, D, D, D, D, 8, D) == SHAPE                # N % 32
    assert f(0, 0, 256, 256, 0, 0, 0, 0, 0, 0, 8, 0) == OK                  # no tokens
    assert f(D, 4, 256, 256, D, D, D, D, D, D, 8, 0) == NULL                # y
    assert f(D, 5, 256, 256, D, D, D, D, D, D, 8, D) == NULL                # workspace needed
    assert f(D, 2, 32 * 520, 32 * 520, D, D, D, D, D, D, 8, D) == NULL      # k > 512: too
    assert f(D, 4, 256, 200, D, D, D, D, D, D, 8, D) == SHAPE               # ldx < N
    assert f(D, 4, 256, 260, D, D, D, D, D, D, 8, D) == ALIGN               # ldx % 8
    assert f(D, 4, 256, 256, D, D + 4, D, D, D, D, 8, D) == ALIGN           # B
    assert f(D, 4, 256, 256, D, D, D, D, D, D, 8, D, layout=7) == UNSUPPORTED


def test_linear_noalloc_argument_errors(bq):
    """Every check runs before the first HIP call (which looks up the device scratch), so
    these return on a host without a GPU; beyond the 64 MiB scratch: BATQ_ERR_TOO_LARGE."""
    f = bq.linear_w4a4_noalloc_raw
    T = bq.SCALES_MFMA_TILED
    # (x, S, N, ldx, A, B, r_min, r_max, wq, we, out, y)
    assert f(D, 4, 48, 64, D, D, D, D, D, D, 8, D) == SHAPE                # N % 32
    assert f(0, 0, 256, 256, 0, 0, 0, 0, 0, 0, 8, 0) == OK                  # no tokens
    assert f(D, 4, 256, 256, D, D, D, D, D, D, 8, 0) == NULL                # y
    assert f(D, 4, 256, 256, D, D, D, D, D, 0, 8, D) == NULL                # we
    assert f(D, 4, 256, 200, D, D, D, D, D, D, 8, D) == SHAPE               # ldx < N
    assert f(D, 4, 256, 260, D, D, D, D, D, D, 8, D) == ALIGN               # ldx % 8
    assert f(D, 4, 256, 256, D, D + 4, D, D, D, D, 8, D) == ALIGN           # B
    assert f(D, 4, 256, 256, D, D, D, D, D, D, 8, D, layout=7) == UNSUPPORTED
    # 16384 x 12288: 96 MiB of codes
    assert f(D, 16384, 12288, 12288, D, D, D, D, D, D, 8, D, layout=T) == TOO_LARGE
    # the boundary: 16384 tokens, N = 7680 fits the tiled layout (60 MiB + 3.75 MiB), 7936 not
    fits = lambda n: (16384 * n // 2 + 255) // 256 * 256 + bq.scale_bytes(16384, n, T)
    assert fits(7680) <= bq.NOALLOC_SCRATCH_BYTES < fits(7936)
    assert f(D, 16384, 7936, 7936, D, D, D, D, D, D, 8, D, layout=T) == TOO_LARGE


def test_linear_w4a8_argument_errors(bq):
    f = bq.linear_w4a8_raw
    # (x, S, N, ldx, A, B, r_min, r_max, wq, we, out, y, xq8, xe)
    assert f(D, 4, 48, 64, D, D, D, D, D, D, 8, D) == SHAPE                # N % 32
    assert f(0, 0, 256, 256, 0, 0, 0, 0, 0, 0, 8, 0) == OK                  # no tokens
    assert f(D, 4, 256, 256, D, D, D, D, D, D, 8, 0) == NULL                # y
    assert f(D, 5, 256, 256, D, D, D, D, D, D, 8, D) == NULL                # workspace needed
    assert f(D, 4, 32 * 256, 32 * 256, D, D, D, D, D, D, 8, D) == NULL      # S k > 768: too
    assert f(D, 2, 32 * 520, 32 * 520, D, D, D, D, D, D, 8, D) == NULL      # k > 512
    assert f(D, 4, 256, 200, D, D, D, D, D, D, 8, D) == SHAPE               # ldx < N
    assert f(D, 4, 256, 260, D, D, D, D, D, D, 8, D) == ALIGN               # ldx % 8
    assert f(D, 4, 256, 256, D, D + 4, D, D, D, D, 8, D) == ALIGN           # B
    assert f(D, 4, 256, 256, D, D, D, D, D, D, 8, D, layout=7) == UNSUPPORTED


def test_prepare_weight_argument_errors_and_singular_factors(bq):
    p = bq.prepare_weight_raw
    A = np.eye(8, dtype=np.float32)
    B = np.tile(np.eye(4, dtype=np.float32), (2, 1, 1))
    a, b = A.ctypes.data, B.ctypes.data
    assert p(D, 4, 70, a, b, D, D) == SHAPE
    assert p(D, -4, 64, a, b, D, D) == SHAPE
    assert p(0, 0, 64, 0, 0, 0, 0) == OK
    assert p(D, 4, 64, 0, b, D, D) == NULL
    assert p(D + 4, 4, 64, a, b, D, D) == ALIGN
    # singular factors are detected on the host, before any device work
    As = A.copy()
    As[3] = As[5]
    assert p(D, 4, 64, As.ctypes.data, b, D, D) == SINGULAR
    Bs = B.copy()
    Bs[1, 2] = 0
    assert p(D, 4, 64, a, Bs.ctypes.data, D, D) == SINGULAR
    with pytest.raises(bq.BatqError):
        bq.weight_factors(As, B)


def test_clip_ratios_match_oracle_bit_for_bit(bq, orc):
    for name in ("tiny", "q_proj", "down_proj"):
        L = wl.make_layer(name, with_weight=False)
        for a in (L.alpha_min, L.alpha_max):
            assert np.array_equal(bq.clip_ratios(a), orc.clip_ratio(a))
    extreme = np.array([0.0, 30.0, -30.0, 88.0, -88.0, 1e-8], dtype=np.float32)
    assert np.array_equal(bq.clip_ratios(extreme), orc.clip_ratio(extreme))


def test_weight_factors_match_oracle_exact_inverse(bq, orc):
    for name in ("tiny", "q_proj", "down_proj"):
        L = wl.make_layer(name, with_weight=False)
        Ai, Bi = bq.weight_factors(L.A, L.B)
        Ai_o, Bi_o = orc.weight_factors(L.A, L.B)
        assert np.array_equal(Ai, Ai_o)
        assert np.array_equal(Bi, Bi_o)


def test_binding_fails_loudly_without_library(bq, monkeypatch):
    monkeypatch.setattr(bq._binding, "_lib", None)
    monkeypatch.setattr(bq._binding, "LIB_PATH", "/nonexistent/libbatq.so")
    with pytest.raises(RuntimeError, match="no fallback"):
        bq._binding.lib()


def test_invalid_scale_layout_is_rejected(bq):
    assert bq.quantize_act_raw(D, 4, 64, 64, D, D, D, D, D, D, 7) == UNSUPPORTED
    assert bq.gemm_w4a4_raw(D, D, D, D, 4, 64, 8, D, 2) == UNSUPPORTED
    A = np.eye(8, dtype=np.float32)
    B = np.tile(np.eye(4, dtype=np.float32), (2, 1, 1))
    assert bq.prepare_weight_raw(D, 4, 64, A.ctypes.data, B.ctypes.data, D, D, 5) == UNSUPPORTED


def test_tiled_scale_layout_definition():
    """The tiled index map is a bijection onto distinct bytes of the stated buffer size,
    and matches hand-computed offsets of the layout's definition."""
    from tests.gpu_util import tiled_scale_bytes, tiled_scale_index
    for rows, k in [(32, 8), (37, 131), (64, 128), (1, 3)]:
        idx = tiled_scale_index(rows, k)
        assert len(np.unique(idx)) == rows * k
        assert idx.max() < tiled_scale_bytes(rows, k)
    idx = tiled_scale_index(64, 16)
    # (row 33, block 9): panel 1, group 1 -> unit 1*2 + 1 = 3; row%32 = 1; block%8 = 1 -> 4
    assert idx[33, 9] == 3 * 256 + 1 * 8 + 4 + 0
    # (row 0, blocks 0..7) -> bytes 0,4,1,5,2,6,3,7
    assert list(idx[0, :8]) == [0, 4, 1, 5, 2, 6, 3, 7]
    assert tiled_scale_bytes(17, 128) == 32 * 128
    import w4a4_batq_quantize_amd as bq
    assert bq.scale_bytes(17, 4096, bq.SCALES_MFMA_TILED) == tiled_scale_bytes(17, 128)
    assert bq.scale_bytes(17, 4096, bq.SCALES_ROW_MAJOR) == 17 * 128


def test_torch_wrappers_check_operands_before_any_launch(bq, monkeypatch):
    """The torch-level wrappers check every operand's type, element count and device before
    they reach the C ABI (which sees raw pointers only): a wrong size raises here, on the
    host, and no library call is made."""
    import torch
    calls = []
    monkeypatch.setattr(bq._binding, "lib", lambda: calls.append(1) or None)
    S, N, out = 4, 256, 64
    k = N // 32
    x = torch.zeros((S, N), dtype=torch.bfloat16)
    A, B = torch.eye(8), torch.eye(4).repeat(k, 1, 1).contiguous()
    r = torch.ones(k)
    bad = [
        lambda: bq.quantize_act(x, A, B[:-1].contiguous(), r, r),                   # short B
        lambda: bq.quantize_act(x, A, B, r[:-1], r),                                # short ratios
        lambda: bq.quantize_act(x, A, B, r, r, e=torch.empty(S * k - 1, dtype=torch.uint8)),
        lambda: bq.quantize_act(x, A, B, r, r, q=torch.empty((S, N // 2 - 1), dtype=torch.uint8)),
        lambda: bq.quantize_act(x, A.double(), B, r, r),                            # dtype
        lambda: bq.quantize_act(x, A.to("meta"), B, r, r),                          # device
        lambda: bq.quantize_act_mxfp8(x, A, B, r, r, q8=torch.empty((S, N // 2), dtype=torch.uint8)),
        lambda: bq.quantize_act_rmsnorm(x, torch.ones(N - 1), 1e-6, A, B, r, r),
    ]
    xq = torch.zeros((S, N // 2), dtype=torch.uint8)
    xe = torch.zeros((S, k), dtype=torch.uint8)
    wq = torch.zeros((out, N // 2), dtype=torch.uint8)
    we = torch.zeros((out, k), dtype=torch.uint8)
    bad += [
        lambda: bq.gemm_w4a4(xq, xe, wq, we[:-1]),                                   # short we
        lambda: bq.gemm_w4a4(xq, xe[:, :-1].contiguous(), wq, we),
        lambda: bq.gemm_w4a4(xq, xe, wq, we, y=torch.empty((S, out - 1))),
        lambda: bq.gemm_w4a4(xq, torch.zeros(S * k, dtype=torch.uint8), wq, we,
                             layout=bq.SCALES_MFMA_TILED),              # tiled scales are padded
        lambda: bq.gemm_w4a8(xq, xe, wq, we),                                       # E4M3 rows are N bytes
        lambda: bq.linear_w4a4(x, A, B, r, r, wq, we[:-1]),
        lambda: bq.linear_w4a4(x, A, B, r, r, wq, we, workspace=(xq[:-1], xe)),
        lambda: bq.linear_w4a8(x, A, B, r, r, wq, we, workspace=(xq, xe)),          # xq8 is [S, N]
        lambda: bq.gemm_out(xq, xe, wq, we, residual=torch.zeros((S, out + 1), dtype=torch.bfloat16)),
        lambda: bq.transform_rows(x, A, B[:-1].contiguous()),
        lambda: bq.quantize_kv(x, torch.zeros(S - 1, dtype=torch.int64), bq.KV_MXFP4, A, B, r, r,
                               torch.zeros((8, N // 2), dtype=torch.uint8),
                               torch.zeros((8, k), dtype=torch.uint8)),
        lambda: bq.dequantize_rows(torch.zeros((8, N // 2), dtype=torch.uint8),
                                   torch.zeros((8, k - 1), dtype=torch.uint8), bq.KV_MXFP4),
    ]
    for i, f in enumerate(bad):
        with pytest.raises(AssertionError):
            f()
        assert not calls, f"case {i} reached the library"
