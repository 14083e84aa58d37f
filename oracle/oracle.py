"""Plain CPU oracle for BATQuant's online W4A4 linear-layer path.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's cpu_baseline
leg may import this module; the product package never does, and this module never imports
the product package.

The arithmetic lives in ``batq_oracle.c`` (plain scalar C, fp32 transform with correctly
rounded ``fmaf`` chains, fp64 GEMM).  This file adds the two offline parameter steps that
are defined exactly and are easiest to state with exact rationals:

* ``clip_ratio``: sigmoid of the learnable clipping logits (daily-arxiv summary, bullet
  "块级可学习裁剪"; gist.science summary, section 2C), evaluated as 1/(1+exp(-a)) in binary64
  and rounded once to fp32;
* ``exact_inverse_f32`` / ``weight_factors``: the inverse factors used to fold P^-1 into the
  weights offline (gist.science section 2D; thelatestinai listing, Figure 3).  Because
  (B (x) A)^-1 = B^-1 (x) A^-1, the weight-side transform needs A^-1 and each B_i^-1; they
  are taken as the fp32 rounding (nearest, ties to even) of the exact rational inverse.

Parity of every function here is pinned by tests that do not reuse this code (closed
forms, exhaustive enumeration, brute force on tiny inputs, special cases reducing to
textbook routines).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "batq_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile batq_oracle.c into liboracle.so next to it (always recompiles)."""
    tmp = _SO + ".tmp"
    cmd = ["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


_lib = None


def lib() -> ctypes.CDLL:
    """Load liboracle.so, building it first only if it does not exist."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        build()
    L = ctypes.CDLL(_SO)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int
    L.orc_quantize_act.argtypes = [P, I64, I64, I64, P, P, P, P, P, P, P, P, I32]
    L.orc_quantize_weight.argtypes = [P, I64, I64, P, P, P, P, I32]
    L.orc_transform_f32.argtypes = [P, I64, I64, P, P, P]
    L.orc_clip_quantize_f32.argtypes = [P, I64, I64, I32, P, P, P, P, P]
    L.orc_e2m1_round_f32.argtypes = [P, I64, P]
    L.orc_e2m1_round_bits.argtypes = [ctypes.c_uint32, ctypes.c_uint32, P]
    L.orc_e8m0_scale_f32.argtypes = [P, I64, P]
    L.orc_dequant.argtypes = [P, P, I64, I64, P]
    L.orc_gemm_w4a4.argtypes = [P, P, P, P, I64, I64, I64, P, I64, P, I64, P, P, I32]
    L.orc_quantize_act_fp8.argtypes = [P, I64, I64, I64, P, P, P, P, P, P, I32]
    L.orc_clip_quantize_fp8_f32.argtypes = [P, I64, I64, P, P, P, P]
    L.orc_e4m3_round_f32.argtypes = [P, I64, P]
    L.orc_e4m3_value.argtypes = [P, I64, P]
    L.orc_e8m0_scale_fp8_f32.argtypes = [P, I64, P]
    L.orc_dequant_fp8.argtypes = [P, P, I64, I64, P]
    L.orc_gemm_w4a8.argtypes = [P, P, P, P, I64, I64, I64, P, I64, P, I64, P, P, I32]
    L.orc_quantize_act_form.argtypes = [P, I64, I64, I64, I32, P, P, P, P, P, P, I32]
    L.orc_rmsnorm_f32.argtypes = [P, I64, I64, I64, P, ctypes.c_float, P, P]
    L.orc_quantize_kv.argtypes = [P, I64, I64, I64, P, I32, P, P, P, P, P, P]
    L.orc_transform_rows.argtypes = [P, I32, I64, I64, I64, P, P, P]
    L.orc_f32_to_bf16.argtypes = [P, I64, P]
    L.orc_quantize_act_rmsnorm.argtypes = [P, I64, I64, I64, P, ctypes.c_float, P, P, P, P, P,
                                           P]
    L.orc_quantize_weight_form.argtypes = [P, I64, I64, I32, P, P, P, P, I32]
    L.orc_transform_form_f32.argtypes = [P, I64, I64, I32, P, P, P]
    L.orc_max_threads.restype = I32
    _lib = L
    return L


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def max_threads() -> int:
    return int(lib().orc_max_threads())


# ----------------------------------------------------------------------------------------
# Offline parameter steps
# ----------------------------------------------------------------------------------------

def clip_ratio(alpha) -> np.ndarray:
    """fp32 clip ratios sigmoid(alpha) = 1 / (1 + exp(-alpha)), binary64 then one rounding."""
    a = np.asarray(alpha, dtype=np.float32).ravel()
    out = np.empty(a.shape, dtype=np.float32)
    for t, v in enumerate(a.tolist()):
        out[t] = np.float32(1.0 / (1.0 + math.exp(-float(v))))
    return out.reshape(np.shape(alpha))


def round_fraction_f32(x: Fraction) -> float:
    """Round an exact rational to the nearest fp32 value, ties to even (binary32 with
    subnormals; finite inputs of magnitude below 2^128 only)."""
    if x == 0:
        return 0.0
    sign = -1.0 if x < 0 else 1.0
    a = abs(x)
    # exponent k with 2^k <= a < 2^(k+1)
    k = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** k > a:
        k -= 1
    if Fraction(2) ** (k + 1) <= a:
        k += 1
    qexp = max(k - 23, -149)  # weight of the last significand bit
    scaled = a / (Fraction(2) ** qexp)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = math.ldexp(float(n), qexp)
    if val >= 2.0 ** 128:
        raise OverflowError("value beyond the fp32 range")
    return sign * val


def exact_inverse(M) -> list[list[Fraction]]:
    """Exact inverse of a square matrix of fp32 entries by Gauss-Jordan elimination over the
    rationals.  Raises ZeroDivisionError if the matrix is singular."""
    M = np.asarray(M, dtype=np.float32)
    n = M.shape[0]
    a = [[Fraction(float(M[i, j])) for j in range(n)] + [Fraction(int(i == j)) for j in range(n)]
         for i in range(n)]
    for col in range(n):
        piv = next((r for r in range(col, n) if a[r][col] != 0), None)
        if piv is None:
            raise ZeroDivisionError("singular matrix")
        a[col], a[piv] = a[piv], a[col]
        p = a[col][col]
        a[col] = [v / p for v in a[col]]
        for r in range(n):
            if r != col and a[r][col] != 0:
                f = a[r][col]
                a[r] = [vr - f * vc for vr, vc in zip(a[r], a[col])]
    return [row[n:] for row in a]


def exact_inverse_f32(M) -> np.ndarray:
    """fp32 rounding (nearest, ties to even) of the exact inverse of M."""
    inv = exact_inverse(M)
    n = len(inv)
    return np.array([[round_fraction_f32(inv[i][j]) for j in range(n)] for i in range(n)],
                    dtype=np.float32)


def weight_factors(A, B):
    """Factors of the weight-side transform W_i -> B_i^-1 W_i A^-T, written in the same
    B'^T W A' form as the activation side: returns A' = (A^-1)^T [8,8] and
    B'_i = (B_i^-1)^T [k,4,4], all fp32."""
    A = np.asarray(A, dtype=np.float32)
    B = np.asarray(B, dtype=np.float32).reshape(-1, 4, 4)
    Ainv_t = np.ascontiguousarray(exact_inverse_f32(A).T)
    Binv_t = np.stack([np.ascontiguousarray(exact_inverse_f32(b).T) for b in B])
    return Ainv_t, np.ascontiguousarray(Binv_t)


# ----------------------------------------------------------------------------------------
# Online path
# ----------------------------------------------------------------------------------------

def quantize_act(x_bits, A, B, r_min, r_max, ldx=None, debug=False, nthreads=1):
    """bf16 activations (uint16 bit patterns [S, ldx]) -> (codes [S, N/2], scales [S, N/32])
    [+ (v [S, N], clipped y [S, N]) with debug=True]."""
    x_bits = np.asarray(x_bits)
    assert x_bits.dtype == np.uint16 and x_bits.ndim == 2
    x_bits = np.ascontiguousarray(x_bits)
    S = x_bits.shape[0]
    B = _c(B, np.float32).reshape(-1, 16)
    k = B.shape[0]
    N = 32 * k
    ldx = x_bits.shape[1] if ldx is None else ldx
    assert ldx >= N
    A = _c(A, np.float32).reshape(64)
    r_min = _c(r_min, np.float32)
    r_max = _c(r_max, np.float32)
    q = np.zeros((S, N // 2), dtype=np.uint8)
    e = np.zeros((S, k), dtype=np.uint8)
    v = np.zeros((S, N), dtype=np.float32) if debug else None
    yc = np.zeros((S, N), dtype=np.float32) if debug else None
    lib().orc_quantize_act(_p(x_bits), S, N, ldx, _p(A), _p(B), _p(r_min), _p(r_max),
                           _p(q), _p(e), _p(v), _p(yc), nthreads)
    return (q, e, v, yc) if debug else (q, e)


def quantize_weight(W, Ainv_t, Binv_t, nthreads=1):
    """fp32 weights [out, N] with the inverse factors -> (codes [out, N/2], scales)."""
    W = _c(W, np.float32)
    rows, N = W.shape
    Ainv_t = _c(Ainv_t, np.float32).reshape(64)
    Binv_t = _c(Binv_t, np.float32).reshape(-1, 16)
    assert Binv_t.shape[0] * 32 == N
    q = np.zeros((rows, N // 2), dtype=np.uint8)
    e = np.zeros((rows, N // 32), dtype=np.uint8)
    lib().orc_quantize_weight(_p(W), rows, N, _p(Ainv_t), _p(Binv_t), _p(q), _p(e), nthreads)
    return q, e


def prepare_weight(W, A, B, nthreads=1):
    """Offline weight preparation: inverse factors, transform, MXFP4 (no clip)."""
    Ainv_t, Binv_t = weight_factors(A, B)
    return quantize_weight(W, Ainv_t, Binv_t, nthreads=nthreads)


def transform_f32(x, A, B) -> np.ndarray:
    """GPK transform alone on fp32 rows [rows, N]."""
    x = _c(x, np.float32)
    rows, N = x.shape
    y = np.zeros_like(x)
    lib().orc_transform_f32(_p(x), rows, N, _p(_c(A, np.float32)), _p(_c(B, np.float32)),
                            _p(y))
    return y


def clip_quantize_f32(y, r_min=None, r_max=None, clip=True, debug=False):
    """Clip (optional) + MXFP4 of already-transformed fp32 rows."""
    y = _c(y, np.float32)
    rows, N = y.shape
    k = N // 32
    rmin = _c(r_min if clip else np.ones(k), np.float32)
    rmax = _c(r_max if clip else np.ones(k), np.float32)
    q = np.zeros((rows, N // 2), dtype=np.uint8)
    e = np.zeros((rows, k), dtype=np.uint8)
    v = np.zeros((rows, N), dtype=np.float32) if debug else None
    lib().orc_clip_quantize_f32(_p(y), rows, N, int(bool(clip)), _p(rmin), _p(rmax), _p(q),
                                _p(e), _p(v))
    return (q, e, v) if debug else (q, e)


def e2m1_round(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.zeros(v.shape, dtype=np.uint8)
    lib().orc_e2m1_round_f32(_p(v), v.size, _p(out))
    return out


def e2m1_round_bits(start: int, count: int) -> np.ndarray:
    out = np.zeros(count, dtype=np.uint8)
    lib().orc_e2m1_round_bits(start, count, _p(out))
    return out


def e8m0_scale(amax) -> np.ndarray:
    a = _c(amax, np.float32)
    out = np.zeros(a.shape, dtype=np.uint8)
    lib().orc_e8m0_scale_f32(_p(a), a.size, _p(out))
    return out


def dequant(q, e) -> np.ndarray:
    q = _c(q, np.uint8)
    e = _c(e, np.uint8)
    rows = q.shape[0]
    N = q.shape[1] * 2
    out = np.zeros((rows, N), dtype=np.float64)
    lib().orc_dequant(_p(q), _p(e), rows, N, _p(out))
    return out


def gemm(xq, xe, wq, we, rows=None, cols=None, nthreads=1):
    """fp64 reference of the W4A4 product and of sum |terms| for selected outputs."""
    xq, xe, wq, we = (_c(a, np.uint8) for a in (xq, xe, wq, we))
    S, N = xq.shape[0], xq.shape[1] * 2
    out = wq.shape[0]
    assert wq.shape[1] * 2 == N and xe.shape == (S, N // 32) and we.shape == (out, N // 32)
    r = None if rows is None else _c(rows, np.int64)
    c = None if cols is None else _c(cols, np.int64)
    nr = S if r is None else r.size
    nc = out if c is None else c.size
    y = np.zeros((nr, nc), dtype=np.float64)
    t = np.zeros((nr, nc), dtype=np.float64)
    lib().orc_gemm_w4a4(_p(xq), _p(xe), _p(wq), _p(we), S, N, out, _p(r), nr, _p(c), nc,
                        _p(y), _p(t), nthreads)
    return y, t


# ----------------------------------------------------------------------------------------
# W4A8: MXFP8 (E4M3) activations against the same MXFP4 weights
# ----------------------------------------------------------------------------------------

def quantize_act_fp8(x_bits, A, B, r_min, r_max, nthreads=1):
    """bf16 activations [S, N] -> (E4M3 codes [S, N], scales [S, N/32])."""
    x_bits = np.ascontiguousarray(np.asarray(x_bits))
    assert x_bits.dtype == np.uint16 and x_bits.ndim == 2
    S = x_bits.shape[0]
    B = _c(B, np.float32).reshape(-1, 16)
    k = B.shape[0]
    N = 32 * k
    ldx = x_bits.shape[1]
    assert ldx >= N
    q = np.zeros((S, N), dtype=np.uint8)
    e = np.zeros((S, k), dtype=np.uint8)
    lib().orc_quantize_act_fp8(_p(x_bits), S, N, ldx, _p(_c(A, np.float32).reshape(64)), _p(B),
                               _p(_c(r_min, np.float32)), _p(_c(r_max, np.float32)), _p(q),
                               _p(e), nthreads)
    return q, e


def clip_quantize_fp8_f32(y, r_min, r_max):
    """Clip + MXFP8 of already-transformed fp32 rows."""
    y = _c(y, np.float32)
    rows, N = y.shape
    q = np.zeros((rows, N), dtype=np.uint8)
    e = np.zeros((rows, N // 32), dtype=np.uint8)
    lib().orc_clip_quantize_fp8_f32(_p(y), rows, N, _p(_c(r_min, np.float32)),
                                    _p(_c(r_max, np.float32)), _p(q), _p(e))
    return q, e


def e4m3_round(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.zeros(v.shape, dtype=np.uint8)
    lib().orc_e4m3_round_f32(_p(v), v.size, _p(out))
    return out


def e4m3_value(code) -> np.ndarray:
    c = _c(code, np.uint8)
    out = np.zeros(c.shape, dtype=np.float64)
    lib().orc_e4m3_value(_p(c), c.size, _p(out))
    return out


def e8m0_scale_fp8(amax) -> np.ndarray:
    a = _c(amax, np.float32)
    out = np.zeros(a.shape, dtype=np.uint8)
    lib().orc_e8m0_scale_fp8_f32(_p(a), a.size, _p(out))
    return out


def dequant_fp8(q8, e) -> np.ndarray:
    q8 = _c(q8, np.uint8)
    e = _c(e, np.uint8)
    rows, N = q8.shape
    out = np.zeros((rows, N), dtype=np.float64)
    lib().orc_dequant_fp8(_p(q8), _p(e), rows, N, _p(out))
    return out


def gemm_w4a8(xq8, xe, wq, we, rows=None, cols=None, nthreads=1):
    """fp64 reference of the W4A8 product (MXFP8 activations x MXFP4 weights)."""
    xq8, xe, wq, we = (_c(a, np.uint8) for a in (xq8, xe, wq, we))
    S, N = xq8.shape
    out = wq.shape[0]
    assert wq.shape[1] * 2 == N and xe.shape == (S, N // 32) and we.shape == (out, N // 32)
    r = None if rows is None else _c(rows, np.int64)
    c = None if cols is None else _c(cols, np.int64)
    nr = S if r is None else r.size
    nc = out if c is None else c.size
    y = np.zeros((nr, nc), dtype=np.float64)
    t = np.zeros((nr, nc), dtype=np.float64)
    lib().orc_gemm_w4a8(_p(xq8), _p(xe), _p(wq), _p(we), S, N, out, _p(r), nr, _p(c), nc,
                        _p(y), _p(t), nthreads)
    return y, t


# ----------------------------------------------------------------------------------------
# Transform forms compared in thelatestinai listing's Table 1: GPK (form 0), naive
# Kronecker with a private A_i per block (form 1), a full 32x32 P_i per block (form 2)
# ----------------------------------------------------------------------------------------

FORM_GPK, FORM_KRONECKER, FORM_FULL = 0, 1, 2


def _form_factors(form, F0, F1, k):
    if form == FORM_FULL:
        F0 = _c(F0, np.float32).reshape(k, 1024)
        F1 = np.zeros(16 * k, dtype=np.float32)
    else:
        F0 = _c(F0, np.float32).reshape(-1)
        assert F0.size == (64 if form == FORM_GPK else 64 * k)
        F1 = _c(F1, np.float32).reshape(k, 16)
    return F0, F1


def quantize_act_form(x_bits, form, F0, F1, r_min, r_max, nthreads=1):
    """bf16 activations [S, N] -> (codes [S, N/2], scales [S, N/32]) with transform `form`:
    F0 = A [8,8] / A_i [k,8,8] / P_i [k,32,32], F1 = B_i [k,4,4] (unused for the full form)."""
    x_bits = np.ascontiguousarray(np.asarray(x_bits))
    assert x_bits.dtype == np.uint16 and x_bits.ndim == 2
    S, ldx = x_bits.shape
    r_min = _c(r_min, np.float32)
    k = r_min.size
    N = 32 * k
    F0, F1 = _form_factors(form, F0, F1, k)
    q = np.zeros((S, N // 2), dtype=np.uint8)
    e = np.zeros((S, k), dtype=np.uint8)
    lib().orc_quantize_act_form(_p(x_bits), S, N, ldx, form, _p(F0), _p(F1), _p(r_min),
                                _p(_c(r_max, np.float32)), _p(q), _p(e), nthreads)
    return q, e


def transform_form_f32(x, form, F0, F1) -> np.ndarray:
    x = _c(x, np.float32)
    rows, N = x.shape
    F0, F1 = _form_factors(form, F0, F1, N // 32)
    y = np.zeros_like(x)
    lib().orc_transform_form_f32(_p(x), rows, N, form, _p(F0), _p(F1), _p(y))
    return y


def weight_factors_form(form, F0, F1, k):
    """Transposed fp32 inverses of a form's factors (nearest fp32 to the exact inverse):
    the weight block becomes P_i^-1 applied on the right transposed, W_i P_i^-T."""
    if form == FORM_GPK:
        return weight_factors(F0, F1)
    B = np.asarray(F1, dtype=np.float32).reshape(-1, 4, 4) if form != FORM_FULL else None
    if form == FORM_KRONECKER:
        A = np.asarray(F0, dtype=np.float32).reshape(k, 8, 8)
        Ai = np.stack([np.ascontiguousarray(exact_inverse_f32(a).T) for a in A])
        Bi = np.stack([np.ascontiguousarray(exact_inverse_f32(b).T) for b in B])
        return np.ascontiguousarray(Ai), np.ascontiguousarray(Bi)
    P = np.asarray(F0, dtype=np.float32).reshape(k, 32, 32)
    Pi = np.stack([np.ascontiguousarray(exact_inverse_f32(m).T) for m in P])
    return np.ascontiguousarray(Pi), None


def prepare_weight_form(W, form, F0, F1, nthreads=1):
    """Offline weight preparation for a transform form: inverse factors, transform, MXFP4."""
    W = _c(W, np.float32)
    rows, N = W.shape
    k = N // 32
    G0, G1 = weight_factors_form(form, F0, F1, k)
    G0, G1 = _form_factors(form, G0, G1, k)
    q = np.zeros((rows, N // 2), dtype=np.uint8)
    e = np.zeros((rows, k), dtype=np.uint8)
    lib().orc_quantize_weight_form(_p(W), rows, N, form, _p(G0), _p(G1), _p(q), _p(e),
                                   nthreads)
    return q, e


# ----------------------------------------------------------------------------------------
# RMSNorm in front of the quantiser (arithmetic contract in orc_rmsnorm_f32)
# ----------------------------------------------------------------------------------------

def rmsnorm(x_bits, gamma, eps):
    """bf16 rows [S, N] -> (normalised fp32 rows [S, N], r [S])."""
    x_bits = np.ascontiguousarray(np.asarray(x_bits))
    assert x_bits.dtype == np.uint16 and x_bits.ndim == 2
    S, ldx = x_bits.shape
    gamma = _c(gamma, np.float32)
    N = gamma.size
    xh = np.zeros((S, N), dtype=np.float32)
    r = np.zeros(S, dtype=np.float32)
    lib().orc_rmsnorm_f32(_p(x_bits), S, N, ldx, _p(gamma), float(eps), _p(xh), _p(r))
    return xh, r


def quantize_act_rmsnorm(x_bits, gamma, eps, A, B, r_min, r_max):
    """RMSNorm + transform + clip + MXFP4 of bf16 rows [S, N]."""
    x_bits = np.ascontiguousarray(np.asarray(x_bits))
    S, ldx = x_bits.shape
    gamma = _c(gamma, np.float32)
    N = gamma.size
    k = N // 32
    q = np.zeros((S, N // 2), dtype=np.uint8)
    e = np.zeros((S, k), dtype=np.uint8)
    lib().orc_quantize_act_rmsnorm(_p(x_bits), S, N, ldx, _p(gamma), float(eps),
                                   _p(_c(A, np.float32).reshape(64)),
                                   _p(_c(B, np.float32).reshape(-1)), _p(_c(r_min, np.float32)),
                                   _p(_c(r_max, np.float32)), _p(q), _p(e))
    return q, e


# ----------------------------------------------------------------------------------------
# KV caches (W4A8KV8 / W4A8KV4): BAT + MXFP8 / MXFP4 of K and V rows into cache slots;
# queries by P^-T and attention outputs by P^-1 without quantisation
# ----------------------------------------------------------------------------------------

def quantize_kv(x_bits, slots, fmt, A, B, r_min, r_max, cache_q, cache_e):
    """Write the quantised rows of x (bf16 bits [T, N]) into cache rows `slots` (negative:
    skipped); cache_q [num_slots, N/2 (fmt 4) or N (fmt 8)], cache_e [num_slots, N/32] are
    updated in place."""
    x_bits = np.ascontiguousarray(np.asarray(x_bits))
    assert x_bits.dtype == np.uint16 and x_bits.ndim == 2 and fmt in (4, 8)
    T, ldx = x_bits.shape
    B = _c(B, np.float32).reshape(-1)
    N = 32 * (B.size // 16)
    slots = _c(slots, np.int64)
    assert slots.size == T and cache_q.flags.c_contiguous and cache_e.flags.c_contiguous
    assert cache_q.shape[1] == (N if fmt == 8 else N // 2) and cache_e.shape[1] == N // 32
    assert slots.max(initial=-1) < cache_q.shape[0]
    lib().orc_quantize_kv(_p(x_bits), T, N, ldx, _p(slots), fmt,
                          _p(_c(A, np.float32).reshape(64)), _p(B), _p(_c(r_min, np.float32)),
                          _p(_c(r_max, np.float32)), _p(cache_q), _p(cache_e))


def transform_rows(x, A, B, x_is_bf16_bits=False) -> np.ndarray:
    """GPK transform of rows (bf16 bit patterns or fp32 [rows, N]) -> fp32 [rows, N]."""
    x = np.ascontiguousarray(np.asarray(x))
    if x_is_bf16_bits:
        assert x.dtype == np.uint16
    else:
        x = x.astype(np.float32)
    rows, ldx = x.shape
    B = _c(B, np.float32).reshape(-1)
    N = 32 * (B.size // 16)
    y = np.zeros((rows, N), dtype=np.float32)
    lib().orc_transform_rows(_p(x), int(x_is_bf16_bits), rows, N, ldx,
                             _p(_c(A, np.float32).reshape(64)), _p(B), _p(y))
    return y


def f32_to_bf16(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.zeros(v.shape, dtype=np.uint16)
    lib().orc_f32_to_bf16(_p(v), v.size, _p(out))
    return out
