"""ctypes binding over libbatq.so: argument marshalling only.

Every step of the path runs in the library's HIP kernels; PyTorch provides device memory
and the current stream.  If the built library is missing the calls fail loudly; there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbatq.so")

STATUS = {0: "BATQ_OK", 1: "BATQ_ERR_NULL", 2: "BATQ_ERR_SHAPE", 3: "BATQ_ERR_ALIGN",
          4: "BATQ_ERR_UNSUPPORTED", 5: "BATQ_ERR_SINGULAR", 6: "BATQ_ERR_HIP",
          7: "BATQ_ERR_TOO_LARGE"}

# Every exported entry point and its ctypes signature (the names of include/batq.h).
_P, _I64, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
SIGNATURES = {
    "batq_quantize_act": [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _I, _P],
    "batq_prepare_weight": [_P, _I64, _I64, _P, _P, _P, _P, _I, _P],
    "batq_gemm_w4a4": [_P, _P, _P, _P, _I, _I64, _I64, _I64, _P, _P],
    "batq_quantize_act_mxfp8": [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _I, _P],
    "batq_gemm_w4a8": [_P, _P, _P, _P, _I, _I64, _I64, _I64, _P, _P],
    "batq_quantize_act_rmsnorm": [_P, _I64, _I64, _I64, _P, ctypes.c_float, _P, _P, _P, _P, _P,
                                  _P, _I, _P],
    "batq_gemm_w4a4_out": [_P, _P, _P, _P, _I, _I64, _I64, _I64, _P, _I, _P, _P],
    "batq_gemm_w4a8_out": [_P, _P, _P, _P, _I, _I64, _I64, _I64, _P, _I, _P, _P],
    "batq_quantize_act_form": [_P, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _I, _P],
    "batq_prepare_weight_form": [_P, _I64, _I64, _I, _P, _P, _P, _P, _I, _P],
    "batq_quantize_kv": [_P, _I64, _I64, _I64, _P, _I64, _I, _P, _P, _P, _P, _P, _P, _P],
    "batq_transform_rows": [_P, _I, _I64, _I64, _I64, _P, _P, _P, _I, _P],
    "batq_dequantize_rows": [_P, _P, _I64, _I64, _I, _P, _I64, _P, _I, _P],
    "batq_linear_w4a4": [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _I, _I64, _P, _P, _P, _P],
    "batq_linear_w4a8": [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _I, _I64, _P, _P, _P, _P],
    "batq_linear_w4a4_noalloc": [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _I, _I64, _P, _P],
    "batq_clip_ratios": [_P, _I64, _P],
    "batq_weight_factors": [_P, _P, _I64, _P, _P],
    "batq_status_string": [_I],
}


# Scale layouts (batq_scale_layout): row-major [rows, N/32], or the MFMA-tiled order in which
# the GEMM consumes them (32-row x 8-block units of 256 bytes).
SCALES_ROW_MAJOR = 0
SCALES_MFMA_TILED = 1

# bytes of batq_linear_w4a4_noalloc's device scratch (BATQ_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20

# batq_linear_w4a4 runs in one kernel up to this many tokens (BATQ_LINEAR_FUSED_TOKENS)
LINEAR_FUSED_TOKENS = 4
LINEAR_W4A8_FUSED_BLOCKS = 768

# Element types (batq_out_type) of GEMM outputs and of transformed / dequantised rows.
OUT_F32 = 0
OUT_BF16 = 1

# Transform forms (batq_transform): GPK, naive Kronecker with a private A_i per block, full
# 32x32 P_i per block.
TRANSFORM_GPK = 0
TRANSFORM_KRONECKER = 1
TRANSFORM_FULL = 2

# KV-cache element formats (batq_kv_format).
KV_MXFP4 = 4
KV_MXFP8 = 8


def scale_bytes(rows: int, N: int, layout: int) -> int:
    """Size in bytes of the scale array of a rows x N MXFP4 tensor in `layout`."""
    k = N // 32
    if layout == SCALES_ROW_MAJOR:
        return rows * k
    return ((rows + 31) // 32) * 32 * ((k + 7) // 8) * 8


class BatqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load the built library (build it with __graft_entry__.build() or
    ``python w4a4_batq_quantize_amd/build.py``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; the HIP path has no fallback")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name == "batq_status_string" else ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().batq_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise BatqError(fn, status)


# ---------------------------------------------------------------------------------------
# raw entry points (integer device pointers, integer stream handle)
# ---------------------------------------------------------------------------------------

def quantize_act_raw(x, S, N, ldx, A, B, r_min, r_max, q, e, layout=SCALES_ROW_MAJOR,
                     stream=0) -> int:
    return lib().batq_quantize_act(x, S, N, ldx, A, B, r_min, r_max, q, e, layout, stream)


def gemm_w4a4_raw(xq, xe, wq, we, S, N, out, y, layout=SCALES_ROW_MAJOR, stream=0) -> int:
    return lib().batq_gemm_w4a4(xq, xe, wq, we, layout, S, N, out, y, stream)


def quantize_act_mxfp8_raw(x, S, N, ldx, A, B, r_min, r_max, q8, e, layout=SCALES_ROW_MAJOR,
                           stream=0) -> int:
    return lib().batq_quantize_act_mxfp8(x, S, N, ldx, A, B, r_min, r_max, q8, e, layout,
                                         stream)


def gemm_w4a8_raw(xq8, xe, wq, we, S, N, out, y, layout=SCALES_ROW_MAJOR, stream=0) -> int:
    return lib().batq_gemm_w4a8(xq8, xe, wq, we, layout, S, N, out, y, stream)


def quantize_act_form_raw(x, S, N, ldx, form, F0, F1, r_min, r_max, q, e,
                          layout=SCALES_ROW_MAJOR, stream=0) -> int:
    return lib().batq_quantize_act_form(x, S, N, ldx, form, F0, F1, r_min, r_max, q, e, layout,
                                        stream)


def prepare_weight_form_raw(W, out, N, form, F0_host, F1_host, wq, we,
                            layout=SCALES_ROW_MAJOR, stream=0) -> int:
    return lib().batq_prepare_weight_form(W, out, N, form, F0_host, F1_host, wq, we, layout,
                                          stream)


def gemm_w4a4_out_raw(xq, xe, wq, we, S, N, out, y, y_type=0, residual=0,
                      layout=SCALES_ROW_MAJOR, stream=0) -> int:
    return lib().batq_gemm_w4a4_out(xq, xe, wq, we, layout, S, N, out, y, y_type, residual,
                                    stream)


def gemm_w4a8_out_raw(xq8, xe, wq, we, S, N, out, y, y_type=0, residual=0,
                      layout=SCALES_ROW_MAJOR, stream=0) -> int:
    return lib().batq_gemm_w4a8_out(xq8, xe, wq, we, layout, S, N, out, y, y_type, residual,
                                    stream)


def quantize_act_rmsnorm_raw(x, S, N, ldx, gamma, eps, A, B, r_min, r_max, q, e,
                             layout=SCALES_ROW_MAJOR, stream=0) -> int:
    return lib().batq_quantize_act_rmsnorm(x, S, N, ldx, gamma, eps, A, B, r_min, r_max, q, e,
                                           layout, stream)


def linear_w4a4_raw(x, S, N, ldx, A, B, r_min, r_max, wq, we, out, y, xq=0, xe=0,
                    layout=SCALES_ROW_MAJOR, stream=0) -> int:
    return lib().batq_linear_w4a4(x, S, N, ldx, A, B, r_min, r_max, wq, we, layout, out, y, xq,
                                  xe, stream)


def linear_w4a4_noalloc_raw(x, S, N, ldx, A, B, r_min, r_max, wq, we, out, y,
                            layout=SCALES_ROW_MAJOR, stream=0) -> int:
    return lib().batq_linear_w4a4_noalloc(x, S, N, ldx, A, B, r_min, r_max, wq, we, layout, out,
                                          y, stream)


def linear_w4a8_raw(x, S, N, ldx, A, B, r_min, r_max, wq, we, out, y, xq8=0, xe=0,
                    layout=SCALES_ROW_MAJOR, stream=0) -> int:
    return lib().batq_linear_w4a8(x, S, N, ldx, A, B, r_min, r_max, wq, we, layout, out, y, xq8,
                                  xe, stream)


def quantize_kv_raw(x, T, N, ldx, slots, num_slots, fmt, A, B, r_min, r_max, cache_q, cache_e,
                    stream=0) -> int:
    return lib().batq_quantize_kv(x, T, N, ldx, slots, num_slots, fmt, A, B, r_min, r_max,
                                  cache_q, cache_e, stream)


def transform_rows_raw(x, x_type, rows, N, ldx, A, B, y, y_type, stream=0) -> int:
    return lib().batq_transform_rows(x, x_type, rows, N, ldx, A, B, y, y_type, stream)


def dequantize_rows_raw(q, e, src_rows, N, fmt, index, rows, y, y_type, stream=0) -> int:
    return lib().batq_dequantize_rows(q, e, src_rows, N, fmt, index, rows, y, y_type, stream)


def prepare_weight_raw(W, out, N, A_host, B_host, wq, we, layout=SCALES_ROW_MAJOR,
                       stream=0) -> int:
    return lib().batq_prepare_weight(W, out, N, A_host, B_host, wq, we, layout, stream)


# ---------------------------------------------------------------------------------------
# host helpers
# ---------------------------------------------------------------------------------------

def _host_f32(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def clip_ratios(alpha) -> np.ndarray:
    """fp32 sigmoid(alpha) per block (host)."""
    a = _host_f32(alpha).ravel()
    r = np.empty_like(a)
    _check("batq_clip_ratios", lib().batq_clip_ratios(a.ctypes.data, a.size, r.ctypes.data))
    return r


def weight_factors(A, B):
    """Host fp32 factors (A^-1)^T [8,8] and (B_i^-1)^T [k,4,4] of the offline weight side."""
    A = _host_f32(A).reshape(8, 8)
    B = _host_f32(B).reshape(-1, 4, 4)
    Ai = np.empty_like(A)
    Bi = np.empty_like(B)
    _check("batq_weight_factors", lib().batq_weight_factors(
        A.ctypes.data, B.ctypes.data, B.shape[0], Ai.ctypes.data, Bi.ctypes.data))
    return Ai, Bi


# ---------------------------------------------------------------------------------------
# torch-tensor entry points
# ---------------------------------------------------------------------------------------

def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t) -> int:
    return t.data_ptr()


def _req(t, name, dtype, numel, device, contiguous=True):
    """Argument check before any launch: the C ABI sees raw pointers only, so a tensor of the
    wrong type, size or device would make a kernel read or write outside it."""
    assert t is not None, f"{name} is required"
    assert t.dtype == dtype, f"{name}: dtype {t.dtype}, expected {dtype}"
    assert t.numel() == numel, f"{name}: {t.numel()} elements, expected {numel}"
    assert t.device == device, f"{name} is on {t.device}, expected {device}"
    if contiguous:
        assert t.is_contiguous(), f"{name} must be contiguous"


def _req_act(x):
    """bf16 activations [S, N] with unit column stride and N a multiple of 32."""
    import torch
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1, \
        "x must be a bf16 [S, N] tensor with unit column stride"
    assert x.shape[1] % 32 == 0, "N must be a multiple of 32"
    return x.shape[0], x.shape[1]


def _req_gpk(A, B, r_min, r_max, k, device):
    import torch
    _req(A, "A", torch.float32, 64, device)
    _req(B, "B", torch.float32, 16 * k, device)
    _req(r_min, "r_min", torch.float32, k, device)
    _req(r_max, "r_max", torch.float32, k, device)


def _scale_tensor(rows, N, layout, device):
    import torch
    if layout == SCALES_ROW_MAJOR:
        return torch.empty((rows, N // 32), dtype=torch.uint8, device=device)
    return torch.empty((scale_bytes(rows, N, layout),), dtype=torch.uint8, device=device)


def quantize_act(x, A, B, r_min, r_max, q=None, e=None, layout=SCALES_ROW_MAJOR, stream=None):
    """Fused transform + clip + MXFP4 of bf16 activations x [S, N] (row stride may exceed
    N).  A fp32 [8,8], B fp32 [k,4,4], r_min/r_max fp32 [k] (device).  Returns the codes
    uint8 [S, N/2] and the scales: uint8 [S, N/32] row-major, or a flat uint8 buffer in the
    MFMA-tiled layout."""
    import torch
    S, N = _req_act(x)
    if q is None:
        q = torch.empty((S, N // 2), dtype=torch.uint8, device=x.device)
    if e is None:
        e = _scale_tensor(S, N, layout, x.device)
    _req_gpk(A, B, r_min, r_max, N // 32, x.device)
    _req(q, "q", torch.uint8, S * (N // 2), x.device)
    _req(e, "e", torch.uint8, scale_bytes(S, N, layout), x.device)
    _check("batq_quantize_act", quantize_act_raw(
        _ptr(x), S, N, x.stride(0), _ptr(A), _ptr(B), _ptr(r_min), _ptr(r_max), _ptr(q),
        _ptr(e), layout, _stream(stream)))
    return q, e


def prepare_weight(W, A_host, B_host, layout=SCALES_ROW_MAJOR, stream=None):
    """Offline: fp32 weights W [out, N] (device) -> MXFP4 codes [out, N/2] and scales of
    W P^-T (in `layout`).  A_host [8,8] and B_host [k,4,4] are host arrays; synchronises
    the stream."""
    import torch
    assert W.dtype == torch.float32 and W.is_contiguous() and W.dim() == 2
    out, N = W.shape
    A = _host_f32(A_host)
    B = _host_f32(B_host)
    assert A.size == 64 and B.size == 16 * (N // 32)
    wq = torch.empty((out, N // 2), dtype=torch.uint8, device=W.device)
    we = _scale_tensor(out, N, layout, W.device)
    _check("batq_prepare_weight", prepare_weight_raw(
        _ptr(W), out, N, A.ctypes.data, B.ctypes.data, _ptr(wq), _ptr(we), layout,
        _stream(stream)))
    return wq, we


def gemm_w4a4(xq, xe, wq, we, y=None, layout=SCALES_ROW_MAJOR, stream=None):
    """fp32 y [S, out] = dq(xq, xe) dq(wq, we)^T on scaled MFMA; xe and we in `layout`."""
    import torch
    S, N = xq.shape[0], xq.shape[1] * 2
    out = wq.shape[0]
    dev = xq.device
    _req(xq, "xq", torch.uint8, S * (N // 2), dev)
    _req(xe, "xe", torch.uint8, scale_bytes(S, N, layout), dev)
    _req(wq, "wq", torch.uint8, out * (N // 2), dev)
    _req(we, "we", torch.uint8, scale_bytes(out, N, layout), dev)
    if y is None:
        y = torch.empty((S, out), dtype=torch.float32, device=dev)
    _req(y, "y", torch.float32, S * out, dev)
    _check("batq_gemm_w4a4", gemm_w4a4_raw(_ptr(xq), _ptr(xe), _ptr(wq), _ptr(we), S, N, out,
                                           _ptr(y), layout, _stream(stream)))
    return y


def linear_w4a4(x, A, B, r_min, r_max, wq, we, layout=SCALES_ROW_MAJOR, y=None,
                workspace=None, stream=None):
    """One pass of the online path through batq_linear_w4a4: quantise the activations and
    multiply with the prepared weights (scales `we` in `layout`).

    `workspace` is the caller's (xq uint8 [S, N/2], xe scales of S x N in `layout`): given
    it, the library picks the faster of its one-kernel path and the two calls.  Without it,
    shapes the one kernel takes (at most LINEAR_FUSED_TOKENS tokens, N/32 a multiple of 8
    up to 512) run with no workspace at all; any other shape gets one allocated here."""
    import torch
    S, N = _req_act(x)
    out = wq.shape[0]
    dev = x.device
    k = N // 32
    _req_gpk(A, B, r_min, r_max, k, dev)
    _req(wq, "wq", torch.uint8, out * (N // 2), dev)
    _req(we, "we", torch.uint8, scale_bytes(out, N, layout), dev)
    if y is None:
        y = torch.empty((S, out), dtype=torch.float32, device=dev)
    _req(y, "y", torch.float32, S * out, dev)
    if workspace is not None:
        xq, xe = workspace
        _req(xq, "workspace xq", torch.uint8, S * (N // 2), dev)
        _req(xe, "workspace xe", torch.uint8, scale_bytes(S, N, layout), dev)
    elif S <= LINEAR_FUSED_TOKENS and k <= 512 and k % 8 == 0:
        xq = xe = None
    else:
        xq = torch.empty((S, N // 2), dtype=torch.uint8, device=dev)
        xe = _scale_tensor(S, N, layout, dev)
    _check("batq_linear_w4a4", linear_w4a4_raw(
        _ptr(x), S, N, x.stride(0), _ptr(A), _ptr(B), _ptr(r_min), _ptr(r_max), _ptr(wq),
        _ptr(we), out, _ptr(y), _ptr(xq) if xq is not None else 0,
        _ptr(xe) if xe is not None else 0, layout, _stream(stream)))
    return y


# ---------------------------------------------------------------------------------------
# W4A8: MXFP8 (E4M3) activations against the same MXFP4 weights
# ---------------------------------------------------------------------------------------

def quantize_act_mxfp8(x, A, B, r_min, r_max, q8=None, e=None, layout=SCALES_ROW_MAJOR,
                       stream=None):
    """Fused transform + clip + MXFP8 of bf16 activations x [S, N].  Returns the E4M3 codes
    uint8 [S, N] and the scales (as quantize_act)."""
    import torch
    S, N = _req_act(x)
    if q8 is None:
        q8 = torch.empty((S, N), dtype=torch.uint8, device=x.device)
    if e is None:
        e = _scale_tensor(S, N, layout, x.device)
    _req_gpk(A, B, r_min, r_max, N // 32, x.device)
    _req(q8, "q8", torch.uint8, S * N, x.device)
    _req(e, "e", torch.uint8, scale_bytes(S, N, layout), x.device)
    _check("batq_quantize_act_mxfp8", quantize_act_mxfp8_raw(
        _ptr(x), S, N, x.stride(0), _ptr(A), _ptr(B), _ptr(r_min), _ptr(r_max), _ptr(q8),
        _ptr(e), layout, _stream(stream)))
    return q8, e


def gemm_w4a8(xq8, xe, wq, we, y=None, layout=SCALES_ROW_MAJOR, stream=None):
    """fp32 y [S, out] = dq8(xq8, xe) dq(wq, we)^T on scaled MFMA; xe and we in `layout`."""
    import torch
    S, N = xq8.shape
    out = wq.shape[0]
    dev = xq8.device
    _req(xq8, "xq8", torch.uint8, S * N, dev)
    _req(xe, "xe", torch.uint8, scale_bytes(S, N, layout), dev)
    _req(wq, "wq", torch.uint8, out * (N // 2), dev)
    _req(we, "we", torch.uint8, scale_bytes(out, N, layout), dev)
    if y is None:
        y = torch.empty((S, out), dtype=torch.float32, device=dev)
    _req(y, "y", torch.float32, S * out, dev)
    _check("batq_gemm_w4a8", gemm_w4a8_raw(_ptr(xq8), _ptr(xe), _ptr(wq), _ptr(we), S, N, out,
                                           _ptr(y), layout, _stream(stream)))
    return y


def linear_w4a8(x, A, B, r_min, r_max, wq, we, layout=SCALES_ROW_MAJOR, y=None,
                workspace=None, stream=None):
    """The W4A8 layer through batq_linear_w4a8: transform, clip and MXFP8 of the activations,
    then the W4A8 product with the prepared weights (scales `we` in `layout`): one kernel up
    to LINEAR_FUSED_TOKENS tokens and LINEAR_W4A8_FUSED_BLOCKS token blocks, else the two
    calls through `workspace` (the caller's (xq8 uint8 [S, N], xe scales), or one allocated
    here when none is given)."""
    import torch
    S, N = _req_act(x)
    out = wq.shape[0]
    dev = x.device
    k = N // 32
    _req_gpk(A, B, r_min, r_max, k, dev)
    _req(wq, "wq", torch.uint8, out * (N // 2), dev)
    _req(we, "we", torch.uint8, scale_bytes(out, N, layout), dev)
    if y is None:
        y = torch.empty((S, out), dtype=torch.float32, device=dev)
    _req(y, "y", torch.float32, S * out, dev)
    if workspace is not None:
        xq8, xe = workspace
        _req(xq8, "workspace xq8", torch.uint8, S * N, dev)
        _req(xe, "workspace xe", torch.uint8, scale_bytes(S, N, layout), dev)
    elif (S <= LINEAR_FUSED_TOKENS and k <= 512 and k % 8 == 0
          and S * k <= LINEAR_W4A8_FUSED_BLOCKS):
        xq8 = xe = None
    else:
        xq8 = torch.empty((S, N), dtype=torch.uint8, device=dev)
        xe = _scale_tensor(S, N, layout, dev)
    _check("batq_linear_w4a8", linear_w4a8_raw(
        _ptr(x), S, N, x.stride(0), _ptr(A), _ptr(B), _ptr(r_min), _ptr(r_max), _ptr(wq),
        _ptr(we), out, _ptr(y), _ptr(xq8) if xq8 is not None else 0,
        _ptr(xe) if xe is not None else 0, layout, _stream(stream)))
    return y


# ---------------------------------------------------------------------------------------
# Transform forms (GPK, naive Kronecker, full P_i)
# ---------------------------------------------------------------------------------------

def quantize_act_form(x, form, F0, F1, r_min, r_max, q=None, e=None, layout=SCALES_ROW_MAJOR,
                      stream=None):
    """Transform (of the given form) + clip + MXFP4 of bf16 activations x [S, N].  F0 / F1
    device fp32: GPK A [8,8] / B [k,4,4]; KRONECKER A [k,8,8] / B [k,4,4]; FULL P [k,32,32] /
    None."""
    import torch
    S, N = _req_act(x)
    k = N // 32
    dev = x.device
    if q is None:
        q = torch.empty((S, N // 2), dtype=torch.uint8, device=dev)
    if e is None:
        e = _scale_tensor(S, N, layout, dev)
    f0n = {TRANSFORM_GPK: 64, TRANSFORM_KRONECKER: 64 * k, TRANSFORM_FULL: 1024 * k}[form]
    _req(F0, "F0", torch.float32, f0n, dev)
    if form != TRANSFORM_FULL:
        _req(F1, "F1", torch.float32, 16 * k, dev)
    _req(r_min, "r_min", torch.float32, k, dev)
    _req(r_max, "r_max", torch.float32, k, dev)
    _req(q, "q", torch.uint8, S * (N // 2), dev)
    _req(e, "e", torch.uint8, scale_bytes(S, N, layout), dev)
    _check("batq_quantize_act_form", quantize_act_form_raw(
        _ptr(x), S, N, x.stride(0), form, _ptr(F0), _ptr(F1) if F1 is not None else 0,
        _ptr(r_min), _ptr(r_max), _ptr(q), _ptr(e), layout, _stream(stream)))
    return q, e


def prepare_weight_form(W, form, F0_host, F1_host, layout=SCALES_ROW_MAJOR, stream=None):
    """Offline: fp32 weights W [out, N] (device) -> MXFP4 codes and scales of W P^-T for a
    transform form; F0_host / F1_host host arrays as for quantize_act_form."""
    import torch
    assert W.dtype == torch.float32 and W.is_contiguous() and W.dim() == 2
    out, N = W.shape
    F0 = _host_f32(F0_host)
    F1 = _host_f32(F1_host) if F1_host is not None else None
    wq = torch.empty((out, N // 2), dtype=torch.uint8, device=W.device)
    we = _scale_tensor(out, N, layout, W.device)
    _check("batq_prepare_weight_form", prepare_weight_form_raw(
        _ptr(W), out, N, form, F0.ctypes.data, F1.ctypes.data if F1 is not None else 0,
        _ptr(wq), _ptr(we), layout, _stream(stream)))
    return wq, we


# ---------------------------------------------------------------------------------------
# GEMM epilogue: bf16 output and/or a bf16 residual
# ---------------------------------------------------------------------------------------

def gemm_out(xq, xe, wq, we, out_dtype=None, residual=None, y=None, layout=SCALES_ROW_MAJOR,
             w4a8=False, stream=None):
    """W4A4 (or, with w4a8=True, W4A8: xq holds E4M3 codes [S, N]) GEMM with the fused
    epilogue y = round(acc + residual): out_dtype torch.float32 (default) or torch.bfloat16,
    residual a bf16 [S, out] tensor or None."""
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    assert out_dtype in (torch.float32, torch.bfloat16)
    S = xq.shape[0]
    N = xq.shape[1] if w4a8 else xq.shape[1] * 2
    out = wq.shape[0]
    dev = xq.device
    _req(xq, "xq", torch.uint8, S * (N if w4a8 else N // 2), dev)
    _req(xe, "xe", torch.uint8, scale_bytes(S, N, layout), dev)
    _req(wq, "wq", torch.uint8, out * (N // 2), dev)
    _req(we, "we", torch.uint8, scale_bytes(out, N, layout), dev)
    if residual is not None:
        _req(residual, "residual", torch.bfloat16, S * out, dev)
    if y is None:
        y = torch.empty((S, out), dtype=out_dtype, device=dev)
    _req(y, "y", out_dtype, S * out, dev)
    yt = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    fn, raw = (("batq_gemm_w4a8_out", gemm_w4a8_out_raw) if w4a8 else
               ("batq_gemm_w4a4_out", gemm_w4a4_out_raw))
    _check(fn, raw(_ptr(xq), _ptr(xe), _ptr(wq), _ptr(we), S, N, out, _ptr(y), yt,
                   _ptr(residual) if residual is not None else 0, layout, _stream(stream)))
    return y


# ---------------------------------------------------------------------------------------
# RMSNorm fused in front of the quantiser
# ---------------------------------------------------------------------------------------

def quantize_act_rmsnorm(x, gamma, eps, A, B, r_min, r_max, q=None, e=None,
                         layout=SCALES_ROW_MAJOR, stream=None):
    """RMSNorm (gamma fp32 [N] on the device, eps) + transform + clip + MXFP4 of bf16
    activations x [S, N]; returns the codes and scales as quantize_act."""
    import torch
    S, N = _req_act(x)
    if q is None:
        q = torch.empty((S, N // 2), dtype=torch.uint8, device=x.device)
    if e is None:
        e = _scale_tensor(S, N, layout, x.device)
    _req(gamma, "gamma", torch.float32, N, x.device)
    _req_gpk(A, B, r_min, r_max, N // 32, x.device)
    _req(q, "q", torch.uint8, S * (N // 2), x.device)
    _req(e, "e", torch.uint8, scale_bytes(S, N, layout), x.device)
    _check("batq_quantize_act_rmsnorm", quantize_act_rmsnorm_raw(
        _ptr(x), S, N, x.stride(0), _ptr(gamma), float(eps), _ptr(A), _ptr(B), _ptr(r_min),
        _ptr(r_max), _ptr(q), _ptr(e), layout, _stream(stream)))
    return q, e


# ---------------------------------------------------------------------------------------
# KV caches (MXFP4 / MXFP8 rows written through a slot map) and the transform of rows
# ---------------------------------------------------------------------------------------

def quantize_kv(x, slots, fmt, A, B, r_min, r_max, cache_q, cache_e, stream=None):
    """Transform + clip + MX encoding of K or V rows x (bf16 [T, N]) written into cache rows
    slots[t] (int64 [T]; out-of-range slots skip the token).  cache_q uint8 [num_slots, N/2]
    (KV_MXFP4) or [num_slots, N] (KV_MXFP8), cache_e uint8 [num_slots, N/32]; updated in
    place."""
    import torch
    T, N = _req_act(x)
    dev = x.device
    num_slots = cache_q.shape[0]
    _req(slots, "slots", torch.int64, T, dev)
    _req(cache_q, "cache_q", torch.uint8, num_slots * (N // 2 if fmt == KV_MXFP4 else N), dev)
    _req(cache_e, "cache_e", torch.uint8, num_slots * (N // 32), dev)
    _req_gpk(A, B, r_min, r_max, N // 32, dev)
    _check("batq_quantize_kv", quantize_kv_raw(
        _ptr(x), T, N, x.stride(0), _ptr(slots), num_slots, fmt, _ptr(A), _ptr(B), _ptr(r_min),
        _ptr(r_max), _ptr(cache_q), _ptr(cache_e), _stream(stream)))
    return cache_q, cache_e


def _elem_type(dtype):
    import torch
    assert dtype in (torch.float32, torch.bfloat16)
    return OUT_BF16 if dtype == torch.bfloat16 else OUT_F32


def transform_rows(x, A, B, out_dtype=None, y=None, stream=None):
    """y = block transform of the rows of x (fp32 or bf16 [rows, N]) with factors A [8, 8],
    B [N/32, 4, 4] (device fp32), no quantisation; y fp32 (default) or bf16."""
    import torch
    assert x.dim() == 2 and x.stride(1) == 1
    rows, N = x.shape
    assert N % 32 == 0, "N must be a multiple of 32"
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if y is None:
        y = torch.empty((rows, N), dtype=out_dtype, device=x.device)
    _req(y, "y", out_dtype, rows * N, x.device)
    _req(A, "A", torch.float32, 64, x.device)
    _req(B, "B", torch.float32, 16 * (N // 32), x.device)
    _check("batq_transform_rows", transform_rows_raw(
        _ptr(x), _elem_type(x.dtype), rows, N, x.stride(0), _ptr(A), _ptr(B), _ptr(y),
        _elem_type(out_dtype), _stream(stream)))
    return y


def dequantize_rows(cache_q, cache_e, fmt, index=None, out_dtype=None, y=None, stream=None):
    """Cache rows (all, or those listed in the int64 index) back to fp32 (default) or bf16
    [rows, N]; an index entry outside the cache gives a zero row."""
    import torch
    assert cache_q.dim() == 2
    src_rows = cache_q.shape[0]
    N = cache_q.shape[1] * 2 if fmt == KV_MXFP4 else cache_q.shape[1]
    assert N % 32 == 0, "N must be a multiple of 32"
    dev = cache_q.device
    _req(cache_q, "cache_q", torch.uint8, cache_q.numel(), dev)
    _req(cache_e, "cache_e", torch.uint8, src_rows * (N // 32), dev)
    if index is not None:
        _req(index, "index", torch.int64, index.numel(), dev)
    rows = src_rows if index is None else index.numel()
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if y is None:
        y = torch.empty((rows, N), dtype=out_dtype, device=dev)
    _req(y, "y", out_dtype, rows * N, dev)
    _check("batq_dequantize_rows", dequantize_rows_raw(
        _ptr(cache_q), _ptr(cache_e), src_rows, N, fmt, _ptr(index) if index is not None else 0,
        rows, _ptr(y), _elem_type(out_dtype), _stream(stream)))
    return y
