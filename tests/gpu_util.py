"""Helpers shared by the GPU parity tests: moving seeded inputs to the device and comparing
the HIP path's outputs with the oracle's."""
import os

import numpy as np

ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


def bf16_to_device(x_bits: np.ndarray):
    torch, dev = torch_dev()
    t = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16))
    return t.to(dev).view(torch.bfloat16)


def f32_to_device(a: np.ndarray):
    torch, dev = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def u8_to_device(a: np.ndarray):
    torch, dev = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev)


def to_host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def nibbles(q: np.ndarray) -> np.ndarray:
    return np.stack([q & 0xF, q >> 4], -1).reshape(q.shape[0], -1)


def assert_codes_equal(q_gpu, e_gpu, q_ref, e_ref, exact_zero=None, what=""):
    """Scales bit-exact; codes bit-exact, except that where the oracle's pre-rounding value
    is exactly +-0 either zero code (0x0 or 0x8) is accepted (the sign of an exact zero after
    min/max/clamp is not fixed by the method)."""
    assert e_gpu.shape == e_ref.shape and q_gpu.shape == q_ref.shape, what
    bad_e = np.argwhere(e_gpu != e_ref)
    assert bad_e.size == 0, f"{what}: {len(bad_e)} scale mismatches, first {bad_e[:4].tolist()}"
    if np.array_equal(q_gpu, q_ref):
        return
    cg, cr = nibbles(q_gpu), nibbles(q_ref)
    diff = cg != cr
    if exact_zero is not None:
        diff &= ~(exact_zero & ((cg & 7) == 0) & ((cr & 7) == 0))
    bad = np.argwhere(diff)
    assert bad.size == 0, (f"{what}: {len(bad)} code mismatches, first (row, elem) "
                           f"{bad[:4].tolist()} gpu {cg[tuple(bad[0])]:x} ref {cr[tuple(bad[0])]:x}")


def assert_fp8_codes_equal(q_gpu, e_gpu, q_ref, e_ref, exact_zero, what=""):
    """Scales and E4M3 code bytes bit-exact, except that where the oracle's clipped value is
    exactly +-0 either zero byte (0x00 or 0x80) is accepted."""
    assert q_gpu.shape == q_ref.shape and e_gpu.shape == e_ref.shape, what
    bad_e = np.argwhere(e_gpu != e_ref)
    assert bad_e.size == 0, f"{what}: {len(bad_e)} scale mismatches, first {bad_e[:4].tolist()}"
    diff = q_gpu != q_ref
    diff &= ~(exact_zero & ((q_gpu & 0x7F) == 0) & ((q_ref & 0x7F) == 0))
    bad = np.argwhere(diff)
    assert bad.size == 0, (f"{what}: {len(bad)} code mismatches, first (row, elem) "
                           f"{bad[:4].tolist()} gpu {q_gpu[tuple(bad[0])]:#04x} "
                           f"ref {q_ref[tuple(bad[0])]:#04x}")


def assert_gemm_close(y_gpu, y_ref, t_ref, rel=1e-5, what=""):
    """|y_gpu - y_ref| <= rel * sum|terms| elementwise (fp32 accumulation across blocks)."""
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bound = rel * t_ref
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{what}: {len(bad)} outputs beyond {rel} sum|terms|, first "
                           f"{bad[:3].tolist()} err {err[tuple(bad[0])]:.3e} "
                           f"bound {bound[tuple(bad[0])]:.3e}")
    assert np.all(np.isfinite(y_gpu))


def tiled_scale_index(rows: int, k: int) -> np.ndarray:
    """Byte offsets [rows, k] of the MFMA-tiled scale layout, from its definition: 32-row
    panels x 8-block groups form 256-byte units; within a row's 8 bytes the blocks of the
    group are ordered 0,2,4,6,1,3,5,7."""
    r = np.arange(rows, dtype=np.int64)[:, None]
    b = np.arange(k, dtype=np.int64)[None, :]
    k8 = (k + 7) // 8
    return ((r // 32) * k8 + b // 8) * 256 + (r % 32) * 8 + (b % 2) * 4 + (b % 8) // 2


def tiled_scale_bytes(rows: int, k: int) -> int:
    return ((rows + 31) // 32) * 32 * ((k + 7) // 8) * 8


def to_tiled_scales(e: np.ndarray, pad: int = 0xFF) -> np.ndarray:
    """Row-major scales [rows, k] -> flat MFMA-tiled buffer; padding bytes set to `pad`
    (0xFF is an E8M0 NaN: any use of a padding byte would poison a result)."""
    rows, k = e.shape
    out = np.full(tiled_scale_bytes(rows, k), pad, dtype=np.uint8)
    out[tiled_scale_index(rows, k)] = e
    return out


def from_tiled_scales(buf: np.ndarray, rows: int, k: int) -> np.ndarray:
    return np.asarray(buf).reshape(-1)[tiled_scale_index(rows, k)]
