"""batq_linear_w4a4_noalloc, the entry point for callers that cannot allocate (its
activation codes and scales live in the library's fixed device scratch), against
batq_linear_w4a4 given a caller workspace: the same kernels, so the outputs are identical.
Two calls in a row, the second with a smaller input (it runs over the first call's leftovers
in the scratch), in both scale layouts, and the oracle's product within 1e-5 sum|terms| on
sampled rows."""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import (ORACLE_THREADS, assert_gemm_close, bf16_to_device, f32_to_device,
                            to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bq():
    import torch
    import w4a4_batq_quantize_amd as bq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bq.lib()
    return bq


def layer_args(bq, L, layout):
    wq, we = bq.prepare_weight(f32_to_device(L.W), L.A, L.B, layout=layout)
    return (bf16_to_device(L.x_bits), f32_to_device(L.A), f32_to_device(L.B),
            f32_to_device(bq.clip_ratios(L.alpha_min)),
            f32_to_device(bq.clip_ratios(L.alpha_max)), wq, we)


def noalloc(bq, args, out, layout):
    import torch
    x, A, B, r1, r2, wq, we = args
    S, N = x.shape
    y = torch.full((S, out), float("nan"), dtype=torch.float32, device="cuda")
    st = bq.linear_w4a4_noalloc_raw(x.data_ptr(), S, N, x.stride(0), A.data_ptr(), B.data_ptr(),
                                    r1.data_ptr(), r2.data_ptr(), wq.data_ptr(), we.data_ptr(),
                                    out, y.data_ptr(), layout=layout,
                                    stream=torch.cuda.current_stream().cuda_stream)
    assert st == 0, bq.status_string(st)
    return y


def with_workspace(bq, args, out, layout):
    import torch
    x, A, B, r1, r2, wq, we = args
    S, N = x.shape
    ws = (torch.empty((S, N // 2), dtype=torch.uint8, device="cuda"),
          torch.empty((bq.scale_bytes(S, N, layout),), dtype=torch.uint8, device="cuda"))
    return bq.linear_w4a4(x, A, B, r1, r2, wq, we, layout=layout, workspace=ws)


def check_oracle(orc, L, y, rows):
    rmin, rmax = orc.clip_ratio(L.alpha_min), orc.clip_ratio(L.alpha_max)
    xq, xe = orc.quantize_act(L.x_bits[rows], L.A, L.B, rmin, rmax, nthreads=ORACLE_THREADS)
    wq, we = orc.prepare_weight(L.W, L.A, L.B, nthreads=ORACLE_THREADS)
    y_ref, t_ref = orc.gemm(xq, xe, wq, we, nthreads=ORACLE_THREADS)
    assert_gemm_close(y[rows], y_ref, t_ref, what="noalloc vs oracle")


@pytest.mark.parametrize("tiled", [True, False])
@pytest.mark.parametrize("first,second", [
    ((2048, 4096, 4096), (300, 1024, 520)),     # quantiser + GEMM through the scratch, twice
    ((12, 1024, 1000), (3, 2048, 77)),          # the one kernel (small S k; S <= 4)
    ((512, 8192, 2048), (33, 512, 4100)),       # 32-row few-token kernel after a tiled GEMM
])
def test_noalloc_matches_workspace_entry(bq, orc, first, second, tiled):
    import torch
    layout = bq.SCALES_MFMA_TILED if tiled else bq.SCALES_ROW_MAJOR
    for i, (S, N, out) in enumerate((first, second)):
        print(f"[noalloc] call {i}: S={S} N={N} out={out} tiled={tiled}", flush=True)
        L = wl.make_layer(wl.custom("noalloc", S, N, out, seed=(131, S, N, out)))
        args = layer_args(bq, L, layout)
        y = noalloc(bq, args, out, layout)
        y_ws = with_workspace(bq, args, out, layout)
        torch.cuda.synchronize()
        y, y_ws = to_host(y), to_host(y_ws)
        assert np.array_equal(y, y_ws), f"call {i}: differs from batq_linear_w4a4 with a workspace"
        rows = np.unique(np.concatenate([[0, S - 1], np.arange(0, S, max(1, S // 16))]))
        check_oracle(orc, L, y, rows)


def test_noalloc_beyond_scratch_is_refused(bq):
    """More activation codes and scales than the scratch holds: BATQ_ERR_TOO_LARGE, no launch,
    and the output untouched."""
    import torch
    S, N, out = 16384, 12288, 64
    x = torch.zeros((S, N), dtype=torch.bfloat16, device="cuda")
    A = torch.eye(8, device="cuda")
    B = torch.eye(4, device="cuda").repeat(N // 32, 1, 1).contiguous()
    r = torch.ones(N // 32, device="cuda")
    wq = torch.zeros((out, N // 2), dtype=torch.uint8, device="cuda")
    we = torch.zeros((bq.scale_bytes(out, N, bq.SCALES_MFMA_TILED),), dtype=torch.uint8,
                     device="cuda")
    y = torch.full((S, out), 7.0, device="cuda")
    st = bq.linear_w4a4_noalloc_raw(x.data_ptr(), S, N, N, A.data_ptr(), B.data_ptr(),
                                    r.data_ptr(), r.data_ptr(), wq.data_ptr(), we.data_ptr(), out,
                                    y.data_ptr(), layout=bq.SCALES_MFMA_TILED,
                                    stream=torch.cuda.current_stream().cuda_stream)
    assert bq._binding.STATUS[st] == "BATQ_ERR_TOO_LARGE"
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
