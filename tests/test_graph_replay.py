"""The online calls captured into a HIP graph (as bench.py times them) and replayed: every
replay, with eager work and synchronisations between replays, gives bit for bit the eager
result (quantiser codes and scales, W4A4 and W4A8 GEMM outputs, KV cache rows, transformed
rows, the one-kernel linear layer)."""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import bf16_to_device, f32_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bq():
    import torch
    import w4a4_batq_quantize_amd as bq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bq.lib()
    return bq


def test_graph_replays_match_eager(bq):
    import torch
    T = bq.SCALES_MFMA_TILED
    L = wl.make_layer(wl.custom("graph", 200, 1024, 512, seed=91))
    S, N, out = 200, 1024, 512
    x = bf16_to_device(L.x_bits)
    A, B = f32_to_device(L.A), f32_to_device(L.B)
    r1 = f32_to_device(bq.clip_ratios(L.alpha_min))
    r2 = f32_to_device(bq.clip_ratios(L.alpha_max))
    wq, we = bq.prepare_weight(f32_to_device(L.W), L.A, L.B, layout=T)
    Ls = wl.make_layer(wl.custom("graph-dec", 3, 1024, 512, seed=92), with_weight=False)
    xs = bf16_to_device(Ls.x_bits)
    slots = torch.from_numpy(wl.kv_slots(S, 300, seed=(93,))).cuda()

    # outputs written by the captured calls
    xq = torch.empty((S, N // 2), dtype=torch.uint8, device="cuda")
    xe = torch.empty((bq.scale_bytes(S, N, T),), dtype=torch.uint8, device="cuda")
    xq8 = torch.empty((S, N), dtype=torch.uint8, device="cuda")
    xe8 = torch.empty_like(xe)
    y4 = torch.empty((S, out), dtype=torch.float32, device="cuda")
    y8 = torch.empty_like(y4)
    sq = torch.empty((3, N // 2), dtype=torch.uint8, device="cuda")
    se = torch.empty((bq.scale_bytes(3, N, T),), dtype=torch.uint8, device="cuda")
    ys = torch.empty((3, out), dtype=torch.float32, device="cuda")
    yl = torch.empty_like(ys)
    yl8 = torch.empty_like(ys)
    cq = torch.zeros((300, N // 2), dtype=torch.uint8, device="cuda")
    ce = torch.zeros((300, N // 32), dtype=torch.uint8, device="cuda")
    tr = torch.empty((S, N), dtype=torch.bfloat16, device="cuda")

    def calls():
        bq.quantize_act(x, A, B, r1, r2, q=xq, e=xe, layout=T)
        bq.gemm_w4a4(xq, xe, wq, we, y=y4, layout=T)
        bq.quantize_act_mxfp8(x, A, B, r1, r2, q8=xq8, e=xe8, layout=T)
        bq.gemm_w4a8(xq8, xe8, wq, we, y=y8, layout=T)
        bq.quantize_act(xs, A, B, r1, r2, q=sq, e=se, layout=T)       # few-token GEMM
        bq.gemm_w4a4(sq, se, wq, we, y=ys, layout=T)
        bq.linear_w4a4(xs, A, B, r1, r2, wq, we, layout=T, y=yl)     # one-kernel linear
        bq.linear_w4a8(xs, A, B, r1, r2, wq, we, layout=T, y=yl8)    # and its W4A8 form
        bq.quantize_kv(x, slots, bq.KV_MXFP4, A, B, r1, r2, cq, ce)
        bq.transform_rows(x, A, B, out_dtype=torch.bfloat16, y=tr)

    outs = (xq, xe, y4, xq8, xe8, y8, sq, se, ys, yl, yl8, cq, ce, tr)
    # every output starts from zeros, here and before each replay: the bytes no call writes
    # (the tiled scale buffers' padding rows) then compare equal too
    for t in outs:
        t.zero_()
    calls()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()                                   # warm the side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.zero_()
        scratch = torch.randn(1 << 20, device="cuda")   # unrelated eager work between replays
        (scratch * 2).sum().item()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("xq", "xe", "y4", "xq8", "xe8", "y8", "sq", "se", "ys",
                                    "yl", "yl8", "cq", "ce", "tr"), outs, eager):
            assert torch.equal(got.view(torch.uint8) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.uint8) if want.dtype == torch.bfloat16 else want), \
                f"replay {rep}: {name}"
