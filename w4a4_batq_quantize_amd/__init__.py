"""BATQuant's online W4A4 linear-layer hot path, native on AMD MI355X (gfx950).

The compute lives in libbatq.so (hand-written HIP kernels behind a C ABI, include/batq.h);
this package is the thin Python binding over it.
"""
from ._binding import (  # noqa: F401
    LIB_PATH,
    SCALES_MFMA_TILED,
    SCALES_ROW_MAJOR,
    SIGNATURES,
    TRANSFORM_FULL,
    TRANSFORM_GPK,
    TRANSFORM_KRONECKER,
    BatqError,
    clip_ratios,
    gemm_w4a4,
    gemm_w4a4_raw,
    gemm_w4a8,
    gemm_w4a8_raw,
    lib,
    linear_w4a4,
    linear_w4a8,
    prepare_weight,
    prepare_weight_form,
    prepare_weight_form_raw,
    prepare_weight_raw,
    quantize_act,
    quantize_act_form,
    quantize_act_form_raw,
    quantize_act_mxfp8,
    quantize_act_mxfp8_raw,
    quantize_act_raw,
    scale_bytes,
    status_string,
    weight_factors,
)
