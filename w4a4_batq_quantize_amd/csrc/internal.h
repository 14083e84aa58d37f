// Launchers shared between the host entry points (api.cpp) and the kernels. Arguments are
// validated by the caller; launchers only size grids and enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace batq {

// Fused transform (+ clip) + MXFP4 of `rows` rows of N = 32k elements.
// Activation mode: bf16 input with row stride ldx, clip ratios r_min/r_max.
// Weight mode: fp32 input with row stride ldx, no clip (r_min/r_max unused).
// Scales row-major, or in the MFMA-tiled layout of batq.h when tiled_scales.
// fp8 (activation mode only): MXFP8 output, codes [rows, N] one E4M3 byte per element.
// form: 0 GPK (A [8][8], B [k][4][4]); 1 Kronecker with private A_i (A [k][8][8], B as
// GPK); 2 full P_i (A [k][32][32], B unused).  Forms 1 and 2 need 16-byte aligned A and do
// not combine with fp8 (hipErrorNotSupported).
hipError_t launch_quantize(bool act, const void* x, int64_t rows, int64_t k, int64_t ldx,
                           const float* A, const float* B, const float* r_min,
                           const float* r_max, uint8_t* q, uint8_t* e, bool tiled_scales,
                           hipStream_t stream, bool fp8 = false, int form = 0);

// RMSNorm (gamma fp32 [32k], eps) fused in front of the GPK activation quantiser; 64, 128
// or 256 threads per row (the padded block count, clamped), one or two blocks per thread,
// k <= 512 (hipErrorNotSupported otherwise).
hipError_t launch_rmsnorm_quantize(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx,
                                   const float* gamma, float eps, const float* A,
                                   const float* B, const float* r_min, const float* r_max,
                                   uint8_t* q, uint8_t* e, bool tiled_scales,
                                   hipStream_t stream);

// KV cache: rows of x (bf16, k blocks) transformed, clipped and encoded (MXFP8 when fp8,
// else MXFP4) into cache rows slots[row] (row-major scales); slots < 0 or >= num_slots skip.
hipError_t launch_quantize_kv(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx,
                              const int64_t* slots, int64_t num_slots, bool fp8,
                              const float* A, const float* B, const float* r_min,
                              const float* r_max, uint8_t* q, uint8_t* e, hipStream_t stream);

// y [rows, 32k] = GPK transform of x (bf16 or fp32 rows, stride ldx) with factors A, B;
// y fp32 or bf16 (round to nearest even), dense.
hipError_t launch_transform_rows(const void* x, bool x_bf16, int64_t rows, int64_t k,
                                 int64_t ldx, const float* A, const float* B, void* y,
                                 bool y_bf16, hipStream_t stream);

// y [rows, 32k] = dequantised MX rows (MXFP8 when fp8, else MXFP4; row-major scales);
// output row r reads source row index[r] (r when index is null), zeros when outside
// [0, src_rows).
hipError_t launch_dequantize_rows(const uint8_t* q, const uint8_t* e, int64_t rows, int64_t k,
                                  bool fp8, const int64_t* index, int64_t src_rows, void* y,
                                  bool y_bf16, hipStream_t stream);

// The linear layer for 1 <= S <= 4 tokens in one kernel: the few-token GEMM encodes the
// bf16 token rows itself (bit for bit launch_quantize's codes); k <= 512, k % 8 == 0;
// hipErrorNotSupported outside that.
hipError_t launch_linear_skinny(const uint16_t* x, int64_t S, int64_t k, int64_t ldx,
                                const float* A, const float* B, const float* r_min,
                                const float* r_max, const uint8_t* wq, const uint8_t* we,
                                bool tiled_scales, int64_t out, float* y, hipStream_t stream);

// The W4A8 layer for at most four tokens in one kernel (MXFP8 token rows encoded in the
// 16-row few-token W4A8 GEMM); hipErrorNotSupported outside S <= 4, k <= 512, k % 8 == 0,
// S k <= 768, the scale alignment or the 32-bit weight offsets.
hipError_t launch_linear16_w4a8(const uint16_t* x, int64_t S, int64_t k, int64_t ldx,
                                const float* A, const float* B, const float* r_min,
                                const float* r_max, const uint8_t* wq, const uint8_t* we,
                                bool tiled_scales, int64_t out, float* y, hipStream_t stream);

// MXFP4 x MXFP4 -> fp32 GEMM, y[S, out] = dq(x)[S, N] dq(w)[out, N]^T; both scale
// arrays in the same layout (tiled_scales: MFMA-tiled, else row-major).
// Epilogue (both GEMMs): res, when not null, is a bf16 [S, out] residual added in fp32;
// out_bf16 stores bf16 (round to nearest even) instead of fp32 (y then points at bf16).
hipError_t launch_gemm(const uint8_t* xq, const uint8_t* xe, const uint8_t* wq,
                       const uint8_t* we, bool tiled_scales, int64_t S, int64_t N,
                       int64_t out, float* y, hipStream_t stream,
                       const uint16_t* res = nullptr, bool out_bf16 = false);

// W4A8: MXFP8 (E4M3) activations xq8 [S, N] (one byte per element) x MXFP4 weights.
// Requires N % 256 == 0 and 4-byte (tiled) / 8-byte (row-major) aligned scale arrays;
// returns hipErrorNotSupported otherwise.
hipError_t launch_gemm_w4a8(const uint8_t* xq8, const uint8_t* xe, const uint8_t* wq,
                            const uint8_t* we, bool tiled_scales, int64_t S, int64_t N,
                            int64_t out, float* y, hipStream_t stream,
                            const uint16_t* res = nullptr, bool out_bf16 = false);

// The no-allocation linear layer's device scratch: activation codes, then (from the next
// 256-byte boundary) their scales.  noalloc_scratch gives the current device's copy (its
// address is looked up once per device, with the device current).
constexpr int64_t kNoAllocScratchBytes = 64LL << 20;
hipError_t noalloc_scratch(uint8_t** ptr);

}  // namespace batq
