/*
 * batq.h -- C ABI of the BATQuant online W4A4 linear-layer library for AMD MI355X (gfx950).
 *
 * The method ("BATQuant: Outlier-resilient MXFP4 Quantization via Learnable Block-wise
 * Optimization") inserts a block-aligned affine transform before a linear layer: each
 * 32-element MXFP block x_i of an activation row becomes y_i = x_i P_i with
 * P_i = B_i (x) A (A 8x8 shared by all blocks, B_i 4x4 private to block i), is clipped to
 * [sigmoid(alpha_min_i) min(y_i), sigmoid(alpha_max_i) max(y_i)] and quantised to MXFP4.
 * The weight side is transformed by P^-1 and quantised offline, so the layer output is the
 * MXFP4 x MXFP4 product of the two (gist.science technical summary, sections 2A-2D;
 * daily-arxiv summary, method bullets; thelatestinai listing, Figure 3 and Table 1).
 *
 * Conventions for every entry point:
 *  - Sizes are int64_t.  "dev" pointers are device (HBM) memory owned by the caller (for
 *    example torch tensors); "host" pointers are ordinary host memory.  The library keeps
 *    no pointer after a call returns and holds no global mutable state, except the fixed
 *    device scratch of batq_linear_w4a4_noalloc.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Device work is
 *    enqueued on it and the call returns without waiting, unless noted.  Results are valid
 *    once the stream reaches the work.
 *  - Every argument is validated on the host before any HIP call, so an invalid call
 *    returns its error code without touching the GPU.  No call throws.
 *  - Aliasing between an input and an output buffer is not allowed.  Non-finite inputs
 *    (Inf/NaN activations, weights or factors) are outside the contract.
 *
 * Data formats:
 *  - bf16 activations: uint16_t bit patterns, row-major [S, ldx], element n of row s at
 *    x[s*ldx + n]; block i of a row is elements [32i, 32i+32).
 *  - GPK factors: A fp32 [8][8] row-major; B fp32 [k][4][4] row-major (B[i][r][c] at
 *    B[16i + 4r + c]), k = N/32.  The transform of one block is evaluated on its row-major
 *    4x8 view X (X[r][c] = x[8r + c]) as Y = B_i^T (X A): first Z = X A, then Y = B_i^T Z,
 *    in fp32, each sum a product followed by fused multiply-adds in increasing index order.
 *  - MXFP4 tensor of R rows: codes uint8_t [R, N/2] row-major, two E2M1 codes per byte,
 *    element 2j in the low nibble and 2j+1 in the high nibble (E2M1: sign bit 3, magnitude
 *    codes 0..7 = 0, 0.5, 1, 1.5, 2, 3, 4, 6); scales uint8_t [R, N/32] row-major, E8M0
 *    (value 2^(byte-127)).  Scale of a block: floor(log2(max|v|)) - 2, clamped to
 *    [-127, 127]; codes: nearest E2M1 of v / scale, ties to even, saturating at 6.
 *  - Scale layouts (batq_scale_layout), for a matrix of R rows and k = N/32 blocks:
 *      BATQ_SCALES_ROW_MAJOR: scale (r, b) at byte r*k + b; R*k bytes.
 *      BATQ_SCALES_MFMA_TILED: rows grouped in panels of 32, blocks in groups of 8; each
 *        (panel, group) is one contiguous 256-byte unit holding its 32 rows x 8 bytes, and
 *        within a row's 8 bytes the blocks of the group are ordered 0,2,4,6,1,3,5,7.  Scale
 *        (r, b) is at byte ((r/32)*K8 + b/8)*256 + (r%32)*8 + (b%2)*4 + (b%8)/2 with
 *        K8 = ceil(k/8); the buffer holds ceil(R/32)*32 * K8*8 bytes (equal to R*k when
 *        R % 32 == 0 and k % 8 == 0).  Bytes of padding rows/blocks are never written and
 *        never influence a result.  This is the order in which the W4A4 GEMM's matrix
 *        instructions consume scales: one 256-byte unit per 32 rows per 256 K elements.
 *  - GEMM output: fp32 [S, out] row-major.
 */
#ifndef BATQ_H
#define BATQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum batq_scale_layout {
    BATQ_SCALES_ROW_MAJOR = 0,
    BATQ_SCALES_MFMA_TILED = 1
} batq_scale_layout;

/*
 * Transform forms of the block-wise affine transform P_i (thelatestinai listing, Table 1,
 * which compares their parameter counts and costs): GPK (P_i = B_i (x) A with one A for all
 * blocks, the method), naive Kronecker (P_i = B_i (x) A_i, a private A_i per block) and the
 * full 32x32 P_i ("w/o decomposition").  Block Hadamard is GPK with Hadamard factors.
 */
typedef enum batq_transform {
    BATQ_TRANSFORM_GPK = 0,
    BATQ_TRANSFORM_KRONECKER = 1,
    BATQ_TRANSFORM_FULL = 2
} batq_transform;

/* Output element type of the GEMMs' epilogue variants. */
typedef enum batq_out_type {
    BATQ_OUT_F32 = 0,
    BATQ_OUT_BF16 = 1
} batq_out_type;

typedef enum batq_status {
    BATQ_OK = 0,
    BATQ_ERR_NULL = 1,        /* a required pointer is NULL                                  */
    BATQ_ERR_SHAPE = 2,       /* negative size, N not a multiple of 32, ldx < N, or overflow */
    BATQ_ERR_ALIGN = 3,       /* a pointer or stride breaks the alignment stated below       */
    BATQ_ERR_UNSUPPORTED = 4, /* valid for the format but beyond the library's limits        */
    BATQ_ERR_SINGULAR = 5,    /* a GPK factor is not invertible                              */
    BATQ_ERR_HIP = 6,         /* the HIP runtime reported an error (launch, copy, alloc)     */
    BATQ_ERR_TOO_LARGE = 7    /* the input exceeds batq_linear_w4a4_noalloc's fixed scratch  */
} batq_status;

/*
 * Online activation path: fused block transform + block-wise clipping + MXFP4 quantisation
 * (gist.science summary, sections 2A-2C and 2D "activation side ... online";
 * daily-arxiv summary, clipping formula; thelatestinai listing, Figure 2 caption: values
 * are divided by the block scale before rounding).
 *
 *   x      dev  bf16 bits [S, ldx]; 16-byte aligned; ldx >= N and ldx % 8 == 0
 *   S      rows (tokens), >= 0;  N  in-features, >= 0, N % 32 == 0 (k = N/32 blocks)
 *   A      dev  fp32 [8][8], 4-byte aligned
 *   B      dev  fp32 [k][4][4], 16-byte aligned
 *   r_min, r_max  dev fp32 [k], the clip ratios sigmoid(alpha_min/max) of each block (see
 *          batq_clip_ratios), 4-byte aligned
 *   q      dev  out: codes uint8 [S, N/2], 16-byte aligned
 *   e      dev  out: scales in `e_layout` (see "Scale layouts" above)
 * S == 0 or N == 0 is a no-op returning BATQ_OK without reading any pointer.  Per block:
 * m = min y, M = max y, lo = r_min*m, hi = r_max*M (fp32), y' = min(max(y, lo), hi) (the
 * upper bound wins if lo > hi), then MXFP4 of y'.  Does not allocate or synchronise.
 */
batq_status batq_quantize_act(const uint16_t* x, int64_t S, int64_t N, int64_t ldx,
                              const float* A, const float* B,
                              const float* r_min, const float* r_max,
                              uint8_t* q, uint8_t* e, batq_scale_layout e_layout,
                              void* stream);

/*
 * Offline weight preparation: fold P^-1 into the weights and quantise them to MXFP4 with
 * round-to-nearest (gist.science summary, section 2D "weight side ... fused offline";
 * thelatestinai listing, Figure 3 and Tables 6-7 "RTN" weight quantiser).  Keeping
 * X W^T = (X P)(W P^-T)^T, each weight block becomes B_i^-1 W_i A^-T, computed in the same
 * form as the activation side with A' = (A^-1)^T and B'_i = (B_i^-1)^T (see
 * batq_weight_factors), without clipping.
 *
 *   W       dev  fp32 [out, N] row-major, 16-byte aligned;  out >= 0, N % 32 == 0
 *   A_host  host fp32 [8][8];  B_host host fp32 [N/32][4][4]
 *   wq      dev  out: codes uint8 [out, N/2], 16-byte aligned
 *   we      dev  out: scales in `we_layout`
 * Returns BATQ_ERR_SINGULAR if A or any B_i is not invertible.  Offline step: allocates a
 * small device buffer for the factors and synchronises `stream` before returning.
 */
batq_status batq_prepare_weight(const float* W, int64_t out, int64_t N,
                                const float* A_host, const float* B_host,
                                uint8_t* wq, uint8_t* we, batq_scale_layout we_layout,
                                void* stream);

/*
 * W4A4 GEMM: y[s][o] = sum_n dq(xq)[s][n] * dq(wq)[o][n], dq(code, e) = e2m1(code) * 2^(e-127)
 * (the W4A4 linear layer of the gist.science summary, section 4, and thelatestinai
 * listing, abstract), on gfx950 scaled MFMA with fp32 accumulation.  Each 32-element block
 * product is exact; sums across blocks round in fp32.
 *
 *   xq, xe  dev  activation codes [S, N/2] (16-byte aligned) and scales
 *   wq, we  dev  weight codes [out, N/2] (16-byte aligned) and scales
 *   layout  the layout of both xe and we.  BATQ_SCALES_MFMA_TILED with N % 256 == 0 takes
 *           the fastest path (scales 256-byte aligned); any other combination is
 *           supported at lower speed.
 *   S, out >= 0;  N >= 0, N % 32 == 0
 *   y       dev  out: fp32 [S, out], 16-byte aligned, overwritten
 * S == 0 or out == 0 is a no-op; N == 0 writes zeros.  Does not allocate or synchronise.
 */
batq_status batq_gemm_w4a4(const uint8_t* xq, const uint8_t* xe,
                           const uint8_t* wq, const uint8_t* we, batq_scale_layout layout,
                           int64_t S, int64_t N, int64_t out, float* y, void* stream);

/*
 * W4A8 activation side: the same transform and clip as batq_quantize_act, with each
 * clipped block encoded as MXFP8 instead of MXFP4 (the W4A8 setting of the gist.science
 * summary, section 4, and of the daily-arxiv summary, results bullet, W4A8KV16): 32 OCP
 * E4M3 elements (the FP8 variant without infinities, largest magnitude 448) and one E8M0
 * scale.  The scale exponent is floor(log2(amax)) - 8 (E4M3's largest exponent is 8),
 * clamped below at 0; each element is y / 2^(e-127) rounded to the nearest E4M3 value, ties
 * to the even code, magnitudes beyond 448 saturating to 448.  An all-zero block gets scale 0
 * and zero codes.
 *
 *   x, S, N, ldx, A, B, r_min, r_max, stream: as batq_quantize_act
 *   q8  dev  out: codes uint8 [S, N] (one E4M3 byte per element), 16-byte aligned
 *   e   dev  out: scales in `e_layout`, as batq_quantize_act
 * Same error behaviour as batq_quantize_act.  Does not allocate or synchronise.
 */
batq_status batq_quantize_act_mxfp8(const uint16_t* x, int64_t S, int64_t N, int64_t ldx,
                                    const float* A, const float* B,
                                    const float* r_min, const float* r_max,
                                    uint8_t* q8, uint8_t* e, batq_scale_layout e_layout,
                                    void* stream);

/*
 * W4A8 GEMM: y[s][o] = sum_n dq8(xq8)[s][n] * dq(wq)[o][n] with dq8(code, e) =
 * e4m3(code) * 2^(e-127) and dq as in batq_gemm_w4a4 (the W4A8 setting of the gist.science
 * summary, section 4).  Both operands are dequantised to bf16 on the GPU -- exact for
 * activation scale bytes 9..246 (every byte batq_quantize_act_mxfp8 writes for a block whose
 * largest magnitude is at least 2^-110) and for every weight scale batq_prepare_weight
 * writes -- and multiplied on gfx950's bf16 MFMA with fp32 accumulation: the products are
 * exact and the sums round in fp32 (within 1e-5 of sum|terms| of the exact product).
 *
 *   xq8, xe  dev  activation codes [S, N] (16-byte aligned) and scales (4-byte aligned)
 *   wq, we   dev  weight codes [out, N/2] (16-byte aligned) and scales (4-byte aligned),
 *                 as batq_prepare_weight writes them
 *   layout   the layout of both xe and we
 *   S, out >= 0;  N >= 0, N % 256 == 0 (BATQ_ERR_UNSUPPORTED otherwise, and when S*N or
 *            out*N/2 reaches 2^32)
 *   y        dev  out: fp32 [S, out], 16-byte aligned, overwritten
 * S == 0 or out == 0 is a no-op; N == 0 writes zeros.  Does not allocate or synchronise.
 */
batq_status batq_gemm_w4a8(const uint8_t* xq8, const uint8_t* xe,
                           const uint8_t* wq, const uint8_t* we, batq_scale_layout layout,
                           int64_t S, int64_t N, int64_t out, float* y, void* stream);

/*
 * Activation side with a chosen transform form (thelatestinai listing, Table 1; see
 * batq_transform): the same clip and MXFP4 encode as batq_quantize_act, after
 *   GPK:       Y = B_i^T (X A) on the row-major 4x8 view, as batq_quantize_act;
 *   KRONECKER: the same with A_i in place of A;
 *   FULL:      y_j = x_0 P_i[0][j], then fused multiply-adds over m = 1..31 in increasing m
 *              (y = x P_i, x a row vector).
 *   F0  dev  fp32: GPK A [8][8] (4-byte aligned); KRONECKER A [N/32][8][8]; FULL
 *            P [N/32][32][32] (both 16-byte aligned)
 *   F1  dev  fp32 B [N/32][4][4] (16-byte aligned) for GPK and KRONECKER; ignored (may be
 *            NULL) for FULL
 *   other arguments as batq_quantize_act.  BATQ_ERR_UNSUPPORTED for an unknown form or
 *   layout.  Does not allocate or synchronise.
 */
batq_status batq_quantize_act_form(const uint16_t* x, int64_t S, int64_t N, int64_t ldx,
                                   batq_transform form, const float* F0, const float* F1,
                                   const float* r_min, const float* r_max,
                                   uint8_t* q, uint8_t* e, batq_scale_layout e_layout,
                                   void* stream);

/*
 * Offline weight preparation for a transform form: each weight block becomes W_i P_i^-T
 * (X W^T = (X P)(W P^-T)^T; gist.science summary, section 2D), computed in the activation
 * form with the transposed inverses of the factors (each the fp32 value nearest to the
 * exact inverse, 64-bit-mantissa Gauss-Jordan on the host), then MXFP4 without clipping.
 *   W dev fp32 [out, N] (16-byte aligned); F0_host / F1_host host factors as in
 *   batq_quantize_act_form; wq / we / we_layout as batq_prepare_weight.
 * Returns BATQ_ERR_SINGULAR if a factor is not invertible.  Offline step: allocates a device
 * buffer for the factors and synchronises `stream` before returning.
 */
batq_status batq_prepare_weight_form(const float* W, int64_t out, int64_t N,
                                     batq_transform form, const float* F0_host,
                                     const float* F1_host, uint8_t* wq, uint8_t* we,
                                     batq_scale_layout we_layout, void* stream);

/*
 * The GEMMs with a fused epilogue, for the layer's neighbours (a residual connection and a
 * bf16 consumer): out[s][o] = round(acc[s][o] + res[s][o]) where acc is the fp32 result of
 * batq_gemm_w4a4 / batq_gemm_w4a8 (same kernels, same accumulation), res an optional bf16
 * residual converted exactly to fp32 and added with one fp32 rounding, and round() the
 * identity for BATQ_OUT_F32 or fp32 -> bf16 to nearest, ties to even, for BATQ_OUT_BF16.
 * The pages define the linear layer only (gist.science summary, section 4); this is the
 * plain reading of its output feeding the next layer.
 *   y         dev  out: [S, out] of y_type, 16-byte aligned, overwritten
 *   residual  dev  bf16 [S, out] (16-byte aligned) or NULL
 *   other arguments and errors as batq_gemm_w4a4 / batq_gemm_w4a8 (BATQ_ERR_UNSUPPORTED
 *   also for an unknown y_type).  Does not allocate or synchronise.
 */
batq_status batq_gemm_w4a4_out(const uint8_t* xq, const uint8_t* xe,
                               const uint8_t* wq, const uint8_t* we, batq_scale_layout layout,
                               int64_t S, int64_t N, int64_t out, void* y,
                               batq_out_type y_type, const uint16_t* residual, void* stream);
batq_status batq_gemm_w4a8_out(const uint8_t* xq8, const uint8_t* xe,
                               const uint8_t* wq, const uint8_t* we, batq_scale_layout layout,
                               int64_t S, int64_t N, int64_t out, void* y,
                               batq_out_type y_type, const uint16_t* residual, void* stream);

/*
 * The layer's input RMSNorm fused in front of the activation quantiser (the step before
 * each quantised linear layer of the models the pages evaluate; the pages do not define its
 * arithmetic, so it is fixed here): per row, the sum of squares T is taken per 32-block as
 * x_0^2 followed by fused multiply-adds in increasing index order, and the block sums,
 * zero-padded to the next power of two, are added by repeated halving (t[b] += t[b + h] for
 * h = K/2, K/4, .., 1); r = 1 / sqrt(T / N + eps) with correctly rounded division and square
 * root; x_hat_j = (x_j * r) * gamma_j, each product rounded to fp32.  x_hat then goes
 * through exactly the transform, clip and MXFP4 encode of batq_quantize_act.
 *   x, S, N, ldx, A, B, r_min, r_max, q, e, e_layout, stream: as batq_quantize_act
 *   gamma  dev  fp32 [N] RMSNorm weight, 16-byte aligned;  eps >= 0, finite
 *   N <= 16384 (BATQ_ERR_UNSUPPORTED beyond).  Does not allocate or synchronise.
 */
batq_status batq_quantize_act_rmsnorm(const uint16_t* x, int64_t S, int64_t N, int64_t ldx,
                                      const float* gamma, float eps,
                                      const float* A, const float* B,
                                      const float* r_min, const float* r_max,
                                      uint8_t* q, uint8_t* e, batq_scale_layout e_layout,
                                      void* stream);

/* Element format of a quantised KV cache (W4A8KV4 / W4A8KV8 settings). */
typedef enum batq_kv_format {
    BATQ_KV_MXFP4 = 4,   /* E2M1 codes, two per byte, low nibble first: [rows][N/2] */
    BATQ_KV_MXFP8 = 8,   /* E4M3 codes, one per byte: [rows][N] */
} batq_kv_format;

/*
 * KV cache write: the quantised keys or values of T new tokens stored into a cache of
 * num_slots rows through a slot map.  The pages run the method on attention blocks with
 * their KV caches (gist.science summary, section 2D) and report 8- and 4-bit caches
 * (thelatestinai listing, captions of Tables 2, 3 and 5: W4A8KV8, W4A8KV4); the cache
 * rows go through the same block transform, block clip and MX encoding as activations
 * (plain reading: each K/V row, N = kv heads x head dim, is one activation row), so k P
 * and q P^-T keep the attention scores q k^T.
 *   x       dev  bf16 [T, ldx], rows of N = 32k values (16-byte aligned, ldx % 8 == 0)
 *   slots   dev  int64 [T]: cache row of token t; a value < 0 or >= num_slots skips the
 *                token (the cache row is left as it was)
 *   fmt     BATQ_KV_MXFP4 or BATQ_KV_MXFP8 (element codes as batq_quantize_act or
 *           batq_quantize_act_mxfp8)
 *   A, B, r_min, r_max  dev, as batq_quantize_act
 *   cache_q dev  [num_slots][N/2] (MXFP4) or [num_slots][N] (MXFP8) bytes, 16-byte aligned
 *   cache_e dev  [num_slots][N/32] E8M0 scales, row-major
 * Two tokens mapped to one slot race (either may win).  Does not allocate or synchronise.
 */
batq_status batq_quantize_kv(const uint16_t* x, int64_t T, int64_t N, int64_t ldx,
                             const int64_t* slots, int64_t num_slots, batq_kv_format fmt,
                             const float* A, const float* B, const float* r_min,
                             const float* r_max, uint8_t* cache_q, uint8_t* cache_e,
                             void* stream);

/*
 * The block transform alone, y_i = B_i^T X_i A on each 32-block (same arithmetic as the
 * transform inside batq_quantize_act), for the unquantised side of attention with a
 * transformed cache: queries take the factors of P^-T (batq_weight_factors of the kv head
 * they attend to), attention outputs over transformed values take those of P^-1 (the
 * transposed A^-1, B_i^-1) (gist.science summary, section 2B and 2D).
 *   x       dev  [rows, ldx] of x_type (BATQ_OUT_F32 or BATQ_OUT_BF16 names the element type;
 *                16-byte aligned; ldx % 4 == 0 for fp32, % 8 for bf16)
 *   A, B    dev  fp32 [8][8] and [N/32][4][4] (B 16-byte aligned)
 *   y       dev  [rows, N] dense of y_type; bf16 output is rounded to nearest, ties to even
 * Does not allocate or synchronise.
 */
batq_status batq_transform_rows(const void* x, batq_out_type x_type, int64_t rows, int64_t N,
                                int64_t ldx, const float* A, const float* B, void* y,
                                batq_out_type y_type, void* stream);

/*
 * MX rows back to numbers: y[r][j] = code value * 2^(e - 127) (exact in fp32; bf16 output
 * rounded to nearest, ties to even), reading cache rows selected by an optional index (the
 * slots of a sequence).  OCP MX element decoding (gist.science summary, section 1; the
 * element values of E2M1 and E4M3); NaN encodings (scale 0xFF, E4M3 S.1111.111) give NaN.
 *   q, e     dev  cache as written by batq_quantize_kv ([src_rows] rows; q 16-byte aligned)
 *   index    dev  int64 [rows] or NULL (then rows <= src_rows and row r reads row r); an
 *                 entry outside [0, src_rows) gives a zero row
 *   y        dev  [rows, N] dense of y_type, 16-byte aligned
 * Does not allocate or synchronise.
 */
batq_status batq_dequantize_rows(const uint8_t* q, const uint8_t* e, int64_t src_rows, int64_t N,
                                 batq_kv_format fmt, const int64_t* index, int64_t rows,
                                 void* y, batq_out_type y_type, void* stream);

/* Token count up to which batq_linear_w4a4 runs in one kernel. */
#define BATQ_LINEAR_FUSED_TOKENS 4

/*
 * The online linear layer in one call: y = the W4A4 product of batq_quantize_act(x) with
 * the prepared weights (gist.science summary, sections 2D and 4: activations transformed
 * and clipped online, MXFP4 x MXFP4 product).  For 1 <= S <= BATQ_LINEAR_FUSED_TOKENS (and
 * N/32 <= 512, N/32 % 8 == 0) one kernel can do it: the few-token GEMM encodes the token
 * rows itself, with the quantiser's arithmetic, so the codes are exactly
 * batq_quantize_act's and y agrees with the two-call path within the GEMM's accumulation
 * bound (its K split, and so its fp32 summation order, differs).  In that range xq / xe may
 * be NULL, and the one kernel runs.  When they are given, the library runs whichever of the
 * two paths is faster for the shape (measured: the one kernel while S <= 16,
 * S * N/32 <= 1536 and S * N/32 * ceil(out / 16) <= 196608, the token blocks all its
 * workgroups encode), also for 4 < S <= 16.
 * Otherwise the two calls run, with xq / xe as the caller's workspace for the activation
 * codes and scales (sized as batq_quantize_act's q and e in `layout`).  Either path gives
 * the same result for the same inputs on every call.
 *   x, S, N, ldx, A, B, r_min, r_max: as batq_quantize_act
 *   wq, we, layout, out, y: as batq_gemm_w4a4 (y dev fp32 [S, out], 16-byte aligned)
 *   xq, xe: dev workspace or NULL (see above; BATQ_ERR_NULL when needed and missing,
 *           BATQ_ERR_UNSUPPORTED when the one-kernel path declines aligned-scale or size
 *           limits and no workspace is given)
 * Does not allocate or synchronise.
 */
batq_status batq_linear_w4a4(const uint16_t* x, int64_t S, int64_t N, int64_t ldx,
                             const float* A, const float* B, const float* r_min,
                             const float* r_max, const uint8_t* wq, const uint8_t* we,
                             batq_scale_layout layout, int64_t out, float* y, uint8_t* xq,
                             uint8_t* xe, void* stream);

/* Bytes of batq_linear_w4a4_noalloc's device scratch (activation codes and scales). */
#define BATQ_NOALLOC_SCRATCH_BYTES (64LL << 20)

/*
 * batq_linear_w4a4 for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same layer and the same
 * kernels as batq_linear_w4a4 given a workspace (the result is identical), with the
 * activation codes and scales kept in a fixed device array of BATQ_NOALLOC_SCRATCH_BYTES
 * that the library owns: every GPU it runs on holds one until the process ends, and every
 * call on that GPU shares it (and leaves its contents behind).
 *   arguments: as batq_linear_w4a4 without xq / xe; `stream` must belong to the current
 *              device
 *   Needs round_up(S * N/2, 256) + the scale bytes of S x N in `layout` <= the scratch size,
 *   else BATQ_ERR_TOO_LARGE (checked before any HIP call; e.g. S = 16384 fits up to
 *   N = 7680 in the MFMA-tiled layout, S = 2048 up to N = 61440).  The first call on a device looks up the device
 *   address of its scratch (a HIP call, no allocation).
 * Calls that overlap on one GPU (other streams, other threads) race on the scratch: order
 * them.  Does not allocate or synchronise.
 */
batq_status batq_linear_w4a4_noalloc(const uint16_t* x, int64_t S, int64_t N, int64_t ldx,
                                     const float* A, const float* B, const float* r_min,
                                     const float* r_max, const uint8_t* wq, const uint8_t* we,
                                     batq_scale_layout layout, int64_t out, float* y,
                                     void* stream);

/* Largest S * N/32 the one-kernel W4A8 layer takes (its MXFP8 token codes live in LDS). */
#define BATQ_LINEAR_W4A8_FUSED_BLOCKS 768

/*
 * The W4A8 linear layer in one call: y = the W4A8 product of batq_quantize_act_mxfp8(x)
 * with the prepared MXFP4 weights (gist.science summary, section 4: the W4A8KV16 setting,
 * activations transformed and clipped online as in W4A4, then MXFP8).  For
 * 1 <= S <= BATQ_LINEAR_FUSED_TOKENS with S * N/32 <= BATQ_LINEAR_W4A8_FUSED_BLOCKS (and
 * N/32 % 8 == 0) one kernel can do it: the few-token W4A8 GEMM encodes the token rows to
 * MXFP8 itself with the quantiser's arithmetic, so the codes are exactly
 * batq_quantize_act_mxfp8's and y has batq_gemm_w4a8's accuracy.  In that range the one
 * kernel runs and xq8 / xe are not used (it measured faster than the two calls on every
 * shape it takes; they may be NULL).  Otherwise batq_quantize_act_mxfp8 then
 * batq_gemm_w4a8 run, with xq8 (dev u8 [S, N]) / xe (sized as that call's e in `layout`) as
 * the caller's workspace.  The same inputs give the same result on every call.
 *   x, S, N, ldx, A, B, r_min, r_max: as batq_quantize_act_mxfp8
 *   wq, we, layout, out, y: as batq_gemm_w4a8 (N % 256 == 0, else BATQ_ERR_UNSUPPORTED;
 *           y dev fp32 [S, out], 16-byte aligned)
 *   xq8, xe: dev workspace or NULL (BATQ_ERR_NULL when needed and missing,
 *           BATQ_ERR_UNSUPPORTED when the one-kernel path declines aligned-scale or size
 *           limits and no workspace is given)
 * Does not allocate or synchronise.
 */
batq_status batq_linear_w4a8(const uint16_t* x, int64_t S, int64_t N, int64_t ldx,
                             const float* A, const float* B, const float* r_min,
                             const float* r_max, const uint8_t* wq, const uint8_t* we,
                             batq_scale_layout layout, int64_t out, float* y, uint8_t* xq8,
                             uint8_t* xe, void* stream);

/*
 * Host: clip ratios r[i] = fp32(1 / (1 + exp(-alpha[i]))) evaluated in binary64 and rounded
 * once (daily-arxiv summary, clipping bullet: the sigmoid keeps each ratio in (0, 1);
 * gist.science summary, section 2C).  The logits are per block, shared by all tokens.
 *   alpha host fp32 [k];  ratio host fp32 [k] (out);  k >= 0.
 */
batq_status batq_clip_ratios(const float* alpha, int64_t k, float* ratio);

/*
 * Host: the fp32 factors of the offline weight transform, A' = (A^-1)^T and
 * B'_i = (B_i^-1)^T, each entry the fp32 value nearest to the exact inverse (computed with
 * 64-bit-mantissa Gauss-Jordan elimination with partial pivoting).  Since
 * (B_i (x) A)^-1 = B_i^-1 (x) A^-1, these realise P^-T block by block (gist.science
 * summary, section 2B and 2D).
 *   A host fp32 [8][8];  B host fp32 [k][4][4];  k >= 0
 *   A_inv_t host out fp32 [8][8];  B_inv_t host out fp32 [k][4][4]
 * Returns BATQ_ERR_SINGULAR if a factor is not invertible.
 */
batq_status batq_weight_factors(const float* A, const float* B, int64_t k,
                                float* A_inv_t, float* B_inv_t);

/* Human-readable name of a status code (static storage). */
const char* batq_status_string(batq_status status);

#ifdef __cplusplus
}
#endif

#endif /* BATQ_H */
