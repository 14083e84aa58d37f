// Block arithmetic of the BATQuant quantisers (gfx950), shared by the quantiser kernels and
// the GEMM that encodes its few token rows itself: the block transform (GPK
// Y = B_i^T (X A), or a full 32x32 P_i), the block clip and the MX encode.  The arithmetic
// contract is the quantisers' (quantize.hip's header): every sum a product followed by
// fused multiply-adds in increasing index order, clip min(max(y, lo), hi) with the upper
// bound winning, scale byte max(E(amax) - 2, 0) (MXFP4) or max(E(amax) - 8, 0) (MXFP8),
// conversion by the scaled convert instructions, which round once to nearest-even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace batq {
namespace mx {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Y = B^T (X A) for one block held in registers, X[r][c] = x[8r + c].  Z = X A is formed a
// row at a time and each row s is folded into every row of Y at once, so only one row of Z
// is live; every sum keeps its order (a product, then fused multiply-adds in increasing
// index order: z[s][c] over the 8 terms of A's column, y[r][c] over s = 0..3).
__device__ __forceinline__ void gpk_transform(const float (&x)[32], const float* __restrict__ A,
                                              const float4 (&b)[4], float (&y)[32])
{
    const float bm[4][4] = {{b[0].x, b[0].y, b[0].z, b[0].w},
                            {b[1].x, b[1].y, b[1].z, b[1].w},
                            {b[2].x, b[2].y, b[2].z, b[2].w},
                            {b[3].x, b[3].y, b[3].z, b[3].w}};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        float zs[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float acc = x[8 * s] * A[c];
#pragma unroll
            for (int qi = 1; qi < 8; ++qi) acc = __builtin_fmaf(x[8 * s + qi], A[8 * qi + c], acc);
            zs[c] = acc;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
                y[8 * r + c] = s == 0 ? bm[0][r] * zs[c]
                                      : __builtin_fmaf(bm[s][r], zs[c], y[8 * r + c]);
        }
    }
}

// y = x P for one block with a full 32x32 P (y_j = sum_m x_m P[m][j]): a product for m = 0,
// then one fused multiply-add per m in increasing m (thelatestinai listing, Table 1, the
// "w/o decomposition" form).  The rows of P stream in as 16-byte loads; every row of the
// activations reads the same P_i, so they come from cache.
__device__ __forceinline__ void full_transform(const float (&x)[32], const float* __restrict__ P,
                                               float (&y)[32])
{
    const float4* pr = reinterpret_cast<const float4*>(P);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const float4 v = pr[t];
        y[4 * t] = x[0] * v.x;
        y[4 * t + 1] = x[0] * v.y;
        y[4 * t + 2] = x[0] * v.z;
        y[4 * t + 3] = x[0] * v.w;
    }
#pragma unroll 4
    for (int m = 1; m < 32; ++m) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float4 v = pr[8 * m + t];
            y[4 * t] = __builtin_fmaf(x[m], v.x, y[4 * t]);
            y[4 * t + 1] = __builtin_fmaf(x[m], v.y, y[4 * t + 1]);
            y[4 * t + 2] = __builtin_fmaf(x[m], v.z, y[4 * t + 2]);
            y[4 * t + 3] = __builtin_fmaf(x[m], v.w, y[4 * t + 3]);
        }
    }
}

// The per-block parameters a lane needs besides A: B_i (GPK and Kronecker forms) and the
// two clip ratios (activations).
struct BlockParams {
    float4 b[4];
    float rmin, rmax;
};

template <bool kAct, int kForm>
__device__ __forceinline__ BlockParams load_block_params(const float* __restrict__ B,
                                                         const float* __restrict__ r_min,
                                                         const float* __restrict__ r_max,
                                                         int64_t blk)
{
    BlockParams p;
    if constexpr (kForm != 2) {
        const float4* bp = reinterpret_cast<const float4*>(B + 16 * blk);
#pragma unroll
        for (int t = 0; t < 4; ++t) p.b[t] = bp[t];
    }
    if constexpr (kAct) {
        p.rmin = r_min[blk];
        p.rmax = r_max[blk];
    }
    return p;
}

// The encoded block: E2M1 codes (4 words, element 2j in the low nibble of byte j) or E4M3
// codes (8 words, element j in byte j), and the E8M0 scale byte.
template <bool kFp8>
struct BlockCode {
    uint32_t w[kFp8 ? 8 : 4];
    uint32_t ebyte;
};

// Transform, clip and encode one block held in registers (block index blk of its row).
template <bool kAct, bool kFp8, int kForm>
__device__ __forceinline__ BlockCode<kFp8> encode_block(float (&x)[32], const float* __restrict__ A,
                                                        const BlockParams& p, int64_t blk)
{
    BlockCode<kFp8> c;
    float y[32];
    if constexpr (kForm == 2) {
        full_transform(x, A + 1024 * blk, y);
    } else {
        gpk_transform(x, kForm == 1 ? A + 64 * blk : A, p.b, y);
    }

    float amax;
    float lo = 0.0f, hi = 0.0f;
    if constexpr (kAct) {
        float m = y[0], M = y[0];
#pragma unroll
        for (int j = 1; j < 32; ++j) {
            m = __builtin_fminf(m, y[j]);
            M = __builtin_fmaxf(M, y[j]);
        }
        hi = p.rmax * M;
        lo = __builtin_fminf(p.rmin * m, hi);        // lo > hi: every value -> hi
        amax = __builtin_fmaxf(__builtin_fabsf(__builtin_amdgcn_fmed3f(m, lo, hi)),
                               __builtin_fabsf(__builtin_amdgcn_fmed3f(M, lo, hi)));
    } else {
        amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(y[j]));
    }
    const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFF) - (kFp8 ? 8 : 2);
    c.ebyte = ex > 0 ? (uint32_t)ex : 0u;
    const float scale = __uint_as_float(c.ebyte << 23);

    if constexpr (kFp8) {
        // 448 * 2^(e - 127) = 1.75 * 2^(e - 119): fp32 exponent field e + 8, mantissa 0.75
        const float sat = __uint_as_float(((c.ebyte + 8u) << 23) | 0x00600000u);
        const float L = __builtin_amdgcn_fmed3f(lo, -sat, sat);
        const float H = __builtin_amdgcn_fmed3f(hi, -sat, sat);
        typedef short v2i16 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            v2i16 acc = {0, 0};
            acc = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(
                acc, __builtin_amdgcn_fmed3f(y[4 * d + 0], L, H),
                __builtin_amdgcn_fmed3f(y[4 * d + 1], L, H), scale, false);
            acc = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(
                acc, __builtin_amdgcn_fmed3f(y[4 * d + 2], L, H),
                __builtin_amdgcn_fmed3f(y[4 * d + 3], L, H), scale, true);
            c.w[d] = (uint32_t)(uint16_t)acc[0] | ((uint32_t)(uint16_t)acc[1] << 16);
        }
    } else {
        if constexpr (kAct) {
#pragma unroll
            for (int j = 0; j < 32; ++j) y[j] = __builtin_amdgcn_fmed3f(y[j], lo, hi);
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t acc = 0;
            acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, y[8 * d + 0], y[8 * d + 1], scale, 0);
            acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, y[8 * d + 2], y[8 * d + 3], scale, 1);
            acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, y[8 * d + 4], y[8 * d + 5], scale, 2);
            acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, y[8 * d + 6], y[8 * d + 7], scale, 3);
            c.w[d] = acc;
        }
    }
    return c;
}

}  // namespace mx
}  // namespace batq
