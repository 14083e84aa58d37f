// Fused BATQuant block transform + block-wise clipping + MXFP4 quantisation (gfx950).
//
// One thread owns one 32-element block of one row (one MXFP4 block): it reads the block
// (64 B of bf16, or 128 B of fp32 on the weight side), applies Y = B_i^T (X A) on the
// row-major 4x8 view X of the block (GPK factorisation P_i = B_i (x) A, gist.science
// summary section 2B; thelatestinai listing Table 1: 12 multiply-adds per element instead
// of 32 for a full 32x32 P_i), clips the block to [r_min m, r_max M] (daily-arxiv summary,
// clipping bullet; gist.science section 2C), picks the E8M0 scale from the largest clipped
// magnitude and writes 16 bytes of E2M1 codes plus one scale byte (values divided by the
// scale before rounding: thelatestinai listing, Figure 2 caption).
//
// Layout on the chip: lanes of a wave take consecutive blocks of one row, so a wave reads
// one contiguous 4 KB span of a row and writes one contiguous 1 KB span of codes and 64
// scale bytes; when a row has fewer than 64 blocks a wave covers several whole rows.  A
// (64 floats, the same for every block) is read through the scalar unit into SGPRs and is
// a direct operand of every first-stage multiply-add; B_i and the clip ratios are per-lane
// vector loads that hit in cache (they are 64 B + 8 B per block column for all rows).
//
// Arithmetic contract (must match the plain oracle bit for bit): fp32, each sum a product
// followed by fused multiply-adds in increasing index order, first Z = X A over the
// contiguous 8-index, then Y = B^T Z over the 4-index; clipping min(max(y, lo), hi) with
// lo = r_min * min(y), hi = r_max * max(y) (the upper bound wins when lo > hi); scale byte
// max(E(amax) - 2, 0) with E the fp32 exponent field; E2M1 by v_cvt_scalef32_pk_fp4_f32,
// whose scale operand contributes only its exponent field, so passing e << 23 divides by
// 2^(e-127) exactly and rounds once to nearest-even with saturation at 6.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "mx_block.h"

namespace batq {
namespace {

using namespace mx;

constexpr int kWavesPerGroup = 4;
constexpr int kThreads = 64 * kWavesPerGroup;

// A (8x8, wave-uniform) as four 16-dword scalar loads, taken whole by an empty asm so that
// none of them is left until after the vector loads have completed.
__device__ __forceinline__ void pin_uniform_a(const float* __restrict__ A)
{
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    const f32x16* a = reinterpret_cast<const f32x16*>(A);
    asm volatile("" ::"s"(a[0]), "s"(a[1]), "s"(a[2]), "s"(a[3]));
}

// An empty asm that takes one value of each of the block's loads (A, B_i, the ratios when
// kRatios, and each 16-byte piece of x): every one of them is issued before this point, so
// the lane waits for one round trip instead of a chain (the compiler otherwise issues some
// loads after the arithmetic that precedes their use, and waits for them there).
template <bool kBf16, bool kRatios>
__device__ __forceinline__ void issue_together(const float* __restrict__ A, const BlockParams& p,
                                               const float (&x)[32])
{
    pin_uniform_a(A);
    // x: one value of each 16-byte load (4 for bf16 rows, 8 for fp32 rows)
    if constexpr (kBf16 && kRatios)
        asm volatile("" ::"v"(p.b[0].x), "v"(p.b[1].x), "v"(p.b[2].x), "v"(p.b[3].x),
                     "v"(p.rmin), "v"(p.rmax), "v"(x[0]), "v"(x[8]), "v"(x[16]), "v"(x[24]));
    else if constexpr (kBf16)
        asm volatile("" ::"v"(p.b[0].x), "v"(p.b[1].x), "v"(p.b[2].x), "v"(p.b[3].x),
                     "v"(x[0]), "v"(x[8]), "v"(x[16]), "v"(x[24]));
    else
        asm volatile("" ::"v"(p.b[0].x), "v"(p.b[1].x), "v"(p.b[2].x), "v"(p.b[3].x),
                     "v"(x[0]), "v"(x[4]), "v"(x[8]), "v"(x[12]), "v"(x[16]), "v"(x[20]),
                     "v"(x[24]), "v"(x[28]));
}

// Transform, clip, encode and store one block held in registers (row, blk), shared by the
// quantisers; the parameters come preloaded.
template <bool kAct, bool kFp8, int kForm>
__device__ __forceinline__ void quantize_block(float (&x)[32], const float* __restrict__ A,
                                               const BlockParams& p,
                                               uint8_t* __restrict__ q, uint8_t* __restrict__ e,
                                               int64_t row, int64_t blk, int64_t k,
                                               int tiled_scales, bool store = true)
{
    const BlockCode<kFp8> c = encode_block<kAct, kFp8, kForm>(x, A, p, blk);
    if (store) {
        if constexpr (kFp8) {
            uint4* qp = reinterpret_cast<uint4*>(q + row * (32 * k) + 32 * blk);
            qp[0] = make_uint4(c.w[0], c.w[1], c.w[2], c.w[3]);
            qp[1] = make_uint4(c.w[4], c.w[5], c.w[6], c.w[7]);
        } else {
            *reinterpret_cast<uint4*>(q + row * (16 * k) + 16 * blk) =
                make_uint4(c.w[0], c.w[1], c.w[2], c.w[3]);
        }
    }
    // scale byte: row-major, or the 256-byte (32 rows x 8 blocks) units the GEMM consumes,
    // blocks of a unit ordered 0,2,4,6,1,3,5,7 within each row's 8 bytes
    const int64_t eoff = tiled_scales
        ? (((row >> 5) * ((k + 7) >> 3) + (blk >> 3)) << 8) + ((row & 31) << 3) +
              ((blk & 1) << 2) + ((blk & 7) >> 1)
        : row * k + blk;
    if (store) e[eoff] = (uint8_t)c.ebyte;
}

// The same with the parameters loaded here.
template <bool kAct, bool kFp8, int kForm>
__device__ __forceinline__ void quantize_block(float (&x)[32], const float* __restrict__ A,
                                               const float* __restrict__ B,
                                               const float* __restrict__ r_min,
                                               const float* __restrict__ r_max,
                                               uint8_t* __restrict__ q, uint8_t* __restrict__ e,
                                               int64_t row, int64_t blk, int64_t k,
                                               int tiled_scales)
{
    const BlockParams p = load_block_params<kAct, kForm>(B, r_min, r_max, blk);
    quantize_block<kAct, kFp8, kForm>(x, A, p, q, e, row, blk, k, tiled_scales);
}

// kForm selects the transform (thelatestinai listing, Table 1): 0 GPK, A [8][8] shared by
// every block (read through the scalar unit); 1 naive Kronecker, a private A_i [8][8] per
// block, same reshape evaluation; 2 a full 32x32 P_i per block (A points at P [k][32][32],
// B is unused).  For forms 1 and 2 a workgroup owns one block column (blockIdx.x) and its
// threads take consecutive rows, so A_i / P_i (and B_i) are uniform across the wave and
// come through the scalar unit as FMA operands, like GPK's A.
// kFp8 (activations only): MXFP8 output, one E4M3 code byte per element (the W4A8
// setting).  Same transform and clip; the scale exponent is floor(log2 amax) - 8 (E4M3's
// largest exponent), and the conversion instruction, exact round-to-nearest-even otherwise,
// returns NaN above 448 where MX saturates, so the clip bounds are first clamped into
// [-448 s, 448 s] (a clamp of a clamp is the clamp to the clamped bounds).
// One block of x (bf16 activations or fp32 weights) into fp32 registers.
template <bool kAct>
__device__ __forceinline__ void load_block(const void* __restrict__ xin, int64_t row, int64_t ldx,
                                           int64_t blk, float (&x)[32])
{
    if constexpr (kAct) {
        const uint4* xp = reinterpret_cast<const uint4*>(
            static_cast<const uint16_t*>(xin) + row * ldx + 32 * blk);
        uint4 v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = xp[t];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t w[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                x[8 * t + 2 * d] = bf16_lo(w[d]);
                x[8 * t + 2 * d + 1] = bf16_hi(w[d]);
            }
        }
    } else {
        const float4* xp = reinterpret_cast<const float4*>(
            static_cast<const float*>(xin) + row * ldx + 32 * blk);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float4 v = xp[t];
            x[4 * t] = v.x;
            x[4 * t + 1] = v.y;
            x[4 * t + 2] = v.z;
            x[4 * t + 3] = v.w;
        }
    }
}

template <bool kAct, bool kFp8 = false, int kForm = 0>
__global__ void __launch_bounds__(kThreads)
quantize_kernel(const void* __restrict__ xin, int64_t rows, int64_t k, int64_t ldx,
                const float* __restrict__ A, const float* __restrict__ B,
                const float* __restrict__ r_min, const float* __restrict__ r_max,
                uint8_t* __restrict__ q, uint8_t* __restrict__ e, int lpr_log2,
                int tiled_scales)
{
    static_assert(kAct || !kFp8, "MXFP8 is an activation-side format");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int64_t row, blk;
    if constexpr (kForm != 0) {
        blk = blockIdx.x;
        row = (int64_t)blockIdx.y * kThreads + threadIdx.x;
    } else {
        row = ((((int64_t)blockIdx.x * kWavesPerGroup + wave) << (6 - lpr_log2)) +
               (lane >> lpr_log2));
        blk = (int64_t)blockIdx.y * 64 + (lane & ((1 << lpr_log2) - 1));
    }
    if (row >= rows || blk >= k) return;

    const BlockParams p = load_block_params<kAct, kForm>(B, r_min, r_max, blk);
    float x[32];
    load_block<kAct>(xin, row, ldx, blk, x);
    if constexpr (kForm == 0) issue_together<kAct, kAct>(A, p, x);
    quantize_block<kAct, kFp8, kForm>(x, A, p, q, e, row, blk, k, tiled_scales);
}

// ---------------------------------------------------------------------------------------
// RMSNorm fused in front of the activation quantiser
// ---------------------------------------------------------------------------------------
//
// TPR threads per row (64, 128 or 256: the padded block count clamped to that range), one
// or two blocks per thread held in registers from load to store, 256 / TPR rows per
// workgroup.  Arithmetic contract (as the oracle's orc_rmsnorm_f32): block sums of squares
// x_0^2 then fmaf in increasing j; the block sums, zero-padded to K = the next power of two
// >= k, added by halving (t[b] += t[b + h], h = K/2 .. 1); r = 1 / sqrt(T / N + eps) with
// correctly rounded division and square root; x_hat = (x r) gamma, two roundings; then the
// GPK transform, clip and MXFP4 of quantize_block.  Thread i of a row holds blocks i and
// i + TPR: the step h = TPR (K = 2 TPR) is inside the thread, the steps with 64 <= h < TPR
// cross waves through LDS, those with h < 64 cross lanes inside the wave; fp32 addition is
// commutative, so the operand order of each step does not change its result.
constexpr int kRmsThreads = 256;

__device__ __forceinline__ void load_bf16_block(const uint16_t* __restrict__ src, float (&x)[32])
{
    const uint4* xp = reinterpret_cast<const uint4*>(src);
    uint4 v[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = xp[t];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t w[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            x[8 * t + 2 * d] = bf16_lo(w[d]);
            x[8 * t + 2 * d + 1] = bf16_hi(w[d]);
        }
    }
}

__device__ __forceinline__ float block_sum_squares(const float (&x)[32])
{
    float acc = x[0] * x[0];
#pragma unroll
    for (int j = 1; j < 32; ++j) acc = __builtin_fmaf(x[j], x[j], acc);
    return acc;
}

__device__ __forceinline__ void rms_scale(float (&x)[32], const float* __restrict__ g, float r)
{
    const float4* gp = reinterpret_cast<const float4*>(g);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const float4 v = gp[t];
        x[4 * t] = (x[4 * t] * r) * v.x;
        x[4 * t + 1] = (x[4 * t + 1] * r) * v.y;
        x[4 * t + 2] = (x[4 * t + 2] * r) * v.z;
        x[4 * t + 3] = (x[4 * t + 3] * r) * v.w;
    }
}

template <int TPR>
__global__ void __launch_bounds__(kRmsThreads)
rmsnorm_quantize_kernel(const uint16_t* __restrict__ xin, int64_t rows, int64_t k, int64_t ldx,
                        const float* __restrict__ gamma, float eps,
                        const float* __restrict__ A, const float* __restrict__ B,
                        const float* __restrict__ r_min, const float* __restrict__ r_max,
                        uint8_t* __restrict__ q, uint8_t* __restrict__ e, int kpow2,
                        int tiled_scales)
{
    constexpr int kRows = kRmsThreads / TPR;
    __shared__ float part[kRmsThreads];
    __shared__ float total[kRows];
    const int tid = threadIdx.x, lane = tid & 63;
    const int rt = tid % TPR, rl = tid / TPR;
    const int64_t row = (int64_t)blockIdx.x * kRows + rl;
    const bool live = row < rows;                    // dead rows still take every barrier
    const uint16_t* xr = xin + row * ldx;
    const int64_t b0 = rt, b1 = rt + TPR;
    const bool has0 = live && b0 < k, has1 = live && b1 < k;
    float x0[32], x1[32];
    float s0 = 0.0f, s1 = 0.0f;
    if (has0) {
        load_bf16_block(xr + 32 * b0, x0);
        s0 = block_sum_squares(x0);
    }
    if (has1) {
        load_bf16_block(xr + 32 * b1, x1);
        s1 = block_sum_squares(x1);
    }
    float v = kpow2 > TPR ? s0 + s1 : s0;            // step h = TPR
    for (int h = (kpow2 < TPR ? kpow2 : TPR) / 2; h >= 64; h /= 2) {
        part[tid] = v;
        __syncthreads();
        if (rt < h) v = v + part[tid + h];
        __syncthreads();
    }
    for (int h = (kpow2 < 64 ? kpow2 : 64) / 2; h >= 1; h /= 2) {
        const float o = __shfl_down(v, h, 64);
        if (lane < h) v = v + o;
    }
    if (rt == 0) total[rl] = v;
    __syncthreads();
    const float T = total[rl];
    const float mean = T / (float)(32 * k);
    const float r = 1.0f / __builtin_sqrtf(mean + eps);
    if (has0) {
        rms_scale(x0, gamma + 32 * b0, r);
        quantize_block<true, false, 0>(x0, A, B, r_min, r_max, q, e, row, b0, k, tiled_scales);
    }
    if (has1) {
        rms_scale(x1, gamma + 32 * b1, r);
        quantize_block<true, false, 0>(x1, A, B, r_min, r_max, q, e, row, b1, k, tiled_scales);
    }
}

// ---------------------------------------------------------------------------------------
// KV caches (W4A8KV8 / W4A8KV4) and the transform of rows without quantisation
// ---------------------------------------------------------------------------------------

// The activation quantiser's mapping (lanes take consecutive blocks of a row), each row
// written to cache row slots[row]; negative slots and slots >= num_slots are skipped.
template <bool kFp8>
__global__ void __launch_bounds__(kThreads)
quantize_kv_kernel(const uint16_t* __restrict__ xin, int64_t rows, int64_t k, int64_t ldx,
                   const int64_t* __restrict__ slots, int64_t num_slots,
                   const float* __restrict__ A, const float* __restrict__ B,
                   const float* __restrict__ r_min, const float* __restrict__ r_max,
                   uint8_t* __restrict__ q, uint8_t* __restrict__ e, int lpr_log2)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t row = ((((int64_t)blockIdx.x * kWavesPerGroup + wave) << (6 - lpr_log2)) +
                         (lane >> lpr_log2));
    const int64_t blk = (int64_t)blockIdx.y * 64 + (lane & ((1 << lpr_log2) - 1));
    if (row >= rows || blk >= k) return;
    // the row is in bounds whatever its slot: it is loaded and encoded unconditionally (so
    // its loads go out together with the slot's), and only the stores depend on the slot
    const BlockParams p = load_block_params<true, 0>(B, r_min, r_max, blk);
    const int64_t slot = slots[row];
    float x[32];
    load_bf16_block(xin + row * ldx + 32 * blk, x);
    // as issue_together, with the slot's load among them (instead of the row's loads
    // waiting behind its test)
    pin_uniform_a(A);
    asm volatile("" ::"v"(slot), "v"(p.b[0].x), "v"(p.b[1].x), "v"(p.b[2].x), "v"(p.b[3].x),
                 "v"(p.rmin), "v"(p.rmax), "v"(x[0]), "v"(x[8]), "v"(x[16]), "v"(x[24]));
    const bool keep = slot >= 0 && slot < num_slots;
    quantize_block<true, kFp8, 0>(x, A, p, q, e, keep ? slot : 0, blk, k, 0, keep);
}

// y = GPK transform of x with the given factors (P for K/V rows, the transposed inverses for
// queries, the inverses for attention outputs), one lane per (row, block).
template <bool kInBf16, bool kOutBf16>
__global__ void __launch_bounds__(kThreads)
transform_rows_kernel(const void* __restrict__ xin, int64_t rows, int64_t k, int64_t ldx,
                      const float* __restrict__ A, const float* __restrict__ B,
                      void* __restrict__ yout, int lpr_log2)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t row = ((((int64_t)blockIdx.x * kWavesPerGroup + wave) << (6 - lpr_log2)) +
                         (lane >> lpr_log2));
    const int64_t blk = (int64_t)blockIdx.y * 64 + (lane & ((1 << lpr_log2) - 1));
    if (row >= rows || blk >= k) return;
    const BlockParams p = load_block_params<false, 0>(B, nullptr, nullptr, blk);
    float x[32];
    load_block<kInBf16>(xin, row, ldx, blk, x);
    issue_together<kInBf16, false>(A, p, x);    // every load issued before the first use
    float y[32];
    gpk_transform(x, A, p.b, y);
    const int64_t off = row * 32 * k + 32 * blk;
    if constexpr (kOutBf16) {
        uint4* yp = reinterpret_cast<uint4*>(static_cast<uint16_t*>(yout) + off);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint32_t w[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t u0 = __float_as_uint(y[8 * t + 2 * d]);
                const uint32_t u1 = __float_as_uint(y[8 * t + 2 * d + 1]);
                w[d] = ((u0 + 0x7FFFu + ((u0 >> 16) & 1u)) >> 16) |
                       (((u1 + 0x7FFFu + ((u1 >> 16) & 1u)) >> 16) << 16);
            }
            yp[t] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else {
        float4* yp = reinterpret_cast<float4*>(static_cast<float*>(yout) + off);
#pragma unroll
        for (int t = 0; t < 8; ++t)
            yp[t] = make_float4(y[4 * t], y[4 * t + 1], y[4 * t + 2], y[4 * t + 3]);
    }
}

// Dequantise MX rows (MXFP4 codes [., N/2] or MXFP8 codes [., N], scales [., N/32]
// row-major): output row r is source row index[r] (or r without an index); an index outside
// [0, src_rows) gives a zero row.  Values are code value * 2^(e - 127), exact in fp32 (bf16
// output: rounded to nearest even).
template <bool kFp8, bool kOutBf16>
__global__ void __launch_bounds__(kThreads)
dequantize_rows_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ e,
                       int64_t rows, int64_t k, const int64_t* __restrict__ index,
                       int64_t src_rows, void* __restrict__ yout, int lpr_log2)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t row = ((((int64_t)blockIdx.x * kWavesPerGroup + wave) << (6 - lpr_log2)) +
                         (lane >> lpr_log2));
    const int64_t blk = (int64_t)blockIdx.y * 64 + (lane & ((1 << lpr_log2) - 1));
    if (row >= rows || blk >= k) return;
    const int64_t src = index ? index[row] : row;
    float v[32];
    if (src < 0 || src >= src_rows) {
#pragma unroll
        for (int j = 0; j < 32; ++j) v[j] = 0.0f;
    } else {
        // the scale byte and the codes are loaded together
        const uint32_t eb = e[src * k + blk];
        uint4 c0, c1;
        if constexpr (kFp8) {
            const uint4* qp = reinterpret_cast<const uint4*>(q + src * 32 * k + 32 * blk);
            c0 = qp[0];
            c1 = qp[1];
            asm volatile("" ::"v"(eb), "v"(c0.x), "v"(c1.x));
        } else {
            c0 = *reinterpret_cast<const uint4*>(q + src * 16 * k + 16 * blk);
            c1 = c0;
            asm volatile("" ::"v"(eb), "v"(c0.x));
        }
        // 2^(eb - 127): the exponent field itself, the subnormal 2^-127 for eb = 0, NaN for
        // the E8M0 NaN byte 0xFF
        const float s = eb == 255u ? __uint_as_float(0x7FC00000u)
                        : eb       ? __uint_as_float(eb << 23)
                                   : __uint_as_float(0x00400000u);
        if constexpr (kFp8) {
            const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const uint32_t c = (w[j >> 2] >> (8 * (j & 3))) & 0xFFu;
                const uint32_t f = (c >> 3) & 15u, m = c & 7u;
                // E4M3: (8 + m) 2^(f - 10) for f > 0, m 2^-9 for f = 0 (exact in fp32)
                float mag = f ? (float)(8u + m) * __uint_as_float((f + 117u) << 23)
                              : (float)m * __uint_as_float(118u << 23);
                if ((c & 0x7Fu) == 0x7Fu) mag = __uint_as_float(0x7FC00000u);   // E4M3 NaN
                v[j] = ((c & 0x80u) ? -mag : mag) * s;
            }
        } else {
            const uint32_t w[4] = {c0.x, c0.y, c0.z, c0.w};
            // E2M1 magnitudes in halves: 0, 1, 2, 3, 4, 6, 8, 12
            constexpr uint32_t kHalves = 0xC8643210u;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const uint32_t c = (w[j >> 3] >> (4 * (j & 7))) & 15u;
                const float mag = (float)((kHalves >> (4 * (c & 7u))) & 15u) * 0.5f;
                v[j] = ((c & 8u) ? -mag : mag) * s;
            }
        }
    }
    const int64_t off = row * 32 * k + 32 * blk;
    if constexpr (kOutBf16) {
        uint4* yp = reinterpret_cast<uint4*>(static_cast<uint16_t*>(yout) + off);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint32_t w[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t u0 = __float_as_uint(v[8 * t + 2 * d]);
                const uint32_t u1 = __float_as_uint(v[8 * t + 2 * d + 1]);
                w[d] = ((u0 + 0x7FFFu + ((u0 >> 16) & 1u)) >> 16) |
                       (((u1 + 0x7FFFu + ((u1 >> 16) & 1u)) >> 16) << 16);
            }
            yp[t] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else {
        float4* yp = reinterpret_cast<float4*>(static_cast<float*>(yout) + off);
#pragma unroll
        for (int t = 0; t < 8; ++t)
            yp[t] = make_float4(v[4 * t], v[4 * t + 1], v[4 * t + 2], v[4 * t + 3]);
    }
}

// grid of the lane-per-block kernels for rows of k blocks
dim3 block_grid(int64_t rows, int64_t k, int& lpr_log2, bool& ok)
{
    lpr_log2 = 0;
    while ((1LL << lpr_log2) < k && lpr_log2 < 6) ++lpr_log2;
    const int64_t rows_per_wave = 64 >> lpr_log2;
    const int64_t waves = (rows + rows_per_wave - 1) / rows_per_wave;
    const int64_t gx = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
    const int64_t gy = (k + 63) / 64;
    ok = gx <= 0x7FFFFFFF && gy <= 65535;
    return dim3((unsigned)(ok ? gx : 1), (unsigned)(ok ? gy : 1));
}

}  // namespace

hipError_t launch_quantize(bool act, const void* x, int64_t rows, int64_t k, int64_t ldx,
                           const float* A, const float* B, const float* r_min,
                           const float* r_max, uint8_t* q, uint8_t* e, bool tiled_scales,
                           hipStream_t stream, bool fp8, int form)
{
    if (form < 0 || form > 2 || (fp8 && form != 0)) return hipErrorNotSupported;
    // lanes per row: the smallest power of two >= k, capped at one wave
    int lpr_log2 = 0;
    while ((1LL << lpr_log2) < k && lpr_log2 < 6) ++lpr_log2;
    const int64_t rows_per_wave = 64 >> lpr_log2;
    const int64_t waves = (rows + rows_per_wave - 1) / rows_per_wave;
    const int64_t gy = (k + 63) / 64;
    const int64_t gx = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
    if (gx > 0x7FFFFFFF || gy > 65535) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)gx, (unsigned)gy);
    if (form != 0) {
        // one block column per workgroup, kThreads rows each
        const int64_t gr = (rows + kThreads - 1) / kThreads;
        if (k > 0x7FFFFFFF || gr > 65535) return hipErrorInvalidConfiguration;
        grid = dim3((unsigned)k, (unsigned)gr);
    }
    const int ts = (int)tiled_scales;
    if (form == 1 && act)
        hipLaunchKernelGGL((quantize_kernel<true, false, 1>), grid, dim3(kThreads), 0, stream,
                           x, rows, k, ldx, A, B, r_min, r_max, q, e, lpr_log2, ts);
    else if (form == 1)
        hipLaunchKernelGGL((quantize_kernel<false, false, 1>), grid, dim3(kThreads), 0, stream,
                           x, rows, k, ldx, A, B, r_min, r_max, q, e, lpr_log2, ts);
    else if (form == 2 && act)
        hipLaunchKernelGGL((quantize_kernel<true, false, 2>), grid, dim3(kThreads), 0, stream,
                           x, rows, k, ldx, A, B, r_min, r_max, q, e, lpr_log2, ts);
    else if (form == 2)
        hipLaunchKernelGGL((quantize_kernel<false, false, 2>), grid, dim3(kThreads), 0, stream,
                           x, rows, k, ldx, A, B, r_min, r_max, q, e, lpr_log2, ts);
    else if (act && fp8)
        hipLaunchKernelGGL((quantize_kernel<true, true>), grid, dim3(kThreads), 0, stream, x,
                           rows, k, ldx, A, B, r_min, r_max, q, e, lpr_log2, ts);
    else if (act)
        hipLaunchKernelGGL(quantize_kernel<true>, grid, dim3(kThreads), 0, stream, x, rows, k,
                           ldx, A, B, r_min, r_max, q, e, lpr_log2, ts);
    else
        hipLaunchKernelGGL(quantize_kernel<false>, grid, dim3(kThreads), 0, stream, x, rows,
                           k, ldx, A, B, r_min, r_max, q, e, lpr_log2, (int)tiled_scales);
    return hipGetLastError();
}

}  // namespace batq

namespace batq {

hipError_t launch_rmsnorm_quantize(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx,
                                   const float* gamma, float eps, const float* A,
                                   const float* B, const float* r_min, const float* r_max,
                                   uint8_t* q, uint8_t* e, bool tiled_scales,
                                   hipStream_t stream)
{
    if (k < 1 || k > 2 * kRmsThreads) return hipErrorNotSupported;
    int kpow2 = 1;
    while (kpow2 < k) kpow2 *= 2;
    const int tpr = kpow2 < 64 ? 64 : kpow2 > kRmsThreads ? kRmsThreads : kpow2;
    const int64_t groups = (rows + kRmsThreads / tpr - 1) / (kRmsThreads / tpr);
    if (groups > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)groups), block(kRmsThreads);
    const int ts = (int)tiled_scales;
    if (tpr == 64)
        hipLaunchKernelGGL(rmsnorm_quantize_kernel<64>, grid, block, 0, stream, x, rows, k, ldx,
                           gamma, eps, A, B, r_min, r_max, q, e, kpow2, ts);
    else if (tpr == 128)
        hipLaunchKernelGGL(rmsnorm_quantize_kernel<128>, grid, block, 0, stream, x, rows, k,
                           ldx, gamma, eps, A, B, r_min, r_max, q, e, kpow2, ts);
    else
        hipLaunchKernelGGL(rmsnorm_quantize_kernel<256>, grid, block, 0, stream, x, rows, k,
                           ldx, gamma, eps, A, B, r_min, r_max, q, e, kpow2, ts);
    return hipGetLastError();
}

}  // namespace batq

namespace batq {

hipError_t launch_quantize_kv(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx,
                              const int64_t* slots, int64_t num_slots, bool fp8,
                              const float* A, const float* B, const float* r_min,
                              const float* r_max, uint8_t* q, uint8_t* e, hipStream_t stream)
{
    int lpr;
    bool ok;
    const dim3 grid = block_grid(rows, k, lpr, ok);
    if (!ok) return hipErrorInvalidConfiguration;
    if (fp8)
        hipLaunchKernelGGL(quantize_kv_kernel<true>, grid, dim3(kThreads), 0, stream, x, rows,
                           k, ldx, slots, num_slots, A, B, r_min, r_max, q, e, lpr);
    else
        hipLaunchKernelGGL(quantize_kv_kernel<false>, grid, dim3(kThreads), 0, stream, x, rows,
                           k, ldx, slots, num_slots, A, B, r_min, r_max, q, e, lpr);
    return hipGetLastError();
}

hipError_t launch_transform_rows(const void* x, bool x_bf16, int64_t rows, int64_t k,
                                 int64_t ldx, const float* A, const float* B, void* y,
                                 bool y_bf16, hipStream_t stream)
{
    int lpr;
    bool ok;
    const dim3 grid = block_grid(rows, k, lpr, ok);
    if (!ok) return hipErrorInvalidConfiguration;
    const dim3 blk(kThreads);
    if (x_bf16 && y_bf16)
        hipLaunchKernelGGL((transform_rows_kernel<true, true>), grid, blk, 0, stream, x, rows,
                           k, ldx, A, B, y, lpr);
    else if (x_bf16)
        hipLaunchKernelGGL((transform_rows_kernel<true, false>), grid, blk, 0, stream, x, rows,
                           k, ldx, A, B, y, lpr);
    else if (y_bf16)
        hipLaunchKernelGGL((transform_rows_kernel<false, true>), grid, blk, 0, stream, x, rows,
                           k, ldx, A, B, y, lpr);
    else
        hipLaunchKernelGGL((transform_rows_kernel<false, false>), grid, blk, 0, stream, x, rows,
                           k, ldx, A, B, y, lpr);
    return hipGetLastError();
}

hipError_t launch_dequantize_rows(const uint8_t* q, const uint8_t* e, int64_t rows, int64_t k,
                                  bool fp8, const int64_t* index, int64_t src_rows, void* y,
                                  bool y_bf16, hipStream_t stream)
{
    int lpr;
    bool ok;
    const dim3 grid = block_grid(rows, k, lpr, ok);
    if (!ok) return hipErrorInvalidConfiguration;
    const dim3 blk(kThreads);
    if (fp8 && y_bf16)
        hipLaunchKernelGGL((dequantize_rows_kernel<true, true>), grid, blk, 0, stream, q, e,
                           rows, k, index, src_rows, y, lpr);
    else if (fp8)
        hipLaunchKernelGGL((dequantize_rows_kernel<true, false>), grid, blk, 0, stream, q, e,
                           rows, k, index, src_rows, y, lpr);
    else if (y_bf16)
        hipLaunchKernelGGL((dequantize_rows_kernel<false, true>), grid, blk, 0, stream, q, e,
                           rows, k, index, src_rows, y, lpr);
    else
        hipLaunchKernelGGL((dequantize_rows_kernel<false, false>), grid, blk, 0, stream, q, e,
                           rows, k, index, src_rows, y, lpr);
    return hipGetLastError();
}

}  // namespace batq
