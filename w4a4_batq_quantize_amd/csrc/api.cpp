// Host side of the C ABI declared in include/batq.h: argument validation (always before
// any HIP call), the offline parameter steps (clip ratios, inverse GPK factors) and the
// launches of the fused quantiser and the W4A4 GEMM.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#include "batq.h"
#include "internal.h"

#define BATQ_API extern "C" __attribute__((visibility("default")))

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

batq_status from_hip(hipError_t err) { return err == hipSuccess ? BATQ_OK : BATQ_ERR_HIP; }

// Inverse of an n x n fp32 matrix (n <= 32) by Gauss-Jordan elimination with partial
// pivoting in 64-bit-mantissa arithmetic, stored transposed and rounded once to fp32.
// Returns false if a pivot is zero or a result is not finite.
bool inverse_transposed(const float* M, int n, float* out_t)
{
    static thread_local long double a[32][64];
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < 2 * n; ++j)
            a[i][j] = j < n ? (long double)M[i * n + j] : (long double)(j - n == i);
    for (int col = 0; col < n; ++col) {
        int piv = col;
        for (int r = col + 1; r < n; ++r)
            if (std::fabs(a[r][col]) > std::fabs(a[piv][col])) piv = r;
        if (a[piv][col] == 0.0L) return false;
        if (piv != col)
            for (int j = 0; j < 2 * n; ++j) std::swap(a[piv][j], a[col][j]);
        const long double p = a[col][col];
        for (int j = 0; j < 2 * n; ++j) a[col][j] /= p;
        for (int r = 0; r < n; ++r) {
            if (r == col || a[r][col] == 0.0L) continue;
            const long double f = a[r][col];
            for (int j = 0; j < 2 * n; ++j) a[r][j] -= f * a[col][j];
        }
    }
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) {
            const float v = (float)a[i][n + j];        // (M^-1)[i][j]
            if (!std::isfinite(v)) return false;
            out_t[j * n + i] = v;                       // stored transposed
        }
    return true;
}

bool valid_form(batq_transform t)
{
    return t == BATQ_TRANSFORM_GPK || t == BATQ_TRANSFORM_KRONECKER || t == BATQ_TRANSFORM_FULL;
}

// number of floats of the two factor arrays of a transform form with k blocks
int64_t factor0_floats(batq_transform t, int64_t k)
{
    return t == BATQ_TRANSFORM_GPK ? 64 : t == BATQ_TRANSFORM_KRONECKER ? 64 * k : 1024 * k;
}
int64_t factor1_floats(batq_transform t, int64_t k) { return t == BATQ_TRANSFORM_FULL ? 0 : 16 * k; }

bool valid_layout(batq_scale_layout l)
{
    return l == BATQ_SCALES_ROW_MAJOR || l == BATQ_SCALES_MFMA_TILED;
}

bool mul_overflows(int64_t a, int64_t b)
{
    return a != 0 && b > std::numeric_limits<int64_t>::max() / a;
}

}  // namespace

BATQ_API const char* batq_status_string(batq_status status)
{
    switch (status) {
        case BATQ_OK: return "BATQ_OK";
        case BATQ_ERR_NULL: return "BATQ_ERR_NULL: a required pointer is NULL";
        case BATQ_ERR_SHAPE: return "BATQ_ERR_SHAPE: invalid size";
        case BATQ_ERR_ALIGN: return "BATQ_ERR_ALIGN: misaligned pointer or stride";
        case BATQ_ERR_UNSUPPORTED: return "BATQ_ERR_UNSUPPORTED: valid for the format but beyond the library's limits";
        case BATQ_ERR_SINGULAR: return "BATQ_ERR_SINGULAR: a GPK factor is not invertible";
        case BATQ_ERR_HIP: return "BATQ_ERR_HIP: HIP runtime error";
        case BATQ_ERR_TOO_LARGE: return "BATQ_ERR_TOO_LARGE: the activation codes and scales exceed the no-allocation entry point's 64 MiB scratch";
    }
    return "unknown batq_status";
}

BATQ_API batq_status batq_clip_ratios(const float* alpha, int64_t k, float* ratio)
{
    if (k < 0) return BATQ_ERR_SHAPE;
    if (k == 0) return BATQ_OK;
    if (!alpha || !ratio) return BATQ_ERR_NULL;
    for (int64_t i = 0; i < k; ++i)
        ratio[i] = (float)(1.0 / (1.0 + std::exp(-(double)alpha[i])));
    return BATQ_OK;
}

BATQ_API batq_status batq_weight_factors(const float* A, const float* B, int64_t k,
                                         float* A_inv_t, float* B_inv_t)
{
    if (k < 0) return BATQ_ERR_SHAPE;
    if (!A || !A_inv_t || (k > 0 && (!B || !B_inv_t))) return BATQ_ERR_NULL;
    if (!inverse_transposed(A, 8, A_inv_t)) return BATQ_ERR_SINGULAR;
    for (int64_t i = 0; i < k; ++i)
        if (!inverse_transposed(B + 16 * i, 4, B_inv_t + 16 * i)) return BATQ_ERR_SINGULAR;
    return BATQ_OK;
}

BATQ_API batq_status batq_quantize_act(const uint16_t* x, int64_t S, int64_t N, int64_t ldx,
                                       const float* A, const float* B, const float* r_min,
                                       const float* r_max, uint8_t* q, uint8_t* e,
                                       batq_scale_layout e_layout, void* stream)
{
    if (S < 0 || N < 0 || N % 32 != 0) return BATQ_ERR_SHAPE;
    if (S == 0 || N == 0) return BATQ_OK;
    if (!x || !A || !B || !r_min || !r_max || !q || !e) return BATQ_ERR_NULL;
    if (!valid_layout(e_layout)) return BATQ_ERR_UNSUPPORTED;
    if (ldx < N || mul_overflows(S, ldx)) return BATQ_ERR_SHAPE;
    if (ldx % 8 != 0 || !aligned(x, 16) || !aligned(B, 16) || !aligned(q, 16) ||
        !aligned(A, 4) || !aligned(r_min, 4) || !aligned(r_max, 4))
        return BATQ_ERR_ALIGN;
    const int64_t k = N / 32;
    if (k > 64LL * 65535) return BATQ_ERR_UNSUPPORTED;
    return from_hip(batq::launch_quantize(true, x, S, k, ldx, A, B, r_min, r_max, q, e,
                                          e_layout == BATQ_SCALES_MFMA_TILED,
                                          as_stream(stream)));
}

BATQ_API batq_status batq_prepare_weight(const float* W, int64_t out, int64_t N,
                                         const float* A_host, const float* B_host,
                                         uint8_t* wq, uint8_t* we,
                                         batq_scale_layout we_layout, void* stream)
{
    if (out < 0 || N < 0 || N % 32 != 0) return BATQ_ERR_SHAPE;
    if (out == 0 || N == 0) return BATQ_OK;
    if (!W || !A_host || !B_host || !wq || !we) return BATQ_ERR_NULL;
    if (!valid_layout(we_layout)) return BATQ_ERR_UNSUPPORTED;
    if (mul_overflows(out, N)) return BATQ_ERR_SHAPE;
    if (!aligned(W, 16) || !aligned(wq, 16)) return BATQ_ERR_ALIGN;
    const int64_t k = N / 32;
    if (k > 64LL * 65535) return BATQ_ERR_UNSUPPORTED;

    std::vector<float> factors(64 + 16 * k);
    const batq_status st = batq_weight_factors(A_host, B_host, k, factors.data(),
                                               factors.data() + 64);
    if (st != BATQ_OK) return st;

    hipStream_t s = as_stream(stream);
    float* d = nullptr;
    if (hipMalloc(&d, factors.size() * sizeof(float)) != hipSuccess) return BATQ_ERR_HIP;
    hipError_t err = hipMemcpyAsync(d, factors.data(), factors.size() * sizeof(float),
                                    hipMemcpyHostToDevice, s);
    if (err == hipSuccess)
        err = batq::launch_quantize(false, W, out, k, N, d, d + 64, nullptr, nullptr, wq, we,
                                    we_layout == BATQ_SCALES_MFMA_TILED, s);
    const hipError_t sync = hipStreamSynchronize(s);
    const hipError_t fr = hipFree(d);
    if (err != hipSuccess || sync != hipSuccess || fr != hipSuccess) return BATQ_ERR_HIP;
    return BATQ_OK;
}

BATQ_API batq_status batq_gemm_w4a4(const uint8_t* xq, const uint8_t* xe, const uint8_t* wq,
                                    const uint8_t* we, batq_scale_layout layout, int64_t S,
                                    int64_t N, int64_t out, float* y, void* stream)
{
    if (S < 0 || N < 0 || out < 0 || N % 32 != 0) return BATQ_ERR_SHAPE;
    if (S == 0 || out == 0) return BATQ_OK;
    if (!y || (N > 0 && (!xq || !xe || !wq || !we))) return BATQ_ERR_NULL;
    if (!valid_layout(layout)) return BATQ_ERR_UNSUPPORTED;
    if (mul_overflows(S, out) || mul_overflows(S, N) || mul_overflows(out, N))
        return BATQ_ERR_SHAPE;
    if (!aligned(y, 16) || !aligned(xq, 16) || !aligned(wq, 16)) return BATQ_ERR_ALIGN;
    return from_hip(batq::launch_gemm(xq, xe, wq, we, layout == BATQ_SCALES_MFMA_TILED, S, N,
                                      out, y, as_stream(stream)));
}

BATQ_API batq_status batq_linear_w4a4(const uint16_t* x, int64_t S, int64_t N, int64_t ldx,
                                      const float* A, const float* B, const float* r_min,
                                      const float* r_max, const uint8_t* wq, const uint8_t* we,
                                      batq_scale_layout layout, int64_t out, float* y,
                                      uint8_t* xq, uint8_t* xe, void* stream)
{
    if (S < 0 || N < 0 || out < 0 || N % 32 != 0) return BATQ_ERR_SHAPE;
    if (S == 0 || out == 0) return BATQ_OK;
    if (!valid_layout(layout)) return BATQ_ERR_UNSUPPORTED;
    if (N == 0) return batq_gemm_w4a4(nullptr, nullptr, nullptr, nullptr, layout, S, 0, out, y,
                                      stream);
    const int64_t k = N / 32;
    const bool can_fuse = S <= BATQ_LINEAR_FUSED_TOKENS && k <= 512 && k % 8 == 0;
    if (!y || !x || !A || !B || !r_min || !r_max || !wq || !we) return BATQ_ERR_NULL;
    if (!can_fuse && (!xq || !xe)) return BATQ_ERR_NULL;
    // with a workspace, the one kernel where it measured faster than the two calls (up to
    // 16 tokens on 16-row workgroups): every workgroup encodes the S k token blocks, so the
    // total encoding work decides
    const bool small = S <= 16 && k <= 512 && k % 8 == 0 && S * k <= 1536 &&
                       S * k * ((out + 15) / 16) <= 196608;
    const bool fused = (can_fuse && (!xq || !xe)) || small;
    if (ldx < N || mul_overflows(S, ldx) || mul_overflows(S, out) || mul_overflows(out, N))
        return BATQ_ERR_SHAPE;
    if (ldx % 8 != 0 || !aligned(x, 16) || !aligned(B, 16) || !aligned(y, 16) ||
        !aligned(wq, 16) || !aligned(A, 4) || !aligned(r_min, 4) || !aligned(r_max, 4))
        return BATQ_ERR_ALIGN;
    if (fused) {
        const hipError_t err = batq::launch_linear_skinny(
            x, S, k, ldx, A, B, r_min, r_max, wq, we, layout == BATQ_SCALES_MFMA_TILED, out, y,
            as_stream(stream));
        if (err != hipErrorNotSupported) return from_hip(err);
        // outside the one-kernel path's limits (scale alignment, operand size): two steps
        if (!xq || !xe) return BATQ_ERR_UNSUPPORTED;
    }
    const batq_status st =
        batq_quantize_act(x, S, N, ldx, A, B, r_min, r_max, xq, xe, layout, stream);
    if (st != BATQ_OK) return st;
    return batq_gemm_w4a4(xq, xe, wq, we, layout, S, N, out, y, stream);
}

BATQ_API batq_status batq_linear_w4a4_noalloc(const uint16_t* x, int64_t S, int64_t N,
                                              int64_t ldx, const float* A, const float* B,
                                              const float* r_min, const float* r_max,
                                              const uint8_t* wq, const uint8_t* we,
                                              batq_scale_layout layout, int64_t out, float* y,
                                              void* stream)
{
    if (S < 0 || N < 0 || out < 0 || N % 32 != 0) return BATQ_ERR_SHAPE;
    if (S == 0 || out == 0) return BATQ_OK;
    if (!valid_layout(layout)) return BATQ_ERR_UNSUPPORTED;
    if (N == 0) return batq_gemm_w4a4(nullptr, nullptr, nullptr, nullptr, layout, S, 0, out, y,
                                      stream);
    if (!y || !x || !A || !B || !r_min || !r_max || !wq || !we) return BATQ_ERR_NULL;
    if (ldx < N || mul_overflows(S, ldx) || mul_overflows(S, out) || mul_overflows(out, N))
        return BATQ_ERR_SHAPE;
    if (ldx % 8 != 0 || !aligned(x, 16) || !aligned(B, 16) || !aligned(y, 16) ||
        !aligned(wq, 16) || !aligned(A, 4) || !aligned(r_min, 4) || !aligned(r_max, 4))
        return BATQ_ERR_ALIGN;
    const int64_t k = N / 32;
    if (mul_overflows(S, k)) return BATQ_ERR_SHAPE;
    // codes, then the scales from the next 256-byte boundary (the tiled layout's alignment)
    const int64_t code_span = (S * (N / 2) + 255) / 256 * 256;
    const int64_t scale_span = layout == BATQ_SCALES_MFMA_TILED
                                   ? ((S + 31) / 32) * 32 * ((k + 7) / 8) * 8
                                   : S * k;
    if (code_span > batq::kNoAllocScratchBytes ||
        scale_span > batq::kNoAllocScratchBytes - code_span)
        return BATQ_ERR_TOO_LARGE;
    uint8_t* scratch = nullptr;
    if (batq::noalloc_scratch(&scratch) != hipSuccess) return BATQ_ERR_HIP;
    return batq_linear_w4a4(x, S, N, ldx, A, B, r_min, r_max, wq, we, layout, out, y, scratch,
                            scratch + code_span, stream);
}

BATQ_API batq_status batq_linear_w4a8(const uint16_t* x, int64_t S, int64_t N, int64_t ldx,
                                      const float* A, const float* B, const float* r_min,
                                      const float* r_max, const uint8_t* wq, const uint8_t* we,
                                      batq_scale_layout layout, int64_t out, float* y,
                                      uint8_t* xq8, uint8_t* xe, void* stream)
{
    if (S < 0 || N < 0 || out < 0 || N % 32 != 0) return BATQ_ERR_SHAPE;
    if (S == 0 || out == 0) return BATQ_OK;
    if (!valid_layout(layout)) return BATQ_ERR_UNSUPPORTED;
    if (N == 0) return batq_gemm_w4a8(nullptr, nullptr, nullptr, nullptr, layout, S, 0, out, y,
                                      stream);
    const int64_t k = N / 32;
    const bool can_fuse = S <= BATQ_LINEAR_FUSED_TOKENS && k <= 512 && k % 8 == 0 &&
                          S * k <= BATQ_LINEAR_W4A8_FUSED_BLOCKS;
    if (!y || !x || !A || !B || !r_min || !r_max || !wq || !we) return BATQ_ERR_NULL;
    if (!can_fuse && (!xq8 || !xe)) return BATQ_ERR_NULL;
    if (ldx < N || mul_overflows(S, ldx) || mul_overflows(S, out) || mul_overflows(out, N))
        return BATQ_ERR_SHAPE;
    if (ldx % 8 != 0 || !aligned(x, 16) || !aligned(B, 16) || !aligned(y, 16) ||
        !aligned(wq, 16) || !aligned(A, 4) || !aligned(r_min, 4) || !aligned(r_max, 4))
        return BATQ_ERR_ALIGN;
    // the one kernel wherever it applies: measured faster than the two calls on every
    // shape it takes (its token rows are at most 768 blocks)
    if (can_fuse) {
        const hipError_t err = batq::launch_linear16_w4a8(
            x, S, k, ldx, A, B, r_min, r_max, wq, we, layout == BATQ_SCALES_MFMA_TILED, out, y,
            as_stream(stream));
        if (err != hipErrorNotSupported) return from_hip(err);
        if (!xq8 || !xe) return BATQ_ERR_UNSUPPORTED;
    }
    const batq_status st =
        batq_quantize_act_mxfp8(x, S, N, ldx, A, B, r_min, r_max, xq8, xe, layout, stream);
    if (st != BATQ_OK) return st;
    return batq_gemm_w4a8(xq8, xe, wq, we, layout, S, N, out, y, stream);
}

BATQ_API batq_status batq_quantize_act_mxfp8(const uint16_t* x, int64_t S, int64_t N,
                                             int64_t ldx, const float* A, const float* B,
                                             const float* r_min, const float* r_max,
                                             uint8_t* q8, uint8_t* e, batq_scale_layout e_layout,
                                             void* stream)
{
    if (S < 0 || N < 0 || N % 32 != 0) return BATQ_ERR_SHAPE;
    if (S == 0 || N == 0) return BATQ_OK;
    if (!x || !A || !B || !r_min || !r_max || !q8 || !e) return BATQ_ERR_NULL;
    if (!valid_layout(e_layout)) return BATQ_ERR_UNSUPPORTED;
    if (ldx < N || mul_overflows(S, ldx)) return BATQ_ERR_SHAPE;
    if (ldx % 8 != 0 || !aligned(x, 16) || !aligned(B, 16) || !aligned(q8, 16) ||
        !aligned(A, 4) || !aligned(r_min, 4) || !aligned(r_max, 4))
        return BATQ_ERR_ALIGN;
    const int64_t k = N / 32;
    if (k > 64LL * 65535) return BATQ_ERR_UNSUPPORTED;
    return from_hip(batq::launch_quantize(true, x, S, k, ldx, A, B, r_min, r_max, q8, e,
                                          e_layout == BATQ_SCALES_MFMA_TILED,
                                          as_stream(stream), /*fp8=*/true));
}

BATQ_API batq_status batq_gemm_w4a8(const uint8_t* xq8, const uint8_t* xe, const uint8_t* wq,
                                    const uint8_t* we, batq_scale_layout layout, int64_t S,
                                    int64_t N, int64_t out, float* y, void* stream)
{
    if (S < 0 || N < 0 || out < 0 || N % 32 != 0) return BATQ_ERR_SHAPE;
    if (S == 0 || out == 0) return BATQ_OK;
    if (!y || (N > 0 && (!xq8 || !xe || !wq || !we))) return BATQ_ERR_NULL;
    if (!valid_layout(layout)) return BATQ_ERR_UNSUPPORTED;
    if (mul_overflows(S, out) || mul_overflows(S, N) || mul_overflows(out, N))
        return BATQ_ERR_SHAPE;
    if (!aligned(y, 16) || !aligned(xq8, 16) || !aligned(wq, 16) || !aligned(xe, 4) ||
        !aligned(we, 4))
        return BATQ_ERR_ALIGN;
    if (N % 256 != 0 || S * N >= (1LL << 32) || out * (N / 2) >= (1LL << 32))
        return BATQ_ERR_UNSUPPORTED;
    return from_hip(batq::launch_gemm_w4a8(xq8, xe, wq, we, layout == BATQ_SCALES_MFMA_TILED,
                                           S, N, out, y, as_stream(stream)));
}

BATQ_API batq_status batq_quantize_act_form(const uint16_t* x, int64_t S, int64_t N, int64_t ldx,
                                            batq_transform form, const float* F0,
                                            const float* F1, const float* r_min,
                                            const float* r_max, uint8_t* q, uint8_t* e,
                                            batq_scale_layout e_layout, void* stream)
{
    if (S < 0 || N < 0 || N % 32 != 0) return BATQ_ERR_SHAPE;
    if (S == 0 || N == 0) return BATQ_OK;
    if (!valid_form(form) || !valid_layout(e_layout)) return BATQ_ERR_UNSUPPORTED;
    if (!x || !F0 || (form != BATQ_TRANSFORM_FULL && !F1) || !r_min || !r_max || !q || !e)
        return BATQ_ERR_NULL;
    if (ldx < N || mul_overflows(S, ldx)) return BATQ_ERR_SHAPE;
    if (ldx % 8 != 0 || !aligned(x, 16) || !aligned(q, 16) || !aligned(r_min, 4) ||
        !aligned(r_max, 4) || !aligned(F0, form == BATQ_TRANSFORM_GPK ? 4 : 16) ||
        (form != BATQ_TRANSFORM_FULL && !aligned(F1, 16)))
        return BATQ_ERR_ALIGN;
    const int64_t k = N / 32;
    if (k > 64LL * 65535) return BATQ_ERR_UNSUPPORTED;
    return from_hip(batq::launch_quantize(true, x, S, k, ldx, F0, F1, r_min, r_max, q, e,
                                          e_layout == BATQ_SCALES_MFMA_TILED,
                                          as_stream(stream), false, (int)form));
}

BATQ_API batq_status batq_prepare_weight_form(const float* W, int64_t out, int64_t N,
                                              batq_transform form, const float* F0_host,
                                              const float* F1_host, uint8_t* wq, uint8_t* we,
                                              batq_scale_layout we_layout, void* stream)
{
    if (out < 0 || N < 0 || N % 32 != 0) return BATQ_ERR_SHAPE;
    if (out == 0 || N == 0) return BATQ_OK;
    if (!valid_form(form) || !valid_layout(we_layout)) return BATQ_ERR_UNSUPPORTED;
    if (!W || !F0_host || (form != BATQ_TRANSFORM_FULL && !F1_host) || !wq || !we)
        return BATQ_ERR_NULL;
    if (mul_overflows(out, N)) return BATQ_ERR_SHAPE;
    if (!aligned(W, 16) || !aligned(wq, 16)) return BATQ_ERR_ALIGN;
    const int64_t k = N / 32;
    if (k > 64LL * 65535) return BATQ_ERR_UNSUPPORTED;

    // transposed inverses of every factor: F0 part then F1 part, each 16-byte aligned
    const int64_t n0 = factor0_floats(form, k), n1 = factor1_floats(form, k);
    std::vector<float> factors(n0 + n1);
    const int64_t m0 = form == BATQ_TRANSFORM_GPK ? 1 : k;
    const int d0 = form == BATQ_TRANSFORM_FULL ? 32 : 8;
    for (int64_t i = 0; i < m0; ++i)
        if (!inverse_transposed(F0_host + i * d0 * d0, d0, factors.data() + i * d0 * d0))
            return BATQ_ERR_SINGULAR;
    for (int64_t i = 0; i < n1 / 16; ++i)
        if (!inverse_transposed(F1_host + 16 * i, 4, factors.data() + n0 + 16 * i))
            return BATQ_ERR_SINGULAR;

    hipStream_t s = as_stream(stream);
    float* d = nullptr;
    if (hipMalloc(&d, factors.size() * sizeof(float)) != hipSuccess) return BATQ_ERR_HIP;
    hipError_t err = hipMemcpyAsync(d, factors.data(), factors.size() * sizeof(float),
                                    hipMemcpyHostToDevice, s);
    if (err == hipSuccess)
        err = batq::launch_quantize(false, W, out, k, N, d, n1 ? d + n0 : nullptr, nullptr,
                                    nullptr, wq, we, we_layout == BATQ_SCALES_MFMA_TILED, s,
                                    false, (int)form);
    const hipError_t sync = hipStreamSynchronize(s);
    const hipError_t fr = hipFree(d);
    if (err != hipSuccess || sync != hipSuccess || fr != hipSuccess) return BATQ_ERR_HIP;
    return BATQ_OK;
}

BATQ_API batq_status batq_gemm_w4a4_out(const uint8_t* xq, const uint8_t* xe, const uint8_t* wq,
                                        const uint8_t* we, batq_scale_layout layout, int64_t S,
                                        int64_t N, int64_t out, void* y, batq_out_type y_type,
                                        const uint16_t* residual, void* stream)
{
    if (S < 0 || N < 0 || out < 0 || N % 32 != 0) return BATQ_ERR_SHAPE;
    if (S == 0 || out == 0) return BATQ_OK;
    if (!y || (N > 0 && (!xq || !xe || !wq || !we))) return BATQ_ERR_NULL;
    if (!valid_layout(layout) || (y_type != BATQ_OUT_F32 && y_type != BATQ_OUT_BF16))
        return BATQ_ERR_UNSUPPORTED;
    if (mul_overflows(S, out) || mul_overflows(S, N) || mul_overflows(out, N))
        return BATQ_ERR_SHAPE;
    if (!aligned(y, 16) || !aligned(xq, 16) || !aligned(wq, 16) || !aligned(residual, 16))
        return BATQ_ERR_ALIGN;
    return from_hip(batq::launch_gemm(xq, xe, wq, we, layout == BATQ_SCALES_MFMA_TILED, S, N,
                                      out, static_cast<float*>(y), as_stream(stream), residual,
                                      y_type == BATQ_OUT_BF16));
}

BATQ_API batq_status batq_gemm_w4a8_out(const uint8_t* xq8, const uint8_t* xe, const uint8_t* wq,
                                        const uint8_t* we, batq_scale_layout layout, int64_t S,
                                        int64_t N, int64_t out, void* y, batq_out_type y_type,
                                        const uint16_t* residual, void* stream)
{
    if (S < 0 || N < 0 || out < 0 || N % 32 != 0) return BATQ_ERR_SHAPE;
    if (S == 0 || out == 0) return BATQ_OK;
    if (!y || (N > 0 && (!xq8 || !xe || !wq || !we))) return BATQ_ERR_NULL;
    if (!valid_layout(layout) || (y_type != BATQ_OUT_F32 && y_type != BATQ_OUT_BF16))
        return BATQ_ERR_UNSUPPORTED;
    if (mul_overflows(S, out) || mul_overflows(S, N) || mul_overflows(out, N))
        return BATQ_ERR_SHAPE;
    if (!aligned(y, 16) || !aligned(xq8, 16) || !aligned(wq, 16) || !aligned(xe, 4) ||
        !aligned(we, 4) || !aligned(residual, 16))
        return BATQ_ERR_ALIGN;
    if (N % 256 != 0 || S * N >= (1LL << 32) || out * (N / 2) >= (1LL << 32))
        return BATQ_ERR_UNSUPPORTED;
    return from_hip(batq::launch_gemm_w4a8(xq8, xe, wq, we, layout == BATQ_SCALES_MFMA_TILED,
                                           S, N, out, static_cast<float*>(y), as_stream(stream),
                                           residual, y_type == BATQ_OUT_BF16));
}

BATQ_API batq_status batq_quantize_act_rmsnorm(const uint16_t* x, int64_t S, int64_t N,
                                               int64_t ldx, const float* gamma, float eps,
                                               const float* A, const float* B,
                                               const float* r_min, const float* r_max,
                                               uint8_t* q, uint8_t* e,
                                               batq_scale_layout e_layout, void* stream)
{
    if (S < 0 || N < 0 || N % 32 != 0) return BATQ_ERR_SHAPE;
    if (S == 0 || N == 0) return BATQ_OK;
    if (!x || !gamma || !A || !B || !r_min || !r_max || !q || !e) return BATQ_ERR_NULL;
    if (!valid_layout(e_layout)) return BATQ_ERR_UNSUPPORTED;
    if (ldx < N || mul_overflows(S, ldx)) return BATQ_ERR_SHAPE;
    if (ldx % 8 != 0 || !aligned(x, 16) || !aligned(B, 16) || !aligned(q, 16) ||
        !aligned(gamma, 16) || !aligned(A, 4) || !aligned(r_min, 4) || !aligned(r_max, 4))
        return BATQ_ERR_ALIGN;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return BATQ_ERR_SHAPE;
    const int64_t k = N / 32;
    if (k > 512 || S > 0x7FFFFFFF) return BATQ_ERR_UNSUPPORTED;
    return from_hip(batq::launch_rmsnorm_quantize(x, S, k, ldx, gamma, eps, A, B, r_min, r_max,
                                                  q, e, e_layout == BATQ_SCALES_MFMA_TILED,
                                                  as_stream(stream)));
}

BATQ_API batq_status batq_quantize_kv(const uint16_t* x, int64_t T, int64_t N, int64_t ldx,
                                      const int64_t* slots, int64_t num_slots,
                                      batq_kv_format fmt, const float* A, const float* B,
                                      const float* r_min, const float* r_max,
                                      uint8_t* cache_q, uint8_t* cache_e, void* stream)
{
    if (T < 0 || N < 0 || N % 32 != 0 || num_slots < 0) return BATQ_ERR_SHAPE;
    if (fmt != BATQ_KV_MXFP4 && fmt != BATQ_KV_MXFP8) return BATQ_ERR_UNSUPPORTED;
    if (T == 0 || N == 0) return BATQ_OK;
    if (!x || !slots || !A || !B || !r_min || !r_max || !cache_q || !cache_e)
        return BATQ_ERR_NULL;
    if (ldx < N || mul_overflows(T, ldx) || mul_overflows(num_slots, N)) return BATQ_ERR_SHAPE;
    if (ldx % 8 != 0 || !aligned(x, 16) || !aligned(B, 16) || !aligned(cache_q, 16) ||
        !aligned(slots, 8) || !aligned(A, 4) || !aligned(r_min, 4) || !aligned(r_max, 4))
        return BATQ_ERR_ALIGN;
    return from_hip(batq::launch_quantize_kv(x, T, N / 32, ldx, slots, num_slots,
                                             fmt == BATQ_KV_MXFP8, A, B, r_min, r_max,
                                             cache_q, cache_e, as_stream(stream)));
}

BATQ_API batq_status batq_transform_rows(const void* x, batq_out_type x_type, int64_t rows,
                                         int64_t N, int64_t ldx, const float* A,
                                         const float* B, void* y, batq_out_type y_type,
                                         void* stream)
{
    if (rows < 0 || N < 0 || N % 32 != 0) return BATQ_ERR_SHAPE;
    if ((x_type != BATQ_OUT_F32 && x_type != BATQ_OUT_BF16) ||
        (y_type != BATQ_OUT_F32 && y_type != BATQ_OUT_BF16))
        return BATQ_ERR_UNSUPPORTED;
    if (rows == 0 || N == 0) return BATQ_OK;
    if (!x || !A || !B || !y) return BATQ_ERR_NULL;
    if (ldx < N || mul_overflows(rows, ldx) || mul_overflows(rows, N)) return BATQ_ERR_SHAPE;
    const bool xb = x_type == BATQ_OUT_BF16;
    if (ldx % (xb ? 8 : 4) != 0 || !aligned(x, 16) || !aligned(B, 16) || !aligned(y, 16) ||
        !aligned(A, 4))
        return BATQ_ERR_ALIGN;
    return from_hip(batq::launch_transform_rows(x, xb, rows, N / 32, ldx, A, B, y,
                                                y_type == BATQ_OUT_BF16, as_stream(stream)));
}

BATQ_API batq_status batq_dequantize_rows(const uint8_t* q, const uint8_t* e, int64_t src_rows,
                                          int64_t N, batq_kv_format fmt, const int64_t* index,
                                          int64_t rows, void* y, batq_out_type y_type,
                                          void* stream)
{
    if (src_rows < 0 || rows < 0 || N < 0 || N % 32 != 0) return BATQ_ERR_SHAPE;
    if ((fmt != BATQ_KV_MXFP4 && fmt != BATQ_KV_MXFP8) ||
        (y_type != BATQ_OUT_F32 && y_type != BATQ_OUT_BF16))
        return BATQ_ERR_UNSUPPORTED;
    if (!index && rows > src_rows) return BATQ_ERR_SHAPE;
    if (rows == 0 || N == 0) return BATQ_OK;
    if (!y || (src_rows > 0 && (!q || !e)) || (!index && !q)) return BATQ_ERR_NULL;
    if (mul_overflows(rows, N) || mul_overflows(src_rows, N)) return BATQ_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(y, 16) || (index && !aligned(index, 8)))
        return BATQ_ERR_ALIGN;
    return from_hip(batq::launch_dequantize_rows(q, e, rows, N / 32, fmt == BATQ_KV_MXFP8,
                                                 index, src_rows, y, y_type == BATQ_OUT_BF16,
                                                 as_stream(stream)));
}
