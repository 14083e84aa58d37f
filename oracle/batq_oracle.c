/*
 * batq_oracle.c -- plain, slow CPU oracle for BATQuant's online W4A4 linear-layer path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
 * cpu_baseline leg load this file's shared object.  The product library shares no code,
 * header, table or helper with it, and it never calls the product library.
 *
 * What it computes follows the BATQuant pages ("BATQuant: Outlier-resilient MXFP4
 * Quantization via Learnable Block-wise Optimization"):
 *   - block-aligned affine transform y_i = x_i P_i on each 32-element MXFP block
 *     (daily-arxiv summary, method bullet "块对齐仿射变换"; gist.science summary, section 2A);
 *   - GPK factorisation P_i = B_i (x) A, A 8x8 global, B_i 4x4 private, evaluated with the
 *     Kronecker reshape trick (gist.science section 2B; thelatestinai listing, Table 1:
 *     g = 32, g1 = 8, g2 = 4, cost O(SN(g1+g2)) for XP);
 *   - block-wise clipping to [sigmoid(a_min) min(y), sigmoid(a_max) max(y)]
 *     (daily-arxiv summary, bullet "块级可学习裁剪"; gist.science section 2C);
 *   - MXFP4: 32 elements share one E8M0 scale, values are divided by the scale before
 *     rounding to E2M1 (thelatestinai listing, Figure 2 caption and the DuQuant++ abstract
 *     on that page; ARCQuant blog, "理论保证" on E8M0 being exponent-only);
 *   - the W4A4 product with weights transformed offline by P^-1 (gist.science section 2D;
 *     thelatestinai listing, Figure 3);
 *   - the W4A8 setting: the same transform and clip with the activations encoded as MXFP8
 *     (E4M3 elements, one E8M0 scale per 32) against the same MXFP4 weights (gist.science
 *     section 4 and the daily-arxiv results bullet, W4A8KV16);
 *   - the layer's input normalisation fused in front of the quantiser (RMSNorm, the step
 *     before every linear layer of the models the pages quantise; not defined on the pages,
 *     so its arithmetic is this file's contract: see orc_rmsnorm_f32);
 *   - the KV-cache settings (W4A8KV8, W4A8KV4: thelatestinai listing, Tables 2, 3 and 5;
 *     BAT covers self-attention including the KV caches: gist.science section 2D): K/V rows
 *     transformed, clipped and encoded as MXFP8 or MXFP4 into cache slots; queries
 *     transformed by P^-T (and attention outputs by P^-1) without quantisation;
 *   - the other transform forms that thelatestinai listing's Table 1 compares against GPK:
 *     a full 32x32 P_i per block ("w/o decomposition") and P_i = B_i (x) A_i with a private
 *     A_i per block (naive Kronecker); block Hadamard is GPK with Hadamard factors.
 *
 * Where the pages leave a step open, the plainest reading is taken (listed with reasons in
 * the design notes): fp32 arithmetic for the transform with sequential fused multiply-add
 * chains in index order (inner sum over the contiguous 8-index first, i.e. Z = X A, then
 * Y = B^T Z); torch.clamp-style clipping min(max(y, lo), hi); OCP MX scale exponent
 * floor(log2(amax)) - 2 clamped to the E8M0 range; E2M1 nearest value with ties to the
 * even code and saturation at 6; two codes per byte, even element in the low nibble.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -fPIC -shared
 * (fmaf is C99's correctly rounded fused multiply-add; contraction is off so that every
 * other product and sum rounds separately).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------ */
/* Element formats                                                                       */
/* ------------------------------------------------------------------------------------ */

/* bf16 -> fp32 is exact: the bf16 bit pattern is the top half of the fp32 pattern. */
static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* The eight E2M1 magnitudes, indexed by the 3-bit magnitude code (1 exponent bit pair,
 * 1 mantissa bit, exponent bias 1): 0, 0.5 (subnormal), 1, 1.5, 2, 3, 4, 6. */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Round v to the nearest E2M1 value; on a tie take the code with an even magnitude code
 * (round-half-to-even on the 1-bit mantissa); values beyond 6 take 6 (E2M1 has no
 * infinity).  The sign bit is copied from v, so a negative value that rounds to zero
 * gives the code 0x8 (negative zero). */
static uint8_t e2m1_round(double v)
{
    double a = fabs(v);
    /* Saturate first: E2M1 has no infinity, so every magnitude beyond the largest value 6
     * becomes 6.  (Without this the binary64 distances below round to equal values for huge
     * magnitudes and the tie rule would wrongly pick 4.)  For a <= 6 the distances are exact
     * wherever two of them can be equal, i.e. near the midpoints. */
    if (a > 6.0) a = 6.0;
    int best = 0;
    double best_d = a; /* distance to magnitude 0 */
    for (int c = 1; c < 8; ++c) {
        double d = fabs(a - E2M1_MAG[c]);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)((signbit(v) ? 0x8 : 0x0) | best);
}

/* Value of a 4-bit E2M1 code. */
static double e2m1_value(uint8_t code)
{
    double m = E2M1_MAG[code & 0x7];
    return (code & 0x8) ? -m : m;
}

/* Shared E8M0 scale byte of a block whose largest magnitude is amax.  OCP MX rule: the
 * block exponent is floor(log2(amax)) minus E2M1's largest exponent (2), clamped to the
 * E8M0 range [-127, 127]; the byte stores it with bias 127.  An all-zero block takes the
 * smallest scale (byte 0). */
static uint8_t e8m0_scale(float amax)
{
    if (amax == 0.0f) return 0;
    int ex;
    (void)frexpf(amax, &ex);          /* amax = m * 2^ex with m in [0.5, 1) */
    int x = (ex - 1) - 2;             /* floor(log2 amax) - emax(E2M1) */
    if (x < -127) x = -127;
    if (x > 127) x = 127;
    return (uint8_t)(x + 127);
}

/* E4M3 (OCP FP8, the variant without infinities): 4 exponent bits with bias 7, 3 mantissa
 * bits; magnitude code c = 8E + m gives m/8 * 2^-6 for E = 0 (subnormal) and
 * (1 + m/8) * 2^(E-7) for E = 1..15, except that E = 15, m = 7 is NaN, so the finite
 * magnitudes are the 127 codes 0..126 and the largest is 448. */
static double e4m3_mag(int c)
{
    int E = c >> 3, m = c & 7;
    return E == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, E - 7);
}

/* Round v to the nearest E4M3 value; on a tie take the even magnitude code (ties to even on
 * the 3-bit mantissa); magnitudes beyond 448 take 448 (the MX conversion saturates); the
 * sign bit is copied from v.  A plain search over the 127 finite magnitudes: for |v| <= 448
 * every distance below is exact in binary64, so ties are seen exactly. */
static uint8_t e4m3_round(double v)
{
    double a = fabs(v);
    if (a > 448.0) a = 448.0;
    int best = 0;
    double best_d = a;
    for (int c = 1; c <= 126; ++c) {
        double d = fabs(a - e4m3_mag(c));
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)((signbit(v) ? 0x80 : 0x00) | best);
}

static double e4m3_value(uint8_t code)
{
    double m = e4m3_mag(code & 0x7F);
    return (code & 0x80) ? -m : m;
}

/* MXFP8 scale byte: OCP MX rule with E4M3's largest exponent (8): floor(log2(amax)) - 8,
 * clamped to the E8M0 range, bias 127; an all-zero block takes byte 0. */
static uint8_t e8m0_scale_fp8(float amax)
{
    if (amax == 0.0f) return 0;
    int ex;
    (void)frexpf(amax, &ex);
    int x = (ex - 1) - 8;
    if (x < -127) x = -127;
    if (x > 127) x = 127;
    return (uint8_t)(x + 127);
}

/* ------------------------------------------------------------------------------------ */
/* GPK block transform                                                                   */
/* ------------------------------------------------------------------------------------ */

/* y = x (B (x) A) for one 32-element block x, using the reshape identity
 *   x (B (x) A) = vec_row(B^T X A),   X = 4x8 row-major view of x (X[r][c] = x[8r + c]).
 * A is 8x8 row-major, B is 4x4 row-major.  Evaluation order (fp32, one rounding per
 * operation): Z[r][c] = sum_q X[r][q] A[q][c], then Y[r][c] = sum_q B[q][r] Z[q][c]; each
 * sum starts with a plain product and adds the remaining terms in increasing q with fmaf. */
static void gpk_transform_block(const float x[32], const float A[64], const float B[16],
                                float y[32])
{
    float Z[32];
    for (int r = 0; r < 4; ++r) {
        for (int c = 0; c < 8; ++c) {
            float acc = x[8 * r + 0] * A[0 * 8 + c];
            for (int q = 1; q < 8; ++q) acc = fmaf(x[8 * r + q], A[q * 8 + c], acc);
            Z[8 * r + c] = acc;
        }
    }
    for (int r = 0; r < 4; ++r) {
        for (int c = 0; c < 8; ++c) {
            float acc = B[0 * 4 + r] * Z[0 * 8 + c];
            for (int q = 1; q < 4; ++q) acc = fmaf(B[q * 4 + r], Z[q * 8 + c], acc);
            y[8 * r + c] = acc;
        }
    }
}

/* y = x P for one block with a full 32x32 P (row-major, y_j = sum_m x_m P[m][j]): each
 * y_j is a plain product for m = 0 followed by fmaf for m = 1..31 in increasing m. */
static void full_transform_block(const float x[32], const float P[1024], float y[32])
{
    for (int j = 0; j < 32; ++j) {
        float acc = x[0] * P[j];
        for (int m = 1; m < 32; ++m) acc = fmaf(x[m], P[32 * m + j], acc);
        y[j] = acc;
    }
}

/* Transform selector shared by the variant entry points:
 *   0 GPK:       F0 = A [8][8] (one for all blocks), F1 = B [k][4][4]
 *   1 Kronecker: F0 = A [k][8][8] (private per block), F1 = B [k][4][4]
 *   2 full:      F0 = P [k][32][32], F1 unused
 * Forms 0 and 1 use the reshape evaluation of gpk_transform_block. */
static void transform_block(int form, const float x[32], const float* F0, const float* F1,
                            int64_t i, float y[32])
{
    if (form == 2)
        full_transform_block(x, F0 + 1024 * i, y);
    else
        gpk_transform_block(x, F0 + (form == 1 ? 64 * i : 0), F1 + 16 * i, y);
}

/* ------------------------------------------------------------------------------------ */
/* Clip + MXFP4 quantisation of one transformed block                                    */
/* ------------------------------------------------------------------------------------ */

/* Clip y to [r_min * min(y), r_max * max(y)] (torch.clamp semantics: the upper bound wins
 * when lo > hi), then quantise to MXFP4.  With clip == 0 the block is quantised as is.
 * Writes 16 code bytes (even element in the low nibble), the scale byte, and optionally the
 * values after division by the scale and before rounding (v32) and the clipped values
 * (yc32). */
static void clip_quantize_block(const float y[32], int clip, float r_min, float r_max,
                                uint8_t codes[16], uint8_t* scale, float* v32, float* yc32)
{
    float yc[32];
    if (clip) {
        float m = y[0], M = y[0];
        for (int j = 1; j < 32; ++j) {
            if (y[j] < m) m = y[j];
            if (y[j] > M) M = y[j];
        }
        float lo = r_min * m;
        float hi = r_max * M;
        for (int j = 0; j < 32; ++j) {
            float t = y[j] < lo ? lo : y[j]; /* max(y, lo) */
            yc[j] = t > hi ? hi : t;         /* min(., hi)  */
        }
    } else {
        for (int j = 0; j < 32; ++j) yc[j] = y[j];
    }

    float amax = 0.0f;
    for (int j = 0; j < 32; ++j) {
        float a = fabsf(yc[j]);
        if (a > amax) amax = a;
    }
    uint8_t e = e8m0_scale(amax);
    double s = ldexp(1.0, (int)e - 127); /* the shared scale 2^(e - 127) */

    uint8_t code[32];
    for (int j = 0; j < 32; ++j) {
        double v = (double)yc[j] / s;    /* exact in double */
        code[j] = e2m1_round(v);
        if (v32) v32[j] = (float)v;
        if (yc32) yc32[j] = yc[j];
    }
    for (int b = 0; b < 16; ++b) codes[b] = (uint8_t)(code[2 * b] | (code[2 * b + 1] << 4));
    *scale = e;
}

/* Clip (as above) + MXFP8 quantisation of one transformed block: 32 E4M3 code bytes and
 * the scale byte. */
static void clip_quantize_block_fp8(const float y[32], float r_min, float r_max,
                                    uint8_t codes[32], uint8_t* scale)
{
    float m = y[0], M = y[0];
    for (int j = 1; j < 32; ++j) {
        if (y[j] < m) m = y[j];
        if (y[j] > M) M = y[j];
    }
    float lo = r_min * m;
    float hi = r_max * M;
    float yc[32];
    float amax = 0.0f;
    for (int j = 0; j < 32; ++j) {
        float t = y[j] < lo ? lo : y[j];
        yc[j] = t > hi ? hi : t;
        if (fabsf(yc[j]) > amax) amax = fabsf(yc[j]);
    }
    uint8_t e = e8m0_scale_fp8(amax);
    double s = ldexp(1.0, (int)e - 127);
    for (int j = 0; j < 32; ++j) codes[j] = e4m3_round((double)yc[j] / s);
    *scale = e;
}

/* ------------------------------------------------------------------------------------ */
/* Exported entry points                                                                 */
/* ------------------------------------------------------------------------------------ */

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Activation side (online path): bf16 X [rows, ldx] -> transform -> clip -> MXFP4.
 * A [8][8], B [N/32][4][4], r_min/r_max [N/32] (fp32 clip ratios sigmoid(alpha)).
 * q [rows, N/2], e [rows, N/32].  v_dbg and yc_dbg ([rows, N] fp32) may be NULL. */
void orc_quantize_act(const uint16_t* x, int64_t rows, int64_t N, int64_t ldx,
                      const float* A, const float* B, const float* r_min, const float* r_max,
                      uint8_t* q, uint8_t* e, float* v_dbg, float* yc_dbg, int nthreads)
{
    int64_t k = N / 32;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < rows; ++s) {
        for (int64_t i = 0; i < k; ++i) {
            float xb[32], y[32];
            for (int j = 0; j < 32; ++j) xb[j] = bf16_to_float(x[s * ldx + 32 * i + j]);
            gpk_transform_block(xb, A, B + 16 * i, y);
            clip_quantize_block(y, 1, r_min[i], r_max[i], q + s * (N / 2) + 16 * i,
                                e + s * k + i, v_dbg ? v_dbg + s * N + 32 * i : NULL,
                                yc_dbg ? yc_dbg + s * N + 32 * i : NULL);
        }
    }
}

/* Weight side (offline): fp32 W [rows, N] -> transform with the inverse factors
 * (Ainv_t = (A^-1)^T, Binv_t[i] = (B_i^-1)^T, so that the block becomes B_i^-1 W_i A^-T)
 * -> MXFP4 without clipping. */
void orc_quantize_weight(const float* W, int64_t rows, int64_t N,
                         const float* Ainv_t, const float* Binv_t,
                         uint8_t* q, uint8_t* e, int nthreads)
{
    int64_t k = N / 32;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < rows; ++o) {
        for (int64_t i = 0; i < k; ++i) {
            float y[32];
            gpk_transform_block(W + o * N + 32 * i, Ainv_t, Binv_t + 16 * i, y);
            clip_quantize_block(y, 0, 1.0f, 1.0f, q + o * (N / 2) + 16 * i, e + o * k + i,
                                NULL, NULL);
        }
    }
}

/* Activation side with a transform form (see transform_block): bf16 X -> transform ->
 * clip -> MXFP4. */
void orc_quantize_act_form(const uint16_t* x, int64_t rows, int64_t N, int64_t ldx, int form,
                           const float* F0, const float* F1, const float* r_min,
                           const float* r_max, uint8_t* q, uint8_t* e, int nthreads)
{
    int64_t k = N / 32;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < rows; ++s) {
        for (int64_t i = 0; i < k; ++i) {
            float xb[32], y[32];
            for (int j = 0; j < 32; ++j) xb[j] = bf16_to_float(x[s * ldx + 32 * i + j]);
            transform_block(form, xb, F0, F1, i, y);
            clip_quantize_block(y, 1, r_min[i], r_max[i], q + s * (N / 2) + 16 * i,
                                e + s * k + i, NULL, NULL);
        }
    }
}

/* Weight side with a transform form: fp32 W -> transform with the inverse factors of that
 * form (transposed inverses, as for orc_quantize_weight) -> MXFP4 without clipping. */
void orc_quantize_weight_form(const float* W, int64_t rows, int64_t N, int form,
                              const float* F0, const float* F1, uint8_t* q, uint8_t* e,
                              int nthreads)
{
    int64_t k = N / 32;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < rows; ++o) {
        for (int64_t i = 0; i < k; ++i) {
            float y[32];
            transform_block(form, W + o * N + 32 * i, F0, F1, i, y);
            clip_quantize_block(y, 0, 1.0f, 1.0f, q + o * (N / 2) + 16 * i, e + o * k + i,
                                NULL, NULL);
        }
    }
}

/* The transform of a form alone on fp32 rows (for the pins). */
void orc_transform_form_f32(const float* x, int64_t rows, int64_t N, int form,
                            const float* F0, const float* F1, float* y)
{
    int64_t k = N / 32;
    for (int64_t s = 0; s < rows; ++s)
        for (int64_t i = 0; i < k; ++i)
            transform_block(form, x + s * N + 32 * i, F0, F1, i, y + s * N + 32 * i);
}

/* RMSNorm of bf16 rows: x_hat[j] = (x[j] * r) * gamma[j], r = 1 / sqrt(T / N + eps), where
 * T is the row's sum of squares taken as: per 32-element block, x_0^2 then fmaf(x_j, x_j, .)
 * in increasing j; the k block sums, padded with zeros to the next power of two K, are
 * added by halving (for h = K/2, K/4, .., 1: t[b] += t[b + h] for b < h); T = t[0].  Every
 * operation is one fp32 rounding (division and square root correctly rounded).
 * x_hat [rows, N] fp32; r_out [rows] (may be NULL). */
void orc_rmsnorm_f32(const uint16_t* x, int64_t rows, int64_t N, int64_t ldx,
                     const float* gamma, float eps, float* x_hat, float* r_out)
{
    int64_t k = N / 32;
    int64_t K = 1;
    while (K < k) K *= 2;
    for (int64_t s = 0; s < rows; ++s) {
        float t[1 << 16];
        for (int64_t b = 0; b < K; ++b) t[b] = 0.0f;
        for (int64_t b = 0; b < k; ++b) {
            float v0 = bf16_to_float(x[s * ldx + 32 * b]);
            float acc = v0 * v0;
            for (int j = 1; j < 32; ++j) {
                float v = bf16_to_float(x[s * ldx + 32 * b + j]);
                acc = fmaf(v, v, acc);
            }
            t[b] = acc;
        }
        for (int64_t h = K / 2; h >= 1; h /= 2)
            for (int64_t b = 0; b < h; ++b) t[b] = t[b] + t[b + h];
        float mean = t[0] / (float)N;
        float d = mean + eps;
        float r = 1.0f / sqrtf(d);
        if (r_out) r_out[s] = r;
        for (int64_t j = 0; j < N; ++j) {
            float v = bf16_to_float(x[s * ldx + j]);
            float u = v * r;
            x_hat[s * N + j] = u * gamma[j];
        }
    }
}

/* RMSNorm (as orc_rmsnorm_f32) fused in front of the activation quantiser: transform, clip
 * and MXFP4 of the normalised fp32 rows, as orc_quantize_act. */
void orc_quantize_act_rmsnorm(const uint16_t* x, int64_t rows, int64_t N, int64_t ldx,
                              const float* gamma, float eps, const float* A, const float* B,
                              const float* r_min, const float* r_max, uint8_t* q, uint8_t* e)
{
    int64_t k = N / 32;
    float* xh = (float*)malloc(sizeof(float) * (size_t)N);
    for (int64_t s = 0; s < rows; ++s) {
        orc_rmsnorm_f32(x + s * ldx, 1, N, ldx, gamma, eps, xh, NULL);
        for (int64_t i = 0; i < k; ++i) {
            float y[32];
            gpk_transform_block(xh + 32 * i, A, B + 16 * i, y);
            clip_quantize_block(y, 1, r_min[i], r_max[i], q + s * (N / 2) + 16 * i,
                                e + s * k + i, NULL, NULL);
        }
    }
    free(xh);
}

/* KV cache: row t of x (bf16 [T, ldx], N = heads x head_dim) is transformed, clipped and
 * encoded (fmt 4: MXFP4, codes [slots, N/2]; fmt 8: MXFP8, codes [slots, N]) into cache row
 * slots[t] (scales [slots, N/32] row-major); a negative slot skips the row and leaves the
 * cache untouched there. */
void orc_quantize_kv(const uint16_t* x, int64_t T, int64_t N, int64_t ldx, const int64_t* slots,
                     int fmt, const float* A, const float* B, const float* r_min,
                     const float* r_max, uint8_t* cache_q, uint8_t* cache_e)
{
    int64_t k = N / 32;
    int64_t qrow = fmt == 8 ? N : N / 2;
    for (int64_t t = 0; t < T; ++t) {
        int64_t slot = slots[t];
        if (slot < 0) continue;
        for (int64_t i = 0; i < k; ++i) {
            float xb[32], y[32];
            for (int j = 0; j < 32; ++j) xb[j] = bf16_to_float(x[t * ldx + 32 * i + j]);
            gpk_transform_block(xb, A, B + 16 * i, y);
            if (fmt == 8)
                clip_quantize_block_fp8(y, r_min[i], r_max[i], cache_q + slot * qrow + 32 * i,
                                        cache_e + slot * k + i);
            else
                clip_quantize_block(y, 1, r_min[i], r_max[i], cache_q + slot * qrow + 16 * i,
                                    cache_e + slot * k + i, NULL, NULL);
        }
    }
}

/* The GPK transform of rows without quantisation: x bf16 (x_bf16 != 0) or fp32 [rows, ldx]
 * -> y fp32 [rows, N], with whatever factors the caller passes (P for K/V rows, the
 * transposed inverses for queries, the inverses for attention outputs). */
void orc_transform_rows(const void* x, int x_bf16, int64_t rows, int64_t N, int64_t ldx,
                        const float* A, const float* B, float* y)
{
    int64_t k = N / 32;
    for (int64_t s = 0; s < rows; ++s)
        for (int64_t i = 0; i < k; ++i) {
            float xb[32];
            for (int j = 0; j < 32; ++j)
                xb[j] = x_bf16 ? bf16_to_float(((const uint16_t*)x)[s * ldx + 32 * i + j])
                               : ((const float*)x)[s * ldx + 32 * i + j];
            gpk_transform_block(xb, A, B + 16 * i, y + s * N + 32 * i);
        }
}

/* fp32 -> bf16 bit pattern, nearest with ties to the even pattern, by comparing the two
 * neighbouring bf16 values exactly (finite inputs whose rounding stays finite). */
void orc_f32_to_bf16(const float* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &v[i], 4);
        uint32_t lo = u & 0xFFFF0000u, hi = lo + 0x10000u; /* truncation and the next one */
        float flo, fhi;
        memcpy(&flo, &lo, 4);
        memcpy(&fhi, &hi, 4);
        double dlo = fabs((double)v[i] - (double)flo), dhi = fabs((double)fhi - (double)v[i]);
        uint32_t pick = dlo < dhi ? lo : dhi < dlo ? hi : (((lo >> 16) & 1) ? hi : lo);
        out[i] = (uint16_t)(pick >> 16);
    }
}

/* The transform alone (fp32 y [rows, N]) on fp32 input, for the structural pins. */
void orc_transform_f32(const float* x, int64_t rows, int64_t N, const float* A,
                       const float* B, float* y)
{
    int64_t k = N / 32;
    for (int64_t s = 0; s < rows; ++s)
        for (int64_t i = 0; i < k; ++i)
            gpk_transform_block(x + s * N + 32 * i, A, B + 16 * i, y + s * N + 32 * i);
}

/* Clip + quantise already-transformed fp32 rows (for the reduction pins). */
void orc_clip_quantize_f32(const float* y, int64_t rows, int64_t N, int clip,
                           const float* r_min, const float* r_max, uint8_t* q, uint8_t* e,
                           float* v_dbg)
{
    int64_t k = N / 32;
    for (int64_t s = 0; s < rows; ++s)
        for (int64_t i = 0; i < k; ++i)
            clip_quantize_block(y + s * N + 32 * i, clip, clip ? r_min[i] : 1.0f,
                                clip ? r_max[i] : 1.0f, q + s * (N / 2) + 16 * i,
                                e + s * k + i, v_dbg ? v_dbg + s * N + 32 * i : NULL, NULL);
}

/* Element encoder over an array (for the exhaustive E2M1 pin). */
void orc_e2m1_round_f32(const float* v, int64_t n, uint8_t* code)
{
    for (int64_t t = 0; t < n; ++t) code[t] = e2m1_round((double)v[t]);
}

/* E2M1 round of every fp32 bit pattern in [start, start + count) (non-finite patterns give
 * 0xFF), one code per byte. */
void orc_e2m1_round_bits(uint32_t start, uint32_t count, uint8_t* code)
{
    for (uint32_t t = 0; t < count; ++t) {
        uint32_t u = start + t;
        float f;
        memcpy(&f, &u, sizeof f);
        code[t] = isfinite(f) ? e2m1_round((double)f) : 0xFF;
    }
}

/* Scale byte for each amax (for the E8M0 pin). */
void orc_e8m0_scale_f32(const float* amax, int64_t n, uint8_t* e)
{
    for (int64_t t = 0; t < n; ++t) e[t] = e8m0_scale(amax[t]);
}

/* Dequantise MXFP4 rows to fp64: value = e2m1(code) * 2^(e - 127). */
void orc_dequant(const uint8_t* q, const uint8_t* e, int64_t rows, int64_t N, double* out)
{
    int64_t k = N / 32;
    for (int64_t s = 0; s < rows; ++s)
        for (int64_t n = 0; n < N; ++n) {
            uint8_t byte = q[s * (N / 2) + n / 2];
            uint8_t code = (n & 1) ? (byte >> 4) : (byte & 0xF);
            out[s * N + n] = ldexp(e2m1_value(code), (int)e[s * k + n / 32] - 127);
        }
}

/* W4A4 GEMM reference in fp64: y[a][b] = sum_n dq(xq)[rows[a]][n] * dq(wq)[cols[b]][n] and
 * t[a][b] = sum_n |same products|, for the selected output rows and columns (rows == NULL
 * selects all S rows, cols == NULL all `out` columns).  Each product of two dequantised
 * values is exact in fp64; the sum runs in increasing n. */
void orc_gemm_w4a4(const uint8_t* xq, const uint8_t* xe, const uint8_t* wq, const uint8_t* we,
                   int64_t S, int64_t N, int64_t out, const int64_t* rows, int64_t nrows,
                   const int64_t* cols, int64_t ncols, double* y, double* t, int nthreads)
{
    int64_t k = N / 32;
    if (!rows) nrows = S;
    if (!cols) ncols = out;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t a = 0; a < nrows; ++a) {
        int64_t s = rows ? rows[a] : a;
        for (int64_t b = 0; b < ncols; ++b) {
            int64_t o = cols ? cols[b] : b;
            double acc = 0.0, abs_acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                uint8_t xb = xq[s * (N / 2) + n / 2], wb = wq[o * (N / 2) + n / 2];
                uint8_t xc = (n & 1) ? (xb >> 4) : (xb & 0xF);
                uint8_t wc = (n & 1) ? (wb >> 4) : (wb & 0xF);
                double xv = ldexp(e2m1_value(xc), (int)xe[s * k + n / 32] - 127);
                double wv = ldexp(e2m1_value(wc), (int)we[o * k + n / 32] - 127);
                acc += xv * wv;
                abs_acc += fabs(xv * wv);
            }
            y[a * ncols + b] = acc;
            t[a * ncols + b] = abs_acc;
        }
    }
}

/* W4A8 activation side: bf16 X [rows, ldx] -> transform -> clip -> MXFP8.
 * q8 [rows, N] (one E4M3 code per byte), e [rows, N/32]. */
void orc_quantize_act_fp8(const uint16_t* x, int64_t rows, int64_t N, int64_t ldx,
                          const float* A, const float* B, const float* r_min,
                          const float* r_max, uint8_t* q8, uint8_t* e, int nthreads)
{
    int64_t k = N / 32;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < rows; ++s) {
        for (int64_t i = 0; i < k; ++i) {
            float xb[32], y[32];
            for (int j = 0; j < 32; ++j) xb[j] = bf16_to_float(x[s * ldx + 32 * i + j]);
            gpk_transform_block(xb, A, B + 16 * i, y);
            clip_quantize_block_fp8(y, r_min[i], r_max[i], q8 + s * N + 32 * i, e + s * k + i);
        }
    }
}

/* Clip + MXFP8 of already-transformed fp32 rows (for the reduction pin). */
void orc_clip_quantize_fp8_f32(const float* y, int64_t rows, int64_t N, const float* r_min,
                               const float* r_max, uint8_t* q8, uint8_t* e)
{
    int64_t k = N / 32;
    for (int64_t s = 0; s < rows; ++s)
        for (int64_t i = 0; i < k; ++i)
            clip_quantize_block_fp8(y + s * N + 32 * i, r_min[i], r_max[i], q8 + s * N + 32 * i,
                                    e + s * k + i);
}

void orc_e4m3_round_f32(const float* v, int64_t n, uint8_t* code)
{
    for (int64_t t = 0; t < n; ++t) code[t] = e4m3_round((double)v[t]);
}

void orc_e4m3_value(const uint8_t* code, int64_t n, double* v)
{
    for (int64_t t = 0; t < n; ++t) v[t] = e4m3_value(code[t]);
}

void orc_e8m0_scale_fp8_f32(const float* amax, int64_t n, uint8_t* e)
{
    for (int64_t t = 0; t < n; ++t) e[t] = e8m0_scale_fp8(amax[t]);
}

/* Dequantise MXFP8 rows to fp64. */
void orc_dequant_fp8(const uint8_t* q8, const uint8_t* e, int64_t rows, int64_t N, double* out)
{
    int64_t k = N / 32;
    for (int64_t s = 0; s < rows; ++s)
        for (int64_t n = 0; n < N; ++n)
            out[s * N + n] = ldexp(e4m3_value(q8[s * N + n]), (int)e[s * k + n / 32] - 127);
}

/* W4A8 GEMM reference in fp64: MXFP8 activations [S, N] x MXFP4 weights [out, N]; same
 * conventions as orc_gemm_w4a4. */
void orc_gemm_w4a8(const uint8_t* xq8, const uint8_t* xe, const uint8_t* wq, const uint8_t* we,
                   int64_t S, int64_t N, int64_t out, const int64_t* rows, int64_t nrows,
                   const int64_t* cols, int64_t ncols, double* y, double* t, int nthreads)
{
    int64_t k = N / 32;
    if (!rows) nrows = S;
    if (!cols) ncols = out;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t a = 0; a < nrows; ++a) {
        int64_t s = rows ? rows[a] : a;
        for (int64_t b = 0; b < ncols; ++b) {
            int64_t o = cols ? cols[b] : b;
            double acc = 0.0, abs_acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                uint8_t wb = wq[o * (N / 2) + n / 2];
                uint8_t wc = (n & 1) ? (wb >> 4) : (wb & 0xF);
                double xv = ldexp(e4m3_value(xq8[s * N + n]), (int)xe[s * k + n / 32] - 127);
                double wv = ldexp(e2m1_value(wc), (int)we[o * k + n / 32] - 127);
                acc += xv * wv;
                abs_acc += fabs(xv * wv);
            }
            y[a * ncols + b] = acc;
            t[a * ncols + b] = abs_acc;
        }
    }
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
