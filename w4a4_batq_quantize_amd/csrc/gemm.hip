// MXFP4 x MXFP4 -> fp32 GEMM on gfx950 scaled MFMA (the W4A4 linear layer).
//
// y[s][o] = sum_n dq(x)[s][n] dq(w)[o][n] with dq = e2m1(code) * 2^(e-127) per 32-element
// block.  The contraction runs on V_MFMA_SCALE_F32_16X16X128_F8F6F4 with both operands in
// E2M1 (format code 4): one instruction multiplies a 16x128 by a 128x16 tile, every lane
// supplying 32 consecutive K values (16 bytes) of one row and the E8M0 scale of exactly
// that 32-element block, so MX blocks map onto lanes one to one and the scales are applied
// inside the instruction.  Lane l holds row l%16 and K block l/16; the 16x16 fp32 result
// gives lane l the column l%16 and rows 4(l/16)..4(l/16)+3.
//
// The MFMA "row" operand is the weight tile (out dimension) and the "column" operand is the
// activation tile (token dimension), so each lane's four accumulator values are four
// consecutive output features of one token: one 16-byte store into row-major y.
//
// Work decomposition: a 256-thread workgroup (4 waves, 2 x 2) owns a BO x BS output tile;
// each wave owns (BO/2) x (BS/2).  The K loop advances 128 elements (64 code bytes and 4
// scale bytes per row) per step; the next step's tiles are fetched into registers while the
// current step is multiplied out of LDS (two LDS stages, one barrier per step).  Rows past
// the end of the matrices and K blocks past N/32 are filled with zero codes, which add
// nothing whatever the scale.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace batq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kCodeBytes = 64;          // code bytes per row per K step (128 elements)
constexpr int kPitch = kCodeBytes + 16; // LDS row pitch; the 16-byte pad spreads rows over banks
constexpr int kFmtE2M1 = 4;

template <int BO, int BS>
struct Smem {
    uint8_t w[2][BO][kPitch];
    uint8_t x[2][BS][kPitch];
    uint8_t ws[2][BO][4];
    uint8_t xs[2][BS][4];
};

// Per-thread staging registers of one K step.
template <int BO, int BS>
struct Stage {
    static constexpr int kChunks = (BO + BS) * 4;              // 16-byte code chunks
    static constexpr int kPerThread = kChunks / kThreads;
    uint4 code[kPerThread];
    uint32_t scale;                                           // 4 scale bytes of one row
};

template <int BO, int BS>
__device__ __forceinline__ void load_stage(Stage<BO, BS>& st, const uint8_t* __restrict__ xq,
                                           const uint8_t* __restrict__ xe,
                                           const uint8_t* __restrict__ wq,
                                           const uint8_t* __restrict__ we, int64_t S,
                                           int64_t out, int64_t k, int64_t o0, int64_t s0,
                                           int64_t kt)
{
    const int tid = threadIdx.x;
    const int64_t rowbytes = 16 * k;
#pragma unroll
    for (int j = 0; j < Stage<BO, BS>::kPerThread; ++j) {
        const int c = tid + kThreads * j;
        const int r = c >> 2, part = c & 3;
        const int64_t blk = 4 * kt + part;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < BO) {
            const int64_t o = o0 + r;
            if (o < out && blk < k)
                v = *reinterpret_cast<const uint4*>(wq + o * rowbytes + 16 * blk);
        } else {
            const int64_t s = s0 + (r - BO);
            if (s < S && blk < k)
                v = *reinterpret_cast<const uint4*>(xq + s * rowbytes + 16 * blk);
        }
        st.code[j] = v;
    }
    // scale bytes: threads [0, BO) take weight rows, [BO, BO + BS) activation rows
    uint32_t sc = 0x7F7F7F7Fu;
    if (tid < BO + BS) {
        const bool isw = tid < BO;
        const int64_t row = isw ? o0 + tid : s0 + (tid - BO);
        const bool ok = isw ? row < out : row < S;
        const uint8_t* src = (isw ? we : xe) + row * k;
        if (ok) {
            sc = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int64_t blk = 4 * kt + b;
                const uint32_t v = blk < k ? src[blk] : 0x7Fu;
                sc |= v << (8 * b);
            }
        }
    }
    st.scale = sc;
}

template <int BO, int BS>
__device__ __forceinline__ void store_stage(Smem<BO, BS>& sm, int buf, const Stage<BO, BS>& st)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < Stage<BO, BS>::kPerThread; ++j) {
        const int c = tid + kThreads * j;
        const int r = c >> 2, part = c & 3;
        uint8_t* dst = r < BO ? &sm.w[buf][r][16 * part] : &sm.x[buf][r - BO][16 * part];
        *reinterpret_cast<uint4*>(dst) = st.code[j];
    }
    if (tid < BO + BS) {
        uint8_t* dst = tid < BO ? sm.ws[buf][tid] : sm.xs[buf][tid - BO];
        *reinterpret_cast<uint32_t*>(dst) = st.scale;
    }
}

template <int BO, int BS>
__global__ void __launch_bounds__(kThreads)
gemm_kernel(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xe,
            const uint8_t* __restrict__ wq, const uint8_t* __restrict__ we, int64_t S,
            int64_t k, int64_t out, float* __restrict__ y, int64_t tiles_o)
{
    constexpr int WO = BO / 2, WS = BS / 2;     // per-wave tile
    constexpr int TO = WO / 16, TS = WS / 16;   // 16x16 MFMA tiles per wave
    __shared__ Smem<BO, BS> sm;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wo = wave >> 1, ws = wave & 1;
    const int64_t tile = blockIdx.x;
    const int64_t o0 = (tile % tiles_o) * BO;
    const int64_t s0 = (tile / tiles_o) * BS;
    const int64_t ksteps = (k + 3) / 4;

    v4f acc[TO][TS];
#pragma unroll
    for (int a = 0; a < TO; ++a)
#pragma unroll
        for (int b = 0; b < TS; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

    Stage<BO, BS> st;
    load_stage<BO, BS>(st, xq, xe, wq, we, S, out, k, o0, s0, 0);
    store_stage<BO, BS>(sm, 0, st);
    __syncthreads();

    const int lr = lane & 15;   // row within a 16-row MFMA tile
    const int lg = lane >> 4;   // K block within the 128-element step
    for (int64_t kt = 0; kt < ksteps; ++kt) {
        const int buf = (int)(kt & 1);
        const bool more = kt + 1 < ksteps;
        if (more) load_stage<BO, BS>(st, xq, xe, wq, we, S, out, k, o0, s0, kt + 1);

        uint4 af[TO], bf[TS];
        int asc[TO], bsc[TS];
#pragma unroll
        for (int a = 0; a < TO; ++a) {
            const int r = wo * WO + 16 * a + lr;
            af[a] = *reinterpret_cast<const uint4*>(&sm.w[buf][r][16 * lg]);
            asc[a] = sm.ws[buf][r][lg];
        }
#pragma unroll
        for (int b = 0; b < TS; ++b) {
            const int r = ws * WS + 16 * b + lr;
            bf[b] = *reinterpret_cast<const uint4*>(&sm.x[buf][r][16 * lg]);
            bsc[b] = sm.xs[buf][r][lg];
        }
#pragma unroll
        for (int a = 0; a < TO; ++a) {
            const v8i av = {(int)af[a].x, (int)af[a].y, (int)af[a].z, (int)af[a].w, 0, 0, 0, 0};
#pragma unroll
            for (int b = 0; b < TS; ++b) {
                const v8i bv = {(int)bf[b].x, (int)bf[b].y, (int)bf[b].z, (int)bf[b].w, 0, 0, 0, 0};
                acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    av, bv, acc[a][b], kFmtE2M1, kFmtE2M1, 0, asc[a], 0, bsc[b]);
            }
        }
        if (more) store_stage<BO, BS>(sm, buf ^ 1, st);
        __syncthreads();
    }

    // epilogue: lane holds y[s][o .. o+3] for s = column l%16, o = rows 4(l/16) .. +3
    const bool vec_ok = (out & 3) == 0;
#pragma unroll
    for (int a = 0; a < TO; ++a) {
        const int64_t o = o0 + wo * WO + 16 * a + 4 * lg;
#pragma unroll
        for (int b = 0; b < TS; ++b) {
            const int64_t s = s0 + ws * WS + 16 * b + lr;
            if (s >= S) continue;
            float* dst = y + s * out + o;
            if (vec_ok && o + 3 < out) {
                *reinterpret_cast<float4*>(dst) =
                    make_float4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (o + j < out) dst[j] = acc[a][b][j];
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* xq, const uint8_t* xe, const uint8_t* wq,
                       const uint8_t* we, int64_t S, int64_t N, int64_t out, float* y,
                       hipStream_t stream)
{
    constexpr int BO = 128, BS = 128;
    const int64_t k = N / 32;
    const int64_t tiles_o = (out + BO - 1) / BO;
    const int64_t tiles_s = (S + BS - 1) / BS;
    const int64_t tiles = tiles_o * tiles_s;
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemm_kernel<BO, BS>), dim3((unsigned)tiles), dim3(kThreads), 0, stream,
                       xq, xe, wq, we, S, k, out, y, tiles_o);
    return hipGetLastError();
}

}  // namespace batq
