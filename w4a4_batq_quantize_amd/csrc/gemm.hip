// MXFP4 x MXFP4 (and E2M1 x E4M3) -> fp32 GEMMs on gfx950 matrix cores: the product of the
// W4A4 (W4A8) linear layer, and the layer in one kernel for a few tokens.
//
// y[s][o] = sum_n dq(x)[s][n] dq(w)[o][n] with dq = code value * 2^(e-127) per 32-element
// block.  W4A4: the contraction runs on the scaled MFMA instructions: each lane supplies the
// K values of one MX block of one row (16 bytes of E2M1) together with the E8M0 scale of
// exactly that block, so blocks map onto lanes one to one and the block scales are applied
// inside the instruction.  W4A8: the same lane-to-block mapping, but both operands are
// dequantised to bf16 in registers and multiplied on the bf16 MFMAs, which (unlike the scaled
// MFMA with an E4M3 operand) return the product to within fp32 summation rounding.
//
// Kernels, by token count S (the launchers below choose):
//  - gemm_pc_kernel / gemm_dma_kernel (S > 64; MFMA-tiled / row-major scales):
//    V_MFMA_SCALE_F32_32X32X64_F8F6F4 on 256 (out) x 128 (token) tiles, operands moved
//    HBM/L2 -> LDS by buffer_load ... lds without passing through registers, three LDS
//    stages; producer waves issue the DMA and consumer waves the MFMAs in the first;
//  - gemm_big_kernel (two or more rounds of 256 x 256 tiles, MFMA-tiled scales, fp32
//    output without residual): persistent workgroups whose waves all stream and multiply,
//    256-element K stages moved as whole 128-byte lines, the stage DMA running on from one
//    tile into the next;
//  - gemm_w4a8_kernel (S > 64, E4M3 tokens): the 256 x 128 tile and DMA, bf16 MFMAs;
//  - gemm_skinny16_kernel (S <= 16, by a workgroup-rounds rule) and gemm_skinny_kernel
//    (S <= 64 otherwise): weight streaming, 16 or 32 output rows per workgroup and K split
//    across its waves;
//  - gemm_linear16_kernel / gemm_linear_skinny_kernel: the few-token GEMM that encodes its
//    token rows itself (the whole layer in one kernel, S <= 4);
//  - gemm_generic_kernel for any other N (ragged K) or alignment: the 16x16x128 form with
//    register-staged, bounds-checked loads.
// In the tiled kernels the activation tile is the MFMA row operand and the weight tile the
// column operand, so a lane's accumulators are one output feature of 16 tokens and every
// dword store instruction writes whole 128-byte lines of y.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <utility>

#include "internal.h"
#include "mx_block.h"

namespace batq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

constexpr int kThreads = 256;
constexpr int kFmtE2M1 = 4;
constexpr int kXcds = 8;

// ---------------------------------------------------------------------------------------
// W4A8 products, exactly
// ---------------------------------------------------------------------------------------
//
// The scaled MFMA with an E4M3 operand does not return the exact product: measured on
// gfx950, it forms the products of each group of 8 consecutive K positions aligned to the
// largest of them and truncates them to 2^(E-13) (E that product's exponent sum), so a
// product more than 9 octaves below its group's largest is cut (448 + 31 * 2^-6 comes out as
// 448).  The W4A8 kernels therefore dequantise both operands to bf16 -- an E4M3 or E2M1 value
// times its E8M0 scale is exact in bf16 for activation scale bytes 9..246 and weight scale
// bytes 0..252, which covers every scale the quantisers produce from finite inputs above
// 2^-110 -- and multiply them on the bf16 MFMAs, whose products are exact and whose sums
// stayed within 1.3e-6 of the sum of |terms| in every measured case (wide and narrow scales,
// 64 to 12288 K positions).  Each lane converts the 8 elements one bf16 MFMA takes from the
// MX block it holds, so the MFMAs of one scaled step cover the same K positions on both
// operands, in a different order (the sum is invariant to it).
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// E8M0 byte as the scale operand of the scaled conversions (they read its exponent field)
__device__ __forceinline__ float e8m0_operand(uint32_t byte) { return __uint_as_float(byte << 23); }

// elements 8q .. 8q + 7 of an E2M1 block (16 bytes) times 2^(s - 127), as bf16
__device__ __forceinline__ v8bf dequant_e2m1_bf16(const v4u& c, int q, float s)
{
    const uint32_t w = c[q];
    const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
    const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
    const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
    const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
    return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// elements 8q .. 8q + 7 of an E4M3 block (32 bytes) times 2^(s - 127), as bf16
__device__ __forceinline__ v8bf dequant_e4m3_bf16(const v8i& c, int q, float s)
{
    const uint32_t w0 = (uint32_t)c[2 * q], w1 = (uint32_t)c[2 * q + 1];
    const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, false);
    const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, true);
    const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, false);
    const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, true);
    return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}


// acc (32 x 32) += the 64-position K-step whose block the lane holds (16 bytes of E2M1 codes
// w, 32 bytes of E4M3 codes x, their scale bytes): four bf16 MFMAs.  kWeightsA: the weights
// are the row operand (A) of the instruction, else the tokens are.
template <bool kWeightsA>
__device__ __forceinline__ v16f w4a8_step32(v16f acc, const v4u& w, const v8i& x, uint32_t wbyte,
                                            uint32_t xbyte)
{
    const float sw = e8m0_operand(wbyte & 0xFFu), sx = e8m0_operand(xbyte & 0xFFu);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const v8bf a = dequant_e2m1_bf16(w, q, sw), b = dequant_e4m3_bf16(x, q, sx);
        acc = kWeightsA ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0)
                        : __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc, 0, 0, 0);
        // (one MFMA's conversions at a time: they run while the previous MFMA does, and the
        // bf16 operands do not all stay live)
        __builtin_amdgcn_sched_barrier(0);
    }
    return acc;
}

// acc (16 x 16, weights as the row operand) += the 128-position K-step whose block the lane
// holds: four bf16 16x16x32 MFMAs
__device__ __forceinline__ v4f w4a8_step16(v4f acc, const v4u& w, const v8i& x, uint32_t wbyte,
                                           uint32_t xbyte)
{
    const float sw = e8m0_operand(wbyte & 0xFFu), sx = e8m0_operand(xbyte & 0xFFu);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant_e2m1_bf16(w, q, sw),
                                                       dequant_e4m3_bf16(x, q, sx), acc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    return acc;
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8])
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// Workgroup barrier without the memory fence __syncthreads() adds (which would wait for the
// LDS DMA of the stages still in flight).  The asm statement orders all memory accesses at
// compiler level; the hardware-level completion of this wave's LDS reads and of the DMA it
// needs is established by the explicit s_waitcnt placed before it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// K rotation of a tile when the grid has more tiles than CUs: the tile starts its K loop at
// stage (weight tile + token tile) mod nst and wraps.  Tiles that share an operand tile then
// request its stages at different times, so most of their requests find the lines a
// neighbour has already brought into L2, where with every tile in step each request waits
// for the same fill.  Measured on the producer/consumer kernel: gate_up and the S = 16384
// prefills 4-7% faster; with a single round of tiles (q_proj, down_proj) no gain, so it is
// off there (and in the W4A8 kernel, whose waves issue the DMA between their MFMAs, it
// gained 2-3% on those shapes and cost 3% on the single-round ones).  Any order sums the
// same terms (within the accumulation bound), and the rotation is fixed per tile.
__device__ __forceinline__ int64_t k_rotation(int64_t tiles_o, int64_t tiles_s, int64_t o0,
                                              int64_t s0, int64_t BO, int64_t BS, int64_t nst)
{
    if (nst == 0 || tiles_o * tiles_s <= 256) return 0;
    return (o0 / BO + s0 / BS) % nst;
}

// Tile numbering: when the tile count divides evenly, each XCD (own L2) receives a
// contiguous run of tiles; within the run, groups of `group_o` weight tiles are swept
// across the activation tiles so neighbouring workgroups share operands.
__device__ __forceinline__ void tile_origin(int64_t tiles_o, int64_t tiles_s, int64_t group_o,
                                           int64_t BO, int64_t BS, int64_t& o0, int64_t& s0)
{
    const int64_t total = tiles_o * tiles_s;
    int64_t id = blockIdx.x;
    if (total % kXcds == 0) id = (id % kXcds) * (total / kXcds) + id / kXcds;
    const int64_t span = group_o * tiles_s;
    const int64_t first_o = (id / span) * group_o;
    const int64_t gsize = tiles_o - first_o < group_o ? tiles_o - first_o : group_o;
    const int64_t rem = id % span;
    o0 = (first_o + rem % gsize) * BO;
    s0 = (rem / gsize) * BS;
}

// =======================================================================================
// gemm_dma_kernel<Cfg>: BO (out) x BS (tokens) tile per workgroup
// =======================================================================================
//
// Waves are arranged WO x WS; each owns (BO/WO) x (BS/WS) outputs = TM x TN MFMA tiles of
// 32 x 32.  A K stage is 256 elements: per tile row 128 code bytes and 8 scale bytes.  LDS
// stage layout: rows [0, BO) weight rows, [BO, BO+BS) activation rows, 128 bytes each,
// followed by (BO+BS) x 8 scale bytes.  Within a row the 16-byte chunk c is stored at
// position c ^ ((row / 2) % 8): the DMA writes 64 lanes x 16 bytes contiguously, so the
// layout cannot be padded.  gfx950's LDS has 64 banks (256 bytes per bank row, measured: a
// conflict-free ds_read_b128 pattern reaches ~217 B/clk per CU, and an XOR by row % 8 only
// ~120), so two 128-byte rows share a bank row and the XOR key is the row pair: the 16
// lanes served together (rows r..r+15 of one operand, one chunk) then hit 16 distinct
// 16-byte bank groups.  NB stages are in flight (prefetch distance NB-1).
//
// The 32x32x64 operand layout: lane l holds row l%32 and K block l/32 of the K-step, the
// result gives lane l column l%32 and rows 8(r/4) + 4(l/32) + r%4 for register r.

constexpr int kStageBlocks = 8;
constexpr int kRowBytes = 16 * kStageBlocks;   // 128

template <int BO_, int BS_, int WO_, int WS_, int NB_, bool TS_, int SB_ = 4, bool SW_ = false>
struct DmaCfg {
    static constexpr int BO = BO_, BS = BS_, WO = WO_, WS = WS_, NB = NB_;
    static constexpr bool TS = TS_;   // scales in the MFMA-tiled layout (else row-major)
    // SW: activations as the MFMA's row operand and weights as its column operand, so a
    // lane's accumulator column is one output feature and a register row one token: each
    // dword store of the epilogue writes 32 consecutive outputs (whole 128-byte lines)
    static constexpr bool SW = SW_;
    static constexpr int SB = TS_ ? 4 : SB_;                        // scale DMA bytes per lane
    static constexpr int kWaves = WO * WS;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int TM = BO / WO / 32, TN = BS / WS / 32;
    static constexpr int kRows = BO + BS;
    static constexpr int kCodeBytes = kRows * kRowBytes;
    static constexpr int kScaleBytes = kRows * kStageBlocks;
    static constexpr int kBufBytes = kCodeBytes + kScaleBytes;
    static constexpr int kCodeDma = kCodeBytes / 1024 / kWaves;     // 1 KB instructions / wave
    // tiled: one 256-byte unit per 32-row panel per stage; row-major: 8 bytes per row
    static constexpr int kScaleDma = kScaleBytes / (64 * SB) / kWaves;  // per wave
    static constexpr int kDmaPerStage = kCodeDma + kScaleDma;
    static_assert(TM >= 1 && TN >= 1 && BO % (WO * 32) == 0 && BS % (WS * 32) == 0, "tiles");
    static_assert(kCodeBytes % (1024 * kWaves) == 0, "code DMA split");
    static_assert((SB == 4 || SB == 2) && kScaleBytes % (64 * SB * kWaves) == 0, "scale DMA");
    static_assert(BO % 8 == 0 && BO % 32 == 0, "weight rows fill whole DMA instructions");
    static_assert(NB >= 2 && NB * kBufBytes <= 160 * 1024, "LDS");
    static_assert(kDmaPerStage * (NB - 1) <= 63, "vmcnt range");
};

struct DmaArgs {
    const uint8_t* xq;
    const uint8_t* xe;
    const uint8_t* wq;
    const uint8_t* we;
    int64_t S, k, out;
    // epilogue: optional bf16 residual [S, out] added in fp32, and bf16 output (round to
    // nearest even) instead of fp32
    const uint16_t* res;
    int out_bf16;
};

// fp32 -> bf16, round to nearest, ties to even (outputs are finite)
__device__ __forceinline__ uint32_t bf16_rne(float v)
{
    const uint32_t u = __float_as_uint(v);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Four consecutive outputs y[s][o .. o+3] (the first `valid` of them inside the matrix)
// through the epilogue; `vec`: 16-byte fp32 / 8-byte bf16 accesses are aligned and legal.
__device__ __forceinline__ void epi_store4(const DmaArgs& p, float* __restrict__ y, int64_t s,
                                           int64_t o, float v0, float v1, float v2, float v3,
                                           int valid, bool vec)
{
    float v[4] = {v0, v1, v2, v3};
    const int64_t idx = s * p.out + o;
    const bool full = vec && valid >= 4;
    if (p.res) {
        if (full) {
            const uint2 r = *reinterpret_cast<const uint2*>(p.res + idx);
            v[0] += __uint_as_float(r.x << 16);
            v[1] += __uint_as_float(r.x & 0xFFFF0000u);
            v[2] += __uint_as_float(r.y << 16);
            v[3] += __uint_as_float(r.y & 0xFFFF0000u);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (j < valid) v[j] += __uint_as_float((uint32_t)p.res[idx + j] << 16);
        }
    }
    if (p.out_bf16) {
        uint16_t* d = reinterpret_cast<uint16_t*>(y) + idx;
        if (full) {
            *reinterpret_cast<uint2*>(d) = make_uint2(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16),
                                                      bf16_rne(v[2]) | (bf16_rne(v[3]) << 16));
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (j < valid) d[j] = (uint16_t)bf16_rne(v[j]);
        }
    } else {
        float* d = y + idx;
        if (full) {
            *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (j < valid) d[j] = v[j];
        }
    }
}

// Per-lane source offsets of this wave's DMA instructions for the tile (stage 0); the
// stage offset is uniform and added to the base.  Rows past the end are clamped to the
// last row: their products land in outputs that are never stored.
template <class C>
struct DmaPlan {
    uint32_t code_off[C::kCodeDma];
    uint32_t scale_off[C::kScaleDma];
};

template <class C>
__device__ __forceinline__ void dma_plan(DmaPlan<C>& pl, const DmaArgs& p, int64_t o0,
                                         int64_t s0, int wave, int lane)
{
    const int64_t rowbytes = 16 * p.k;
#pragma unroll
    for (int i = 0; i < C::kCodeDma; ++i) {
        const int inst = wave * C::kCodeDma + i;
        const int r = inst * 8 + (lane >> 3);              // tile row of this lane
        const int c = (lane & 7) ^ ((r >> 1) & 7);        // global chunk for LDS slot lane&7
        int64_t row = r < C::BO ? o0 + r : s0 + (r - C::BO);
        const int64_t last = (r < C::BO ? p.out : p.S) - 1;
        row = row < last ? row : last;
        pl.code_off[i] = (uint32_t)(row * rowbytes + 16 * c);
    }
    if constexpr (C::TS) {
        // the unit of panel P at stage ks starts at (P*k/8 + ks)*256; lanes take 4 bytes each
#pragma unroll
        for (int j = 0; j < C::kScaleDma; ++j) {
            const int inst = wave * C::kScaleDma + j;         // panel within the tile
            const int r = inst * 32;
            int64_t row = r < C::BO ? o0 + r : s0 + (r - C::BO);
            const int64_t last = (r < C::BO ? p.out : p.S) - 1;
            row = row < last ? row : last;
            pl.scale_off[j] = (uint32_t)((row >> 5) * (p.k >> 3) * 256 + 4 * lane);
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < C::kScaleDma; ++j) {
        constexpr int kLanesPerRow = kStageBlocks / C::SB;
        const int inst = wave * C::kScaleDma + j;
        const int r = inst * (64 / kLanesPerRow) + lane / kLanesPerRow;
        int64_t row = r < C::BO ? o0 + r : s0 + (r - C::BO);
        const int64_t last = (r < C::BO ? p.out : p.S) - 1;
        row = row < last ? row : last;
        pl.scale_off[j] = (uint32_t)(row * p.k + C::SB * (lane % kLanesPerRow));
    }
}

// A raw (untyped) buffer resource over `bytes` bytes at `base` (dword 3 = 0x00020000 on gfx9):
// loads through it take a 32-bit lane offset plus a uniform offset, so the DMA issue needs no
// per-lane 64-bit address arithmetic on the SIMDs that run the MFMAs (measured: that VALU work
// slowed the DMA and the MFMAs down when they shared SIMDs); offsets past `bytes` read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const uint8_t* base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// DMA instruction d (of kDmaPerStage) of this wave for stage ks: the code instructions
// first, then the scale instructions.  The launcher guarantees every operand array is
// smaller than 4 GB.
template <class C>
__device__ __forceinline__ void dma_one(uint8_t* buf, const DmaPlan<C>& pl, const DmaArgs& p,
                                        int64_t ks, int wave, int d)
{
#if defined(__HIP_DEVICE_COMPILE__)   // the LDS-load builtins exist for the device only
    if (d < C::kCodeDma) {
        const int inst = wave * C::kCodeDma + d;
        const bool w = inst * 8 < C::BO;
        const __amdgpu_buffer_rsrc_t r =
            buffer_rsrc(w ? p.wq : p.xq, (w ? p.out : p.S) * 16 * p.k);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(buf + inst * 1024), 16,
                                                 pl.code_off[d], (int)(ks * kRowBytes), 0, 0);
    } else {
        constexpr int kRowsPerInst = C::TS ? 32 : 64 * C::SB / kStageBlocks;
        const int j = d - C::kCodeDma;
        const int inst = wave * C::kScaleDma + j;
        const bool w = inst * kRowsPerInst < C::BO;
        const int64_t rows = w ? p.out : p.S;
        const int64_t bytes = C::TS ? ((rows + 31) / 32) * 32 * p.k : rows * p.k;
        const __amdgpu_buffer_rsrc_t r = buffer_rsrc(w ? p.we : p.xe, bytes);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (lds_void_t*)(buf + C::kCodeBytes + inst * 64 * C::SB), C::SB, pl.scale_off[j],
            (int)(ks * (C::TS ? 256 : kStageBlocks)), 0, 0);
    }
#endif
}

template <class C>
__device__ __forceinline__ void dma_stage(uint8_t* buf, const DmaPlan<C>& pl, const DmaArgs& p,
                                          int64_t ks, int wave)
{
#pragma unroll
    for (int d = 0; d < C::kDmaPerStage; ++d) dma_one<C>(buf, pl, p, ks, wave, d);
}

// The DMA of a prefetched stage, issued in pieces between the MFMAs of the current one so
// that the address unit drains it while the matrix cores work (a DMA instruction holds its
// wave until the unit accepts it).
template <class C>
struct DmaIssue {
    uint8_t* buf;
    const DmaPlan<C>* pl;
    const DmaArgs* p;
    int64_t ks;
    int wave;                 // < 0: no DMA issued from this wave
    __device__ __forceinline__ void operator()(int d) const
    {
        if (wave >= 0 && d < C::kDmaPerStage) dma_one<C>(buf, *pl, *p, ks, wave, d);
    }
};

// Operand fragments of one K-step T (64 elements) out of an LDS stage, 16 bytes per lane
// per 32-row MFMA operand.
template <int TM, int TN>
struct Frags {
    uint4 a[TM];
    uint4 b[TN];
};

template <class C, int T>
__device__ __forceinline__ void dma_load_frags(Frags<C::TM, C::TN>& f, const uint8_t* buf,
                                               uint32_t wrow_off, uint32_t xrow_off, int lg,
                                               int lr7)
{
    const uint32_t pos = 16u * (uint32_t)((2 * T + lg) ^ lr7);
#pragma unroll
    for (int a = 0; a < C::TM; ++a)
        f.a[a] = *reinterpret_cast<const uint4*>(buf + wrow_off + pos + 32 * kRowBytes * a);
#pragma unroll
    for (int b = 0; b < C::TN; ++b)
        f.b[b] = *reinterpret_cast<const uint4*>(buf + xrow_off + pos + 32 * kRowBytes * b);
}

template <class C, int T>
__device__ __forceinline__ void dma_mfma_frags(v16f (&acc)[C::TM][C::TN],
                                               const Frags<C::TM, C::TN>& f,
                                               const uint32_t (&wsc)[2][C::TM],
                                               const uint32_t (&xsc)[2][C::TN],
                                               const DmaIssue<C>& dma)
{
    // DMA slots per K-step: one after each row of TN MFMAs
    constexpr int kSlots = (C::kDmaPerStage + 3) / 4;
    // tiled scales: byte T of the one dword; row-major: byte 2*(T%2) of word T/2
    constexpr int kSel = C::TS ? T : 2 * (T & 1);
    constexpr int kWord = C::TS ? 0 : T >> 1;
#pragma unroll
    for (int a = 0; a < C::TM; ++a) {
        const v8i av = {(int)f.a[a].x, (int)f.a[a].y, (int)f.a[a].z, (int)f.a[a].w, 0, 0, 0, 0};
#pragma unroll
        for (int b = 0; b < C::TN; ++b) {
            const v8i bv = {(int)f.b[b].x, (int)f.b[b].y, (int)f.b[b].z, (int)f.b[b].w, 0, 0, 0, 0};
            if constexpr (C::SW)
                acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    bv, av, acc[a][b], kFmtE2M1, kFmtE2M1, kSel, (int)xsc[kWord][b], kSel,
                    (int)wsc[kWord][a]);
            else
                acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    av, bv, acc[a][b], kFmtE2M1, kFmtE2M1, kSel, (int)wsc[kWord][a], kSel,
                    (int)xsc[kWord][b]);
        }
        // this row's share of the K-step's DMA slots
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = a * kSlots / C::TM; d < (a + 1) * kSlots / C::TM; ++d) dma(T * kSlots + d);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The four K-steps of a stage, software-pipelined: the fragments of step T+1 are requested
// from LDS before the MFMAs of step T are issued (scheduling fences keep that order), so the
// LDS latency hides behind the matrix-core work of the previous step.
template <class C>
__device__ __forceinline__ void dma_mfma_stage(v16f (&acc)[C::TM][C::TN], const uint8_t* buf,
                                               int wrow0, int xrow0, int lane,
                                               const DmaIssue<C>& dma)
{
    const int lr = lane & 31, lg = lane >> 5, lr7 = (lane >> 1) & 7;
    const uint32_t wrow_off = (uint32_t)(wrow0 + lr) * kRowBytes;
    const uint32_t xrow_off = (uint32_t)(C::BO + xrow0 + lr) * kRowBytes;
    uint32_t wsc[2][C::TM], xsc[2][C::TN];
    Frags<C::TM, C::TN> f0, f1;
    if constexpr (C::TS) {
        // tiled: lane (row, l/32) finds the blocks 2T + l/32 of its row as bytes T of one
        // dword (the row's 8 bytes are read whole, which keeps these reads distinguishable
        // from the stage DMA still in flight); both words alias it.  The fragment reads go
        // out first so the scale reads and selects overlap their latency.
        dma_load_frags<C, 0>(f0, buf, wrow_off, xrow_off, lg, lr7);
        dma_load_frags<C, 1>(f1, buf, wrow_off, xrow_off, lg, lr7);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int a = 0; a < C::TM; ++a) {
            const uint2 v = *reinterpret_cast<const uint2*>(
                buf + C::kCodeBytes + (wrow0 / 32 + a) * 256 + lr * 8);
            wsc[0][a] = wsc[1][a] = lg ? v.y : v.x;
        }
#pragma unroll
        for (int b = 0; b < C::TN; ++b) {
            const uint2 v = *reinterpret_cast<const uint2*>(
                buf + C::kCodeBytes + ((C::BO + xrow0) / 32 + b) * 256 + lr * 8);
            xsc[0][b] = xsc[1][b] = lg ? v.y : v.x;
        }
    } else {
        // row-major: the stage's 8 scale bytes of each operand row, pre-shifted so that the
        // byte select 2*(T%2) picks block 2T + lane/32 from the low (T < 2) or high word
        uint2 wv[C::TM], xv[C::TN];
#pragma unroll
        for (int a = 0; a < C::TM; ++a)
            wv[a] = *reinterpret_cast<const uint2*>(buf + C::kCodeBytes +
                                                    (wrow0 + 32 * a + lr) * kStageBlocks);
#pragma unroll
        for (int b = 0; b < C::TN; ++b)
            xv[b] = *reinterpret_cast<const uint2*>(buf + C::kCodeBytes +
                                                    (C::BO + xrow0 + 32 * b + lr) * kStageBlocks);
        dma_load_frags<C, 0>(f0, buf, wrow_off, xrow_off, lg, lr7);
        dma_load_frags<C, 1>(f1, buf, wrow_off, xrow_off, lg, lr7);
#pragma unroll
        for (int a = 0; a < C::TM; ++a) {
            wsc[0][a] = wv[a].x >> (8 * lg);
            wsc[1][a] = wv[a].y >> (8 * lg);
        }
#pragma unroll
        for (int b = 0; b < C::TN; ++b) {
            xsc[0][b] = xv[b].x >> (8 * lg);
            xsc[1][b] = xv[b].y >> (8 * lg);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    dma_mfma_frags<C, 0>(acc, f0, wsc, xsc, dma);
    __builtin_amdgcn_sched_barrier(0);
    dma_load_frags<C, 2>(f0, buf, wrow_off, xrow_off, lg, lr7);
    __builtin_amdgcn_sched_barrier(0);
    dma_mfma_frags<C, 1>(acc, f1, wsc, xsc, dma);
    __builtin_amdgcn_sched_barrier(0);
    dma_load_frags<C, 3>(f1, buf, wrow_off, xrow_off, lg, lr7);
    __builtin_amdgcn_sched_barrier(0);
    dma_mfma_frags<C, 2>(acc, f0, wsc, xsc, dma);
    __builtin_amdgcn_sched_barrier(0);
    dma_mfma_frags<C, 3>(acc, f1, wsc, xsc, dma);
}

// ---- consumer pipeline of gemm_pc_kernel ----
// The scale bytes of one stage for this lane, in the selects the MFMAs take (as in
// dma_mfma_stage).
template <class C>
struct StageScales {
    uint32_t w[2][C::TM], x[2][C::TN];
};

template <class C>
__device__ __forceinline__ void pc_read_scales(StageScales<C>& sc, const uint8_t* buf, int wrow0,
                                               int xrow0, int lr, int lg)
{
    if constexpr (C::TS) {
        // the lane's own dword of its row's 8 bytes (64 lanes, 64 distinct dwords)
#pragma unroll
        for (int a = 0; a < C::TM; ++a)
            sc.w[0][a] = sc.w[1][a] = *reinterpret_cast<const uint32_t*>(
                buf + C::kCodeBytes + (wrow0 / 32 + a) * 256 + lr * 8 + 4 * lg);
#pragma unroll
        for (int b = 0; b < C::TN; ++b)
            sc.x[0][b] = sc.x[1][b] = *reinterpret_cast<const uint32_t*>(
                buf + C::kCodeBytes + ((C::BO + xrow0) / 32 + b) * 256 + lr * 8 + 4 * lg);
    } else {
#pragma unroll
        for (int a = 0; a < C::TM; ++a) {
            const uint2 v = *reinterpret_cast<const uint2*>(buf + C::kCodeBytes +
                                                            (wrow0 + 32 * a + lr) * kStageBlocks);
            sc.w[0][a] = v.x >> (8 * lg);
            sc.w[1][a] = v.y >> (8 * lg);
        }
#pragma unroll
        for (int b = 0; b < C::TN; ++b) {
            const uint2 v = *reinterpret_cast<const uint2*>(
                buf + C::kCodeBytes + (C::BO + xrow0 + 32 * b + lr) * kStageBlocks);
            sc.x[0][b] = v.x >> (8 * lg);
            sc.x[1][b] = v.y >> (8 * lg);
        }
    }
}

// One stage of a consumer wave.  On entry f0 holds K-step 0 of `cur`, f1 K-step 1 (maybe in
// flight) and sc its scales.  The barrier that hands over the next stage sits before the
// stage's last MFMA group rather than at the start of the next stage: by then every LDS
// read of `cur` has been issued, and once they have landed (lgkmcnt(0)) the producers may
// refill `cur`'s buffer while the last MFMAs run; the next stage's scales and first
// fragments are read in their shadow, so a stage starts without waiting on LDS.
template <class C, bool kNext>
__device__ __forceinline__ void pc_stage(v16f (&acc)[C::TM][C::TN], const uint8_t* cur,
                                         const uint8_t* nxt,
                                         Frags<C::TM, C::TN>& f0, Frags<C::TM, C::TN>& f1,
                                         StageScales<C>& sc, int wrow0, int xrow0, int lane)
{
    const int lr = lane & 31, lg = lane >> 5, lr7 = (lane >> 1) & 7;
    const uint32_t wrow_off = (uint32_t)(wrow0 + lr) * kRowBytes;
    const uint32_t xrow_off = (uint32_t)(C::BO + xrow0 + lr) * kRowBytes;
    const DmaIssue<C> none{nullptr, nullptr, nullptr, 0, -1};
    dma_mfma_frags<C, 0>(acc, f0, sc.w, sc.x, none);
    __builtin_amdgcn_sched_barrier(0);
    dma_load_frags<C, 2>(f0, cur, wrow_off, xrow_off, lg, lr7);
    __builtin_amdgcn_sched_barrier(0);
    dma_mfma_frags<C, 1>(acc, f1, sc.w, sc.x, none);
    __builtin_amdgcn_sched_barrier(0);
    dma_load_frags<C, 3>(f1, cur, wrow_off, xrow_off, lg, lr7);
    __builtin_amdgcn_sched_barrier(0);
    dma_mfma_frags<C, 2>(acc, f0, sc.w, sc.x, none);
    __builtin_amdgcn_sched_barrier(0);
    StageScales<C> sn;
    if constexpr (kNext) {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
        barrier_only();
        pc_read_scales<C>(sn, nxt, wrow0, xrow0, lr, lg);
        dma_load_frags<C, 0>(f0, nxt, wrow_off, xrow_off, lg, lr7);
    }
    __builtin_amdgcn_sched_barrier(0);
    dma_mfma_frags<C, 3>(acc, f1, sc.w, sc.x, none);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kNext) {
        dma_load_frags<C, 1>(f1, nxt, wrow_off, xrow_off, lg, lr7);
        sc = sn;
    }
}

// One pipeline step: once at most the DMA instructions of the NB-2 following stages are
// still in flight for this wave, this wave's part of stage s is in `cur`; after the barrier
// all of it is, and every wave has finished reading `nxt` (stage s-1).  Stage s is then
// multiplied out of `cur` while stage s+NB-1 is fetched into `nxt` (the final stage again
// once the end is reached, so the body has no branch and the wait count is constant).
template <class C>
__device__ __forceinline__ void dma_pipeline_step(v16f (&acc)[C::TM][C::TN], uint8_t* cur,
                                                  uint8_t* nxt, const DmaPlan<C>& pl,
                                                  const DmaArgs& p, int64_t s, int64_t nst,
                                                  int wave, int wrow0, int xrow0, int lane)
{
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(C::kDmaPerStage * (C::NB - 2), 0));
    barrier_only();
    const int64_t ahead = s + C::NB - 1;
    const DmaIssue<C> dma{nxt, &pl, &p, ahead < nst ? ahead : nst - 1, wave};
    dma_mfma_stage<C>(acc, cur, wrow0, xrow0, lane, dma);
}

// Store a consumer wave's TM x TN accumulator tiles: lane l of tile (a, b) holds, in its
// register group g, y[s][o .. o+3] with s = 32b + l%32 and o = 32a + 8g + 4(l/32) relative to
// the wave's origin.
// One output through the epilogue (residual add, fp32 or bf16 store).
__device__ __forceinline__ void epi_store1(const DmaArgs& p, float* __restrict__ y, int64_t s,
                                           int64_t o, float v)
{
    const int64_t idx = s * p.out + o;
    if (p.res) v += __uint_as_float((uint32_t)p.res[idx] << 16);
    if (p.out_bf16)
        reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)bf16_rne(v);
    else
        y[idx] = v;
}

// Store of the swapped orientation (C::SW): lane l of tile (a, b) holds, in register r,
// y[s][o] with o = 32a + l%32 and s = 32b + 8(r/4) + 4(l/32) + r%4 relative to the wave's
// origin; each store instruction writes two tokens' 32 consecutive outputs.  Interior tiles
// store with the non-temporal hint: the output is written once and never read back here, so
// it should not displace operand lines that other tiles still read from the caches
// (graph-timed on one box: q_proj 25.5 -> 23.7 us, down_proj 58.9 -> 56.6 us).
template <class C>
__device__ __forceinline__ void store_tile_sw(const v16f (&acc)[C::TM][C::TN], const DmaArgs& p,
                                              float* __restrict__ y, int64_t o0, int64_t s0,
                                              int wrow0, int xrow0, int lane)
{
    const int lr = lane & 31, lg = lane >> 5;
    const bool interior = !p.res && !p.out_bf16 && o0 + C::BO <= p.out && s0 + C::BS <= p.S;
    if (interior) {
        float* base = y + (s0 + xrow0 + 4 * lg) * p.out + o0 + wrow0 + lr;
#pragma unroll
        for (int b = 0; b < C::TN; ++b) {
#pragma unroll
            for (int a = 0; a < C::TM; ++a) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    __builtin_nontemporal_store(
                        acc[a][b][r], &base[(32 * b + 8 * (r >> 2) + (r & 3)) * p.out + 32 * a]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        return;
    }
#pragma unroll
    for (int a = 0; a < C::TM; ++a) {
        const int64_t o = o0 + wrow0 + 32 * a + lr;
        if (o >= p.out) continue;
#pragma unroll
        for (int b = 0; b < C::TN; ++b) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t s = s0 + xrow0 + 32 * b + 8 * (r >> 2) + 4 * lg + (r & 3);
                if (s < p.S) epi_store1(p, y, s, o, acc[a][b][r]);
            }
        }
    }
}

template <class C>
__device__ __forceinline__ void store_tile(const v16f (&acc)[C::TM][C::TN], const DmaArgs& p,
                                           float* __restrict__ y, int64_t o0, int64_t s0,
                                           int wrow0, int xrow0, int lane)
{
    if constexpr (C::SW) {
        store_tile_sw<C>(acc, p, y, o0, s0, wrow0, xrow0, lane);
        return;
    }
    const int lr = lane & 31, lg = lane >> 5;
    if (p.res || p.out_bf16) {
        // epilogue with a residual and/or bf16 output
        const bool vec = (p.out & 3) == 0;
#pragma unroll
        for (int b = 0; b < C::TN; ++b) {
            const int64_t s = s0 + xrow0 + 32 * b + lr;
            if (s >= p.S) continue;
#pragma unroll
            for (int a = 0; a < C::TM; ++a) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t o = o0 + wrow0 + 32 * a + 8 * g + 4 * lg;
                    if (o >= p.out) continue;
                    epi_store4(p, y, s, o, acc[a][b][4 * g], acc[a][b][4 * g + 1],
                               acc[a][b][4 * g + 2], acc[a][b][4 * g + 3],
                               (int)(p.out - o < 4 ? p.out - o : 4), vec);
                }
            }
        }
        return;
    }
    const bool interior = (p.out & 3) == 0 && o0 + C::BO <= p.out && s0 + C::BS <= p.S;
    if (interior) {
        // whole tile inside the output: unconditional 16-byte stores, one 32x32 tile at a
        // time (keeps the accumulator-to-VGPR copies short-lived)
        float* base = y + (s0 + xrow0 + lr) * p.out + o0 + wrow0 + 4 * lg;
#pragma unroll
        for (int b = 0; b < C::TN; ++b) {
#pragma unroll
            for (int a = 0; a < C::TM; ++a) {
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<float4*>(base + 32 * b * p.out + 32 * a + 8 * g) =
                        make_float4(acc[a][b][4 * g], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2],
                                    acc[a][b][4 * g + 3]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        return;
    }
    const bool vec_ok = (p.out & 3) == 0;
#pragma unroll
    for (int b = 0; b < C::TN; ++b) {
        const int64_t s = s0 + xrow0 + 32 * b + lr;
        if (s >= p.S) continue;
#pragma unroll
        for (int a = 0; a < C::TM; ++a) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t o = o0 + wrow0 + 32 * a + 8 * g + 4 * lg;
                float* dst = y + s * p.out + o;
                const float v0 = acc[a][b][4 * g], v1 = acc[a][b][4 * g + 1];
                const float v2 = acc[a][b][4 * g + 2], v3 = acc[a][b][4 * g + 3];
                if (vec_ok && o + 3 < p.out) {
                    *reinterpret_cast<float4*>(dst) = make_float4(v0, v1, v2, v3);
                } else {
                    if (o < p.out) dst[0] = v0;
                    if (o + 1 < p.out) dst[1] = v1;
                    if (o + 2 < p.out) dst[2] = v2;
                    if (o + 3 < p.out) dst[3] = v3;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <class C>
__global__ void __launch_bounds__(C::kThreads)
gemm_dma_kernel(DmaArgs p, float* __restrict__ y, int64_t tiles_o, int64_t tiles_s)
{
    constexpr int NB = C::NB;
    __shared__ __attribute__((aligned(16))) uint8_t lds0[C::kBufBytes];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[C::kBufBytes];
    __shared__ __attribute__((aligned(16))) uint8_t lds2[NB > 2 ? C::kBufBytes : 16];
    __shared__ __attribute__((aligned(16))) uint8_t lds3[NB > 3 ? C::kBufBytes : 16];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wrow0 = (wave / C::WS) * (C::BO / C::WO);
    const int xrow0 = (wave % C::WS) * (C::BS / C::WS);
    int64_t o0, s0;
    tile_origin(tiles_o, tiles_s, 4, C::BO, C::BS, o0, s0);

    v16f acc[C::TM][C::TN];
#pragma unroll
    for (int a = 0; a < C::TM; ++a)
#pragma unroll
        for (int b = 0; b < C::TN; ++b) acc[a][b] = v16f{};

    const int64_t nst = p.k / kStageBlocks;
    if (nst > 0) {
        DmaPlan<C> pl;
        dma_plan<C>(pl, p, o0, s0, wave, lane);
        uint8_t* bufs[4] = {lds0, lds1, lds2, lds3};
#pragma unroll
        for (int i = 0; i < NB - 1; ++i) dma_stage<C>(bufs[i], pl, p, i < nst ? i : nst - 1, wave);
        // whole rounds of NB stages (buffers rotate), then the remainder
        const int64_t nfull = nst - nst % NB;
        int64_t s = 0;
        for (; s < nfull; s += NB) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
                dma_pipeline_step<C>(acc, bufs[i], bufs[(i + NB - 1) % NB], pl, p, s + i, nst,
                                     wave, wrow0, xrow0, lane);
        }
#pragma unroll
        for (int i = 0; i < NB - 1; ++i)
            if (s + i < nst)
                dma_pipeline_step<C>(acc, bufs[i], bufs[(i + NB - 1) % NB], pl, p, s + i, nst,
                                     wave, wrow0, xrow0, lane);
        // the trailing prefetches must land before the workgroup's LDS is released
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    }

    store_tile<C>(acc, p, y, o0, s0, wrow0, xrow0, lane);
}

// =======================================================================================
// gemm_pc_kernel<Cfg>: the same tile with producer and consumer waves
// =======================================================================================
//
// 2x the waves of the configuration: waves [0, W) multiply (the MFMA issue of a wave never
// waits on the address unit), waves [W, 2W) only stream stages into LDS with the same
// per-wave DMA split.  One barrier per stage orders the two roles: before barrier s every
// producer has waited for its part of stage s; after it, consumers multiply stage s and
// producers fetch stage s+NB-1 into the buffer consumers finished before the barrier (they
// drain their LDS reads, lgkmcnt(0), before every barrier).
template <class C>
__global__ void __launch_bounds__(2 * C::kThreads)
gemm_pc_kernel(DmaArgs p, float* __restrict__ y, int64_t tiles_o, int64_t tiles_s)
{
    constexpr int NB = C::NB;
    __shared__ __attribute__((aligned(16))) uint8_t lds0[C::kBufBytes];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[C::kBufBytes];
    __shared__ __attribute__((aligned(16))) uint8_t lds2[NB > 2 ? C::kBufBytes : 16];
    __shared__ __attribute__((aligned(16))) uint8_t lds3[NB > 3 ? C::kBufBytes : 16];
    uint8_t* bufs[4] = {lds0, lds1, lds2, lds3};

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int64_t o0, s0;
    tile_origin(tiles_o, tiles_s, 4, C::BO, C::BS, o0, s0);
    const int64_t nst = p.k / kStageBlocks;

    if (wave >= C::kWaves) {
        // ---------------- producer ----------------
        if (nst == 0) return;
        const int pw = wave - C::kWaves;
        DmaPlan<C> pl;
        dma_plan<C>(pl, p, o0, s0, pw, lane);
        const int64_t rot = k_rotation(tiles_o, tiles_s, o0, s0, C::BO, C::BS, nst);
        auto phys = [&](int64_t ks) { const int64_t t = ks + rot; return t >= nst ? t - nst : t; };
#pragma unroll
        for (int i = 0; i < NB - 1; ++i)
            dma_stage<C>(bufs[i], pl, p, phys(i < nst ? i : nst - 1), pw);
        const int64_t nfull = nst - nst % NB;
        int64_t s = 0;
        for (; s < nfull; s += NB) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(C::kDmaPerStage * (NB - 2), 0));
                barrier_only();
                const int64_t ahead = s + i + NB - 1;
                dma_stage<C>(bufs[(i + NB - 1) % NB], pl, p, phys(ahead < nst ? ahead : nst - 1),
                             pw);
            }
        }
#pragma unroll
        for (int i = 0; i < NB - 1; ++i)
            if (s + i < nst) {
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(C::kDmaPerStage * (NB - 2), 0));
                barrier_only();
                const int64_t ahead = s + i + NB - 1;
                dma_stage<C>(bufs[(i + NB - 1) % NB], pl, p, phys(ahead < nst ? ahead : nst - 1),
                             pw);
            }
        // the trailing prefetches must land before the workgroup's LDS is released
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        return;
    }

    // ---------------- consumer ----------------
    const int wrow0 = (wave / C::WS) * (C::BO / C::WO);
    const int xrow0 = (wave % C::WS) * (C::BS / C::WS);
    v16f acc[C::TM][C::TN];
#pragma unroll
    for (int a = 0; a < C::TM; ++a)
#pragma unroll
        for (int b = 0; b < C::TN; ++b) acc[a][b] = v16f{};
    if (nst > 0) {
        // barrier 0 hands over stage 0; barrier s (s >= 1) is taken inside stage s-1
        const int lr = lane & 31, lg = lane >> 5, lr7 = (lane >> 1) & 7;
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
        barrier_only();
        Frags<C::TM, C::TN> f0, f1;
        StageScales<C> sc;
        pc_read_scales<C>(sc, bufs[0], wrow0, xrow0, lr, lg);
        const uint32_t wrow_off = (uint32_t)(wrow0 + lr) * kRowBytes;
        const uint32_t xrow_off = (uint32_t)(C::BO + xrow0 + lr) * kRowBytes;
        dma_load_frags<C, 0>(f0, bufs[0], wrow_off, xrow_off, lg, lr7);
        dma_load_frags<C, 1>(f1, bufs[0], wrow_off, xrow_off, lg, lr7);
        // stages 0 .. nst-2 are followed by another (stage t lives in buffer t % NB); the
        // last one is peeled so that every buffer index stays a compile-time constant
        const int64_t nmain = nst - 1;
        const int64_t nfull = nmain - nmain % NB;
        int64_t s = 0;
        for (; s < nfull; s += NB) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
                pc_stage<C, true>(acc, bufs[i], bufs[(i + 1) % NB], f0, f1, sc, wrow0, xrow0,
                                  lane);
        }
#pragma unroll
        for (int i = 0; i < NB - 1; ++i)
            if (s + i < nmain)
                pc_stage<C, true>(acc, bufs[i], bufs[(i + 1) % NB], f0, f1, sc, wrow0, xrow0,
                                  lane);
        const int last = (int)(nmain % NB);
#pragma unroll
        for (int i = 0; i < NB; ++i)
            if (last == i)
                pc_stage<C, false>(acc, bufs[i], bufs[i], f0, f1, sc, wrow0, xrow0, lane);
    }
    store_tile<C>(acc, p, y, o0, s0, wrow0, xrow0, lane);
}

// =======================================================================================
// gemm_big_kernel<WO, WS>: persistent 256 x 256 tiles, every wave streams and multiplies
// =======================================================================================
//
// For grids of several rounds of tiles.  A 256 x 256 tile moves half the operand bytes per
// flop of a 256 x 128 one (512 rows per K element for 2 x 256 x 256 flops).  One workgroup
// per CU walks its tiles in turn (tile b, b + grid, ...), and the stage DMA runs on from one
// tile into the next, so a tile's first stages arrive while the previous one finishes and
// its output stores drain under the next tile's matrix-core work (measured with in-kernel
// timestamps: a tile's first stage waited ~6 us for its data and its stores took ~3.5-6 us
// when every tile began and ended in a round of its own).
//
// K stages are 256 elements: 128 code bytes per operand row, so each DMA instruction moves
// 8 whole 128-byte lines (a DMA probe on this chip: 54 B/clk per CU for whole lines against
// 29 for 16 half lines of 64 bytes per instruction, whatever the bytes in flight; at the
// matrix cores' full rate this tile consumes 33).  Two stage buffers of 64 KB and two 4 KB
// scale units (the MFMA-tiled layout's 256-byte unit of a 32-row panel is one stage) fill
// the LDS: during stage s the buffers hold stages s and s+1, and once every wave has read
// stage s (a barrier before its last K-step, which also finds all of stage s+1 landed) its
// buffer is refilled with stage s+2, of this tile or the next, between the last K-step's
// MFMAs.  Each wave's DMA per stage: 8 code instructions (rows 64 v .. 64 v + 63 of the
// tile, weights for waves 0-3) and two 4-byte-per-lane scale instructions (panels 2 (v % 4)
// and 2 (v % 4) + 1 of its operand), the same count for every wave, so nothing in the
// MFMA stream depends on the wave (a per-wave branch there spilled every register).
//
// LDS layout of a code buffer: tile rows 0..255 weights, 256..511 tokens, 128 bytes each;
// the 16-byte chunk c of row r sits at slot c ^ ((r / 2) % 8), the conflict-free layout of
// the tiled kernels above.  Lane offsets are the same for every tile; the tile's first row
// enters as the instruction's uniform offset, and rows past the end of an operand read
// zeros (the buffer descriptor's size), which no stored output uses.
//
// Waves: WO x WS, each owning (256/WO) x (256/WS) outputs as TM x TN 32 x 32 MFMA tiles (the
// activation tile is the MFMA row operand: line-wide epilogue stores as in the tiled
// kernels above).  Each K-step issues its MFMAs one at a time with the memory instructions
// of the wave in between (the next K-step's fragments; in the last K-step the DMA of stage
// s+2 and the next stage's scales and first fragments).
namespace big {
constexpr int BO = 256, BS = 256;
constexpr int kRowB = 128;                       // code bytes per operand row per stage
constexpr int kRows = BO + BS;
constexpr int kCodeBytes = kRows * kRowB;        // 64 KB
constexpr int kUnitBytes = (kRows / 32) * 256;   // 4 KB: the scales of one stage
}  // namespace big

template <int WO_, int WS_, bool ROT_ = true, int GO_ = 4>
struct BigCfg {
    static constexpr int WO = WO_, WS = WS_;
    static constexpr bool kRotate = ROT_;        // K rotation of the tiles (see k_rotation)
    static constexpr int kGroupO = GO_;          // weight tiles per XCD sweep (see tile_origin)
    static constexpr int BO = big::BO, BS = big::BS;
    static constexpr int kWaves = WO * WS, kThreads = 64 * kWaves;
    static constexpr int TM = BO / WO / 32, TN = BS / WS / 32;
    static constexpr int kCodeDma = big::kCodeBytes / 1024 / kWaves;   // per wave per stage
    static constexpr int kDma = kCodeDma + 2;                           // with the two scale ones
    static_assert(kWaves == 8 && kCodeDma == 8, "a wave streams 64 rows of one operand");
    static_assert(BO % (WO * 32) == 0 && BS % (WS * 32) == 0, "tiles");
    static_assert(2 * big::kCodeBytes + 2 * big::kUnitBytes <= 160 * 1024, "LDS");
};

// This wave's DMA: its operand (weights or tokens), the lane offsets of its instructions
// (the same for every tile), and the operand's bytes per row and per 32-row scale panel.
struct BigPlan {
    __amdgpu_buffer_rsrc_t code, scale;
    uint32_t code_off[8];                        // per code instruction
    uint32_t scale_off[2];                       // per scale instruction
    uint32_t row_bytes, panel_bytes;             // 16 k, 32 k
    bool weights;
};

template <class C>
__device__ __forceinline__ void big_plan(BigPlan& pl, const DmaArgs& p, int wave, int lane)
{
    const bool w = wave < 4;                     // rows 64 wave .. 64 wave + 63 of the tile
    const int64_t rows = w ? p.out : p.S;
    const int tile0 = w ? 0 : C::BO;
    pl.weights = w;
    pl.code = buffer_rsrc(w ? p.wq : p.xq, rows * 16 * p.k);
    pl.scale = buffer_rsrc(w ? p.we : p.xe, ((rows + 31) / 32) * 32 * p.k);
    pl.row_bytes = (uint32_t)(16 * p.k);
    pl.panel_bytes = (uint32_t)(32 * p.k);
#pragma unroll
    for (int i = 0; i < C::kCodeDma; ++i) {
        const int r = (wave * C::kCodeDma + i) * 8 + (lane >> 3) - tile0;   // operand row in tile
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        pl.code_off[i] = (uint32_t)r * pl.row_bytes + 16u * (uint32_t)c;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
        pl.scale_off[j] = (uint32_t)(2 * (wave & 3) + j) * pl.panel_bytes + 4u * (uint32_t)lane;
}

// A tile as the DMA sees it: the uniform byte offsets of this wave's operand rows and scale
// panels, and the K rotation of the tile's stages.
struct BigTile {
    uint32_t code_base, scale_base;
    int rot;
};

template <class C>
__device__ __forceinline__ BigTile big_tile(const BigPlan& pl, int64_t o0, int64_t s0, int rot)
{
    const uint32_t first = (uint32_t)(pl.weights ? o0 : s0);
    return BigTile{(uint32_t)__builtin_amdgcn_readfirstlane((int)(first * pl.row_bytes)),
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)((first / 32) * pl.panel_bytes)),
                   __builtin_amdgcn_readfirstlane(rot)};
}

// The LDS of the big-tile kernel: two code buffers and two scale-unit buffers, each an array
// of its own (the compiler orders an LDS read only after DMA into the same array).
__shared__ __attribute__((aligned(16))) uint8_t big_c0[big::kCodeBytes];
__shared__ __attribute__((aligned(16))) uint8_t big_c1[big::kCodeBytes];
__shared__ __attribute__((aligned(16))) uint8_t big_u0[big::kUnitBytes];
__shared__ __attribute__((aligned(16))) uint8_t big_u1[big::kUnitBytes];

template <int I>
__device__ __forceinline__ uint8_t* big_code()
{
    if constexpr (I % 2 == 0) return big_c0;
    else return big_c1;
}

template <int I>
__device__ __forceinline__ uint8_t* big_unit()
{
    if constexpr (I % 2 == 0) return big_u0;
    else return big_u1;
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 (unrolled, i a constant).
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>)
{
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Instruction D of this wave's DMA of one stage (physical stage ph of tile t) into buffer I:
// D = 0, 1 its two scale panels, D = 2 .. 9 its code rows, one call per instruction so that
// the caller can spread them between MFMAs.
template <class C, int I, int D>
__device__ __forceinline__ void big_dma(const BigPlan& pl, const BigTile& t, int ph, int wave)
{
#if defined(__HIP_DEVICE_COMPILE__)
    // the wave's byte offset in the buffer, made opaque here so that the compiler forms each
    // instruction's LDS address when it is issued instead of keeping one register per buffer
    // and instruction alive across the loop (that ran out of scalar registers)
    uint32_t woff = (uint32_t)wave;
    asm volatile("" : "+s"(woff));
    if constexpr (D < 2) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            pl.scale, (lds_void_t*)(big_unit<I>() + (2u * woff + D) * 256u), 4, pl.scale_off[D],
            (int)(t.scale_base + (uint32_t)ph * 256u), 0, 0);
    } else {
        constexpr int c = D - 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            pl.code, (lds_void_t*)(big_code<I>() + (woff * C::kCodeDma + c) * 1024), 16,
            pl.code_off[c], (int)(t.code_base + (uint32_t)ph * big::kRowB), 0, 0);
    }
#endif
}

template <int TM, int TN>
struct BigFrags {
    uint4 a[TM];      // weight fragments
    uint4 b[TN];      // token fragments
};

template <int TM, int TN>
struct BigScales {
    uint32_t w[TM], x[TN];
};

// Fragment P of K-step T (blocks 2T, 2T + 1 of the stage) in the order the MFMAs consume
// them: weight 0, tokens 0..TN-1, weights 1..TM-1.
template <class C, int T, int P>
__device__ __forceinline__ void big_frag_piece(BigFrags<C::TM, C::TN>& f, const uint8_t* buf,
                                               int wrow0, int xrow0, int lr, int lg)
{
    const uint32_t slot = 16u * (uint32_t)((2 * T + lg) ^ ((lr >> 1) & 7));
    if constexpr (P >= 1 && P <= C::TN) {
        constexpr int b = P - 1;
        f.b[b] = *reinterpret_cast<const uint4*>(buf + (C::BO + xrow0 + 32 * b + lr) * big::kRowB +
                                                 slot);
    } else {
        constexpr int a = P == 0 ? 0 : P - C::TN;
        f.a[a] = *reinterpret_cast<const uint4*>(buf + (wrow0 + 32 * a + lr) * big::kRowB + slot);
    }
}

// Scale dword R of a unit buffer for this lane: weights 0..TM-1, then tokens 0..TN-1 (the
// lane's dword of its row's 8 bytes: byte T selects K-step T).
template <class C, int R>
__device__ __forceinline__ void big_scale_piece(BigScales<C::TM, C::TN>& sc, const uint8_t* u,
                                                int wrow0, int xrow0, int lr, int lg)
{
    if constexpr (R < C::TM)
        sc.w[R] = *reinterpret_cast<const uint32_t*>(u + (wrow0 / 32 + R) * 256 + lr * 8 + 4 * lg);
    else
        sc.x[R - C::TM] = *reinterpret_cast<const uint32_t*>(
            u + ((C::BO + xrow0) / 32 + R - C::TM) * 256 + lr * 8 + 4 * lg);
}

// The TM x TN MFMAs of one K-step (SEL = the K-step's byte in the scale dwords), each
// followed by extra(i): the memory instructions issued in the matrix cores' shadow, one
// slot per MFMA, in a fixed order (scheduling fences around every piece).
template <class C, int SEL, class X>
__device__ __forceinline__ void big_kstep(v16f (&acc)[C::TM][C::TN],
                                          const BigFrags<C::TM, C::TN>& f,
                                          const BigScales<C::TM, C::TN>& sc, X&& extra)
{
    static_for<C::TM * C::TN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int a = i / C::TN, b = i % C::TN;
        const v8i av = {(int)f.a[a].x, (int)f.a[a].y, (int)f.a[a].z, (int)f.a[a].w, 0, 0, 0, 0};
        const v8i bv = {(int)f.b[b].x, (int)f.b[b].y, (int)f.b[b].z, (int)f.b[b].w, 0, 0, 0, 0};
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            bv, av, acc[a][b], kFmtE2M1, kFmtE2M1, SEL, (int)sc.x[b], SEL, (int)sc.w[a]);
        __builtin_amdgcn_sched_barrier(0);
        extra(ic);
        __builtin_amdgcn_sched_barrier(0);
    });
}

struct BigWave {
    int wave, wrow0, xrow0, lr, lg;
};

// Stage s (buffer I = s % 2).  On entry f0 holds (or is loading) K-step 0 of stage s and sc
// its scales.  K-steps 0-2 read the next K-step's fragments in their shadow.  Then the wave
// waits for its DMA of stage s+1 and its reads of stage s, and the barrier follows: all of
// stage s+1 has landed and no wave reads buffer I again.  K-step 3 issues the DMA of stage
// s+2 into buffer I (`nt`, physical stage `ph`: of this tile, the next, or, past the last,
// a refetch into a buffer never read again) and reads stage s+1's scales and K-step 0
// fragments, all between its MFMAs (after the last stage of all, reads of a buffer whose
// contents are not used).
template <class C, int I>
__device__ __forceinline__ void big_stage(v16f (&acc)[C::TM][C::TN], const BigPlan& pl,
                                          const BigWave& wv, const BigTile& nt, int ph,
                                          BigFrags<C::TM, C::TN>& f0,
                                          BigFrags<C::TM, C::TN>& f1,
                                          BigScales<C::TM, C::TN>& sc)
{
    constexpr int kPieces = C::TM + C::TN;
    constexpr int kSlots = C::TM * C::TN;
    static_assert(kPieces <= kSlots, "one fragment per MFMA slot");
    static_assert(2 * kSlots >= C::kDma && 2 * (kSlots - 1) >= 2 * kPieces, "last K-step slots");
    big_kstep<C, 0>(acc, f0, sc, [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i < kPieces)
            big_frag_piece<C, 1, i>(f1, big_code<I>(), wv.wrow0, wv.xrow0, wv.lr, wv.lg);
    });
    big_kstep<C, 1>(acc, f1, sc, [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i < kPieces)
            big_frag_piece<C, 2, i>(f0, big_code<I>(), wv.wrow0, wv.xrow0, wv.lr, wv.lg);
    });
    big_kstep<C, 2>(acc, f0, sc, [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i < kPieces)
            big_frag_piece<C, 3, i>(f1, big_code<I>(), wv.wrow0, wv.xrow0, wv.lr, wv.lg);
    });
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    barrier_only();
    BigScales<C::TM, C::TN> sn = sc;
    constexpr int J = 1 - I;
    big_kstep<C, 3>(acc, f1, sc, [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        // two DMA instructions per slot, then (from slot 1) two reads
        static_for<2>([&](auto jc) {
            constexpr int d = 2 * i + decltype(jc)::value;
            if constexpr (d < C::kDma) big_dma<C, I, d>(pl, nt, ph, wv.wave);
        });
        static_for<2>([&](auto jc) {
            constexpr int r = 2 * (i - 1) + decltype(jc)::value;
            if constexpr (i >= 1 && r < 2 * kPieces) {
                if constexpr (r < kPieces)
                    big_scale_piece<C, r>(sn, big_unit<J>(), wv.wrow0, wv.xrow0, wv.lr, wv.lg);
                else
                    big_frag_piece<C, 0, r - kPieces>(f0, big_code<J>(), wv.wrow0, wv.xrow0,
                                                      wv.lr, wv.lg);
            }
        });
    });
    sc = sn;
}

// Tile number i of the launch: XCD-aware order (as tile_origin does for one round per
// workgroup), so that the 32 tiles an XCD runs at once share operand rows.
template <int64_t group_o>
__device__ __forceinline__ void big_tile_origin(int64_t i, int64_t tiles_o, int64_t tiles_s,
                                                int64_t& o0, int64_t& s0)
{
    const int64_t total = tiles_o * tiles_s;
    int64_t id = i;
    if (total % kXcds == 0) id = (id % kXcds) * (total / kXcds) + id / kXcds;
    const int64_t span = group_o * tiles_s;
    const int64_t first_o = (id / span) * group_o;
    const int64_t gsize = tiles_o - first_o < group_o ? tiles_o - first_o : group_o;
    const int64_t rem = id % span;
    o0 = (first_o + rem % gsize) * big::BO;
    s0 = (rem / gsize) * big::BS;
}

// fp32 output of a wave's TM x TN accumulator tiles: lane l of tile (a, b) holds, in register
// r, y[s][o] with o = 32a + l%32 and s = 32b + 8(r/4) + 4(l/32) + r%4 relative to the wave's
// origin; each store instruction writes two tokens' 32 consecutive outputs, non-temporal as
// in store_tile_sw (S = 16384: N = 12288 397 -> 392 us, N = 4096 155 -> 146 us).
template <int TM, int TN>
__device__ __forceinline__ void big_store(const v16f (&acc)[TM][TN], const DmaArgs& p,
                                          float* __restrict__ y, int64_t o0, int64_t s0,
                                          const BigWave& wv, int lane)
{
    const int lr = lane & 31, lg = lane >> 5;
    const int64_t ob = o0 + wv.wrow0 + lr, sb = s0 + wv.xrow0 + 4 * lg;
    float* base = y + sb * p.out + ob;
    if (o0 + big::BO <= p.out && s0 + big::BS <= p.S) {
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int a = 0; a < TM; ++a) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    __builtin_nontemporal_store(
                        acc[a][b][r], &base[(32 * b + 8 * (r >> 2) + (r & 3)) * p.out + 32 * a]);
                __builtin_amdgcn_sched_barrier(0);
            }
        return;
    }
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t ds = 32 * b + 8 * (r >> 2) + (r & 3);
                if (ob + 32 * a < p.out && sb + ds < p.S)
                    base[ds * p.out + 32 * a] = acc[a][b][r];
            }
}

template <class C>
__global__ void __launch_bounds__(C::kThreads)
gemm_big_kernel(DmaArgs p, float* __restrict__ y, int64_t tiles_o, int64_t tiles_s)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const BigWave wv{wave, (wave / C::WS) * (C::BO / C::WO), (wave % C::WS) * (C::BS / C::WS),
                     lane & 31, lane >> 5};
    const int64_t ntiles = tiles_o * tiles_s;
    const int nst = (int)(p.k / 8);              // 256-element stages, a multiple of 4 (> 0)
    const int64_t grid = gridDim.x;
    BigPlan pl;
    big_plan<C>(pl, p, wave, lane);
    auto tile_of = [&](int64_t t, int64_t& o0, int64_t& s0) {
        big_tile_origin<C::kGroupO>(t, tiles_o, tiles_s, o0, s0);
        return big_tile<C>(pl, o0, s0,
                           C::kRotate ? (int)k_rotation(tiles_o, tiles_s, o0, s0, C::BO, C::BS, nst)
                                      : 0);
    };
    int64_t t = blockIdx.x;                      // this workgroup's tiles: t, t + grid, ...
    int64_t o0, s0;
    BigTile cur = tile_of(t, o0, s0);
    // the first tile's stages 0 and 1
    static_for<2>([&](auto ic) {
        constexpr int I = decltype(ic)::value;
        const int ph = I + cur.rot < nst ? I + cur.rot : I + cur.rot - nst;
        static_for<C::kDma>([&](auto dc) {
            big_dma<C, I, decltype(dc)::value>(pl, cur, ph, wave);
        });
    });
    // stage 0: this wave's part once stage 1 remains in flight, then all of it
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(C::kDma, 0));
    barrier_only();
    BigFrags<C::TM, C::TN> f0, f1;
    BigScales<C::TM, C::TN> sc;
    static_for<C::TM + C::TN>([&](auto rc) {
        big_scale_piece<C, decltype(rc)::value>(sc, big_unit<0>(), wv.wrow0, wv.xrow0, wv.lr, wv.lg);
    });
    static_for<C::TM + C::TN>([&](auto rc) {
        big_frag_piece<C, 0, decltype(rc)::value>(f0, big_code<0>(), wv.wrow0, wv.xrow0, wv.lr,
                                                  wv.lg);
    });

    v16f acc[C::TM][C::TN];
#pragma unroll
    for (int a = 0; a < C::TM; ++a)
#pragma unroll
        for (int b = 0; b < C::TN; ++b) acc[a][b] = v16f{};
    const int64_t my_tiles = (ntiles - t + grid - 1) / grid;
    for (int64_t it = 0; it < my_tiles; ++it) {
        const bool has_next = it + 1 < my_tiles;
        int64_t o1 = o0, s1 = s0;
        const BigTile nxt = has_next ? tile_of(t + grid, o1, s1) : cur;
        // the DMA target of stage s is stage s + 2 of this tile (all but the last two
        // stages), else stage s + 2 - nst of the next tile, else (past the last tile) this
        // tile's last stage again, into a buffer that is never read
        int s = 0;
        for (; s < nst - 2; s += 2) {
            static_for<2>([&](auto ic) {
                constexpr int I = decltype(ic)::value;
                const int q = s + I + 2 + cur.rot;
                big_stage<C, I>(acc, pl, wv, cur, q >= nst ? q - nst : q, f0, f1, sc);
            });
        }
        const int last = nst - 1 + cur.rot >= nst ? cur.rot - 1 : nst - 1 + cur.rot;
        static_for<2>([&](auto ic) {
            constexpr int I = decltype(ic)::value;
            const int q = I + nxt.rot;
            big_stage<C, I>(acc, pl, wv, nxt, has_next ? (q >= nst ? q - nst : q) : last, f0, f1,
                            sc);
        });
        big_store(acc, p, y, o0, s0, wv, lane);
#pragma unroll
        for (int a = 0; a < C::TM; ++a)
#pragma unroll
            for (int b = 0; b < C::TN; ++b) acc[a][b] = v16f{};
        t += grid;
        o0 = o1;
        s0 = s1;
        cur = nxt;
    }
    // the trailing refetches must land before the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
}

// 256 x 256 tiles, 8 waves of 128 x 64 outputs each (measured against 4 x 2 waves of
// 64 x 128, 2 or 8 weight tiles per XCD sweep, four DMA instructions per MFMA slot and no K
// rotation: each equal or slower)
using CfgBig = BigCfg<2, 4>;

// Whether the persistent big-tile kernel takes a GEMM: MFMA-tiled scales, fp32 output with no
// residual, N a multiple of 1024 (whole pairs of 256-element stages per tile, at least
// four), and at least two rounds of its tiles.  Measured against the 256 x 128
// producer/consumer kernel (graph-timed, rotated buffers, best of two), in its first form
// with 128-element stages: S = 16384, N = 12288, out = 4096 (1024 tiles) 428 -> 418 us;
// S = 16384, N = 4096 (1024 tiles) 192 -> 177 us; S = 2048, N = 4096, out = 24576 (768
// tiles) 138 -> 133 us; with 128 tiles (q_proj, down_proj: half the CUs idle) 26 -> 40 us and
// 58 -> 94 us, which is what the round count excludes.  The 256-element stages (whole-line
// DMA) against that form, same box, outputs bit-identical: 377 -> 365 us, 146 -> 140 us and
// 122 -> 117 us on the three multi-round shapes.
inline bool use_big(int64_t S, int64_t k, int64_t out, bool tiled, const uint16_t* res,
                    bool out_bf16)
{
    if (!tiled || res || out_bf16 || k % 32 != 0 || k == 0) return false;
    const int64_t tiles = ((S + 255) / 256) * ((out + 255) / 256);
    return tiles >= 2 * 256;                        // two rounds on MI355X's 256 CUs
}

using CfgQ = DmaCfg<256, 128, 2, 2, 3, false, 4, true>;    // 256 tiles for a 2048 x 4096 output
using CfgQT = DmaCfg<256, 128, 2, 2, 3, true, 4, true>;

// =======================================================================================
// gemm_generic_kernel: any N % 32 == 0, any alignment of the scale arrays
// =======================================================================================
//
// V_MFMA_SCALE_F32_16X16X128_F8F6F4: lane l holds row l%16, K block l/16; the 16x16
// result gives lane l column l%16 and rows 4(l/16)..4(l/16)+3.  128 x 128 tile, 2 x 2
// waves, K step of 128 elements (4 blocks) staged through padded LDS rows; the next step is
// fetched into registers (kept unpacked until they are written to LDS, so nothing waits on
// them early) while the current one is multiplied.  Rows past the end and K blocks past
// N/32 are zero codes, which contribute nothing whatever their scale.

constexpr int kGBO = 128, kGBS = 128;
constexpr int kGPitch = 64 + 16;

struct GenericSmem {
    uint8_t w[2][kGBO][kGPitch];
    uint8_t x[2][kGBS][kGPitch];
    uint8_t ws[2][kGBO][4];
    uint8_t xs[2][kGBS][4];
};

struct GenericStage {
    uint4 code[(kGBO + kGBS) * 4 / kThreads];
    uint32_t scale[4];
};

// Byte offset of scale (row, blk) in either layout.
__device__ __forceinline__ int64_t scale_index(int64_t row, int64_t blk, int64_t k, int tiled)
{
    return tiled ? (((row >> 5) * ((k + 7) >> 3) + (blk >> 3)) << 8) + ((row & 31) << 3) +
                       ((blk & 1) << 2) + ((blk & 7) >> 1)
                 : row * k + blk;
}

__device__ __forceinline__ void generic_load(GenericStage& st, const DmaArgs& p, int tiled,
                                             int64_t o0, int64_t s0, int64_t kt)
{
    const int tid = threadIdx.x;
    const int64_t rowbytes = 16 * p.k;
#pragma unroll
    for (int j = 0; j < (kGBO + kGBS) * 4 / kThreads; ++j) {
        const int c = tid + kThreads * j;
        const int r = c >> 2, part = c & 3;
        const int64_t blk = 4 * kt + part;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < kGBO) {
            const int64_t o = o0 + r;
            if (o < p.out && blk < p.k)
                v = *reinterpret_cast<const uint4*>(p.wq + o * rowbytes + 16 * blk);
        } else {
            const int64_t s = s0 + (r - kGBO);
            if (s < p.S && blk < p.k)
                v = *reinterpret_cast<const uint4*>(p.xq + s * rowbytes + 16 * blk);
        }
        st.code[j] = v;
    }
    const bool isw = tid < kGBO;
    const int64_t row = isw ? o0 + tid : s0 + (tid - kGBO);
    const bool ok = isw ? row < p.out : row < p.S;
    const uint8_t* src = isw ? p.we : p.xe;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int64_t blk = 4 * kt + b;
        st.scale[b] = (ok && blk < p.k) ? src[scale_index(row, blk, p.k, tiled)] : 0x7Fu;
    }
}

__device__ __forceinline__ void generic_store(GenericSmem& sm, int buf, const GenericStage& st)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < (kGBO + kGBS) * 4 / kThreads; ++j) {
        const int c = tid + kThreads * j;
        const int r = c >> 2, part = c & 3;
        uint8_t* dst = r < kGBO ? &sm.w[buf][r][16 * part] : &sm.x[buf][r - kGBO][16 * part];
        *reinterpret_cast<uint4*>(dst) = st.code[j];
    }
    const uint32_t packed = st.scale[0] | (st.scale[1] << 8) | (st.scale[2] << 16) |
                            (st.scale[3] << 24);
    uint8_t* dst = tid < kGBO ? sm.ws[buf][tid] : sm.xs[buf][tid - kGBO];
    *reinterpret_cast<uint32_t*>(dst) = packed;
}

__global__ void __launch_bounds__(kThreads)
gemm_generic_kernel(DmaArgs p, int tiled, float* __restrict__ y, int64_t tiles_o,
                    int64_t tiles_s)
{
    __shared__ GenericSmem sm;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wo = wave >> 1, wsx = wave & 1;
    int64_t o0, s0;
    tile_origin(tiles_o, tiles_s, 1, kGBO, kGBS, o0, s0);
    const int64_t ksteps = (p.k + 3) / 4;

    v4f acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

    GenericStage st;
    generic_load(st, p, tiled, o0, s0, 0);
    generic_store(sm, 0, st);
    __syncthreads();

    const int lr = lane & 15, lg = lane >> 4;
    for (int64_t kt = 0; kt < ksteps; ++kt) {
        const int buf = (int)(kt & 1);
        const bool more = kt + 1 < ksteps;
        if (more) generic_load(st, p, tiled, o0, s0, kt + 1);
        uint4 af[4], bf[4];
        int asc[4], bsc[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int r = wo * 64 + 16 * a + lr;
            af[a] = *reinterpret_cast<const uint4*>(&sm.w[buf][r][16 * lg]);
            asc[a] = sm.ws[buf][r][lg];
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int r = wsx * 64 + 16 * b + lr;
            bf[b] = *reinterpret_cast<const uint4*>(&sm.x[buf][r][16 * lg]);
            bsc[b] = sm.xs[buf][r][lg];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const v8i av = {(int)af[a].x, (int)af[a].y, (int)af[a].z, (int)af[a].w, 0, 0, 0, 0};
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const v8i bv = {(int)bf[b].x, (int)bf[b].y, (int)bf[b].z, (int)bf[b].w, 0, 0, 0, 0};
                acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    av, bv, acc[a][b], kFmtE2M1, kFmtE2M1, 0, asc[a], 0, bsc[b]);
            }
        }
        if (more) generic_store(sm, buf ^ 1, st);
        __syncthreads();
    }

    const bool vec_ok = (p.out & 3) == 0;
    const bool epi = p.res || p.out_bf16;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int64_t o = o0 + wo * 64 + 16 * a + 4 * lg;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t s = s0 + wsx * 64 + 16 * b + lr;
            if (s >= p.S) continue;
            if (epi) {
                if (o < p.out)
                    epi_store4(p, y, s, o, acc[a][b][0], acc[a][b][1], acc[a][b][2],
                               acc[a][b][3], (int)(p.out - o < 4 ? p.out - o : 4), vec_ok);
                continue;
            }
            float* dst = y + s * p.out + o;
            if (vec_ok && o + 3 < p.out) {
                *reinterpret_cast<float4*>(dst) =
                    make_float4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (o + j < p.out) dst[j] = acc[a][b][j];
            }
        }
    }
}

// =======================================================================================
// gemm_skinny_kernel<TN, TS>: few tokens (S <= 32 TN), weight-streaming bound
// =======================================================================================
//
// With S <= 64 the output is one or two 32-token columns and the work is reading the
// weights once (0.53 B per weight element) at HBM speed; a 256 x 128 tile grid would leave
// most of the chip idle.  Here a workgroup owns 32 output rows and all S tokens, and its
// kSplit waves split the K range.  Each wave streams its part of the 32 weight rows into a
// two-slot LDS ring of its own by DMA, whole 128-byte lines per request (8 rows x 128 B per
// instruction, the 16-byte chunks XOR-swizzled by row pair as in the tiled kernels), so
// every line is requested once; the tokens' codes and the scales (L2-resident) go straight
// into registers.  A stage's weight DMA and its token and scale loads are issued together,
// two stages ahead of use, and a wave reads only its own slots, so its loop has no barrier.
// It multiplies with the 32x32x64 scaled MFMA.  The kSplit partial tiles are then summed
// through LDS (reusing the ring) in wave order (a fixed order: results do not depend on
// timing) and wave (b, g) stores register group g of token column b.
constexpr int kSkinnySlotW = 32 * kRowBytes;                // 32 weight rows x 128 B

// Configuration per token-column count and token format.  XL: the token rows come through
// the LDS ring as well (loaded as MFMA fragments each line is requested four times, and
// with many distinct token rows their bytes outweigh the weights'); the waves are then as
// many as the ring's slots allow in LDS.
template <int TN, bool F8>
struct SkinnyCfg {
    // measured: through LDS for two token columns and for E4M3 tokens; one E2M1 column
    // (at most 32 distinct, mostly repeated rows) is 1-2% faster as direct fragment loads
    static constexpr bool XL = TN == 2 || F8;
    static constexpr int kXBytes = 32 * kRowBytes * (F8 ? 2 : 1);      // token rows / column
    static constexpr int kSlot = kSkinnySlotW + (XL ? TN * kXBytes : 0);
    static constexpr int kFit = (160 * 1024) / (2 * kSlot);
    static constexpr int kMaxWaves = TN == 1 ? 16 : 8;
    static constexpr int waves = !XL ? kMaxWaves : (kFit < kMaxWaves ? kFit : kMaxWaves);
    static_assert(waves >= 2 && 2 * kSlot * waves <= 160 * 1024, "ring in LDS");
};


template <int TN, bool F8, bool XL = false>
struct SkinnyStage {
    v4u x[XL ? 1 : TN][4][F8 ? 2 : 1]; // K-steps 0..3: the lane's token rows (E4M3: 32 bytes,
                                       // two halves); unused with XL
    uint2 ws;                          // scale bytes (tiled: .x only; row-major: both words)
    uint2 xs[TN];
};

// loads per stage issued by skinny_dma (+ skinny_dma_x) + skinny_load, in that order
template <int TN, bool F8, bool XL>
constexpr int kSkinnyGroup = 4 + TN * 4 * (F8 ? 2 : 1) + 1 + TN;

// The 32 weight rows of stage ks into `slot`: instruction q moves rows 8q..8q+7, lane L the
// global chunk (L%8) ^ ((row/2)%8) of row 8q + L/8 into LDS row 8q + L/8, position L%8.
__device__ __forceinline__ void skinny_dma(uint8_t* slot, const __amdgpu_buffer_rsrc_t& rw,
                                           const uint32_t (&woff)[4], int ks)
{
#if defined(__HIP_DEVICE_COMPILE__)   // the LDS-load builtins exist for the device only
#pragma unroll
    for (int q = 0; q < 4; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)(slot + q * 1024), 16,
                                                 woff[q], ks * kRowBytes, 0, 0);
#endif
}

// The token rows of stage ks for XL: column b's 32 rows into slot + b * kXBytes.  E2M1:
// 128-byte rows, as the weights (8 rows per instruction, chunk key (row/2)%8); E4M3:
// 256-byte rows, 4 rows per instruction, the 16 chunks keyed by row%16.
template <int TN, bool F8>
__device__ __forceinline__ void skinny_dma_x(uint8_t* const (&xs)[TN],
                                             const __amdgpu_buffer_rsrc_t& rx,
                                             const uint32_t (&xoff)[TN][F8 ? 8 : 4], int ks)
{
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int q = 0; q < (F8 ? 8 : 4); ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (lds_void_t*)(xs[b] + q * 1024), 16, xoff[b][q],
                ks * kRowBytes * (F8 ? 2 : 1), 0, 0);
#endif
}

template <int TN, bool TS, bool F8, bool XL = false>
__device__ __forceinline__ void skinny_load(SkinnyStage<TN, F8, XL>& st,
                                            const __amdgpu_buffer_rsrc_t& rx,
                                            const __amdgpu_buffer_rsrc_t& rwe,
                                            const __amdgpu_buffer_rsrc_t& rxe,
                                            const uint32_t (&xrow)[TN], uint32_t wse,
                                            const uint32_t (&xse)[TN], int64_t k, int ks,
                                            int lg)
{
    const uint32_t xrb = (F8 ? 32u : 16u) * (uint32_t)k;       // bytes per token code row
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t c = (uint32_t)ks * kRowBytes + 16u * (2 * t + lg);
#pragma unroll
        for (int b = 0; b < (XL ? 0 : TN); ++b) {
            if constexpr (F8) {
                // E4M3 lane half h: block 2t + h, chunks 4t + 2h and 4t + 2h + 1 of the
                // 256-byte stage row
                const uint32_t c8 = (uint32_t)ks * 2 * kRowBytes + 16u * (4 * t + 2 * lg);
                st.x[b][t][0] =
                    __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(xrow[b] * xrb + c8), 0, 0);
                st.x[b][t][1] =
                    __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(xrow[b] * xrb + c8 + 16), 0, 0);
            } else {
                st.x[b][t][0] =
                    __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(xrow[b] * xrb + c), 0, 0);
            }
        }
    }
    if constexpr (TS) {
        const uint32_t so = (uint32_t)ks * 256u;
        st.ws.x = __builtin_amdgcn_raw_buffer_load_b32(rwe, (int)(wse + so), 0, 0);
#pragma unroll
        for (int b = 0; b < TN; ++b)
            st.xs[b].x = __builtin_amdgcn_raw_buffer_load_b32(rxe, (int)(xse[b] + so), 0, 0);
    } else {
        const uint32_t so = (uint32_t)ks * kStageBlocks;
        const v2u wv = __builtin_amdgcn_raw_buffer_load_b64(rwe, (int)(wse + so), 0, 0);
        st.ws = make_uint2(wv.x, wv.y);
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            const v2u xv = __builtin_amdgcn_raw_buffer_load_b64(rxe, (int)(xse[b] + so), 0, 0);
            st.xs[b] = make_uint2(xv.x, xv.y);
        }
    }
}

template <int TN, bool TS, bool F8, bool XL, int T>
__device__ __forceinline__ void skinny_step(v16f (&acc)[TN], const uint4& w,
                                            const uint4 (&xl)[TN][F8 ? 2 : 1],
                                            const SkinnyStage<TN, F8, XL>& st, int lg)
{
    // tiled: byte T of the one dword; row-major: byte 2(T%2) of word T/2, pre-shifted so the
    // lane's half (block 2T + lane/32) sits in that byte
    constexpr int kSel = TS ? T : 2 * (T & 1);
    const uint32_t wsc = TS ? st.ws.x : (((T >> 1) ? st.ws.y : st.ws.x) >> (8 * lg));
    const v8i av = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < TN; ++b) {
        const uint32_t xsc = TS ? st.xs[b].x : (((T >> 1) ? st.xs[b].y : st.xs[b].x) >> (8 * lg));
        v4u u;
        if constexpr (XL)
            u = v4u{xl[b][0].x, xl[b][0].y, xl[b][0].z, xl[b][0].w};
        else
            u = st.x[b][T][0];
        if constexpr (F8) {
            const uint4 h = xl[b][F8 ? 1 : 0];
            const v4u v = XL ? v4u{h.x, h.y, h.z, h.w} : st.x[b][T][F8 ? 1 : 0];
            const v8i bv = {(int)u.x, (int)u.y, (int)u.z, (int)u.w,
                            (int)v.x, (int)v.y, (int)v.z, (int)v.w};
            acc[b] = w4a8_step32<true>(acc[b], v4u{w.x, w.y, w.z, w.w}, bv, wsc >> (8 * kSel),
                                       xsc >> (8 * kSel));
        } else {
            const v8i bv = {(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
            acc[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                av, bv, acc[b], kFmtE2M1, kFmtE2M1, kSel, (int)wsc, kSel, (int)xsc);
        }
    }
}

// One stage out of an LDS slot: the four weight fragments (lane: row lr, K block 2T + lg)
// are read first, then the MFMAs; every read has landed when this returns, so the slot may
// be refilled.
template <int TN, bool TS, bool F8, bool XL>
__device__ __forceinline__ void skinny_stage(v16f (&acc)[TN], const uint8_t* slot,
                                             uint8_t* const (&xs)[TN],
                                             const SkinnyStage<TN, F8, XL>& st, int lr, int lg)
{
    const uint8_t* row = slot + lr * kRowBytes;
    const int key = (lr >> 1) & 7;
    uint4 w[4], x[4][TN][F8 ? 2 : 1];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        w[t] = *reinterpret_cast<const uint4*>(row + 16 * ((2 * t + lg) ^ key));
        if constexpr (XL) {
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                const uint8_t* xr = xs[b];
                if constexpr (F8) {
                    // E4M3 lane half h: block 2t + h, chunks 4t + 2h and 4t + 2h + 1 of the
                    // 256-byte row
                    const uint8_t* r8 = xr + lr * 2 * kRowBytes;
                    x[t][b][0] =
                        *reinterpret_cast<const uint4*>(r8 + 16 * ((4 * t + 2 * lg) ^ (lr & 15)));
                    x[t][b][F8 ? 1 : 0] = *reinterpret_cast<const uint4*>(
                        r8 + 16 * ((4 * t + 2 * lg + 1) ^ (lr & 15)));
                } else {
                    x[t][b][0] = *reinterpret_cast<const uint4*>(xr + lr * kRowBytes +
                                                                 16 * ((2 * t + lg) ^ key));
                }
            }
        }
    }
    skinny_step<TN, TS, F8, XL, 0>(acc, w[0], x[0], st, lg);
    skinny_step<TN, TS, F8, XL, 1>(acc, w[1], x[1], st, lg);
    skinny_step<TN, TS, F8, XL, 2>(acc, w[2], x[2], st, lg);
    skinny_step<TN, TS, F8, XL, 3>(acc, w[3], x[3], st, lg);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    __builtin_amdgcn_sched_barrier(0);
}

// A wave's two-slot ring over its stages s0..s1-1: stage s0 + 2i in slot 0, s0 + 2i + 1 in
// slot 1, each stage's group of loads issued two stages ahead.  The steady-state loop
// refills both slots unconditionally and the last two or three stages are peeled, so that
// every wait point sees the same loads in flight on every path into it: the compiler's own
// waits (for the registers a group loads, and for the LDS its DMA writes, tracked per LDS
// array) then match the explicit ones, where a conditional refill inside the loop made
// them wait for everything in flight.  kPrimed: the caller has issued stages s0 and s0 + 1
// (the second one a refetch into slot 1 when the wave has a single stage).
template <int kGroup, bool kPrimed, class I0, class I1, class C0, class C1>
__device__ __forceinline__ void ring_pipeline(int s0, int s1, I0&& issue0, I1&& issue1,
                                              C0&& compute0, C1&& compute1)
{
    const int n = s1 - s0;
    if (n <= 0) return;
    if constexpr (!kPrimed) issue0(s0);
    if (n == 1) {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
        compute0(s0);
        return;
    }
    if constexpr (!kPrimed) issue1(s0 + 1);
    int s = s0;
    for (; s + 3 < s1; s += 2) {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(kGroup, 15));
        compute0(s);
        issue0(s + 2);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(kGroup, 15));
        compute1(s + 1);
        issue1(s + 3);
    }
    if (s + 2 < s1) {                     // three stages left
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(kGroup, 15));
        compute0(s);
        issue0(s + 2);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(kGroup, 15));
        compute1(s + 1);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
        compute0(s + 2);
    } else {                              // two stages left
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(kGroup, 15));
        compute0(s);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
        compute1(s + 1);
    }
}

// F8: the tokens' codes are E4M3 (one byte per element, the W4A8 setting)
template <int TN, bool TS, bool F8 = false>
__global__ void __launch_bounds__((64 * SkinnyCfg<TN, F8>::waves))
gemm_skinny_kernel(DmaArgs p, float* __restrict__ y)
{
    constexpr bool XL = SkinnyCfg<TN, F8>::XL;
    constexpr int kSplit = SkinnyCfg<TN, F8>::waves;
    constexpr int kXBytes = SkinnyCfg<TN, F8>::kXBytes;             // token rows / column
    constexpr int kRingBytes = kSplit * kSkinnySlotW;              // weight rows, one slot
    constexpr int kXRing = XL ? kSplit * kXBytes : 16;             // token rows, one slot
    static_assert(kSplit * 16 * 64 * 4 <= kRingBytes, "a column's reduction in one array");
    static_assert(2 * (kRingBytes + TN * kXRing) <= 160 * 1024 || !XL, "ring in LDS");
    // every region the DMA writes in an array of its own (weight rows of slot 0 and 1, token
    // column b of slot 0 and 1): the compiler keeps one representative DMA per array and
    // orders a read after the DMA into the same array, so a slot's reads do not wait for
    // the other slot's refill
    __shared__ __attribute__((aligned(16))) uint8_t smem[kRingBytes];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[kRingBytes];
    __shared__ __attribute__((aligned(16))) uint8_t x00[kXRing], x10[kXRing];
    __shared__ __attribute__((aligned(16))) uint8_t x01[TN > 1 ? kXRing : 16];
    __shared__ __attribute__((aligned(16))) uint8_t x11[TN > 1 ? kXRing : 16];
    constexpr int kGroup = kSkinnyGroup<TN, F8, XL>;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lr = lane & 31, lg = lane >> 5;
    // more than 32 tokens with one token column: two workgroups per 32-row tile, one per
    // 32-token half, the pair on one XCD (workgroup i runs on XCD i % 8) so that both read
    // the tile's weight lines from the same L2
    int64_t tile = blockIdx.x, tb = 0;
    if (TN == 1 && p.S > 32) {
        const int64_t g = (int64_t)blockIdx.x >> 4, r = blockIdx.x & 15;
        tile = g * 8 + (r & 7);
        tb = 32 * (r >> 3);
        if (tile * 32 >= p.out) return;                   // the grid is rounded up to 16
    }
    const int64_t o0 = tile * 32;
    const int64_t k = p.k;
    const int nst = (int)(k / kStageBlocks);
    const int s0 = (int)((int64_t)wave * nst / kSplit), s1 = (int)((int64_t)(wave + 1) * nst / kSplit);

    // operand rows of this lane, clamped to the last row (their products are never stored)
    const uint32_t wrow = (uint32_t)(o0 + lr < p.out ? o0 + lr : p.out - 1);
    uint32_t xrow[TN];
#pragma unroll
    for (int b = 0; b < TN; ++b)
        xrow[b] = (uint32_t)(tb + 32 * b + lr < p.S ? tb + 32 * b + lr : p.S - 1);
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(p.wq, p.out * 16 * k);
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(p.xq, p.S * (F8 ? 32 : 16) * k);
    const int64_t k8 = k / 8;
    const __amdgpu_buffer_rsrc_t rwe =
        buffer_rsrc(p.we, TS ? ((p.out + 31) / 32) * 256 * k8 : p.out * k);
    const __amdgpu_buffer_rsrc_t rxe =
        buffer_rsrc(p.xe, TS ? ((p.S + 31) / 32) * 256 * k8 : p.S * k);
    // scale offsets of stage 0: tiled (panel unit, row, half) / row-major (row start)
    const uint32_t wse = TS ? (uint32_t)((wrow >> 5) * k8 * 256 + (wrow & 31) * 8 + 4 * lg)
                            : wrow * (uint32_t)k;
    uint32_t xse[TN];
#pragma unroll
    for (int b = 0; b < TN; ++b)
        xse[b] = TS ? (uint32_t)((xrow[b] >> 5) * k8 * 256 + (xrow[b] & 31) * 8 + 4 * lg)
                    : xrow[b] * (uint32_t)k;
    // weight DMA offsets (stage 0) of this lane's four instructions
    uint32_t woff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = 8 * q + (lane >> 3);
        const int64_t row = o0 + r < p.out ? o0 + r : p.out - 1;
        woff[q] = (uint32_t)(row * 16 * k + 16 * ((lane & 7) ^ ((r >> 1) & 7)));
    }
    // token-row DMA offsets (XL): column b, instruction q
    uint32_t xoff[TN][F8 ? 8 : 4];
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int q = 0; q < (F8 ? 8 : 4); ++q) {
            const int r = F8 ? 4 * q + (lane >> 4) : 8 * q + (lane >> 3);
            const int64_t row = tb + 32 * b + r < p.S ? tb + 32 * b + r : p.S - 1;
            xoff[b][q] = F8 ? (uint32_t)(row * 32 * k + 16 * ((lane & 15) ^ (r & 15)))
                            : (uint32_t)(row * 16 * k + 16 * ((lane & 7) ^ ((r >> 1) & 7)));
        }
    uint8_t* slot0 = smem + wave * kSkinnySlotW;
    uint8_t* slot1 = ring1 + wave * kSkinnySlotW;
    const int xw = XL ? wave * kXBytes : 0;
    uint8_t* xs0[TN];
    uint8_t* xs1[TN];
    xs0[0] = x00 + xw;
    xs1[0] = x10 + xw;
    if constexpr (TN > 1) {
        xs0[TN - 1] = x01 + xw;
        xs1[TN - 1] = x11 + xw;
    }
    auto issue = [&](uint8_t* slot, uint8_t* const (&xs)[TN], SkinnyStage<TN, F8, XL>& st,
                     int ks) {
        skinny_dma(slot, rw, woff, ks);
        if constexpr (XL) skinny_dma_x<TN, F8>(xs, rx, xoff, ks);
        skinny_load<TN, TS, F8, XL>(st, rx, rwe, rxe, xrow, wse, xse, k, ks, lg);
    };

    v16f acc[TN];
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[b] = v16f{};
    {
        // stage s0 + 2i in (slot0, st0), s0 + 2i + 1 in (slot1, st1); a stage's group is
        // issued two stages ahead, so at most one other group is in flight at each wait
        SkinnyStage<TN, F8, XL> st0, st1;
        ring_pipeline<kGroup, false>(
            s0, s1, [&](int ks) { issue(slot0, xs0, st0, ks); },
            [&](int ks) { issue(slot1, xs1, st1, ks); },
            [&](int) { skinny_stage<TN, TS, F8, XL>(acc, slot0, xs0, st0, lr, lg); },
            [&](int) { skinny_stage<TN, TS, F8, XL>(acc, slot1, xs1, st1, lr, lg); });
    }
    // every wave's DMA has landed (its last wait was vmcnt(0)); the weight arrays become the
    // reduction buffers (token column b in slot b's) once all waves are past their last read
    __syncthreads();
    auto red = [&](int b) {
        return reinterpret_cast<float (*)[16][64]>(b == 0 ? smem : ring1);
    };
    // sum the kSplit partial tiles in wave order
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) red(b)[wave][r][lane] = acc[b][r];
    __syncthreads();
    // (token column b, register group g) pairs, kSplit waves taking them in turn
    for (int bg = wave; bg < 4 * TN; bg += kSplit) {
        const int b = bg / 4, g = bg % 4;
        float (*rb)[16][64] = red(b);
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float t = rb[0][4 * g + i][lane];
#pragma unroll
            for (int w = 1; w < kSplit; ++w) t += rb[w][4 * g + i][lane];
            v[i] = t;
        }
        const int64_t srow = tb + 32 * b + lr;
        const int64_t o = o0 + 8 * g + 4 * lg;
        if (srow < p.S && (p.res || p.out_bf16)) {
            if (o < p.out)
                epi_store4(p, y, srow, o, v[0], v[1], v[2], v[3],
                           (int)(p.out - o < 4 ? p.out - o : 4), (p.out & 3) == 0);
        } else if (srow < p.S) {
            float* dst = y + srow * p.out + o;
            if ((p.out & 3) == 0 && o + 3 < p.out) {
                *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (o + i < p.out) dst[i] = v[i];
            }
        }
    }
}


// =======================================================================================
// gemm_w4a8_kernel<TS>: MXFP8 (E4M3) activations x MXFP4 weights, the W4A8 setting
// =======================================================================================
//
// Both operands dequantised to bf16 in registers and multiplied on the 32x32x16 bf16 MFMA
// (exact products, see w4a8_step32): per 64-position K-step, lane half h holds block h of the
// step in both operands, and four bf16 MFMAs cover it.  Tile 256 (out) x 128 (tokens), four
// waves (2 x 2, each 4 x 2 MFMA tiles) at one wave per SIMD, so the 8-dword activation
// fragments, their bf16 forms and the accumulators fit in registers; each wave
// issues its quarter of the next stage's DMA between the MFMA rows of the current stage's
// first K-step; two stages in LDS, one barrier per stage.  A stage is 8
// blocks: 256 weight rows of 128 bytes, 128 activation rows of 256 bytes, then the scale
// bytes (384 rows x 8; tiled: 12 panel units of 256 bytes).  Chunk c (16 bytes) of a weight
// row r sits at slot c ^ ((r / 2) % 8), as in the W4A4 kernels; an activation row fills a
// whole 256-byte bank row, so its chunks are keyed by r % 16.  67 KB per stage, two stages.
namespace w4a8 {
constexpr int BO = 256, BS = 128, WO = 2, WS = 2, TM = 4, TN = 2;
constexpr int kWaves = WO * WS;
constexpr int kXRowBytes = 2 * kRowBytes;                     // 256
constexpr int kWBytes = BO * kRowBytes;                       // 32 KB
constexpr int kCodeBytes = kWBytes + BS * kXRowBytes;         // 64 KB
constexpr int kScaleBytes = (BO + BS) * kStageBlocks;         // 3 KB
constexpr int kBufBytes = kCodeBytes + kScaleBytes;
constexpr int kCodeDma = kCodeBytes / 1024 / kWaves;          // 16 per producer wave
constexpr int kScaleDma = kScaleBytes / 256 / kWaves;         // 3 (4 bytes per lane)
constexpr int kDma = kCodeDma + kScaleDma;
static_assert(kCodeBytes % (1024 * kWaves) == 0 && kScaleBytes % (256 * kWaves) == 0, "split");
static_assert(2 * kBufBytes <= 160 * 1024 && kDma <= 63, "LDS / vmcnt");
}  // namespace w4a8

template <bool TS>
struct W4A8Plan {
    uint32_t code_off[w4a8::kCodeDma];
    uint32_t scale_off[w4a8::kScaleDma];
};

template <bool TS>
__device__ __forceinline__ void w4a8_plan(W4A8Plan<TS>& pl, const DmaArgs& p, int64_t o0,
                                          int64_t s0, int pw, int lane)
{
    using namespace w4a8;
    const int64_t k = p.k;
#pragma unroll
    for (int i = 0; i < kCodeDma; ++i) {
        const int inst = pw * kCodeDma + i;            // 1 KB of LDS each
        if (inst * 1024 < kWBytes) {
            const int r = inst * 8 + (lane >> 3);     // 8 weight rows per instruction
            int64_t row = o0 + r;
            row = row < p.out ? row : p.out - 1;
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            pl.code_off[i] = (uint32_t)(row * 16 * k + 16 * c);
        } else {
            const int r = (inst - kWBytes / 1024) * 4 + (lane >> 4);   // 4 activation rows
            int64_t row = s0 + r;
            row = row < p.S ? row : p.S - 1;
            const int c = (lane & 15) ^ (r & 15);
            pl.code_off[i] = (uint32_t)(row * 32 * k + 16 * c);
        }
    }
#pragma unroll
    for (int j = 0; j < kScaleDma; ++j) {
        const int inst = pw * kScaleDma + j;           // 256 bytes of LDS each
        // tiled: one 32-row panel unit per instruction; row-major: 32 rows x 8 bytes
        const int r = inst * 32 + (TS ? 0 : lane >> 1);
        int64_t row = r < BO ? o0 + r : s0 + (r - BO);
        const int64_t last = (r < BO ? p.out : p.S) - 1;
        row = row < last ? row : last;
        pl.scale_off[j] = TS ? (uint32_t)((row >> 5) * (k >> 3) * 256 + 4 * lane)
                             : (uint32_t)(row * k + 4 * (lane & 1));
    }
}

// DMA instruction d (of kDma) of wave `wave` for stage ks: code instructions, then scales.
template <bool TS>
__device__ __forceinline__ void w4a8_dma_one(uint8_t* buf, const W4A8Plan<TS>& pl,
                                             const DmaArgs& p, int64_t ks, int wave, int d)
{
#if defined(__HIP_DEVICE_COMPILE__)   // the LDS-load builtins exist for the device only
    using namespace w4a8;
    const int64_t k = p.k;
    if (d < kCodeDma) {
        const int inst = wave * kCodeDma + d;
        const bool w = inst * 1024 < kWBytes;
        const __amdgpu_buffer_rsrc_t r =
            w ? buffer_rsrc(p.wq, p.out * 16 * k) : buffer_rsrc(p.xq, p.S * 32 * k);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(buf + inst * 1024), 16,
                                                 pl.code_off[d],
                                                 (int)(ks * (w ? kRowBytes : kXRowBytes)), 0, 0);
    } else {
        const int j = d - kCodeDma;
        const int inst = wave * kScaleDma + j;
        const int64_t k8 = k / 8;
        const __amdgpu_buffer_rsrc_t r =
            inst * 32 < BO ? buffer_rsrc(p.we, TS ? ((p.out + 31) / 32) * 256 * k8 : p.out * k)
                           : buffer_rsrc(p.xe, TS ? ((p.S + 31) / 32) * 256 * k8 : p.S * k);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(buf + kCodeBytes + inst * 256),
                                                 4, pl.scale_off[j],
                                                 (int)(ks * (TS ? 256 : kStageBlocks)), 0, 0);
    }
#endif
}

template <bool TS>
struct W4A8Issue {
    uint8_t* buf;
    const W4A8Plan<TS>* pl;
    const DmaArgs* p;
    int64_t ks;
    int wave;
    __device__ __forceinline__ void operator()(int d) const
    {
        if (d < w4a8::kDma) w4a8_dma_one<TS>(buf, *pl, *p, ks, wave, d);
    }
};

struct W4A8Frags {
    v4u a[w4a8::TM];       // 16 bytes of the lane's weight row
    v8i b[w4a8::TN];       // 32 bytes of the lane's token row
};

// Fragments of K-step T (the step's two blocks: lane half h holds block 2T + h): the 16 bytes
// of the block in the lane's weight row and all 32 bytes of it in the lane's token row
// (16-byte chunks 4T + 2h and 4T + 2h + 1 of the 256-byte stage row).
template <int T>
__device__ __forceinline__ void w4a8_frags(W4A8Frags& f, const uint8_t* buf, int wrow0, int xrow0,
                                           int lr, int lg)
{
    using namespace w4a8;
    const int lr7 = (lr >> 1) & 7, lr15 = lr & 15;
    const uint32_t wpos = 16u * (uint32_t)((2 * T + lg) ^ lr7);
    const uint32_t x0 = 16u * (uint32_t)((4 * T + 2 * lg) ^ lr15);
    const uint32_t x1 = 16u * (uint32_t)((4 * T + 2 * lg + 1) ^ lr15);
#pragma unroll
    for (int a = 0; a < TM; ++a)
        f.a[a] = *reinterpret_cast<const v4u*>(buf + (wrow0 + 32 * a + lr) * kRowBytes + wpos);
#pragma unroll
    for (int b = 0; b < TN; ++b) {
        const uint8_t* row = buf + kWBytes + (xrow0 + 32 * b + lr) * kXRowBytes;
        const v4i lo = *reinterpret_cast<const v4i*>(row + x0);
        const v4i hi = *reinterpret_cast<const v4i*>(row + x1);
        f.b[b] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// The bf16 operands of a K-step that the next one's MFMAs start from: the tokens (all four
// MFMAs' worth) and weight tile 0.
struct W4A8Cvt {
    v8bf x[w4a8::TN][4];
    v8bf w0[4];
};

// Conversion piece P of K-step T's first operands (tokens b = P / 4, q = P % 4, then weight
// tile 0 q = P - 4 TN).
template <bool TS, int T, int P>
__device__ __forceinline__ void w4a8_first_piece(W4A8Cvt& c, const W4A8Frags& f,
                                                 const uint32_t (&wsc)[2][w4a8::TM],
                                                 const uint32_t (&xsc)[2][w4a8::TN])
{
    using namespace w4a8;
    constexpr int kSel = TS ? T : 2 * (T & 1);
    constexpr int kWord = TS ? 0 : T >> 1;
    if constexpr (P < 4 * TN) {
        constexpr int b = P / 4, q = P % 4;
        c.x[b][q] = dequant_e4m3_bf16(f.b[b], q, e8m0_operand((xsc[kWord][b] >> (8 * kSel)) & 0xFFu));
    } else if constexpr (P < 4 * TN + 4) {
        constexpr int q = P - 4 * TN;
        c.w0[q] = dequant_e2m1_bf16(f.a[0], q, e8m0_operand((wsc[kWord][0] >> (8 * kSel)) & 0xFFu));
    }
}

template <bool TS, int T>
__device__ __forceinline__ void w4a8_first(W4A8Cvt& c, const W4A8Frags& f,
                                           const uint32_t (&wsc)[2][w4a8::TM],
                                           const uint32_t (&xsc)[2][w4a8::TN])
{
    static_for<4 * w4a8::TN + 4>([&](auto pc) {
        w4a8_first_piece<TS, T, decltype(pc)::value>(c, f, wsc, xsc);
    });
}

// K-step T: 4 TM TN bf16 MFMAs from `cur` (tokens, weight tile 0) and the step's weight
// fragments, software-pipelined on the one wave of its SIMD: between the MFMAs of weight tile
// a the wave converts tile a+1, and between those of the last tile, when kNext, the next
// K-step's tokens and weight tile 0 (from `fn`) into `nxt`.  The MFMAs run out of registers
// converted a group earlier, so the conversions fill the matrix core's shadow instead of
// stopping it (graph-timed against converting each group right before its MFMAs: S=16384
// N=12288 1355 -> 1334 us, S=2048 N=12288 181 -> 174, three other shapes within +-1.3%).
// The next stage's DMA is issued in K-step 0, its instructions spread over the slots that
// follow each weight tile, so it has the stage's other three K-steps to land before the
// wait that opens the next stage (spread over all four K-steps, the last requests went out
// one weight tile before that wait: S=16384 N=12288 1286 -> 1242 us, N=4096 464 -> 450,
// S=2048 N=12288 167 -> 163, outputs bit-identical).
template <bool TS, int T, bool kNext>
__device__ __forceinline__ void w4a8_mfma(v16f (&acc)[w4a8::TM][w4a8::TN], const W4A8Frags& f,
                                          const W4A8Cvt& cur, const W4A8Frags& fn, W4A8Cvt& nxt,
                                          const uint32_t (&wsc)[2][w4a8::TM],
                                          const uint32_t (&xsc)[2][w4a8::TN],
                                          const W4A8Issue<TS>& dma)
{
    using namespace w4a8;
    constexpr int kSel = TS ? T : 2 * (T & 1);
    constexpr int kWord = TS ? 0 : T >> 1;
    v8bf wv[2][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) wv[0][q] = cur.w0[q];
    static_for<TM>([&](auto ac) {
        constexpr int a = decltype(ac)::value;
        const float swn =
            a + 1 < TM ? e8m0_operand((wsc[kWord][a + 1 < TM ? a + 1 : 0] >> (8 * kSel)) & 0xFFu)
                       : 0.0f;
        static_for<4 * TN>([&](auto mc) {
            constexpr int m = decltype(mc)::value, q = m / TN, b = m % TN;
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.x[b][q], wv[a % 2][q],
                                                                acc[a][b], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (a + 1 < TM) {
                if constexpr (b == TN - 1)
                    wv[(a + 1) % 2][q] = dequant_e2m1_bf16(f.a[a + 1], q, swn);
            } else if constexpr (kNext) {
                // 4 TN + 4 pieces over 4 TN MFMAs: piece m, then piece m + 4 TN
                w4a8_first_piece<TS, T + 1, m>(nxt, fn, wsc, xsc);
                w4a8_first_piece<TS, T + 1, m + 4 * TN>(nxt, fn, wsc, xsc);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (T == 0) {
#pragma unroll
            for (int d = a * kDma / TM; d < (a + 1) * kDma / TM; ++d) dma(d);
        }
        __builtin_amdgcn_sched_barrier(0);
    });
}

// The four K-steps of a stage, the fragments of step T+1 requested before the MFMAs of T.
template <bool TS>
__device__ __forceinline__ void w4a8_stage(v16f (&acc)[w4a8::TM][w4a8::TN], const uint8_t* buf,
                                           int wrow0, int xrow0, int lane,
                                           const W4A8Issue<TS>& dma)
{
    using namespace w4a8;
    const int lr = lane & 31, lg = lane >> 5;
    uint32_t wsc[2][TM], xsc[2][TN];
    W4A8Frags f0, f1;
    w4a8_frags<0>(f0, buf, wrow0, xrow0, lr, lg);
    w4a8_frags<1>(f1, buf, wrow0, xrow0, lr, lg);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (TS) {
        // lane (row, half) finds blocks 2T + half of its row as bytes T of one dword
#pragma unroll
        for (int a = 0; a < TM; ++a) {
            const uint2 v = *reinterpret_cast<const uint2*>(buf + kCodeBytes +
                                                            (wrow0 / 32 + a) * 256 + lr * 8);
            wsc[0][a] = wsc[1][a] = lg ? v.y : v.x;
        }
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            const uint2 v = *reinterpret_cast<const uint2*>(
                buf + kCodeBytes + ((BO + xrow0) / 32 + b) * 256 + lr * 8);
            xsc[0][b] = xsc[1][b] = lg ? v.y : v.x;
        }
    } else {
        // the row's 8 scale bytes, shifted so byte 2(T%2) of word T/2 is block 2T + half
#pragma unroll
        for (int a = 0; a < TM; ++a) {
            const uint2 v = *reinterpret_cast<const uint2*>(
                buf + kCodeBytes + (wrow0 + 32 * a + lr) * kStageBlocks);
            wsc[0][a] = v.x >> (8 * lg);
            wsc[1][a] = v.y >> (8 * lg);
        }
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            const uint2 v = *reinterpret_cast<const uint2*>(
                buf + kCodeBytes + (BO + xrow0 + 32 * b + lr) * kStageBlocks);
            xsc[0][b] = v.x >> (8 * lg);
            xsc[1][b] = v.y >> (8 * lg);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // K-step 0's tokens and weight tile 0 before its MFMAs; every later K-step's are
    // converted under the previous K-step's last MFMAs
    W4A8Cvt c0, c1;
    w4a8_first<TS, 0>(c0, f0, wsc, xsc);
    __builtin_amdgcn_sched_barrier(0);
    w4a8_mfma<TS, 0, true>(acc, f0, c0, f1, c1, wsc, xsc, dma);
    __builtin_amdgcn_sched_barrier(0);
    w4a8_frags<2>(f0, buf, wrow0, xrow0, lr, lg);
    __builtin_amdgcn_sched_barrier(0);
    w4a8_mfma<TS, 1, true>(acc, f1, c1, f0, c0, wsc, xsc, dma);
    __builtin_amdgcn_sched_barrier(0);
    w4a8_frags<3>(f1, buf, wrow0, xrow0, lr, lg);
    __builtin_amdgcn_sched_barrier(0);
    w4a8_mfma<TS, 2, true>(acc, f0, c0, f1, c1, wsc, xsc, dma);
    __builtin_amdgcn_sched_barrier(0);
    w4a8_mfma<TS, 3, false>(acc, f1, c1, f0, c0, wsc, xsc, dma);
}

// Tile config for the shared epilogue (store_tile reads BO, BS, TM, TN only).
using CfgW4A8 = DmaCfg<256, 128, 2, 2, 2, true, 4, true>;

template <bool TS>
__global__ void __launch_bounds__(64 * w4a8::kWaves)
gemm_w4a8_kernel(DmaArgs p, float* __restrict__ y, int64_t tiles_o, int64_t tiles_s)
{
    using namespace w4a8;
    __shared__ __attribute__((aligned(16))) uint8_t lds0[kBufBytes];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[kBufBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wrow0 = (wave / WS) * (BO / WO);
    const int xrow0 = (wave % WS) * (BS / WS);
    int64_t o0, s0;
    tile_origin(tiles_o, tiles_s, 4, BO, BS, o0, s0);
    const int64_t nst = p.k / kStageBlocks;

    v16f acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = v16f{};
    if (nst > 0) {
        W4A8Plan<TS> pl;
        w4a8_plan<TS>(pl, p, o0, s0, wave, lane);
#pragma unroll
        for (int d = 0; d < kDma; ++d) w4a8_dma_one<TS>(lds0, pl, p, 0, wave, d);
        // stage s is multiplied out of one buffer while stage s+1 (the last stage again at
        // the end, so every pass issues the same DMA) streams into the other
        for (int64_t s = 0; s < nst; s += 2) {
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
            barrier_only();
            w4a8_stage<TS>(acc, lds0, wrow0, xrow0, lane,
                           W4A8Issue<TS>{lds1, &pl, &p, s + 1 < nst ? s + 1 : nst - 1, wave});
            if (s + 1 >= nst) break;
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
            barrier_only();
            w4a8_stage<TS>(acc, lds1, wrow0, xrow0, lane,
                           W4A8Issue<TS>{lds0, &pl, &p, s + 2 < nst ? s + 2 : nst - 1, wave});
        }
        // the trailing prefetch must land before the workgroup's LDS is released
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    }
    store_tile<CfgW4A8>(acc, p, y, o0, s0, wrow0, xrow0, lane);
}

// =======================================================================================
// gemm_linear_skinny_kernel<TS>: the whole linear layer for at most four tokens
// =======================================================================================
//
// With S <= 4 the activation quantiser is a launch of its own for a few hundred blocks; here
// the few-token GEMM encodes the tokens itself.  Each workgroup (kLinWaves waves splitting
// K, as gemm_skinny_kernel) first puts its waves' first two weight stages in flight, then
// its lanes transform, clip and encode every block of the S token rows (mx::encode_block,
// the quantiser's own arithmetic, so the codes are bit for bit batq_quantize_act's) into
// a shared LDS buffer, and after a barrier streams the weights as gemm_skinny_kernel does,
// taking the token fragments and scales from that buffer.  Every workgroup encodes the
// same rows (S k blocks, at most three per lane): that costs VALU time the first weight
// stages' latency mostly hides, and saves the quantiser's launch and the codes' round trip.
constexpr int kLinTokens = 4, kLinWaves = 12, kLinMaxK = 512;

template <bool TS>
__global__ void __launch_bounds__(64 * kLinWaves)
gemm_linear_skinny_kernel(DmaArgs p, const uint16_t* __restrict__ x, int64_t ldx,
                          const float* __restrict__ A, const float* __restrict__ B,
                          const float* __restrict__ r_min, const float* __restrict__ r_max,
                          float* __restrict__ y)
{
    constexpr int kRingBytes = kLinWaves * kSkinnySlotW;           // one slot of each wave
    constexpr int kRowStride = kLinMaxK * 16 + 16;                // token code row in LDS
    constexpr int kCodeBytes = kLinTokens * kRowStride;
    constexpr int kRedBytes = kLinWaves * 16 * 64 * 4;
    static_assert(kRedBytes <= kRingBytes, "reduction reuses the first slots");
    // four arrays: the compiler orders an LDS access only after the DMA into the same array,
    // so with each slot and the token buffers in arrays of their own, the encoder's stores
    // and a slot's reads wait for that slot's DMA, not for the other slot's in flight
    __shared__ __attribute__((aligned(16))) uint8_t smem[kRingBytes];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[kRingBytes];
    __shared__ __attribute__((aligned(16))) uint8_t xcode[kCodeBytes];
    __shared__ __attribute__((aligned(16))) uint8_t xscale[kLinTokens * kLinMaxK];
    constexpr int kGroup = 4 + 1;                                 // weight DMA + scale load
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lr = lane & 31, lg = lane >> 5;
    const int64_t o0 = (int64_t)blockIdx.x * 32;
    const int64_t k = p.k, S = p.S;
    const int nst = (int)(k / kStageBlocks);
    const int s0 = (int)((int64_t)wave * nst / kLinWaves);
    const int s1 = (int)((int64_t)(wave + 1) * nst / kLinWaves);

    const uint32_t wrow = (uint32_t)(o0 + lr < p.out ? o0 + lr : p.out - 1);
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(p.wq, p.out * 16 * k);
    const int64_t k8 = k / 8;
    const __amdgpu_buffer_rsrc_t rwe =
        buffer_rsrc(p.we, TS ? ((p.out + 31) / 32) * 256 * k8 : p.out * k);
    const uint32_t wse = TS ? (uint32_t)((wrow >> 5) * k8 * 256 + (wrow & 31) * 8 + 4 * lg)
                            : wrow * (uint32_t)k;
    uint32_t woff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = 8 * q + (lane >> 3);
        const int64_t row = o0 + r < p.out ? o0 + r : p.out - 1;
        woff[q] = (uint32_t)(row * 16 * k + 16 * ((lane & 7) ^ ((r >> 1) & 7)));
    }
    uint8_t* slot0 = smem + wave * kSkinnySlotW;
    uint8_t* slot1 = ring1 + wave * kSkinnySlotW;
    // a stage's group: the weight DMA, then the lane's weight-scale load
    auto issue = [&](uint8_t* slot, uint2& ws, int ks) {
        skinny_dma(slot, rw, woff, ks);
        if constexpr (TS) {
            ws.x = __builtin_amdgcn_raw_buffer_load_b32(rwe, (int)(wse + (uint32_t)ks * 256u), 0, 0);
        } else {
            const v2u v = __builtin_amdgcn_raw_buffer_load_b64(
                rwe, (int)(wse + (uint32_t)ks * kStageBlocks), 0, 0);
            ws = make_uint2(v.x, v.y);
        }
    };
    uint2 ws0 = make_uint2(0, 0), ws1 = make_uint2(0, 0);

    // encode the S token rows into LDS: block q = t k + b, lanes of the workgroup in turn.
    // The token loads go out before the first two weight stages: vector-memory loads retire
    // in issue order, so the encoder then waits for its own rows only, and the weight
    // stages stream in while it runs.
    {
        const uint32_t tid = threadIdx.x, k32 = (uint32_t)k;
        const uint32_t nblk = (uint32_t)(S * k);                  // at most 4 * 512
        constexpr int kPer = (kLinTokens * kLinMaxK + 64 * kLinWaves - 1) / (64 * kLinWaves);
        uint4 xv[kPer][4];
        mx::BlockParams bp[kPer];
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const uint32_t q = tid + (uint32_t)m * 64 * kLinWaves;
            if (q < nblk) {
                const uint32_t t = q / k32, b = q - t * k32;
                bp[m] = mx::load_block_params<true, 0>(B, r_min, r_max, b);
                const uint4* xp = reinterpret_cast<const uint4*>(x + t * ldx + 32 * b);
#pragma unroll
                for (int i = 0; i < 4; ++i) xv[m][i] = xp[i];
            }
        }
        // issued by every wave, so that the compiler's wait for the token rows counts the
        // same ten younger loads on every path; a wave with fewer than two stages of its
        // own refetches the last stage into a slot it never reads
        issue(slot0, ws0, s0 < nst ? s0 : nst - 1);
        issue(slot1, ws1, s0 + 1 < nst ? s0 + 1 : nst - 1);
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const uint32_t q = tid + (uint32_t)m * 64 * kLinWaves;
            if (q < nblk) {
                const uint32_t t = q / k32, b = q - t * k32;
                float xf[32];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t w4[4] = {xv[m][i].x, xv[m][i].y, xv[m][i].z, xv[m][i].w};
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        xf[8 * i + 2 * d] = mx::bf16_lo(w4[d]);
                        xf[8 * i + 2 * d + 1] = mx::bf16_hi(w4[d]);
                    }
                }
                const mx::BlockCode<false> c = mx::encode_block<true, false, 0>(xf, A, bp[m], b);
                *reinterpret_cast<uint4*>(xcode + t * kRowStride + 16 * b) =
                    make_uint4(c.w[0], c.w[1], c.w[2], c.w[3]);
                // the group's 8 bytes in the MFMA-tiled order (block b at (b%2)*4 + (b%8)/2)
                xscale[t * k + 8 * (b >> 3) + ((b & 1) << 2) + ((b & 7) >> 1)] = (uint8_t)c.ebyte;
            }
        }
    }
    // the token buffers are complete once every wave's LDS stores have: a bare barrier after
    // lgkmcnt(0), which leaves the weight stages in flight (the loop waits for them itself)
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    barrier_only();

    const int xr = lr < S ? lr : (int)S - 1;                      // token row of this lane
    const uint8_t* xrow = xcode + xr * kRowStride;
    const uint8_t* xsrow = xscale + xr * k + 4 * lg;
    v16f acc = v16f{};
    auto stage = [&](const uint8_t* slot, const uint2& ws, int ks) {
        const uint8_t* row = slot + lr * kRowBytes;
        const int key = (lr >> 1) & 7;
        uint4 w[4], xv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            w[t] = *reinterpret_cast<const uint4*>(row + 16 * ((2 * t + lg) ^ key));
            xv[t] = *reinterpret_cast<const uint4*>(xrow + 16 * (8 * ks + 2 * t + lg));
        }
        const uint32_t xsc = *reinterpret_cast<const uint32_t*>(xsrow + 8 * ks);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            // weight scale byte: tiled, byte t of the one dword; row-major, byte 2(t%2) of
            // word t/2 pre-shifted by the lane's half; token scales: byte t (tiled order)
            const uint32_t wsc = TS ? ws.x : (((t >> 1) ? ws.y : ws.x) >> (8 * lg));
            const v8i av = {(int)w[t].x, (int)w[t].y, (int)w[t].z, (int)w[t].w, 0, 0, 0, 0};
            const v8i bv = {(int)xv[t].x, (int)xv[t].y, (int)xv[t].z, (int)xv[t].w, 0, 0, 0, 0};
            switch (t) {   // the byte selects are immediates
            case 0:
                acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    av, bv, acc, kFmtE2M1, kFmtE2M1, 0, (int)wsc, 0, (int)xsc);
                break;
            case 1:
                acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    av, bv, acc, kFmtE2M1, kFmtE2M1, TS ? 1 : 2, (int)wsc, 1, (int)xsc);
                break;
            case 2:
                acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    av, bv, acc, kFmtE2M1, kFmtE2M1, TS ? 2 : 0, (int)wsc, 2, (int)xsc);
                break;
            default:
                acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    av, bv, acc, kFmtE2M1, kFmtE2M1, TS ? 3 : 2, (int)wsc, 3, (int)xsc);
                break;
            }
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
        __builtin_amdgcn_sched_barrier(0);
    };
    ring_pipeline<kGroup, true>(
        s0, s1, [&](int ks) { issue(slot0, ws0, ks); }, [&](int ks) { issue(slot1, ws1, ks); },
        [&](int ks) { stage(slot0, ws0, ks); }, [&](int ks) { stage(slot1, ws1, ks); });
    // the partial tiles summed through LDS (the ring, reused) in wave order, once every
    // wave's stage DMA (the unused refetches included) has landed
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
    __syncthreads();
    float (*red)[16][64] = reinterpret_cast<float (*)[16][64]>(smem);
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    if (wave < 4) {
        const int g = wave;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float t = red[0][4 * g + i][lane];
#pragma unroll
            for (int w = 1; w < kLinWaves; ++w) t += red[w][4 * g + i][lane];
            v[i] = t;
        }
        const int64_t o = o0 + 8 * g + 4 * lg;
        if (lr < S) {
            float* dst = y + lr * p.out + o;
            if ((p.out & 3) == 0 && o + 3 < p.out) {
                *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (o + i < p.out) dst[i] = v[i];
            }
        }
    }
}

// =======================================================================================
// gemm_skinny16_kernel<TS, F8>: at most 16 tokens, 16 output rows per workgroup
// =======================================================================================
//
// The few-token GEMM is weight streaming, and its time is the HBM round trips of each
// workgroup's weight panel.  With 32 output rows per workgroup an out = 4096 layer has 128
// workgroups (half the CUs) and, at N = 12288, a panel (196 KB) larger than LDS, so part of
// it waits for a slot to free: a second round trip.  Here a workgroup owns 16 output rows
// (the 16x16x128 scaled MFMA: lane l holds row l%16 and K block l/16 of a 128-element
// K-step), so out = 4096 gives 256 workgroups, and the whole panel (16 rows x 16 k bytes, at
// most 128 KB up to k = 512) is requested at once: each of the kS16Waves waves issues the
// LDS DMA of every stage of its K range together with its token fragments and scales, waits
// once, and multiplies.  The partial tiles are summed through LDS in wave order.  Tokens
// (at most 16) are one MFMA column, loaded as fragments straight into registers: E2M1 16
// bytes per lane (K block l/16); E4M3 the whole 32-byte block l/16, multiplied as four
// bf16 16x16x32 MFMAs (w4a8_step16); a lane's scale byte belongs to K block l/16 either way.
constexpr int kS16Rows = 16, kS16Waves = 8, kS16MaxK = 512, kS16MaxTokens = 16;
constexpr int kS16Stage = kS16Rows * kRowBytes;               // one 128-byte line per row
constexpr int kS16Per = kS16MaxK / kStageBlocks / kS16Waves;  // stages per wave, at most

// dynamic LDS bytes of a launch: the panel, or the reduction buffer if that is larger
inline size_t s16_lds_bytes(int64_t k)
{
    const size_t panel = (size_t)(k / kStageBlocks) * kS16Stage;
    const size_t red = (size_t)kS16Waves * 4 * 64 * 4;
    return panel > red ? panel : red;
}

// Whether the 16-row kernel takes a few-token GEMM (S <= 16, k <= 512).  A workgroup's
// time is about one round trip of its panel (the 32-row kernel's: one or two, its panel
// beyond 128 KB from k = 384 on), so the counts of workgroup rounds decide: rounds =
// ceil(workgroups / (CUs x workgroups per CU)), bounded for the 16-row kernel by the
// panel's LDS and by registers (one for E4M3 tokens, 162 VGPRs x 8 waves; two for E2M1),
// one 32-row workgroup per CU.  Measured on S = 1, 8, N = 4096..16384, out = 4096..12288:
// no more rounds than the 32-row grid is faster (up to 32%, out = 4096 and 12288 at short
// K) but for a few 5% cases; more rounds is 5-13% slower, except at three rounds or more
// (out = 12288): 7-14% faster with E2M1 tokens, 9-15% with one E4M3 token (3-4% slower
// with eight, whose 32-byte rows every workgroup reads again).
constexpr int kNumCUs = 256;                                  // MI355X

// 33..64 tokens: the one-column 32-row kernel on two token halves per tile when the doubled
// grid still fits in one round of workgroups (out <= 4096), else the two-column kernel.
// Measured (S = 33, 48, 64; N = 4096, 12288): at out = 4096 the halves are 8-13% faster with
// E2M1 tokens and 20-30% with E4M3 (16 waves instead of 6 or 4, all CUs); at out = 12288
// they take two rounds instead of one and are up to 24% slower (E2M1).
inline bool skinny_halves(int64_t S, int64_t tiles32)
{
    return S > 32 && 2 * tiles32 <= kNumCUs;
}
inline bool use_skinny16(int64_t S, int64_t k, int64_t out, bool f8)
{
    if (S > kS16MaxTokens || k > kS16MaxK) return false;
    const int64_t by_lds = (int64_t)((160 * 1024) / s16_lds_bytes(k));
    const int64_t per_cu = by_lds < (f8 ? 1 : 2) ? by_lds : (f8 ? 1 : 2);
    const int64_t tiles = (out + kS16Rows - 1) / kS16Rows;
    const int64_t rounds = (tiles + kNumCUs * per_cu - 1) / (kNumCUs * per_cu);
    const int64_t rounds32 = ((out + 31) / 32 + kNumCUs - 1) / kNumCUs;
    return rounds <= rounds32 || (rounds >= 3 && (!f8 || S <= 4));
}

template <bool TS, bool F8>
__global__ void __launch_bounds__(64 * kS16Waves)
gemm_skinny16_kernel(DmaArgs p, float* __restrict__ y)
{
    // dynamic LDS: the panel of this launch's K (k / 8 stages of 2 KB, at least the 8 KB of
    // the reduction), so that several workgroups share a CU when K is short
    extern __shared__ __attribute__((aligned(16))) uint8_t panel[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t o0 = (int64_t)blockIdx.x * kS16Rows;
    const int64_t k = p.k, k8 = k / 8;
    const int nst = (int)(k / kStageBlocks);
    const int s0 = wave * nst / kS16Waves, n = (wave + 1) * nst / kS16Waves - s0;

    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(p.wq, p.out * 16 * k);
    (void)rw;                                   // used by the device-only LDS loads
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(p.xq, p.S * (F8 ? 32 : 16) * k);
    const __amdgpu_buffer_rsrc_t rwe =
        buffer_rsrc(p.we, TS ? ((p.out + 31) / 32) * 256 * k8 : p.out * k);
    const __amdgpu_buffer_rsrc_t rxe =
        buffer_rsrc(p.xe, TS ? ((p.S + 31) / 32) * 256 * k8 : p.S * k);
    // DMA: instruction q moves rows 8q..8q+7, lane L the global chunk (L%8) ^ ((row/2)%8) of
    // row 8q + L/8 into position L%8 of that row's 128 bytes (rows past `out` clamped)
    uint32_t woff[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = 8 * q + (lane >> 3);
        const int64_t row = o0 + r < p.out ? o0 + r : p.out - 1;
        woff[q] = (uint32_t)(row * 16 * k + 16 * ((lane & 7) ^ ((r >> 1) & 7)));
    }
    const uint32_t wrow = (uint32_t)(o0 + lr < p.out ? o0 + lr : p.out - 1);
    const uint32_t xrow = (uint32_t)(lr < p.S ? lr : p.S - 1);
    // scales of stage 0: tiled, the dword of the row's 8 bytes that holds blocks with the
    // lane's parity (blocks 4j + lg of the stage sit at byte 4 (lg%2) + 2j + lg/2);
    // row-major, the row's 8 bytes of the stage (block 4j + lg at byte 4j + lg)
    const uint32_t wse = TS ? (uint32_t)((wrow >> 5) * k8 * 256 + (wrow & 31) * 8 + 4 * (lg & 1))
                            : wrow * (uint32_t)k;
    const uint32_t xse = TS ? (uint32_t)((xrow >> 5) * k8 * 256 + (xrow & 31) * 8 + 4 * (lg & 1))
                            : xrow * (uint32_t)k;
    const uint32_t xrb = (F8 ? 32u : 16u) * (uint32_t)k;          // token code row bytes

    v4u xf[kS16Per][2][F8 ? 2 : 1];
    uint2 ws[kS16Per], xs[kS16Per];
#pragma unroll
    for (int i = 0; i < kS16Per; ++i) {
        if (i < n) {
            const int ks = s0 + i;
#if defined(__HIP_DEVICE_COMPILE__)   // the LDS-load builtins exist for the device only
#pragma unroll
            for (int q = 0; q < 2; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rw, (lds_void_t*)(panel + ks * kS16Stage + q * 1024), 16, woff[q],
                    ks * kRowBytes, 0, 0);
#endif
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if constexpr (F8) {
                    // E4M3 lane group g: all 32 bytes of block 4j + g of the stage
                    const uint32_t c = xrow * xrb + (uint32_t)ks * 256u + 128u * j + 32u * lg;
                    xf[i][j][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)c, 0, 0);
                    xf[i][j][F8 ? 1 : 0] =
                        __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(c + 16), 0, 0);
                } else {
                    const uint32_t c = xrow * xrb + (uint32_t)ks * kRowBytes + 64u * j + 16u * lg;
                    xf[i][j][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)c, 0, 0);
                }
            }
            if constexpr (TS) {
                ws[i].x = __builtin_amdgcn_raw_buffer_load_b32(rwe, (int)(wse + (uint32_t)ks * 256u), 0, 0);
                xs[i].x = __builtin_amdgcn_raw_buffer_load_b32(rxe, (int)(xse + (uint32_t)ks * 256u), 0, 0);
            } else {
                const v2u a = __builtin_amdgcn_raw_buffer_load_b64(rwe, (int)(wse + (uint32_t)ks * 8u), 0, 0);
                const v2u b = __builtin_amdgcn_raw_buffer_load_b64(rxe, (int)(xse + (uint32_t)ks * 8u), 0, 0);
                ws[i] = make_uint2(a.x, a.y);
                xs[i] = make_uint2(b.x, b.y);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));

    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
    const int key = (lr >> 1) & 7;
#pragma unroll
    for (int i = 0; i < kS16Per; ++i) {
        if (i < n) {
            const uint8_t* row = panel + (s0 + i) * kS16Stage + lr * kRowBytes;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint4 a = *reinterpret_cast<const uint4*>(row + 16 * ((4 * j + lg) ^ key));
                const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
                const v4u u = xf[i][j][0];
                // tiled: byte 2j of the dword pre-shifted by the lane's lg/2; row-major: byte
                // 0 of word j pre-shifted by lg
                const uint32_t wsc = TS ? ws[i].x >> (8 * (lg >> 1)) : (j ? ws[i].y : ws[i].x) >> (8 * lg);
                const uint32_t xsc = TS ? xs[i].x >> (8 * (lg >> 1)) : (j ? xs[i].y : xs[i].x) >> (8 * lg);
                if constexpr (F8) {
                    const v4u v = xf[i][j][F8 ? 1 : 0];
                    const v8i bv = {(int)u.x, (int)u.y, (int)u.z, (int)u.w,
                                    (int)v.x, (int)v.y, (int)v.z, (int)v.w};
                    const int sel = (j && TS) ? 16 : 0;
                    acc = w4a8_step16(acc, v4u{a.x, a.y, a.z, a.w}, bv, wsc >> sel, xsc >> sel);
                } else {
                    const v8i bv = {(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
                    if (j == 0)
                        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            av, bv, acc, kFmtE2M1, kFmtE2M1, 0, (int)wsc, 0, (int)xsc);
                    else
                        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            av, bv, acc, kFmtE2M1, kFmtE2M1, TS ? 2 : 0, (int)wsc, TS ? 2 : 0,
                            (int)xsc);
                }
            }
        }
    }

    // the partial tiles summed through LDS (the panel, reused) in wave order
    __syncthreads();
    float (*red)[4][64] = reinterpret_cast<float (*)[4][64]>(panel);
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][i][lane] = acc[i];
    __syncthreads();
    if (wave == 0) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float t = red[0][i][lane];
#pragma unroll
            for (int w = 1; w < kS16Waves; ++w) t += red[w][i][lane];
            v[i] = t;
        }
        const int64_t o = o0 + 4 * lg;
        if (lr < p.S && (p.res || p.out_bf16)) {
            if (o < p.out)
                epi_store4(p, y, lr, o, v[0], v[1], v[2], v[3],
                           (int)(p.out - o < 4 ? p.out - o : 4), (p.out & 3) == 0);
        } else if (lr < p.S) {
            float* dst = y + lr * p.out + o;
            if ((p.out & 3) == 0 && o + 3 < p.out) {
                *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (o + i < p.out) dst[i] = v[i];
            }
        }
    }
}

// =======================================================================================
// gemm_linear16_kernel<TS, NPER>: the layer in one kernel on 16-row workgroups
// =======================================================================================
//
// gemm_skinny16_kernel's structure (16 output rows per workgroup, 16x16x128 scaled MFMA, the
// whole weight panel in flight at once) with the token rows encoded in the kernel, as
// gemm_linear_skinny_kernel does: the lanes' token loads go out first, then every wave's
// weight stages (NPER each; a wave past the last stage refetches it into a scratch slot, so
// every wave issues the same loads and the wait before the encoder counts them exactly),
// then the lanes encode the S k blocks into LDS while the panel streams in.  The token
// buffers are static arrays, apart from the dynamic panel, so the encoder's stores do not
// wait for the weight DMA.  Token fragments and scales then come from LDS (scale bytes in
// plain order, one per lane).  S k <= kLin16MaxSK, so that panel and buffers fit in LDS.
// F8: the tokens encoded to MXFP8 (E4M3, 32 bytes per block: the W4A8 layer), lane group g
// taking block 4j + g whole as in gemm_skinny16_kernel, S k <= kLin16MaxSK8.  W: waves per workgroup
// (E2M1 tokens: 16 when one round of workgroups covers `out`, the encoding spread over
// twice the lanes, measured 7-9% faster there, and 8 otherwise, where 16 measured 3-7%
// slower; E4M3 tokens: 8, where 16 measured up to 25% slower).
constexpr int kLin16MaxSK = 1536, kLin16MaxSK8 = 768;

template <bool TS, int NPER, bool F8 = false, int W = kS16Waves>
__global__ void __launch_bounds__(64 * W)
gemm_linear16_kernel(DmaArgs p, const uint16_t* __restrict__ x, int64_t ldx,
                     const float* __restrict__ A, const float* __restrict__ B,
                     const float* __restrict__ r_min, const float* __restrict__ r_max,
                     float* __restrict__ y)
{
    constexpr int kMaxSK = F8 ? kLin16MaxSK8 : kLin16MaxSK;
    constexpr int kCB = F8 ? 32 : 16;                             // code bytes per block
    __shared__ __attribute__((aligned(16))) uint8_t xcode[kMaxSK * kCB];
    __shared__ __attribute__((aligned(16))) uint8_t xscale[kMaxSK];
    extern __shared__ __attribute__((aligned(16))) uint8_t panel[];   // nst stages + scratch
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lr = lane & 15, lg = lane >> 4;
    const int64_t o0 = (int64_t)blockIdx.x * kS16Rows;
    const int64_t k = p.k, k8 = k / 8, S = p.S;
    const int nst = (int)(k / kStageBlocks);
    const int s0 = wave * NPER;

    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(p.wq, p.out * 16 * k);
    (void)rw;                                   // used by the device-only LDS loads
    const __amdgpu_buffer_rsrc_t rwe =
        buffer_rsrc(p.we, TS ? ((p.out + 31) / 32) * 256 * k8 : p.out * k);
    // 32-bit offsets (out * 16 k < 2^32): a 64-bit product truncated here made the compiler
    // read a register still being loaded as its unused high half, a wait ahead of the DMA
    uint32_t woff[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = 8 * q + (lane >> 3);
        const uint32_t row = (uint32_t)(o0 + r < p.out ? o0 + r : p.out - 1);
        woff[q] = row * (uint32_t)(16 * k) + 16u * ((lane & 7) ^ ((r >> 1) & 7));
    }
    const uint32_t wrow = (uint32_t)(o0 + lr < p.out ? o0 + lr : p.out - 1);
    const uint32_t wse = TS ? (uint32_t)((wrow >> 5) * k8 * 256 + (wrow & 31) * 8 + 4 * (lg & 1))
                            : wrow * (uint32_t)k;

    // token loads first: block q = t k + b, lanes of the workgroup in turn
    constexpr int kPer = (kMaxSK + 64 * W - 1) / (64 * W);
    const uint32_t tid = threadIdx.x, k32 = (uint32_t)k, nblk = (uint32_t)(S * k);
    uint4 xv[kPer][4];
    mx::BlockParams bp[kPer];
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
        const uint32_t q = tid + (uint32_t)m * 64 * W;
        if (q < nblk) {
            const uint32_t t = q / k32, b = q - t * k32;
            bp[m] = mx::load_block_params<true, 0>(B, r_min, r_max, b);
            const uint4* xp = reinterpret_cast<const uint4*>(x + t * ldx + 32 * b);
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[m][i] = xp[i];
        }
    }
    // then the wave's NPER weight stages (past the last stage: a refetch into the scratch slot)
    uint2 ws[NPER];
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
        const int ks = s0 + i < nst ? s0 + i : nst - 1;
        uint8_t* dst = panel + (s0 + i < nst ? ks : nst) * kS16Stage;
        (void)dst;
#if defined(__HIP_DEVICE_COMPILE__)   // the LDS-load builtins exist for the device only
#pragma unroll
        for (int q = 0; q < 2; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)(dst + q * 1024), 16,
                                                     woff[q], ks * kRowBytes, 0, 0);
#endif
        if constexpr (TS) {
            ws[i].x = __builtin_amdgcn_raw_buffer_load_b32(rwe, (int)(wse + (uint32_t)ks * 256u), 0, 0);
        } else {
            const v2u a = __builtin_amdgcn_raw_buffer_load_b64(rwe, (int)(wse + (uint32_t)ks * 8u), 0, 0);
            ws[i] = make_uint2(a.x, a.y);
        }
    }
    // encode the token blocks into LDS (codes row-major, scale bytes in plain order)
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
        const uint32_t q = tid + (uint32_t)m * 64 * W;
        if (q < nblk) {
            const uint32_t t = q / k32, b = q - t * k32;
            float xf[32];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w4[4] = {xv[m][i].x, xv[m][i].y, xv[m][i].z, xv[m][i].w};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    xf[8 * i + 2 * d] = mx::bf16_lo(w4[d]);
                    xf[8 * i + 2 * d + 1] = mx::bf16_hi(w4[d]);
                }
            }
            const mx::BlockCode<F8> c = mx::encode_block<true, F8, 0>(xf, A, bp[m], b);
            *reinterpret_cast<uint4*>(xcode + kCB * q) = make_uint4(c.w[0], c.w[1], c.w[2], c.w[3]);
            if constexpr (F8)
                *reinterpret_cast<uint4*>(xcode + kCB * q + 16) =
                    make_uint4(c.w[F8 ? 4 : 0], c.w[F8 ? 5 : 1], c.w[F8 ? 6 : 2], c.w[F8 ? 7 : 3]);
            xscale[q] = (uint8_t)c.ebyte;
        }
    }
    // the token buffers are complete once every wave's LDS stores have; the weight stages
    // stay in flight across the barrier, and each wave then waits for its own
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    barrier_only();
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));

    const uint32_t xr = (uint32_t)(lr < S ? lr : S - 1);
    const uint8_t* xrow = xcode + kCB * xr * k32;
    const uint8_t* xsrow = xscale + xr * k32;
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
    const int key = (lr >> 1) & 7;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
        if (s0 + i < nst) {
            const int ks = s0 + i;
            const uint8_t* row = panel + ks * kS16Stage + lr * kRowBytes;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int blk = 8 * ks + 4 * j + lg;
                const uint4 a = *reinterpret_cast<const uint4*>(row + 16 * ((4 * j + lg) ^ key));
                const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
                const uint32_t wsc = TS ? ws[i].x >> (8 * (lg >> 1)) : (j ? ws[i].y : ws[i].x) >> (8 * lg);
                const uint32_t xsc = xsrow[blk];
                if constexpr (F8) {
                    // E4M3 lane group g: all 32 bytes of block 4j + g of the K-step
                    const uint8_t* kb = xrow + kCB * blk;
                    const uint4 u = *reinterpret_cast<const uint4*>(kb);
                    const uint4 v = *reinterpret_cast<const uint4*>(kb + 16);
                    const v8i bv = {(int)u.x, (int)u.y, (int)u.z, (int)u.w,
                                    (int)v.x, (int)v.y, (int)v.z, (int)v.w};
                    acc = w4a8_step16(acc, v4u{a.x, a.y, a.z, a.w}, bv,
                                      wsc >> ((j && TS) ? 16 : 0), xsc);
                } else {
                    const uint4 u = *reinterpret_cast<const uint4*>(xrow + kCB * blk);
                    const v8i bv = {(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
                    if (j == 0)
                        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            av, bv, acc, kFmtE2M1, kFmtE2M1, 0, (int)wsc, 0, (int)xsc);
                    else
                        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            av, bv, acc, kFmtE2M1, kFmtE2M1, TS ? 2 : 0, (int)wsc, 0, (int)xsc);
                }
            }
        }
    }

    // the partial tiles summed through LDS (the panel, reused) in wave order
    __syncthreads();
    float (*red)[4][64] = reinterpret_cast<float (*)[4][64]>(panel);
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][i][lane] = acc[i];
    __syncthreads();
    if (wave == 0 && lr < S) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float t = red[0][i][lane];
#pragma unroll
            for (int w = 1; w < W; ++w) t += red[w][i][lane];
            v[i] = t;
        }
        const int64_t o = o0 + 4 * lg;
        float* dst = y + lr * p.out + o;
        if ((p.out & 3) == 0 && o + 3 < p.out) {
            *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (o + i < p.out) dst[i] = v[i];
        }
    }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* xq, const uint8_t* xe, const uint8_t* wq,
                       const uint8_t* we, bool tiled_scales, int64_t S, int64_t N,
                       int64_t out, float* y, hipStream_t stream, const uint16_t* res,
                       bool out_bf16)
{
    const DmaArgs p{xq, xe, wq, we, S, N / 32, out, res, out_bf16 ? 1 : 0};
    const uintptr_t salign = tiled_scales ? 256 : 8;
    const bool dma_ok = (p.k % kStageBlocks) == 0 &&
                        (reinterpret_cast<uintptr_t>(xe) % salign) == 0 &&
                        (reinterpret_cast<uintptr_t>(we) % salign) == 0 &&
                        S * 16 * p.k < (1LL << 32) && out * 16 * p.k < (1LL << 32);
    if (dma_ok && use_skinny16(S, p.k, out, false)) {
        // at most 16 tokens: 16-row workgroups, the whole weight panel requested at once
        const int64_t tiles_o = (out + kS16Rows - 1) / kS16Rows;
        if (tiles_o > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        const size_t lds = s16_lds_bytes(p.k);
        if (tiled_scales)
            hipLaunchKernelGGL((gemm_skinny16_kernel<true, false>), dim3((unsigned)tiles_o),
                               dim3(64 * kS16Waves), lds, stream, p, y);
        else
            hipLaunchKernelGGL((gemm_skinny16_kernel<false, false>), dim3((unsigned)tiles_o),
                               dim3(64 * kS16Waves), lds, stream, p, y);
        return hipGetLastError();
    }
    if (dma_ok && S <= 64) {
        // few tokens: weight streaming, K split across the waves of a 32-row workgroup
        const int64_t tiles_o = (out + 31) / 32;
        if (tiles_o > 0x7FFFFFFF / 2) return hipErrorInvalidConfiguration;
        const dim3 grid((unsigned)tiles_o);
        if (S <= 32 || skinny_halves(S, tiles_o)) {
            // one token column; 33..64 tokens as two halves per tile (the grid rounded up
            // to whole groups of 8 tiles)
            const dim3 grid1((unsigned)(S <= 32 ? tiles_o : (tiles_o + 7) / 8 * 16));
            const dim3 block(64 * SkinnyCfg<1, false>::waves);
            if (tiled_scales)
                hipLaunchKernelGGL((gemm_skinny_kernel<1, true>), grid1, block, 0, stream, p, y);
            else
                hipLaunchKernelGGL((gemm_skinny_kernel<1, false>), grid1, block, 0, stream, p, y);
        } else {
            const dim3 block(64 * SkinnyCfg<2, false>::waves);
            if (tiled_scales)
                hipLaunchKernelGGL((gemm_skinny_kernel<2, true>), grid, block, 0, stream, p, y);
            else
                hipLaunchKernelGGL((gemm_skinny_kernel<2, false>), grid, block, 0, stream, p, y);
        }
        return hipGetLastError();
    }
    if (dma_ok && use_big(S, p.k, out, tiled_scales, res, out_bf16)) {
        // several rounds of 256 x 256 tiles: the persistent big-tile kernel
        const int64_t tiles_o = (out + CfgBig::BO - 1) / CfgBig::BO;
        const int64_t tiles_s = (S + CfgBig::BS - 1) / CfgBig::BS;
        const int64_t grid = tiles_o * tiles_s < kNumCUs ? tiles_o * tiles_s : kNumCUs;
        hipLaunchKernelGGL(gemm_big_kernel<CfgBig>, dim3((unsigned)grid),
                           dim3(CfgBig::kThreads), 0, stream, p, y, tiles_o, tiles_s);
        return hipGetLastError();
    }
    if (dma_ok) {
        const int64_t tiles_o = (out + CfgQ::BO - 1) / CfgQ::BO;
        const int64_t tiles_s = (S + CfgQ::BS - 1) / CfgQ::BS;
        if (tiles_o * tiles_s > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        const dim3 grid((unsigned)(tiles_o * tiles_s));
        if (tiled_scales)
            hipLaunchKernelGGL(gemm_pc_kernel<CfgQT>, grid, dim3(2 * CfgQT::kThreads), 0,
                               stream, p, y, tiles_o, tiles_s);
        else
            hipLaunchKernelGGL(gemm_dma_kernel<CfgQ>, grid, dim3(CfgQ::kThreads), 0, stream,
                               p, y, tiles_o, tiles_s);
        return hipGetLastError();
    }
    const int64_t tiles_o = (out + kGBO - 1) / kGBO;
    const int64_t tiles_s = (S + kGBS - 1) / kGBS;
    if (tiles_o * tiles_s > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(gemm_generic_kernel, dim3((unsigned)(tiles_o * tiles_s)), dim3(kThreads),
                       0, stream, p, (int)tiled_scales, y, tiles_o, tiles_s);
    return hipGetLastError();
}

hipError_t launch_gemm_w4a8(const uint8_t* xq8, const uint8_t* xe, const uint8_t* wq,
                            const uint8_t* we, bool tiled_scales, int64_t S, int64_t N,
                            int64_t out, float* y, hipStream_t stream, const uint16_t* res,
                       bool out_bf16)
{
    const DmaArgs p{xq8, xe, wq, we, S, N / 32, out, res, out_bf16 ? 1 : 0};
    if ((p.k % kStageBlocks) != 0 || (reinterpret_cast<uintptr_t>(xe) % 4) != 0 ||
        (reinterpret_cast<uintptr_t>(we) % 4) != 0 || S * 32 * p.k >= (1LL << 32) ||
        out * 16 * p.k >= (1LL << 32))
        return hipErrorNotSupported;
    const bool s8 = (reinterpret_cast<uintptr_t>(xe) % 8) == 0 &&
                    (reinterpret_cast<uintptr_t>(we) % 8) == 0;
    if (use_skinny16(S, p.k, out, true) && (tiled_scales || s8)) {
        // at most 16 tokens: 16-row workgroups with E4M3 token fragments
        const int64_t tiles_o = (out + kS16Rows - 1) / kS16Rows;
        if (tiles_o > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        const size_t lds = s16_lds_bytes(p.k);
        if (tiled_scales)
            hipLaunchKernelGGL((gemm_skinny16_kernel<true, true>), dim3((unsigned)tiles_o),
                               dim3(64 * kS16Waves), lds, stream, p, y);
        else
            hipLaunchKernelGGL((gemm_skinny16_kernel<false, true>), dim3((unsigned)tiles_o),
                               dim3(64 * kS16Waves), lds, stream, p, y);
        return hipGetLastError();
    }
    if (S <= 64 && (tiled_scales || s8)) {
        // few tokens: the weight-streaming kernel with E4M3 token codes
        const int64_t tiles_w = (out + 31) / 32;
        if (tiles_w > 0x7FFFFFFF / 2) return hipErrorInvalidConfiguration;
        const dim3 grid((unsigned)tiles_w);
        if (S <= 32 || skinny_halves(S, tiles_w)) {
            const dim3 grid1((unsigned)(S <= 32 ? tiles_w : (tiles_w + 7) / 8 * 16));
            const dim3 block(64 * SkinnyCfg<1, true>::waves);
            if (tiled_scales)
                hipLaunchKernelGGL((gemm_skinny_kernel<1, true, true>), grid1, block, 0, stream, p, y);
            else
                hipLaunchKernelGGL((gemm_skinny_kernel<1, false, true>), grid1, block, 0, stream, p, y);
        } else {
            const dim3 block(64 * SkinnyCfg<2, true>::waves);
            if (tiled_scales)
                hipLaunchKernelGGL((gemm_skinny_kernel<2, true, true>), grid, block, 0, stream, p, y);
            else
                hipLaunchKernelGGL((gemm_skinny_kernel<2, false, true>), grid, block, 0, stream, p, y);
        }
        return hipGetLastError();
    }
    const int64_t tiles_o = (out + w4a8::BO - 1) / w4a8::BO;
    const int64_t tiles_s = (S + w4a8::BS - 1) / w4a8::BS;
    if (tiles_o * tiles_s > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)(tiles_o * tiles_s)), block(64 * w4a8::kWaves);
    if (tiled_scales)
        hipLaunchKernelGGL(gemm_w4a8_kernel<true>, grid, block, 0, stream, p, y, tiles_o,
                           tiles_s);
    else
        hipLaunchKernelGGL(gemm_w4a8_kernel<false>, grid, block, 0, stream, p, y, tiles_o,
                           tiles_s);
    return hipGetLastError();
}

}  // namespace batq

namespace batq {

template <bool TS, int NPER, bool F8, int W>
static void launch_linear16_n(const DmaArgs& p, const uint16_t* x, int64_t ldx, const float* A,
                              const float* B, const float* r_min, const float* r_max, float* y,
                              hipStream_t stream)
{
    const int64_t tiles = (p.out + kS16Rows - 1) / kS16Rows;
    const size_t panel = (size_t)(p.k / kStageBlocks + 1) * kS16Stage;   // + the scratch slot
    const size_t red = (size_t)W * 4 * 64 * 4;
    hipLaunchKernelGGL((gemm_linear16_kernel<TS, NPER, F8, W>), dim3((unsigned)tiles),
                       dim3(64 * W), panel > red ? panel : red, stream, p, x, ldx, A, B, r_min,
                       r_max, y);
}

template <bool TS, bool F8, int W = kS16Waves>
static void launch_linear16(const DmaArgs& p, const uint16_t* x, int64_t ldx, const float* A,
                            const float* B, const float* r_min, const float* r_max, float* y,
                            hipStream_t stream)
{
    // stages per wave: at most kS16MaxK / 8 / W (8 with 8 waves, 4 with 16)
    constexpr int kMaxPer = kS16MaxK / kStageBlocks / W;
    const int nper = (int)((p.k / kStageBlocks + W - 1) / W);
    switch (nper) {
    case 1: launch_linear16_n<TS, 1, F8, W>(p, x, ldx, A, B, r_min, r_max, y, stream); break;
    case 2: launch_linear16_n<TS, 2, F8, W>(p, x, ldx, A, B, r_min, r_max, y, stream); break;
    case 3: launch_linear16_n<TS, 3, F8, W>(p, x, ldx, A, B, r_min, r_max, y, stream); break;
    case 4: launch_linear16_n<TS, 4, F8, W>(p, x, ldx, A, B, r_min, r_max, y, stream); break;
    default:
        if constexpr (kMaxPer > 4) {
            switch (nper) {
            case 5: launch_linear16_n<TS, 5, F8, W>(p, x, ldx, A, B, r_min, r_max, y, stream); break;
            case 6: launch_linear16_n<TS, 6, F8, W>(p, x, ldx, A, B, r_min, r_max, y, stream); break;
            case 7: launch_linear16_n<TS, 7, F8, W>(p, x, ldx, A, B, r_min, r_max, y, stream); break;
            default: launch_linear16_n<TS, kMaxPer, F8, W>(p, x, ldx, A, B, r_min, r_max, y, stream); break;
            }
        }
        break;
    }
}

hipError_t launch_linear_skinny(const uint16_t* x, int64_t S, int64_t k, int64_t ldx,
                                const float* A, const float* B, const float* r_min,
                                const float* r_max, const uint8_t* wq, const uint8_t* we,
                                bool tiled_scales, int64_t out, float* y, hipStream_t stream)
{
    // up to 4 tokens any k <= 512; up to 16 (one MFMA token column) on 16-row workgroups
    if (S < 1 || S > kS16MaxTokens || k < 1 || k > kLinMaxK || k % kStageBlocks != 0 ||
        (S > kLinTokens && S * k > kLin16MaxSK))
        return hipErrorNotSupported;
    const uintptr_t salign = tiled_scales ? 256 : 8;
    if ((reinterpret_cast<uintptr_t>(we) % salign) != 0 || out * 16 * k >= (1LL << 32))
        return hipErrorNotSupported;
    const DmaArgs p{nullptr, nullptr, wq, we, S, k, out, nullptr, 0};
    if (S * k <= kLin16MaxSK && k <= kS16MaxK) {
        // 16-row workgroups, the whole panel in flight
        if ((out + kS16Rows - 1) / kS16Rows > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        // 16 waves when one round of workgroups covers out
        const bool wide = (out + kS16Rows - 1) / kS16Rows <= kNumCUs;
        if (tiled_scales) {
            if (wide) launch_linear16<true, false, 16>(p, x, ldx, A, B, r_min, r_max, y, stream);
            else launch_linear16<true, false>(p, x, ldx, A, B, r_min, r_max, y, stream);
        } else {
            if (wide) launch_linear16<false, false, 16>(p, x, ldx, A, B, r_min, r_max, y, stream);
            else launch_linear16<false, false>(p, x, ldx, A, B, r_min, r_max, y, stream);
        }
        return hipGetLastError();
    }
    const int64_t tiles_o = (out + 31) / 32;
    if (tiles_o > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)tiles_o), block(64 * kLinWaves);
    if (tiled_scales)
        hipLaunchKernelGGL(gemm_linear_skinny_kernel<true>, grid, block, 0, stream, p, x, ldx, A,
                           B, r_min, r_max, y);
    else
        hipLaunchKernelGGL(gemm_linear_skinny_kernel<false>, grid, block, 0, stream, p, x, ldx,
                           A, B, r_min, r_max, y);
    return hipGetLastError();
}

hipError_t launch_linear16_w4a8(const uint16_t* x, int64_t S, int64_t k, int64_t ldx,
                                const float* A, const float* B, const float* r_min,
                                const float* r_max, const uint8_t* wq, const uint8_t* we,
                                bool tiled_scales, int64_t out, float* y, hipStream_t stream)
{
    if (S < 1 || S > kLinTokens || k < 1 || k > kS16MaxK || k % kStageBlocks != 0 ||
        S * k > kLin16MaxSK8)
        return hipErrorNotSupported;
    const uintptr_t salign = tiled_scales ? 256 : 8;
    if ((reinterpret_cast<uintptr_t>(we) % salign) != 0 || out * 16 * k >= (1LL << 32))
        return hipErrorNotSupported;
    if ((out + kS16Rows - 1) / kS16Rows > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const DmaArgs p{nullptr, nullptr, wq, we, S, k, out, nullptr, 0};
    if (tiled_scales)
        launch_linear16<true, true>(p, x, ldx, A, B, r_min, r_max, y, stream);
    else
        launch_linear16<false, true>(p, x, ldx, A, B, r_min, r_max, y, stream);
    return hipGetLastError();
}

}  // namespace batq

// =======================================================================================
// Device scratch of the no-allocation linear layer (batq_linear_w4a4_noalloc)
// =======================================================================================
namespace batq {
namespace {

// The activation codes and scales of batq_linear_w4a4_noalloc.  Every GPU the library runs
// on holds its own copy (loaded with the code object) until the process ends.  In host code
// this name stands for a host-side shadow, not device memory: the device address comes from
// hipGetSymbolAddress, once per device, and only that address reaches kernels and copies.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
uint8_t* g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(uint8_t** ptr)
{
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        // first use on this device, with the device current: its copy's address
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace batq
