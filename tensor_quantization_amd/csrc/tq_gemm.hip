// tq_gemm.hip -- the GEMMs that consume the quantized operands, on the gfx950
// matrix cores: the W8A8 quantized linear (baracuda_kernels::quantize,
// quantized_linear) and the block-scaled FP8 GEMM (smile.llm.quant
// Fp8BlockGemm: E4M3 activations with one fp32 scale per 1 x 128 group, E4M3
// weights with one fp32 scale per 128 x 128 tile, out = x W^T):
//
//   y[m][n] = sum_kb (sa[m][kb] * sw[n/128][kb]) * sum_{k in kb} val(qa[m][k]) val(qw[n][k])
//
// Each 128-wide K block is one unit: its fp8 dot products come out of one
// v_mfma_scale_f32_16x16x128_f8f6f4 step per 16 x 16 tile (E8M0 operand
// scales fixed at 1), then the block sum is scaled by sa * sw and added to
// the binary32 total.  Scaling per block keeps the matrix core's own
// summation short: inside a step it cuts products toward zero 13 bits below
// the largest exponent of each group of eight consecutive K, and keeps about
// 24 bits across groups, so its error is bounded per block and never grows
// with K.
//
// k_fp8_gemm: a 256-thread workgroup owns a 128 x 128 output tile; wave w
// computes the 64 x 64 quarter (w / 2, w % 2) as 4 x 4 tiles of 16 x 16,
// sixteen independent products per block, so the scale-and-accumulate of
// one tile overlaps the products of the next.  Lane l holds row l % 16 of A
// (column l % 16 of B) and bytes 32 (l / 16) .. + 31 of the block; result
// element r of lane l is D[4 (l / 16) + r][l % 16], so a lane meets 16
// distinct rows per block (16 scale products).
//
// The A and B K-slices (128 x 128 bytes each) and the block's 128 row scales
// move by direct global -> LDS loads (global_load_lds) into two LDS stages,
// one block ahead; 66.5 KB of LDS and under 256 VGPRs let two workgroups
// share a CU, so one fills the other's waits.  LDS rows are 128 bytes whose
// eight 16-byte chunks sit at slot chunk ^ ((row / 2) % 8): sixteen
// consecutive rows read at one chunk then cover all 64 banks.  A DMA lane
// writes 16 bytes at (wave base + 16 * lane), so each lane fetches the
// global chunk that the swizzle puts in its slot.  Waits and barriers are
// explicit: before block kb is read every wave waits for its own loads, then
// all waves meet; only after that meeting is the buffer that block kb - 1
// used refilled.
#include "tq_device.h"
#include "tq_host.h"

namespace tq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int GT = 128;                  // output tile and K block
constexpr int SLICE = GT * GT;           // bytes of one operand K-slice

__device__ __forceinline__ int64_t min_i64(int64_t a, int64_t b) { return a < b ? a : b; }
__device__ __forceinline__ int swz_key(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * GT + ((chunk ^ swz_key(row)) << 4); }

typedef __attribute__((address_space(3))) void lds_void;

// Direct global -> LDS loads, issued from asm so that the compiler adds no
// wait of its own for them: every lane of the wave writes `bytes` bytes at
// M0 + bytes * lane (M0 = `lds` byte address, wave-uniform).  They count in
// vmcnt; the kernel waits for them explicitly.  Nothing else in the kernel
// uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, const lds_void* lds)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)lds);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, const lds_void* lds)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)lds);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int YT>
__global__ __launch_bounds__(256) void k_fp8_gemm(const uint8_t* __restrict__ qa, const float* __restrict__ sa,
                                                  const uint8_t* __restrict__ qw, const float* __restrict__ sw,
                                                  int64_t M, int64_t K, int64_t N, void* __restrict__ y)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][SLICE];
    __shared__ __attribute__((aligned(16))) float lds_sa[2][GT];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = w >> 1, wn = w & 1;
    const int g4 = lane >> 4, l16 = lane & 15;
    const int64_t m0 = (int64_t)blockIdx.y * GT, n0 = (int64_t)blockIdx.x * GT;
    const int64_t nkb = K / GT;
    const float* gsw = sw + (n0 / GT) * nkb;

    // fill: LDS rows 8 w + lane / 8 + 32 i (i < 4), slot lane % 8; rows past
    // M (a ragged last tile) re-read row M - 1 and their results are dropped
    const int frow = 8 * w + (lane >> 3);
    const int fchunk = (lane & 7) ^ swz_key(frow);
    const uint8_t* fa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = qa + min_i64(m0 + frow + 32 * i, M - 1) * K + fchunk * 16;
    const uint8_t* fb = qw + (n0 + frow) * K + fchunk * 16;
    const float* fs = sa + min_i64(m0 + 32 * w + (lane & 31), M - 1) * nkb;

    auto issue = [&](int64_t kb) {
        const int buf = (int)(kb & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dma16(fa[i] + kb * GT, (const lds_void*)&lds[buf][0][(32 * i + 8 * w) * GT]);
            dma16(fb + (int64_t)32 * i * K + kb * GT, (const lds_void*)&lds[buf][1][(32 * i + 8 * w) * GT]);
        }
        if (lane < 32) dma4(fs + kb, (const lds_void*)&lds_sa[buf][32 * w]);
    };

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{};

    issue(0);
    for (int64_t kb = 0; kb < nkb; ++kb) {
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if (kb + 1 < nkb) issue(kb + 1);

        const int cur = (int)(kb & 1);
        const uint8_t* la = lds[cur][0];
        const uint8_t* lb = lds[cur][1];
        const float swv = gsw[kb];
        v8i av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ar = wm * 64 + i * 16 + l16;
            const int br = wn * 64 + i * 16 + l16;
            const uint4 a0 = *reinterpret_cast<const uint4*>(&la[swz(ar, 2 * g4)]);
            const uint4 a1 = *reinterpret_cast<const uint4*>(&la[swz(ar, 2 * g4 + 1)]);
            const uint4 b0 = *reinterpret_cast<const uint4*>(&lb[swz(br, 2 * g4)]);
            const uint4 b1 = *reinterpret_cast<const uint4*>(&lb[swz(br, 2 * g4 + 1)]);
            av[i] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            bv[i] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
        }
        float c[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 s4 = *reinterpret_cast<const float4*>(&lds_sa[cur][wm * 64 + i * 16 + 4 * g4]);
            c[i][0] = s4.x * swv; c[i][1] = s4.y * swv; c[i][2] = s4.z * swv; c[i][3] = s4.w * swv;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v4f blk = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[i], bv[j], v4f{}, 0, 0, 0, 127, 0, 127);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(blk[r], c[i][r], acc[i][j][r]);
            }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm * 64 + i * 16 + 4 * g4 + r;
                const int64_t col = n0 + wn * 64 + j * 16 + l16;
                if (row < M) store1<YT>(y, row * N + col, acc[i][j][r]);
            }
}

// k_w8a8_gemm: the W8A8 quantized linear on the same tile and load pipeline.
// Each 128-wide K block is two v_mfma_i32_16x16x64_i8 steps per 16 x 16 tile
// (lane l: row l % 16 of A / column l % 16 of B, bytes 16 (l / 16) .. + 15
// of the 64-wide step), accumulated exactly in int32 inside the matrix core;
// the per-row and per-channel scales are applied once, in the epilogue:
// y = ((float)acc * sx[row]) * sw[col], each product rounded in binary32.
typedef int v4i __attribute__((ext_vector_type(4)));

template <int YT>
__global__ __launch_bounds__(256) void k_w8a8_gemm(const int8_t* __restrict__ qx, const float* __restrict__ sx,
                                                   const int8_t* __restrict__ qw, const float* __restrict__ sw,
                                                   int64_t M, int64_t K, int64_t N, void* __restrict__ y)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][SLICE];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = w >> 1, wn = w & 1;
    const int g4 = lane >> 4, l16 = lane & 15;
    const int64_t m0 = (int64_t)blockIdx.y * GT, n0 = (int64_t)blockIdx.x * GT;
    const int64_t nkb = K / GT;

    const int frow = 8 * w + (lane >> 3);
    const int fchunk = (lane & 7) ^ swz_key(frow);
    const int8_t* fa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = qx + min_i64(m0 + frow + 32 * i, M - 1) * K + fchunk * 16;
    const int8_t* fb = qw + (n0 + frow) * K + fchunk * 16;

    auto issue = [&](int64_t kb) {
        const int buf = (int)(kb & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dma16(fa[i] + kb * GT, (const lds_void*)&lds[buf][0][(32 * i + 8 * w) * GT]);
            dma16(fb + (int64_t)32 * i * K + kb * GT, (const lds_void*)&lds[buf][1][(32 * i + 8 * w) * GT]);
        }
    };

    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4i{};

    issue(0);
    for (int64_t kb = 0; kb < nkb; ++kb) {
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if (kb + 1 < nkb) issue(kb + 1);

        const int cur = (int)(kb & 1);
        const uint8_t* la = lds[cur][0];
        const uint8_t* lb = lds[cur][1];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            v4i av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 a = *reinterpret_cast<const uint4*>(&la[swz(wm * 64 + i * 16 + l16, 4 * s + g4)]);
                const uint4 b = *reinterpret_cast<const uint4*>(&lb[swz(wn * 64 + i * 16 + l16, 4 * s + g4)]);
                av[i] = v4i{(int)a.x, (int)a.y, (int)a.z, (int)a.w};
                bv[i] = v4i{(int)b.x, (int)b.y, (int)b.z, (int)b.w};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
    }
    float swc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) swc[j] = sw[n0 + wn * 64 + j * 16 + l16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + wm * 64 + i * 16 + 4 * g4 + r;
            if (row >= M) continue;
            const float sxv = sx[row];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float v = (float)acc[i][j][r];
                v = v * sxv;
                v = v * swc[j];
                store1<YT>(y, row * N + n0 + wn * 64 + j * 16 + l16, v);
            }
        }
}

// k_w8a8_gemm_256: the W8A8 linear on a 256 x 256 output tile (half the
// operand traffic per product of the 128 x 128 tile, a third less LDS traffic
// per product); eight waves, two per SIMD, each computing 64 x 128 as 4 x 8
// tiles; two LDS stages of 64 KB, one workgroup per CU.  Used when N is a
// multiple of 256 (1.70 against 1.44 POP/s on 8192 x 11008 x 4096); the
// 128 x 128 kernel covers the other N.
template <int YT>
__global__ __launch_bounds__(512) void k_w8a8_gemm_256(const int8_t* __restrict__ qx, const float* __restrict__ sx,
                                                       const int8_t* __restrict__ qw, const float* __restrict__ sw,
                                                       int64_t M, int64_t K, int64_t N, void* __restrict__ y)
{
    constexpr int BT = 256;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][BT * GT];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = w >> 1, wn = w & 1;
    const int g4 = lane >> 4, l16 = lane & 15;
    const int64_t m0 = (int64_t)blockIdx.y * BT, n0 = (int64_t)blockIdx.x * BT;
    const int64_t nkb = K / GT;

    // fill: LDS rows 8 w + lane / 8 + 64 i (i < 4), slot lane % 8
    const int frow = 8 * w + (lane >> 3);
    const int fchunk = (lane & 7) ^ swz_key(frow);
    const int8_t* fa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = qx + min_i64(m0 + frow + 64 * i, M - 1) * K + fchunk * 16;
    const int8_t* fb = qw + (n0 + frow) * K + fchunk * 16;

    auto issue = [&](int64_t kb) {
        const int buf = (int)(kb & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dma16(fa[i] + kb * GT, (const lds_void*)&lds[buf][0][(64 * i + 8 * w) * GT]);
            dma16(fb + (int64_t)64 * i * K + kb * GT, (const lds_void*)&lds[buf][1][(64 * i + 8 * w) * GT]);
        }
    };

    v4i acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = v4i{};

    issue(0);
    for (int64_t kb = 0; kb < nkb; ++kb) {
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if (kb + 1 < nkb) issue(kb + 1);

        const int cur = (int)(kb & 1);
        const uint8_t* la = lds[cur][0];
        const uint8_t* lb = lds[cur][1];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            v4i av[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 a = *reinterpret_cast<const uint4*>(&la[swz(wm * 64 + i * 16 + l16, 4 * s + g4)]);
                av[i] = v4i{(int)a.x, (int)a.y, (int)a.z, (int)a.w};
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint4 b = *reinterpret_cast<const uint4*>(&lb[swz(wn * 128 + j * 16 + l16, 4 * s + g4)]);
                const v4i bv = v4i{(int)b.x, (int)b.y, (int)b.z, (int)b.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[i], bv, acc[i][j], 0, 0, 0);
            }
        }
    }
    float swc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) swc[j] = sw[n0 + wn * 128 + j * 16 + l16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + wm * 64 + i * 16 + 4 * g4 + r;
            if (row >= M) continue;
            const float sxv = sx[row];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float v = (float)acc[i][j][r];
                v = v * sxv;
                v = v * swc[j];
                store1<YT>(y, row * N + n0 + wn * 128 + j * 16 + l16, v);
            }
        }
}

// k_fp4_linear: bf16 activations x [M, K] times an FP4 weight in the
// quantizer's own layout (packed [N, K/2] low nibble first, block scales
// [N, K/gs]): K-contiguous rows are what the matrix-core B operand wants, so
// the GEMM reads that layout directly and needs no transposed twin.  Same
// 128 x 128 tile as above with 64-wide K blocks.  The activation slice
// (128 rows x 128 bytes) moves by DMA into two LDS stages.  The weight is
// expanded once per workgroup: thread t loads half a row (16 packed bytes,
// 32 values) of the next block and its scale bytes into registers while the
// matrix cores work on the current block, then writes them as exact bf16
// into the other of two LDS weight buffers, laid out (128-byte rows, same
// swizzle) like the activation slice.  MXFP4 expands by
// v_cvt_scalef32_pk_bf16_fp4, whose scale operand applies the power of two
// 2^(e8m0 - 127) exactly; NVFP4 by the same conversion to f32 at scale 1, a
// binary32 multiply by the E4M3 block scale and a bf16 pack (E2M1 x E4M3 has
// at most 6 significant bits, so the bf16 weight is exact).  Two
// v_mfma_f32_16x16x32_bf16 steps per block chain in the matrix core from
// zero; the block sum is added to a binary32 accumulator (the matrix core's
// own accumulator input joins its truncating alignment, so the chain is kept
// short), and the NVFP4 per-tensor scale multiplies the total once.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
constexpr int FKB = 64;                  // K per block
enum { FP4_NV = 0, FP4_MX = 1 };

__device__ __forceinline__ v2bf fp4_pair_nv(uint32_t word, int sel, float sc)
{
    v2f f;
    switch (sel) {
    case 0: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0); break;
    case 1: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1); break;
    case 2: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2); break;
    default: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3); break;
    }
    return v2bf{(__bf16)(f.x * sc), (__bf16)(f.y * sc)};
}
__device__ __forceinline__ v2bf fp4_pair_mx(uint32_t word, int sel, float sc)
{
    switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 3);
    }
}

// 8 weight values (one packed dword) as a 16-byte bf16 chunk
template <int KIND>
__device__ __forceinline__ uint4 fp4_expand8(uint32_t word, float sc)
{
    v2bf p0, p1, p2, p3;
    if (KIND == FP4_NV) {
        p0 = fp4_pair_nv(word, 0, sc); p1 = fp4_pair_nv(word, 1, sc);
        p2 = fp4_pair_nv(word, 2, sc); p3 = fp4_pair_nv(word, 3, sc);
    } else {
        p0 = fp4_pair_mx(word, 0, sc); p1 = fp4_pair_mx(word, 1, sc);
        p2 = fp4_pair_mx(word, 2, sc); p3 = fp4_pair_mx(word, 3, sc);
    }
    return make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                      __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
}

template <int KIND, int YT>
__global__ __launch_bounds__(256) void k_fp4_linear(const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed,
                                                    const uint8_t* __restrict__ bscale,
                                                    const float* __restrict__ global_scale, int64_t M, int64_t K,
                                                    int64_t N, void* __restrict__ y)
{
    constexpr int GS = KIND == FP4_NV ? 16 : 32;
    constexpr int SPB = FKB / GS;        // scale bytes per weight row per block
    __shared__ __attribute__((aligned(16))) uint8_t la[2][GT * 2 * FKB];
    __shared__ __attribute__((aligned(16))) uint8_t lw[2][GT * 2 * FKB];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = w >> 1, wn = w & 1;
    const int g4 = lane >> 4, l16 = lane & 15;
    const int64_t m0 = (int64_t)blockIdx.y * GT, n0 = (int64_t)blockIdx.x * GT;
    const int64_t nkb = K / FKB;
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
    const float sg = KIND == FP4_NV ? *global_scale : 1.0f;

    // activation rows are 128 bytes per block (64 bf16): the FP8 kernel's fill and swizzle
    const int frow = 8 * w + (lane >> 3);
    const int fchunk = (lane & 7) ^ swz_key(frow);
    const uint8_t* fa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = xb + min_i64(m0 + frow + 32 * i, M - 1) * (2 * K) + fchunk * 16;
    auto issue = [&](int64_t kb) {
        const int buf = (int)(kb & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(fa[i] + kb * 2 * FKB, (const lds_void*)&la[buf][(32 * i + 8 * w) * GT]);
    };

    // weight expansion: thread t owns half h = t % 2 of weight row r = t / 2 (32 values = chunks 4h .. 4h+3)
    const int wr = t >> 1, wh = t & 1;
    const uint8_t* fw = packed + (n0 + wr) * (K / 2) + wh * 16;
    const uint8_t* fsc = bscale + (n0 + wr) * (K / GS);
    uint4 pk;
    uint32_t sbytes;
    auto fetch_w = [&](int64_t kb) {
        pk = *reinterpret_cast<const uint4*>(fw + kb * (FKB / 2));
        sbytes = KIND == FP4_NV ? *reinterpret_cast<const uint32_t*>(fsc + kb * SPB)
                                : (uint32_t)*reinterpret_cast<const uint16_t*>(fsc + kb * SPB);
    };
    auto expand_w = [&](int buf) {
        const uint32_t d[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            // values 32 wh + 8 c .. + 7 of the block: NVFP4 group 2 wh + c / 2, MXFP4 group wh
            const float sc = KIND == FP4_NV ? e4m3_val(sbytes >> (8 * (2 * wh + (c >> 1))), 0)
                                            : __uint_as_float(((sbytes >> (8 * wh)) & 0xff) << 23);
            *reinterpret_cast<uint4*>(&lw[buf][swz(wr, 4 * wh + c)]) = fp4_expand8<KIND>(d[c], sc);
        }
    };

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{};

    issue(0);
    fetch_w(0);
    expand_w(0);
    for (int64_t kb = 0; kb < nkb; ++kb) {
        // block kb's activations have landed and its expanded weights are written
        // by every thread; every wave is done with the buffers of block kb - 1
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const bool more = kb + 1 < nkb;
        if (more) {
            issue(kb + 1);
            fetch_w(kb + 1);
        }

        const int cur = (int)(kb & 1);
        v4f blk[4][4];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            v8bf av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(
                                                     &la[cur][swz(wm * 64 + i * 16 + l16, 4 * s + g4)]));
                bv[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(
                                                     &lw[cur][swz(wn * 64 + i * 16 + l16, 4 * s + g4)]));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    blk[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[j], s == 0 ? v4f{} : blk[i][j], 0, 0, 0);
        }
        if (more) expand_w(cur ^ 1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] = acc[i][j][r] + blk[i][j][r];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm * 64 + i * 16 + 4 * g4 + r;
                const int64_t col = n0 + wn * 64 + j * 16 + l16;
                const float v = KIND == FP4_NV ? acc[i][j][r] * sg : acc[i][j][r];   // NVFP4 per-tensor scale
                if (row < M) store1<YT>(y, row * N + col, v);
            }
}

__global__ __launch_bounds__(256) void k_zero_bytes(uint8_t* __restrict__ p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

}  // namespace tq

using namespace tq;

extern "C" {

tq_status tq_fp8_block_gemm(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw, int64_t M,
                            int64_t N, int64_t K, void* y, int y_dtype, void* stream)
{
    if (!valid_ftype(y_dtype) || M < 0 || N < 0 || K < 0 || N % GT || K % GT) return TQ_ERR_INVALID;
    if (M == 0 || N == 0) return TQ_OK;
    if (!y || (K > 0 && (!qa || !sa || !qw || !sw))) return TQ_ERR_INVALID;
    if (K > 0 && (!aligned16(qa) || !aligned16(qw))) return TQ_ERR_ALIGN;
    if ((M + GT - 1) / GT > 65535 || N / GT > 0x7fffffff) return TQ_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)(N / GT), (unsigned)((M + GT - 1) / GT));
    hipStream_t st = as_stream(stream);
    if (K == 0) {   // empty sums: zeros (a fill kernel, not a memset node, so the call can be graph-captured)
        const int64_t nbytes = M * N * (y_dtype == TQ_F32 ? 4 : 2);
        hipLaunchKernelGGL(k_zero_bytes, dim3((unsigned)std::min<int64_t>((nbytes + 255) / 256, 1 << 20)), dim3(256),
                           0, st, static_cast<uint8_t*>(y), nbytes);
        return launch_status();
    }
    switch (y_dtype) {
    case TQ_F32: hipLaunchKernelGGL(k_fp8_gemm<F32>, grid, dim3(256), 0, st, qa, sa, qw, sw, M, K, N, y); break;
    case TQ_F16: hipLaunchKernelGGL(k_fp8_gemm<F16>, grid, dim3(256), 0, st, qa, sa, qw, sw, M, K, N, y); break;
    default: hipLaunchKernelGGL(k_fp8_gemm<BF16>, grid, dim3(256), 0, st, qa, sa, qw, sw, M, K, N, y); break;
    }
    return launch_status();
}

tq_status tq_w8a8_linear(const int8_t* qx, const float* sx, const int8_t* qw, const float* sw, int64_t M, int64_t N,
                         int64_t K, void* y, int y_dtype, void* stream)
{
    if (!valid_ftype(y_dtype) || M < 0 || N < 0 || K < 0) return TQ_ERR_INVALID;
    if (M == 0 || N == 0) return TQ_OK;
    if (N % GT || K % GT || K > 131071 || (M + GT - 1) / GT > 65535 || N / GT > 0x7fffffff) return TQ_ERR_UNSUPPORTED;
    if (!y || !sx || !sw || (K > 0 && (!qx || !qw))) return TQ_ERR_INVALID;
    if (K > 0 && (!aligned16(qx) || !aligned16(qw))) return TQ_ERR_ALIGN;
    hipStream_t st = as_stream(stream);
    if (K == 0) {   // empty sums: zeros (a fill kernel, not a memset node, so the call can be graph-captured)
        const int64_t nbytes = M * N * (y_dtype == TQ_F32 ? 4 : 2);
        hipLaunchKernelGGL(k_zero_bytes, dim3((unsigned)std::min<int64_t>((nbytes + 255) / 256, 1 << 20)), dim3(256),
                           0, st, static_cast<uint8_t*>(y), nbytes);
        return launch_status();
    }
    if (N % 256 == 0 && (M + 255) / 256 <= 65535) {     // the 256 x 256 tile where N allows it
        const dim3 g2((unsigned)(N / 256), (unsigned)((M + 255) / 256));
        switch (y_dtype) {
        case TQ_F32: hipLaunchKernelGGL(k_w8a8_gemm_256<F32>, g2, dim3(512), 0, st, qx, sx, qw, sw, M, K, N, y); break;
        case TQ_F16: hipLaunchKernelGGL(k_w8a8_gemm_256<F16>, g2, dim3(512), 0, st, qx, sx, qw, sw, M, K, N, y); break;
        default: hipLaunchKernelGGL(k_w8a8_gemm_256<BF16>, g2, dim3(512), 0, st, qx, sx, qw, sw, M, K, N, y); break;
        }
        return launch_status();
    }
    const dim3 grid((unsigned)(N / GT), (unsigned)((M + GT - 1) / GT));
    switch (y_dtype) {
    case TQ_F32: hipLaunchKernelGGL(k_w8a8_gemm<F32>, grid, dim3(256), 0, st, qx, sx, qw, sw, M, K, N, y); break;
    case TQ_F16: hipLaunchKernelGGL(k_w8a8_gemm<F16>, grid, dim3(256), 0, st, qx, sx, qw, sw, M, K, N, y); break;
    default: hipLaunchKernelGGL(k_w8a8_gemm<BF16>, grid, dim3(256), 0, st, qx, sx, qw, sw, M, K, N, y); break;
    }
    return launch_status();
}

tq_status tq_fp4_linear(const void* x, int x_dtype, const uint8_t* packed, const uint8_t* block_scale,
                        const float* global_scale, int kind, int64_t M, int64_t N, int64_t K, void* y,
                        int y_dtype, void* stream)
{
    if (!valid_ftype(y_dtype) || (kind != TQ_NVFP4 && kind != TQ_MXFP4) || M < 0 || N < 0 || K < 0)
        return TQ_ERR_INVALID;
    if (kind == TQ_NVFP4 && !global_scale) return TQ_ERR_INVALID;
    if (M == 0 || N == 0) return TQ_OK;
    if (x_dtype != TQ_BF16 || N % GT || K % FKB || (M + GT - 1) / GT > 65535 || N / GT > 0x7fffffff)
        return TQ_ERR_UNSUPPORTED;
    if (!y || (K > 0 && (!x || !packed || !block_scale))) return TQ_ERR_INVALID;
    if (K > 0 && (!aligned16(x) || !aligned16(packed) || ((uintptr_t)block_scale & 3))) return TQ_ERR_ALIGN;
    hipStream_t st = as_stream(stream);
    if (K == 0) {   // empty sums: zeros (a fill kernel, not a memset node, so the call can be graph-captured)
        const int64_t nbytes = M * N * (y_dtype == TQ_F32 ? 4 : 2);
        hipLaunchKernelGGL(k_zero_bytes, dim3((unsigned)std::min<int64_t>((nbytes + 255) / 256, 1 << 20)), dim3(256),
                           0, st, static_cast<uint8_t*>(y), nbytes);
        return launch_status();
    }
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    const dim3 grid((unsigned)(N / GT), (unsigned)((M + GT - 1) / GT));
#define TQ_FP4_LAUNCH(KD, YD) \
    hipLaunchKernelGGL((k_fp4_linear<KD, YD>), grid, dim3(256), 0, st, xs, packed, block_scale, global_scale, M, K, N, y)
    if (kind == TQ_NVFP4) {
        if (y_dtype == TQ_F32) TQ_FP4_LAUNCH(FP4_NV, F32);
        else if (y_dtype == TQ_F16) TQ_FP4_LAUNCH(FP4_NV, F16);
        else TQ_FP4_LAUNCH(FP4_NV, BF16);
    } else {
        if (y_dtype == TQ_F32) TQ_FP4_LAUNCH(FP4_MX, F32);
        else if (y_dtype == TQ_F16) TQ_FP4_LAUNCH(FP4_MX, F16);
        else TQ_FP4_LAUNCH(FP4_MX, BF16);
    }
#undef TQ_FP4_LAUNCH
    return launch_status();
}

}  // extern "C"
