// tq_fp4.hip -- FP4 E2M1 block quantization with NVFP4 / MXFP4 scales and
// the transposes to GEMM layout (metrale QuantizedWeight: fields weight,
// weight_scale, weight_scale_2; transpose_for_gemm, transpose_for_gemm_gs;
// smile.llm.quant MxFp8 for the E8M0-per-32 scale of the MX family).
//
//   NVFP4: s_g = amax / 2688 (6 * 448; 1 if 0) or the caller's static value;
//          sb = E4M3(amax_16 / (6 * s_g)) (0x38 if it encodes to 0);
//          eff = val(sb) * s_g;                   q = E2M1(x / eff)
//   MXFP4: sb = E8M0 byte of 2^(floor(log2 amax_32) - 2) (127 if all zero);
//          eff = 2^(sb - 127);                   q = E2M1(x * 2^(127 - sb))
//          (x * 2^(127-sb) is exactly RN(x / eff): one rounding of the same
//          real number)
// Codes are packed two per byte along K, even index in the low nibble.
//
// Kernels:
//   k_amax_partial   dynamic NVFP4 s_g, pass 1: chunk maxima.
//   k_fp4_quant      a team of 2 (NVFP4) / 4 (MXFP4) lanes per block, block max
//                    through DPP, U rounds per wave; NVFP4 reads s_g from
//                    global_scale.
//   k_nv_quant_dyn   dynamic NVFP4 s_g, pass 2: one lane per block; every
//                    workgroup merges the chunk maxima, workgroup 0 publishes s_g.
//   k_fp4_ew         dequant / STE / dequant-backward, 8 elements per step.
//   k_transpose_jobs byte transposes through 256 x 256-byte LDS tiles with
//                    4 x 4 register transposes and 16-byte stores, into a
//                    destination of any row stride (concatenation, padding).
//   k_fp4_to_fp8     FP4 -> E4M3 with the per-tensor scale folded in.
#include "tq_device.h"
#include "tq_host.h"

#include <string.h>

namespace tq {

enum { NV = 0, MX = 1 };

// Per-tensor max |x|, pass 1 (block partials into ws).  Plain loads, four
// in flight per thread (non-temporal loads measured 3% slower; two or eight
// in flight and 512- or 1024-thread blocks within 1%).
template <int FT>
__global__ __launch_bounds__(256) void k_amax_partial(const void* __restrict__ x, int64_t numel, int64_t chunk,
                                                      float* __restrict__ ws)
{
    __shared__ float sm[4];
    const int64_t blk = blockIdx.x;
    const int64_t b0 = blk * chunk;
    const int64_t b1 = b0 + chunk < numel ? b0 + chunk : numel;
    float a = 0.0f;
    for (int64_t e = b0 + (int64_t)threadIdx.x * 8; e < b1; e += 256 * 8 * 4) {
        Raw8<FT> r[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t ek = e + k * 256 * 8;
            if (ek < b1) r[k] = load8<FT>(x, ek);
            else r[k] = Raw8<FT>{};
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float v[8];
            widen8<FT>(r[k], v);
#pragma unroll
            for (int i = 0; i < 8; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
        }
    }
    a = team_max<64>(a);
    if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) ws[blk] = __builtin_fmaxf(__builtin_fmaxf(sm[0], sm[1]), __builtin_fmaxf(sm[2], sm[3]));
}

struct BP {
    float eff, y;
    uint32_t sb;
    bool fast;
};

// amax is an element magnitude of type FT (or 0); y6 = RN(1/(6 s_g)) when
// 6 s_g is inside the fast divisor range, else 0.
template <int FT>
__device__ __forceinline__ BP nv_params(float amax, float sg, float six_sg, float y6)
{
    BP p;
    const float q = (y6 != 0.0f && (value_in_fast_range(amax) || amax == 0.0f)) ? div_q<FT>(amax, six_sg, y6)
                                                                                  : amax / six_sg;
    const float v = __builtin_amdgcn_fmed3f(q, 0.0f, 448.0f);
    uint32_t sb = e4m3_pack4(v, 0.0f, 0.0f, 0.0f) & 0xffu;
    if ((sb & 0x7fu) == 0) sb = 0x38;
    p.sb = sb;
    p.eff = e4m3_val(sb, 0) * sg;
    p.fast = scale_in_fast_range(p.eff);
    p.y = p.fast ? rcp_rn(p.eff) : 0.0f;
    return p;
}

__device__ __forceinline__ BP mx_params(float amax)
{
    BP p;
    p.sb = e8m0_mx_byte(amax);
    p.eff = e8m0_val(p.sb);
    p.y = e8m0_inv(p.sb);
    p.fast = true;
    return p;
}

// Quotients x / eff for 8 values (E2M1 keeps the sign of zero, so a fast
// quotient gets x's sign back).
template <int FT, int KIND, bool FAST>
__device__ __forceinline__ void fp4_div8(const float v[8], const BP& p, float t[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if constexpr (KIND == MX) t[i] = v[i] * p.y;
        else t[i] = FAST ? with_sign_of(div_q<FT>(v[i], p.eff, p.y), v[i]) : v[i] / p.eff;
    }
}

// A team of T = GS/8 lanes per block (2 for NVFP4, 4 for MXFP4): lane j holds
// elements 8j..8j+7 of its block, so each load instruction of a wave reads
// 1 KB contiguously and each code store writes 256 bytes contiguously; the
// block max takes one or two DPP steps.  U rounds of 64/T blocks per wave.
template <int FT, int KIND, int U>
__global__ __launch_bounds__(256) void k_fp4_quant(const void* __restrict__ x, int64_t nblocks,
                                                   const float* __restrict__ global_scale,
                                                   uint8_t* __restrict__ packed, uint8_t* __restrict__ bscale)
{
    constexpr int GS = KIND == NV ? 16 : 32;
    constexpr int T = GS / 8;
    constexpr int P = 64 / T;
    const int lane = threadIdx.x & 63;
    const int j = lane % T;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t b0 = wave * (U * P) + lane / T;
    Raw8<FT> raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t b = b0 + (int64_t)u * P;
        if (b < nblocks) raw[u] = load8<FT, true>(x, b * GS + j * 8);
        else raw[u] = Raw8<FT>{};
    }
    const float sg = KIND == NV ? global_scale[0] : 1.0f;
    const float six_sg = 6.0f * sg;
    const float y6 = scale_in_fast_range(six_sg) ? rcp_rn(six_sg) : 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float v[8];
        widen8<FT>(raw[u], v);
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
        a = team_max<T>(a);
        const int64_t b = b0 + (int64_t)u * P;
        if (b >= nblocks) continue;
        const BP p = KIND == NV ? nv_params<FT>(a, sg, six_sg, y6) : mx_params(a);
        float t[8];
        if (p.fast) fp4_div8<FT, KIND, true>(v, p, t);
        else fp4_div8<FT, KIND, false>(v, p, t);
        st4<true>(packed + ((b * GS + j * 8) >> 1), e2m1_pack8(t));
        if (j == 0) bscale[b] = (uint8_t)p.sb;
    }
}

// Dynamic NVFP4, encode pass: one lane per 16-element block, so the block
// scale is computed once per 16 elements (the lane pairs of k_fp4_quant each
// repeat it) and the block max needs no lane exchange.  Lane l of a wave
// takes block (wave * U + u) * 64 + l; each of its two 16-byte loads covers
// half of every 128-byte line of a 2 KB span.  Right after the max pass these
// non-temporal loads measured 7% faster than k_fp4_quant's (the static
// quantize, which reads x cold, stays with k_fp4_quant: 9% slower here).
// Every workgroup merges the chunk maxima; workgroup 0 publishes s_g.
template <int FT, int U>
__global__ __launch_bounds__(256) void k_nv_quant_dyn(const void* __restrict__ x, int64_t nblocks,
                                                      float* __restrict__ global_scale, const float* __restrict__ parts,
                                                      int nparts, uint8_t* __restrict__ packed,
                                                      uint8_t* __restrict__ bscale)
{
    const Part4 pp = load_partials<false>(parts, nparts);
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t b0 = wave * (U * 64) + lane;
    Raw8<FT> lo[U], hi[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t b = b0 + (int64_t)u * 64;
        if (b < nblocks) {
            lo[u] = load8<FT, true>(x, b * 16);
            hi[u] = load8<FT, true>(x, b * 16 + 8);
        } else {
            lo[u] = Raw8<FT>{};
            hi[u] = Raw8<FT>{};
        }
    }
    float amax, unused;
    merge_partials<false>(pp, amax, unused);
    const float g = amax / 2688.0f;
    const float sg = (g == 0.0f) ? 1.0f : g;
    if (blockIdx.x == 0 && threadIdx.x == 0) global_scale[0] = sg;
    const float six_sg = 6.0f * sg;
    const float y6 = scale_in_fast_range(six_sg) ? rcp_rn(six_sg) : 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t b = b0 + (int64_t)u * 64;
        if (b >= nblocks) continue;
        float v[16];
        widen8<FT>(lo[u], v);
        widen8<FT>(hi[u], v + 8);
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
        const BP p = nv_params<FT>(a, sg, six_sg, y6);
        float t0[8], t1[8];
        if (p.fast) {
            fp4_div8<FT, NV, true>(v, p, t0);
            fp4_div8<FT, NV, true>(v + 8, p, t1);
        } else {
            fp4_div8<FT, NV, false>(v, p, t0);
            fp4_div8<FT, NV, false>(v + 8, p, t1);
        }
        st8<true>(packed + b * 8, make_uint2(e2m1_pack8(t0), e2m1_pack8(t1)));
        bscale[b] = (uint8_t)p.sb;
    }
}

// ------------------------------------------------------------ elementwise
enum { OP_DEQ = 0, OP_STE = 1, OP_DQB = 2 };
// Plain code loads in the dequantizer (non-temporal ones measured no faster).
constexpr bool EW_NT = false;

__device__ __forceinline__ float fp4_eff(int kind, uint32_t sb, float sg)
{
    return kind == NV ? e4m3_val(sb, 0) * sg : e8m0_val(sb);
}

template <int OP, int KIND, int FT>
__global__ __launch_bounds__(256) void k_fp4_ew(const void* __restrict__ a, const void* __restrict__ b,
                                                const uint8_t* __restrict__ bscale,
                                                const float* __restrict__ global_scale, int64_t nvec,
                                                void* __restrict__ out)
{
    constexpr int GS = KIND == NV ? 16 : 32;
    const float sg = KIND == NV ? global_scale[0] : 1.0f;
    if constexpr (OP == OP_DEQ) {
        for (int64_t base = (int64_t)blockIdx.x * 256 * DEQ_V; base < nvec;
             base += (int64_t)gridDim.x * 256 * DEQ_V) {
            uint32_t w[DEQ_V], sb[DEQ_V];
#pragma unroll
            for (int k = 0; k < DEQ_V; ++k) {
                const int64_t vi = base + k * 256 + threadIdx.x;
                if (vi < nvec)
                    w[k] = EW_NT ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(
                                       static_cast<const uint8_t*>(a) + vi * 4))
                                 : *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(a) + vi * 4);
            }
#pragma unroll
            for (int k = 0; k < DEQ_V; ++k) {
                const int64_t vi = base + k * 256 + threadIdx.x;
                if (vi < nvec) sb[k] = bscale[vi * 8 / GS];
            }
#pragma unroll
            for (int k = 0; k < DEQ_V; ++k) {
                const int64_t vi = base + k * 256 + threadIdx.x;
                if (vi >= nvec) break;
                const float eff = fp4_eff(KIND, sb[k], sg);
                float o[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f2v d = e2m1_val2(w[k], i);
                    o[2 * i] = d.x * eff;
                    o[2 * i + 1] = d.y * eff;
                }
                store8<FT, WT>(out, vi * 8, o);
            }
        }
        return;
    }
    for (int64_t vi = (int64_t)blockIdx.x * 256 + threadIdx.x; vi < nvec; vi += (int64_t)gridDim.x * 256) {
        const int64_t e = vi * 8;
        const uint32_t sb = bscale[e / GS];
        float o[8];
        if constexpr (OP == OP_DQB) {
            const float eff = fp4_eff(KIND, sb, sg);
            float d[8];
            widen8<FT>(load8<FT, true>(a, e), d);
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = d[i] * eff;
        } else {
            float xv[8], d[8], t[8], g[8];
            widen8<FT>(load8<FT, true>(a, e), xv);
            widen8<FT>(load8<FT, true>(b, e), d);
            if constexpr (KIND == MX) {
                const float inv = e8m0_inv(sb);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    t[i] = xv[i] * inv;
                    g[i] = d[i] * inv;
                }
            } else {
                const float eff = fp4_eff(KIND, sb, sg);
                const bool ok = scale_in_fast_range(eff) & values_fast8(d) & codes_fast8(xv);
                if (ok) {
                    const float y = rcp_rn(eff);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        t[i] = with_sign_of(div_q<FT>(xv[i], eff, y), xv[i]);
                        g[i] = div_q<FT>(d[i], eff, y);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        t[i] = xv[i] / eff;
                        g[i] = d[i] / eff;
                    }
                }
            }
            const uint32_t w = e2m1_pack8(t);
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = g[i] * (((w >> (4 * i)) & 7u) != 7u ? 1.0f : 0.0f);
        }
        store8<FT, OP == OP_DQB ? WT : 1>(out, e, o);
    }
}

// ------------------------------------------------------------ transpose
// dst[c * ldd + off + r] = src[r][c] for a [R, C] byte matrix: the transpose
// written into columns off..off+R-1 of a [C, ldd] matrix (ldd = R, off = 0 for
// a plain transpose).  Fast path: R, C, ldd and off multiples of 16 and
// 16-byte aligned bases; tiles of 256 x 256 bytes staged through LDS, so that
// every input row is read and every output row written in 256-byte segments
// (measured on the FP4 weight transposes: 128 x 128 tiles reach about 55% of
// HBM peak, 256 x 256 tiles about 62%).
constexpr int TRR = 256, TRC = 256, TR_PITCH = TRC / 4 + 1;   // dwords per LDS row, padded
// 65 KB of LDS per workgroup: two resident per CU, 512 on the chip; the
// launch never asks for more, and each workgroup walks its share of tiles.
constexpr int64_t TR_GRID = 512;   // (128, 256 or 384 workgroups walking 2-4 tiles each: 14-79% slower)

__device__ __forceinline__ void transpose4x4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3, uint32_t o[4])
{
    // o[c] byte i = row i byte c
    const uint32_t t01lo = __builtin_amdgcn_perm(r1, r0, 0x05010400u);   // r0b0 r1b0 r0b1 r1b1
    const uint32_t t01hi = __builtin_amdgcn_perm(r1, r0, 0x07030602u);   // r0b2 r1b2 r0b3 r1b3
    const uint32_t t23lo = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
    const uint32_t t23hi = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
    o[0] = __builtin_amdgcn_perm(t23lo, t01lo, 0x05040100u);              // r0b0 r1b0 r2b0 r3b0
    o[1] = __builtin_amdgcn_perm(t23lo, t01lo, 0x07060302u);              // r0b1 r1b1 r2b1 r3b1
    o[2] = __builtin_amdgcn_perm(t23hi, t01hi, 0x05040100u);
    o[3] = __builtin_amdgcn_perm(t23hi, t01hi, 0x07060302u);
}

// One TRR x TRC-byte tile (rows R0.., columns C0.. of src) of a transpose job.
struct TileAt {
    const uint8_t* src;
    uint8_t* dst;
    int64_t R, C, ldd, R0, C0;
};

// Tiles of TRR rows x TRC bytes.  Load: TRC/16 threads share an input row, so
// each wave instruction reads whole lines; read-out: thread (m, d) owns input
// columns 4d..4d+3 and input rows 16m..16m+15, reads 16 dwords from LDS,
// transposes four 4x4 byte blocks in registers and writes 16 bytes to each of
// 4 output rows; the TRR/16 threads with the same d write one TRR-byte output
// segment per row.
constexpr int TR_LOADS = TRR * TRC / 16 / 256, TR_OUTS = TRR * TRC / 64 / 256;

__device__ __forceinline__ void tile_load(const TileAt& T, uint4 w[TR_LOADS])
{
    const int t = threadIdx.x;
    constexpr int TPR = TRC / 16, RPP = 256 / TPR;    // threads per row, rows per pass
#pragma unroll
    for (int k = 0; k < TR_LOADS; ++k) {
        const int r = t / TPR + RPP * k;
        const int cq = (t % TPR) * 16;
        w[k] = make_uint4(0, 0, 0, 0);
        if (T.R0 + r < T.R && T.C0 + cq < T.C) w[k] = ld16<true>(T.src + (T.R0 + r) * T.C + T.C0 + cq);
    }
}

// LDS dword column c of tile row r sits at r * TR_PITCH + (c ^ tr_swz(r)).
// The read-out has sixteen row groups 16 m apart in one wave instruction; with
// the 65-dword pitch alone rows 64 apart share banks (4 lanes per bank), and
// flipping column bits 2-3 by (r / 64) % 4 spreads them over distinct banks.
// The stage writes stay conflict-free: the flip moves whole 4-dword chunks
// (NVFP4 / MXFP4 weight transpose 12.7 / 12.3 -> 12.3 / 11.8 us).
__device__ __forceinline__ int tr_swz(int r) { return 4 * ((r >> 6) & 3); }

__device__ __forceinline__ void tile_stage(const uint4 w[TR_LOADS], uint32_t* tile)
{
    const int t = threadIdx.x;
    constexpr int TPR = TRC / 16, RPP = 256 / TPR;
#pragma unroll
    for (int k = 0; k < TR_LOADS; ++k) {
        const int r = t / TPR + RPP * k;
        uint32_t* row = tile + r * TR_PITCH + (((t % TPR) * 4) ^ tr_swz(r));
        row[0] = w[k].x;
        row[1] = w[k].y;
        row[2] = w[k].z;
        row[3] = w[k].w;
    }
}

__device__ __forceinline__ void tile_store(const TileAt& T, const uint32_t* tile)
{
#pragma unroll
    for (int p = 0; p < TR_OUTS; ++p) {
        const int t = threadIdx.x + 256 * p;
        const int m = t % (TRR / 16), d = t / (TRR / 16);
        const int ds = d ^ tr_swz(16 * m);      // rows 16m .. 16m + 15 share the flip
        uint32_t o[4][4];                       // o[c][qd]: output row 4d+c, bytes 4*qd.. of this 16-byte piece
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int rb = 16 * m + 4 * qd;
            uint32_t tr[4];
            transpose4x4(tile[(rb + 0) * TR_PITCH + ds], tile[(rb + 1) * TR_PITCH + ds],
                         tile[(rb + 2) * TR_PITCH + ds], tile[(rb + 3) * TR_PITCH + ds], tr);
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c][qd] = tr[c];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int64_t oc = T.C0 + 4 * d + c;      // output row = input column
            const int64_t orr = T.R0 + 16 * m;        // output column = input row
            if (oc < T.C && orr < T.R)
                st16<true>(T.dst + oc * T.ldd + orr, make_uint4(o[c][0], o[c][1], o[c][2], o[c][3]));
        }
    }
}

// Several transposes in one launch (codes and block scales of a weight, every
// part of a concatenation): tile b belongs to the job whose range holds b, so
// small matrices (the block scales) fill the chip together with the large ones
// instead of running as a separate under-occupied launch.
struct TJob {
    const uint8_t* src;
    uint8_t* dst;
    int64_t R, C, ldd;
    int64_t tile0, tiles_c;
};
constexpr int MAX_TJOBS = 8;
struct TJobs {
    TJob j[MAX_TJOBS];
    int n;
    int64_t tiles;
};

__device__ __forceinline__ TileAt tile_at(const TJobs& jobs, int64_t b)
{
    int k = 0;
    for (int i = 1; i < jobs.n; ++i)
        if (b >= jobs.j[i].tile0) k = i;
    const TJob& J = jobs.j[k];
    const int64_t tl = b - J.tile0;
    return TileAt{J.src, J.dst, J.R, J.C, J.ldd, (tl / J.tiles_c) * TRR, (tl % J.tiles_c) * TRC};
}

// A workgroup walks tiles b, b + gridDim.x, ...; the next tile's loads are
// issued as soon as the current one sits in LDS, so they are in flight while
// the current tile is read out and stored (with one tile per workgroup every
// workgroup on the chip would read, then write, in lock step).
__global__ __launch_bounds__(256) void k_transpose_jobs(const TJobs jobs)
{
    __shared__ uint32_t tile[TRR * TR_PITCH];
    int64_t b = blockIdx.x;
    TileAt T = tile_at(jobs, b);
    uint4 w[TR_LOADS];
    tile_load(T, w);
    for (;;) {
        tile_stage(w, tile);
        __syncthreads();
        const int64_t nb = b + gridDim.x;
        const bool more = nb < jobs.tiles;
        TileAt Tn = T;
        if (more) {
            Tn = tile_at(jobs, nb);
            tile_load(Tn, w);
        }
        tile_store(T, tile);
        if (!more) break;
        __syncthreads();
        b = nb;
        T = Tn;
    }
}

__global__ __launch_bounds__(256) void k_transpose_u8_generic(const uint8_t* __restrict__ src, int64_t R, int64_t C,
                                                              uint8_t* __restrict__ dst, int64_t ldd)
{
    __shared__ uint8_t tile[64][65];
    const int64_t R0 = (int64_t)blockIdx.y * 64, C0 = (int64_t)blockIdx.x * 64;
    for (int k = threadIdx.x; k < 64 * 64; k += 256) {
        const int r = k / 64, c = k % 64;
        if (R0 + r < R && C0 + c < C) tile[r][c] = src[(R0 + r) * C + C0 + c];
    }
    __syncthreads();
    for (int k = threadIdx.x; k < 64 * 64; k += 256) {
        const int c = k / 64, r = k % 64;
        if (R0 + r < R && C0 + c < C) dst[(C0 + c) * ldd + R0 + r] = tile[r][c];
    }
}

// Zero columns c0..c1-1 of each of `rows` rows of a byte matrix with row
// stride ld (the pad of a concatenated transpose).
__global__ __launch_bounds__(256) void k_zero_cols(uint8_t* __restrict__ dst, int64_t rows, int64_t ld, int64_t c0,
                                                   int64_t c1)
{
    const int64_t w = c1 - c0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows * w; i += (int64_t)gridDim.x * 256)
        dst[(i / w) * ld + c0 + i % w] = 0;
}

// ------------------------------------------------------------ row concat
// Up to four byte ranges copied in one launch; each range moves in the widest
// unit (16, 8 or 1 bytes) that its source, destination and length allow.
// Block b copies 256 units of the range whose block span holds b.
struct CSeg {
    const uint8_t* src;
    uint8_t* dst;
    int64_t units;
    int64_t block0;
    int32_t unit;
};
struct CSegs {
    CSeg s[4];
    int n;
};

__global__ __launch_bounds__(256) void k_copy_segments(const CSegs segs)
{
    const int64_t b = blockIdx.x;
    int k = 0;
    for (int i = 1; i < segs.n; ++i)
        if (b >= segs.s[i].block0) k = i;
    const CSeg S = segs.s[k];
    const int64_t i = (b - S.block0) * 256 + threadIdx.x;
    if (i >= S.units) return;
    if (S.unit == 16) st16<WT>(S.dst + i * 16, ld16<true>(S.src + i * 16));
    else if (S.unit == 8) st8<true>(S.dst + i * 8, ld8<true>(S.src + i * 8));
    else S.dst[i] = S.src[i];
}

// ------------------------------------------------------------ FP4 -> FP8
// out = E4M3(val(q) * eff) per element, eff as in dequantization.  One lane
// per 16 elements: an 8-byte code load (a wave reads 512 contiguous bytes) and
// one 16-byte E4M3 store (1 KB per wave instruction).
template <int KIND>
__global__ __launch_bounds__(256) void k_fp4_to_fp8(const uint8_t* __restrict__ packed,
                                                    const uint8_t* __restrict__ bscale, float sg, int64_t n16,
                                                    uint8_t* __restrict__ out)
{
    constexpr int U = 2;
    const int64_t base = (int64_t)blockIdx.x * (256 * U) + threadIdx.x;
    uint2 w[U];
    uint32_t sb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + u * 256;
        w[u] = make_uint2(0, 0);
        sb[u] = 0;
        if (i < n16) {
            w[u] = ld8<true>(packed + i * 8);
            sb[u] = bscale[KIND == NV ? i : i / 2];
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + u * 256;
        if (i >= n16) break;
        const float eff = fp4_eff(KIND, sb[u], sg);
        float d[16];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const f2v lo = e2m1_val2(w[u].x, b), hi = e2m1_val2(w[u].y, b);
            d[2 * b] = lo.x * eff;
            d[2 * b + 1] = lo.y * eff;
            d[8 + 2 * b] = hi.x * eff;
            d[8 + 2 * b + 1] = hi.y * eff;
        }
        st16<WT>(out + i * 16, make_uint4(e4m3_pack4(d[0], d[1], d[2], d[3]), e4m3_pack4(d[4], d[5], d[6], d[7]),
                                          e4m3_pack4(d[8], d[9], d[10], d[11]),
                                          e4m3_pack4(d[12], d[13], d[14], d[15])));
    }
}

// ============================================================ host side

#define TQ_FT_SWITCH(ft, ...)                                     \
    switch (ft) {                                                 \
    case TQ_F32: { constexpr int FTV = F32; __VA_ARGS__; } break; \
    case TQ_F16: { constexpr int FTV = F16; __VA_ARGS__; } break; \
    default: { constexpr int FTV = BF16; __VA_ARGS__; } break;    \
    }

// Transposes dst[c * ldd + r] = src[r][c] collected into job launches.  A
// job takes the tiled kernel when R, C and ldd are multiples of 16 and both
// bases 16-byte aligned (dst already points at the job's column offset);
// others run the generic kernel at once.  flush() launches what is queued.
struct TransposeBatch {
    TJobs jobs{};
    int64_t tiles = 0;
    hipStream_t st;
    tq_status err = TQ_OK;
    explicit TransposeBatch(hipStream_t s) : st(s) { jobs.n = 0; }
    void flush()
    {
        if (jobs.n == 0 || err) return;
        if (tiles > 0x7fffffff) {
            err = TQ_ERR_UNSUPPORTED;
            return;
        }
        jobs.tiles = tiles;
        const int64_t grid = tiles < TR_GRID ? tiles : TR_GRID;
        hipLaunchKernelGGL(k_transpose_jobs, dim3((unsigned)grid), dim3(256), 0, st, jobs);
        err = launch_status();
        jobs.n = 0;
        tiles = 0;
    }
    void add(const uint8_t* src, int64_t R, int64_t C, uint8_t* dst, int64_t ldd)
    {
        if (R == 0 || C == 0 || err) return;
        if (R % 16 == 0 && C % 16 == 0 && ldd % 16 == 0 && aligned16(src) && aligned16(dst)) {
            if (jobs.n == MAX_TJOBS) flush();
            TJob& j = jobs.j[jobs.n++];
            j.src = src;
            j.dst = dst;
            j.R = R;
            j.C = C;
            j.ldd = ldd;
            j.tile0 = tiles;
            j.tiles_c = cdiv(C, TRC);
            tiles += j.tiles_c * cdiv(R, TRR);
        } else {
            if (cdiv(R, 64) > 65535) {
                err = TQ_ERR_UNSUPPORTED;
                return;
            }
            hipLaunchKernelGGL(k_transpose_u8_generic, dim3((unsigned)cdiv(C, 64), (unsigned)cdiv(R, 64)), dim3(256), 0,
                               st, src, R, C, dst, ldd);
            err = launch_status();
        }
    }
    tq_status finish()
    {
        flush();
        return err;
    }
};

static tq_status check_fp4(int64_t rows, int64_t k, int kind)
{
    if (kind != TQ_NVFP4 && kind != TQ_MXFP4) return TQ_ERR_INVALID;
    if (rows < 0 || k < 0) return TQ_ERR_INVALID;
    if (k % (kind == TQ_NVFP4 ? 16 : 32)) return TQ_ERR_INVALID;
    return TQ_OK;
}

tq_status check_fp4_quant(const void* x, int x_dtype, int64_t rows, int64_t k, int kind, const uint8_t* packed,
                          const uint8_t* block_scale, const float* global_scale)
{
    if (!valid_ftype(x_dtype)) return TQ_ERR_INVALID;
    tq_status s = check_fp4(rows, k, kind);
    if (s || rows * k == 0) return s;
    if (!x || !packed || !block_scale) return TQ_ERR_INVALID;
    if (kind == TQ_NVFP4 && !global_scale) return TQ_ERR_INVALID;
    if (!aligned16(x) || !aligned16(packed)) return TQ_ERR_ALIGN;
    return TQ_OK;
}

// The quantize launches.  A dynamic NVFP4 s_g takes two: the chunk maxima
// into ws (TENSOR_PARTS floats at most, 16-byte aligned), then the encode,
// whose every workgroup merges them.
tq_status fp4_quant_launch(const void* x, int x_dtype, int64_t numel, int kind, uint8_t* packed,
                           uint8_t* block_scale, float* global_scale, int static_global, float* ws, hipStream_t st)
{
    constexpr int U = 2;   // 16- or 32-element blocks per lane in flight (1, 4 and 8 measured slower)
    if (kind == TQ_NVFP4) {
        const int64_t nb = numel / 16;
        const dim3 grid((unsigned)cdiv(cdiv(nb, U * 32), 4));
        if (static_global) {
            TQ_FT_SWITCH(x_dtype, hipLaunchKernelGGL((k_fp4_quant<FTV, NV, U>), grid, dim3(256), 0, st, x, nb,
                                                     global_scale, packed, block_scale));
        } else {
            // (one workgroup publishing s_g between the passes measured the same; at most 256
            // larger chunks instead of 1024 made the call 16% slower)
            int nparts;
            const int64_t chunk = tensor_chunk(numel, &nparts);
            // (the encode in k_fp4_quant's lane pairs, 2 or 4 blocks per lane, measured 3-7% slower)
            const dim3 gridd((unsigned)cdiv(cdiv(nb, U * 64), 4));
            TQ_FT_SWITCH(x_dtype, {
                hipLaunchKernelGGL((k_amax_partial<FTV>), dim3(nparts), dim3(256), 0, st, x, numel, chunk, ws);
                hipLaunchKernelGGL((k_nv_quant_dyn<FTV, U>), gridd, dim3(256), 0, st, x, nb, global_scale, ws, nparts,
                                   packed, block_scale);
            });
        }
    } else {
        const int64_t nb = numel / 32;
        const dim3 grid((unsigned)cdiv(cdiv(nb, U * 16), 4));
        TQ_FT_SWITCH(x_dtype, hipLaunchKernelGGL((k_fp4_quant<FTV, MX, U>), grid, dim3(256), 0, st, x, nb, nullptr,
                                                 packed, block_scale));
    }
    return launch_status();
}

template <int OP>
static tq_status fp4_elementwise(const void* a, const void* b, int ft, const uint8_t* bscale, const float* sg,
                                 int64_t rows, int64_t k, int kind, void* out, hipStream_t st)
{
    const int64_t nvec = rows * k / 8;
    if (nvec == 0) return TQ_OK;
    const dim3 grid(grid_for(nvec, 256 * (OP == OP_DEQ ? DEQ_V : 1))), block(256);
    if (kind == TQ_NVFP4) {
        TQ_FT_SWITCH(ft, hipLaunchKernelGGL((k_fp4_ew<OP, NV, FTV>), grid, block, 0, st, a, b, bscale, sg, nvec, out));
    } else {
        TQ_FT_SWITCH(ft, hipLaunchKernelGGL((k_fp4_ew<OP, MX, FTV>), grid, block, 0, st, a, b, bscale, sg, nvec, out));
    }
    return launch_status();
}

}  // namespace tq

using namespace tq;

extern "C" {

tq_status tq_quant_fp4_block(const void* x, int x_dtype, int64_t rows, int64_t k, int kind, uint8_t* packed,
                             uint8_t* block_scale, float* global_scale, int static_global, void* workspace,
                             size_t workspace_bytes, void* stream)
{
    tq_status s = check_fp4_quant(x, x_dtype, rows, k, kind, packed, block_scale, global_scale);
    if (s || rows * k == 0) return s;
    if (kind == TQ_NVFP4 && !static_global) {
        if (!workspace || workspace_bytes < tq_workspace_bytes(1, rows * k)) return TQ_ERR_INVALID;
        if (!aligned16(workspace)) return TQ_ERR_ALIGN;
    }
    return fp4_quant_launch(x, x_dtype, rows * k, kind, packed, block_scale, global_scale, static_global,
                            static_cast<float*>(workspace), as_stream(stream));
}

tq_status tq_dequant_fp4_block(const uint8_t* packed, const uint8_t* block_scale, const float* global_scale,
                               int64_t rows, int64_t k, int kind, void* y, int y_dtype, void* stream)
{
    if (!valid_ftype(y_dtype)) return TQ_ERR_INVALID;
    tq_status s = check_fp4(rows, k, kind);
    if (s || rows * k == 0) return s;
    if (!packed || !block_scale || !y) return TQ_ERR_INVALID;
    if (kind == TQ_NVFP4 && !global_scale) return TQ_ERR_INVALID;
    if (!aligned16(packed) || !aligned16(y)) return TQ_ERR_ALIGN;
    return fp4_elementwise<OP_DEQ>(packed, nullptr, y_dtype, block_scale, global_scale, rows, k, kind, y,
                                   as_stream(stream));
}

tq_status tq_quant_fp4_block_backward(const void* x, int x_dtype, const uint8_t* block_scale,
                                      const float* global_scale, int64_t rows, int64_t k, int kind, const void* dy,
                                      void* dx, void* stream)
{
    if (!valid_ftype(x_dtype)) return TQ_ERR_INVALID;
    tq_status s = check_fp4(rows, k, kind);
    if (s || rows * k == 0) return s;
    if (!x || !dy || !dx || !block_scale) return TQ_ERR_INVALID;
    if (kind == TQ_NVFP4 && !global_scale) return TQ_ERR_INVALID;
    if (!aligned16(x) || !aligned16(dy) || !aligned16(dx)) return TQ_ERR_ALIGN;
    return fp4_elementwise<OP_STE>(x, dy, x_dtype, block_scale, global_scale, rows, k, kind, dx, as_stream(stream));
}

tq_status tq_dequant_fp4_block_backward(const void* dy, int dy_dtype, const uint8_t* block_scale,
                                        const float* global_scale, int64_t rows, int64_t k, int kind, void* dq,
                                        void* stream)
{
    if (!valid_ftype(dy_dtype)) return TQ_ERR_INVALID;
    tq_status s = check_fp4(rows, k, kind);
    if (s || rows * k == 0) return s;
    if (!dy || !dq || !block_scale) return TQ_ERR_INVALID;
    if (kind == TQ_NVFP4 && !global_scale) return TQ_ERR_INVALID;
    if (!aligned16(dy) || !aligned16(dq)) return TQ_ERR_ALIGN;
    return fp4_elementwise<OP_DQB>(dy, nullptr, dy_dtype, block_scale, global_scale, rows, k, kind, dq,
                                   as_stream(stream));
}

tq_status tq_fp4_transpose_for_gemm(const uint8_t* packed, const uint8_t* block_scale, int64_t n, int64_t k,
                                    int32_t group_size, uint8_t* packed_t, uint8_t* block_scale_t, void* stream)
{
    if (n < 0 || k < 0 || (k & 1) || group_size <= 0 || k % group_size) return TQ_ERR_INVALID;
    if (n == 0 || k == 0) return TQ_OK;
    if (!packed || !packed_t) return TQ_ERR_INVALID;
    if ((block_scale == nullptr) != (block_scale_t == nullptr)) return TQ_ERR_INVALID;
    TransposeBatch tb(as_stream(stream));
    tb.add(packed, n, k / 2, packed_t, n);
    if (block_scale) tb.add(block_scale, n, k / group_size, block_scale_t, n);
    return tb.finish();
}

tq_status tq_fp4_transpose_concat_for_gemm(int32_t nparts, const uint8_t* const* host_packed,
                                           const uint8_t* const* host_block_scale, const int64_t* host_n,
                                           int64_t k, int32_t group_size, int64_t align, uint8_t* packed_t,
                                           uint8_t* block_scale_t, int64_t* host_stride, void* stream)
{
    if (nparts <= 0 || !host_packed || !host_n || k < 0 || (k & 1) || group_size <= 0 || k % group_size ||
        align <= 0)
        return TQ_ERR_INVALID;
    int64_t total = 0;
    for (int32_t i = 0; i < nparts; ++i) {
        if (host_n[i] < 0 || host_n[i] > (INT64_MAX >> 2) - total) return TQ_ERR_INVALID;
        total += host_n[i];
    }
    const int64_t stride = cdiv(total, align) * align;
    if (host_stride) *host_stride = stride;
    const bool scales = block_scale_t != nullptr;
    if (scales && !host_block_scale) return TQ_ERR_INVALID;
    if (stride == 0 || k == 0) return TQ_OK;
    if (!packed_t) return TQ_ERR_INVALID;
    for (int32_t i = 0; i < nparts; ++i) {
        if (host_n[i] == 0) continue;
        if (!host_packed[i] || (scales && !host_block_scale[i])) return TQ_ERR_INVALID;
    }
    hipStream_t st = as_stream(stream);
    const int64_t kb = k / 2, nb = k / group_size;
    TransposeBatch tb(st);
    int64_t off = 0;
    for (int32_t i = 0; i < nparts; ++i) {
        tb.add(host_packed[i], host_n[i], kb, packed_t + off, stride);
        if (scales) tb.add(host_block_scale[i], host_n[i], nb, block_scale_t + off, stride);
        off += host_n[i];
    }
    tq_status s = tb.finish();
    if (s) return s;
    if (stride > total) {
        hipLaunchKernelGGL(k_zero_cols, dim3(grid_for(kb * (stride - total), 256)), dim3(256), 0, st, packed_t, kb,
                           stride, total, stride);
        if (scales)
            hipLaunchKernelGGL(k_zero_cols, dim3(grid_for(nb * (stride - total), 256)), dim3(256), 0, st,
                               block_scale_t, nb, stride, total, stride);
        return launch_status();
    }
    return TQ_OK;
}

tq_status tq_fp4_concat_rows(const uint8_t* packed1, const uint8_t* block_scale1, float host_global_scale1,
                             const uint8_t* packed2, const uint8_t* block_scale2, float host_global_scale2,
                             int64_t n1, int64_t n2, int64_t k, uint8_t* packed_out, uint8_t* block_scale_out,
                             void* stream)
{
    if (n1 < 0 || n2 < 0 || k < 0 || k % 16) return TQ_ERR_INVALID;
    uint32_t g1, g2;
    memcpy(&g1, &host_global_scale1, 4);
    memcpy(&g2, &host_global_scale2, 4);
    if (g1 != g2) return TQ_ERR_INVALID;
    const int64_t kb = k / 2, nb = k / 16;
    if ((n1 + n2) * k == 0) return TQ_OK;
    if (!packed_out || !block_scale_out) return TQ_ERR_INVALID;
    if (n1 > 0 && (!packed1 || !block_scale1)) return TQ_ERR_INVALID;
    if (n2 > 0 && (!packed2 || !block_scale2)) return TQ_ERR_INVALID;
    const struct { const uint8_t* src; uint8_t* dst; int64_t bytes; } cp[4] = {
        {packed1, packed_out, n1 * kb}, {packed2, packed_out + n1 * kb, n2 * kb},
        {block_scale1, block_scale_out, n1 * nb}, {block_scale2, block_scale_out + n1 * nb, n2 * nb}};
    CSegs segs{};
    int64_t blocks = 0;
    for (const auto& c : cp) {
        if (c.bytes <= 0) continue;
        const uintptr_t a = reinterpret_cast<uintptr_t>(c.src) | reinterpret_cast<uintptr_t>(c.dst) | (uintptr_t)c.bytes;
        CSeg& g = segs.s[segs.n++];
        g.unit = (a % 16 == 0) ? 16 : (a % 8 == 0) ? 8 : 1;
        g.src = c.src;
        g.dst = c.dst;
        g.units = c.bytes / g.unit;
        g.block0 = blocks;
        blocks += cdiv(g.units, 256);
    }
    if (blocks > 0x7fffffff) return TQ_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(k_copy_segments, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream), segs);
    return launch_status();
}

tq_status tq_fp4_predequant_to_fp8(const uint8_t* packed, const uint8_t* block_scale, float host_global_scale,
                                   int64_t rows, int64_t k, int kind, uint8_t* fp8_out, void* stream)
{
    tq_status s = check_fp4(rows, k, kind);
    if (s || rows * k == 0) return s;
    if (!packed || !block_scale || !fp8_out) return TQ_ERR_INVALID;
    if ((reinterpret_cast<uintptr_t>(packed) & 7) || !aligned16(fp8_out)) return TQ_ERR_ALIGN;
    const int64_t n16 = rows * k / 16;
    const dim3 grid((unsigned)cdiv(n16, 512)), block(256);
    if (cdiv(n16, 512) > 0x7fffffff) return TQ_ERR_UNSUPPORTED;
    hipStream_t st = as_stream(stream);
    if (kind == TQ_NVFP4)
        hipLaunchKernelGGL(k_fp4_to_fp8<NV>, grid, block, 0, st, packed, block_scale, host_global_scale, n16, fp8_out);
    else
        hipLaunchKernelGGL(k_fp4_to_fp8<MX>, grid, block, 0, st, packed, block_scale, 1.0f, n16, fp8_out);
    return launch_status();
}

}  // extern "C"
