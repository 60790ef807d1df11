// tq_fp8.hip -- FP8 E4M3 block quantization (smile.llm.quant package summary:
// Fp8BlockGemm's activation quantizer with one fp32 scale per 1x128 group and
// its weights with one fp32 scale per 128x128 tile; Fp8BlockDequant), with
// the STE backward and the dequantize backward.
//
//   scale = amax / 448 (1 if that is 0),  q = E4M3(x / scale)
//
// E4M3 is the OCP format (bias 7, max 448) that gfx950's v_cvt_pk_fp8_f32
// produces; values are clamped to +-448 before the conversion (saturation),
// the conversion rounds to nearest even.
//
// Kernels:
//   k_fp8_rows   blocks of 1 x bc (bc = 16..512, power of two): a team of
//                bc/8 lanes per block, 8 blocks per team per launch row.
//   k_fp8_tile   blocks of br x bc with bc = 8*T and br = NP * NT/T: one
//                NT-thread workgroup per tile (512 for 128 x 128, else 256),
//                the tile in registers, the tile max through DPP, bpermute
//                and LDS.
//   k_fp8_generic  any block shape, partial edge blocks included: one
//                  workgroup per block, two passes.
//   k_fp8_ew     dequant / STE / dequant-backward, elementwise, 16-byte I/O.
//
// MXFP8 (smile.llm.quant MxFp8; OCP MX v1.0): E4M3 elements with one E8M0
// scale X = 2^(floor(log2 amax) - 8) per 32 consecutive elements along K;
// q = E4M3(x * 2^(127 - sb)), which is exactly RN(x / X).
//   k_mxfp8_quant  a team of 4 lanes per block (8 elements each): each load
//                  instruction of a wave reads 1 KB, each code store 512 B.
//   k_mxfp8_ew     dequant / STE / dequant-backward, 8 elements per step.
#include "tq_device.h"
#include "tq_host.h"

namespace tq {

struct FP {
    float s, y;
    bool fast;
};

constexpr float Y448 = 1.0f / 448.0f;   // RN(1/448), folded at compile time

// amax is an element magnitude of type FT (or 0).
template <int FT>
__device__ __forceinline__ FP fp8_params(float amax)
{
    FP p;
    const float s = div_by<FT>(amax, 448.0f, Y448);
    p.s = (s == 0.0f) ? 1.0f : s;
    p.fast = scale_in_fast_range(p.s);
    p.y = p.fast ? rcp_rn(p.s) : 0.0f;
    return p;
}

// E4M3 keeps the sign of zero, so a fast quotient gets x's sign back.
template <int FT, bool FAST>
__device__ __forceinline__ uint2 fp8_enc8(const float v[8], const FP& p)
{
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = FAST ? with_sign_of(div_q<FT>(v[i], p.s, p.y), v[i]) : v[i] / p.s;
    return make_uint2(e4m3_pack4(t[0], t[1], t[2], t[3]), e4m3_pack4(t[4], t[5], t[6], t[7]));
}

// ------------------------------------------------------------ 1 x bc rows
// Blocks of L = 8*T*W contiguous elements: lane j of a team of T holds
// vectors w*T + j, so a team's load instruction reads 16*T contiguous bytes.
// STRIDED: input rows start every ldx elements (nbc blocks per row); codes
// and scales stay dense.
template <int FT, int T, int W, int U, bool STRIDED = false>
__global__ __launch_bounds__(256) void k_fp8_rows(const void* __restrict__ x, int64_t nblocks, int64_t nbc,
                                                  int64_t ldx, uint8_t* __restrict__ q, float* __restrict__ scale)
{
    constexpr int P = 64 / T;
    constexpr int64_t L = 8 * T * W;
    const int lane = threadIdx.x & 63;
    const int j = lane % T;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t g0 = wave * (U * P) + lane / T;
    Raw8<FT> raw[U][W];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t g = g0 + (int64_t)u * P;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const int64_t xb = STRIDED ? (g / nbc) * ldx + (g % nbc) * L : g * L;
            if (g < nblocks) raw[u][w] = load8<FT, (T >= 8)>(x, xb + (w * T + j) * 8);
            else raw[u][w] = Raw8<FT>{};
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float v[W][8];
        float a = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            widen8<FT>(raw[u][w], v[w]);
#pragma unroll
            for (int i = 0; i < 8; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[w][i]));
        }
        const FP p = fp8_params<FT>(team_max<T>(a));
        const int64_t g = g0 + (int64_t)u * P;
        if (g >= nblocks) continue;
        if constexpr (T == 8 && W == 2) {
            // 1 x 128 groups: lane j encodes vectors j and 8 + j; exchanges within the team give
            // it the codes of vectors 2j and 2j + 1, stored as 16 contiguous bytes, so each store
            // instruction of the wave writes 1 KB of whole lines (3% faster than two 8-byte stores
            // per lane; non-temporal 8-byte stores measured 3% slower)
            uint2 c[2];
#pragma unroll
            for (int w = 0; w < 2; ++w) c[w] = p.fast ? fp8_enc8<FT, true>(v[w], p) : fp8_enc8<FT, false>(v[w], p);
            const int base = lane & ~7;
            const int slo = (base + ((2 * j) & 7)) << 2, shi = (base + ((2 * j + 1) & 7)) << 2;
            const bool upper = j >= 4;   // vectors 2j, 2j + 1 >= 8: the lanes' second vectors
            const uint32_t ax0 = (uint32_t)__builtin_amdgcn_ds_bpermute(slo, (int)c[0].x);
            const uint32_t ay0 = (uint32_t)__builtin_amdgcn_ds_bpermute(slo, (int)c[0].y);
            const uint32_t ax1 = (uint32_t)__builtin_amdgcn_ds_bpermute(slo, (int)c[1].x);
            const uint32_t ay1 = (uint32_t)__builtin_amdgcn_ds_bpermute(slo, (int)c[1].y);
            const uint32_t bx0 = (uint32_t)__builtin_amdgcn_ds_bpermute(shi, (int)c[0].x);
            const uint32_t by0 = (uint32_t)__builtin_amdgcn_ds_bpermute(shi, (int)c[0].y);
            const uint32_t bx1 = (uint32_t)__builtin_amdgcn_ds_bpermute(shi, (int)c[1].x);
            const uint32_t by1 = (uint32_t)__builtin_amdgcn_ds_bpermute(shi, (int)c[1].y);
            st16<1>(q + g * L + 16 * j, make_uint4(upper ? ax1 : ax0, upper ? ay1 : ay0, upper ? bx1 : bx0,
                                                   upper ? by1 : by0));
        } else {
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const uint2 c = p.fast ? fp8_enc8<FT, true>(v[w], p) : fp8_enc8<FT, false>(v[w], p);
                *reinterpret_cast<uint2*>(q + g * L + (w * T + j) * 8) = c;
            }
        }
        if (j == 0) scale[g] = p.s;
    }
}

// ------------------------------------------------------------ br x bc tiles
// Thread t covers columns (t % T) * 8 .. +8 and rows t / T + k * (256 / T),
// k = 0..NP-1, of its tile.  (128 x 128 tiles over 512 or 1024 threads, with
// 8 waves per SIMD resident instead of 5, measured the same or slower.)
template <int FT, int T, int NP, int NT = 256>
__global__ __launch_bounds__(NT) void k_fp8_tile(const void* __restrict__ x, int64_t cols, int64_t nbc,
                                                 uint8_t* __restrict__ q, float* __restrict__ scale)
{
    constexpr int RP = NT / T, NW = NT / 64;
    __shared__ float wmax[NW];
    const int64_t tr = blockIdx.y, tc = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t r0 = tr * (RP * NP) + t / T;
    const int64_t c0 = tc * (8 * T) + (t % T) * 8;
    Raw8<FT> raw[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) raw[k] = load8<FT, (T >= 8)>(x, (r0 + (int64_t)k * RP) * cols + c0);
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        float v[8];
        widen8<FT>(raw[k], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
    }
    a = team_max<64>(a);
    if ((t & 63) == 0) wmax[t >> 6] = a;
    __syncthreads();
    a = wmax[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) a = __builtin_fmaxf(a, wmax[i]);
    const FP p = fp8_params<FT>(a);
    // only the raw inputs live across the barrier; widening them again is
    // cheaper than holding the binary32 copies
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        float v[8];
        widen8<FT>(raw[k], v);
        st8<(T >= 16)>(q + (r0 + (int64_t)k * RP) * cols + c0,
                       p.fast ? fp8_enc8<FT, true>(v, p) : fp8_enc8<FT, false>(v, p));
    }
    if (t == 0) scale[tr * nbc + tc] = p.s;
}

// ------------------------------------------------------------ generic blocks
// One workgroup per block, two passes over it; blocks on the last block row /
// column may be partial (hb x wb of the br x bc that the shape leaves).
template <int FT>
__global__ __launch_bounds__(256) void k_fp8_generic(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                     int64_t br, int64_t bc, int64_t nbc, uint8_t* __restrict__ q,
                                                     float* __restrict__ scale)
{
    __shared__ float wmax[4];
    const int64_t blk = blockIdx.x;
    const int64_t r0 = (blk / nbc) * br, c0 = (blk % nbc) * bc;
    const int64_t hb = rows - r0 < br ? rows - r0 : br;
    const int64_t wb = cols - c0 < bc ? cols - c0 : bc;
    const int64_t n = hb * wb;
    float a = 0.0f;
    for (int64_t j = threadIdx.x; j < n; j += 256)
        a = __builtin_fmaxf(a, __builtin_fabsf(load1<FT>(x, (r0 + j / wb) * cols + c0 + j % wb)));
    a = team_max<64>(a);
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = a;
    __syncthreads();
    a = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
    const FP p = fp8_params<FT>(a);
    for (int64_t j = threadIdx.x; j < n; j += 256) {
        const int64_t e = (r0 + j / wb) * cols + c0 + j % wb;
        const float t = load1<FT>(x, e) / p.s;
        q[e] = (uint8_t)e4m3_pack4(t, 0.0f, 0.0f, 0.0f);
    }
    if (threadIdx.x == 0) scale[blk] = p.s;
}

// ------------------------------------------------------------ elementwise
enum { OP_DEQ = 0, OP_STE = 1, OP_DQB = 2 };
// Plain code loads in the dequantizers (non-temporal ones measured no faster).
constexpr bool EW_NT = false;

__device__ __forceinline__ int64_t fp8_block_of(int64_t e, int64_t cols, int64_t br, int64_t bc, int64_t nbc)
{
    return ((e / cols) / br) * nbc + (e % cols) / bc;
}

// Block index of element e for power-of-two block shapes in a tensor of
// fewer than 2^32 elements: row = e / cols by a multiply-high with a
// host-computed magic number (Granlund and Montgomery's round-up method,
// exact for every 32-bit dividend), the rest by shifts.
struct BlkIdx {
    uint32_t cols, mul, sh;   // cols == 0: not available
    int lbr, lbc;
    uint32_t nbc;
    __device__ __forceinline__ int64_t of(int64_t e) const
    {
        const uint32_t n = (uint32_t)e;
        uint32_t row = n;
        if (cols != 1) {
            const uint32_t t = __umulhi(mul, n);
            row = (t + ((n - t) >> 1)) >> sh;
        }
        const uint32_t col = n - row * cols;
        return (int64_t)(row >> lbr) * nbc + (col >> lbc);
    }
};

static BlkIdx make_blkidx(int64_t n, int64_t cols, int64_t br, int64_t bc, int64_t nbc)
{
    BlkIdx b{};
    const bool pow2 = br > 0 && bc > 0 && (br & (br - 1)) == 0 && (bc & (bc - 1)) == 0;
    if (!pow2 || n > 0xffffffffLL || cols < 1 || cols > 0xffffffffLL) return b;
    b.cols = (uint32_t)cols;
    if (b.cols > 1) {
        int l = 0;
        while (((uint64_t)1 << l) < b.cols) ++l;
        b.mul = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - b.cols)) / b.cols + 1);
        b.sh = (uint32_t)(l - 1);
    }
    while (((int64_t)1 << b.lbr) < br) ++b.lbr;
    while (((int64_t)1 << b.lbc) < bc) ++b.lbc;
    b.nbc = (uint32_t)nbc;
    return b;
}

// Vector path (cols % 8 == 0 and bc % 8 == 0: the 8 elements share a block).
// STE backward of one vector of 8: dx = (dy / s) where the recomputed E4M3
// code of x / s is finite and below the saturating magnitude, else 0.
template <int FT>
__device__ __forceinline__ void fp8_ste8(const Raw8<FT>& rx, const Raw8<FT>& rd, float s, float o[8])
{
    float xv[8], d[8];
    widen8<FT>(rx, xv);
    widen8<FT>(rd, d);
    const bool ok = scale_in_fast_range(s) & values_fast8(d) & codes_fast8(xv);
    float t[8], g[8];
    if (ok) {
        const float y = rcp_rn(s);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            t[i] = with_sign_of(div_q<FT>(xv[i], s, y), xv[i]);
            g[i] = div_q<FT>(d[i], s, y);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            t[i] = xv[i] / s;
            g[i] = d[i] / s;
        }
    }
    const uint32_t c0 = e4m3_pack4(t[0], t[1], t[2], t[3]);
    const uint32_t c1 = e4m3_pack4(t[4], t[5], t[6], t[7]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t c = ((i < 4 ? c0 : c1) >> ((i & 3) * 8)) & 0x7fu;
        o[i] = g[i] * (c < 0x7eu ? 1.0f : 0.0f);
    }
}

// Vectors of 8 per thread and grid step in the FP8 STE backward (one, with
// the loads in flight as below, measured 2.5% slower).
constexpr int FP8_STE_V = 2;

// SHIFT >= 0: 1 x bc blocks with cols % bc == 0 and bc = 2^SHIFT, so the
// block of element e is e >> SHIFT (no 64-bit divisions per vector).
template <int OP, int FT>
__global__ __launch_bounds__(256) void k_fp8_ew(const void* __restrict__ a, const void* __restrict__ b,
                                                int64_t nvec, int64_t cols, int64_t br, int64_t bc, int64_t nbc,
                                                int shift, BlkIdx bi, const float* __restrict__ scale,
                                                void* __restrict__ out)
{
    constexpr int FV = DEQ_V;
    if constexpr (OP == OP_DEQ) {
        for (int64_t base = (int64_t)blockIdx.x * 256 * FV; base < nvec;
             base += (int64_t)gridDim.x * 256 * FV) {
            uint2 w[FV];
            float s[FV];
            if (shift < 0) {
                // general block index: codes and scales at a clamped index with no
                // branch, so all 2 FV loads are in flight (under `if (vi < nvec)`
                // each load was waited for before the next: 128 x 128 blocks 10%
                // slower; the 1 x 2^k blocks below measured 1-3% faster as they are)
#pragma unroll
                for (int k = 0; k < FV; ++k) {
                    const int64_t vk = base + k * 256 + threadIdx.x;
                    const int64_t vi = vk < nvec ? vk : nvec - 1;
                    w[k] = EW_NT ? ld8<true>(static_cast<const uint8_t*>(a) + vi * 8)
                                 : *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(a) + vi * 8);
                    const int64_t e = vi * 8;
                    s[k] = scale[bi.cols ? bi.of(e) : fp8_block_of(e, cols, br, bc, nbc)];
                }
            } else {
#pragma unroll
                for (int k = 0; k < FV; ++k) {
                    const int64_t vi = base + k * 256 + threadIdx.x;
                    if (vi < nvec)
                        w[k] = EW_NT ? ld8<true>(static_cast<const uint8_t*>(a) + vi * 8)
                                     : *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(a) + vi * 8);
                }
#pragma unroll
                for (int k = 0; k < FV; ++k) {
                    const int64_t e = (base + k * 256 + threadIdx.x) * 8;
                    if (e < nvec * 8) s[k] = scale[e >> shift];
                }
            }
#pragma unroll
            for (int k = 0; k < FV; ++k) {
                const int64_t vi = base + k * 256 + threadIdx.x;
                if (vi >= nvec) break;
                float o[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    o[i] = e4m3_val(w[k].x, i) * s[k];
                    o[4 + i] = e4m3_val(w[k].y, i) * s[k];
                }
                store8<FT, WT>(out, vi * 8, o);
            }
        }
        return;
    }
    if constexpr (OP == OP_STE) {
        // FP8_STE_V vectors per grid step; for each, x, dy and the scale are
        // loaded (at a clamped index) ahead of a scheduling barrier, so all of
        // them are in flight before any is used (the compiler otherwise issued
        // the x load only after testing the scale); only the stores are guarded
        for (int64_t base = (int64_t)blockIdx.x * 256 * FP8_STE_V + threadIdx.x; base < nvec;
             base += (int64_t)gridDim.x * 256 * FP8_STE_V) {
            Raw8<FT> rx[FP8_STE_V], rd[FP8_STE_V];
            float sv[FP8_STE_V];
#pragma unroll
            for (int k = 0; k < FP8_STE_V; ++k) {
                const int64_t vk = base + k * 256;
                const int64_t e = (vk < nvec ? vk : nvec - 1) * 8;
                sv[k] = scale[shift >= 0 ? (e >> shift) : bi.cols ? bi.of(e) : fp8_block_of(e, cols, br, bc, nbc)];
                rx[k] = load8<FT, true>(a, e);
                rd[k] = load8<FT, true>(b, e);
            }
            __builtin_amdgcn_sched_barrier(0);
            float o[FP8_STE_V][8];
#pragma unroll
            for (int k = 0; k < FP8_STE_V; ++k) fp8_ste8<FT>(rx[k], rd[k], sv[k], o[k]);
#pragma unroll
            for (int k = 0; k < FP8_STE_V; ++k) {
                const int64_t vk = base + k * 256;
                if (vk < nvec) store8<FT, 1>(out, vk * 8, o[k]);
            }
        }
        return;
    }
    for (int64_t vi = (int64_t)blockIdx.x * 256 + threadIdx.x; vi < nvec; vi += (int64_t)gridDim.x * 256) {
        const int64_t e = vi * 8;
        const float s = scale[shift >= 0 ? (e >> shift) : bi.cols ? bi.of(e) : fp8_block_of(e, cols, br, bc, nbc)];
        // dequantize backward: dq = dy * scale
        float o[8], d[8];
        widen8<FT>(load8<FT, true>(a, e), d);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = d[i] * s;
        store8<FT, WT>(out, e, o);
    }
}

template <int OP, int FT>
__global__ __launch_bounds__(256) void k_fp8_ew_generic(const void* __restrict__ a, const void* __restrict__ b,
                                                        int64_t n, int64_t cols, int64_t br, int64_t bc,
                                                        int64_t nbc, const float* __restrict__ scale,
                                                        void* __restrict__ out)
{
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
        const float s = scale[fp8_block_of(e, cols, br, bc, nbc)];
        float o;
        if constexpr (OP == OP_DEQ) {
            o = e4m3_val(static_cast<const uint8_t*>(a)[e], 0) * s;
        } else if constexpr (OP == OP_DQB) {
            o = load1<FT>(a, e) * s;
        } else {
            const uint32_t c = e4m3_pack4(load1<FT>(a, e) / s, 0.0f, 0.0f, 0.0f) & 0x7fu;
            o = (load1<FT>(b, e) / s) * (c < 0x7eu ? 1.0f : 0.0f);
        }
        store1<FT>(out, e, o);
    }
}

// ------------------------------------------------------------ per tensor
// Pass 1: max |x| of each chunk into ws.  VEC: numel % 8 == 0.
template <int FT, bool VEC>
__global__ __launch_bounds__(256) void k_fp8_tensor_amax(const void* __restrict__ x, int64_t numel, int64_t chunk,
                                                         float* __restrict__ ws)
{
    __shared__ float sm[4];
    const int64_t b0 = (int64_t)blockIdx.x * chunk;
    const int64_t b1 = b0 + chunk < numel ? b0 + chunk : numel;
    float a = 0.0f;
    if constexpr (VEC) {
        for (int64_t e = b0 + (int64_t)threadIdx.x * 8; e < b1; e += 256 * 8 * 4) {
            Raw8<FT> r[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t ek = e + k * 256 * 8;
                r[k] = ek < b1 ? load8<FT>(x, ek) : Raw8<FT>{};
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float v[8];
                widen8<FT>(r[k], v);
#pragma unroll
                for (int i = 0; i < 8; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
            }
        }
    } else {
        for (int64_t e = b0 + threadIdx.x; e < b1; e += 256) a = __builtin_fmaxf(a, __builtin_fabsf(load1<FT>(x, e)));
    }
    a = team_max<64>(a);
    if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0)
        ws[blockIdx.x] = __builtin_fmaxf(__builtin_fmaxf(sm[0], sm[1]), __builtin_fmaxf(sm[2], sm[3]));
}

// Per-tensor FP8 encode: FP8_TENSOR_EV vectors per thread with both loads in
// flight; a static-scale grid gives each thread one such pair, a dynamic one
// two (every workgroup merges the chunk maxima first, so twice the workgroups
// measured 5% slower there; static 18.8 -> 18.0 us on bf16 [8192, 4096])
constexpr int FP8_TENSOR_EV = 2;
constexpr int FP8_TENSOR_VPT_STATIC = 2, FP8_TENSOR_VPT_MERGE = 4;

// Pass 2, by `mode`: 0 one block reduces the (small, <= 65536 elements)
// tensor itself, then encodes; 1 the scale is an input; 2 every block
// merges pass 1's nparts chunk maxima and block 0 publishes the scale.
template <int FT, bool VEC>
__global__ __launch_bounds__(256) void k_fp8_tensor_encode(const void* __restrict__ x, int64_t numel, int mode,
                                                           const float* __restrict__ parts, int nparts,
                                                           float* __restrict__ scale, uint8_t* __restrict__ q)
{
    FP p;
    if (mode == 2) {
        const Part4 pp = load_partials<false>(parts, nparts);
        float amax, unused;
        merge_partials<false>(pp, amax, unused);
        p = fp8_params<FT>(amax);
        if (blockIdx.x == 0 && threadIdx.x == 0) scale[0] = p.s;
    } else {
        __shared__ float sm[4];
        __shared__ FP sp;
        if (mode == 0) {
            float a = 0.0f;
            for (int64_t e = threadIdx.x; e < numel; e += 256)
                a = __builtin_fmaxf(a, __builtin_fabsf(load1<FT>(x, e)));
            a = team_max<64>(a);
            if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = a;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            FP g;
            if (mode == 1) {
                g.s = scale[0];
                g.fast = scale_in_fast_range(g.s);
                g.y = g.fast ? rcp_rn(g.s) : 0.0f;
            } else {
                g = fp8_params<FT>(__builtin_fmaxf(__builtin_fmaxf(sm[0], sm[1]), __builtin_fmaxf(sm[2], sm[3])));
                scale[0] = g.s;
            }
            sp = g;
        }
        __syncthreads();
        p = sp;
    }
    const int64_t stride = (int64_t)gridDim.x * 256;
    if constexpr (VEC) {
        // FP8_TENSOR_EV vectors per grid step, both loads before any store (one
        // vector per step kept one load in flight at a time)
        const int64_t nvec = numel / 8;
        for (int64_t base = (int64_t)blockIdx.x * 256 * FP8_TENSOR_EV + threadIdx.x; base < nvec;
             base += stride * FP8_TENSOR_EV) {
            Raw8<FT> r[FP8_TENSOR_EV];
#pragma unroll
            for (int k = 0; k < FP8_TENSOR_EV; ++k) {
                const int64_t vi = base + (int64_t)k * 256;
                r[k] = vi < nvec ? load8<FT, true>(x, vi * 8) : Raw8<FT>{};
            }
#pragma unroll
            for (int k = 0; k < FP8_TENSOR_EV; ++k) {
                const int64_t vi = base + (int64_t)k * 256;
                if (vi >= nvec) continue;
                float v[8];
                widen8<FT>(r[k], v);
                // a static scale does not bound |x|: keep x / s from overflowing on the fast path
                const bool fast = p.fast & codes_fast8(v);
                st8<true>(q + vi * 8, fast ? fp8_enc8<FT, true>(v, p) : fp8_enc8<FT, false>(v, p));
            }
        }
    } else {
        for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < numel; e += stride)
            q[e] = (uint8_t)e4m3_pack4(load1<FT>(x, e) / p.s, 0.0f, 0.0f, 0.0f);
    }
}

// ------------------------------------------------------------ MXFP8
template <int FT, int U>
__global__ __launch_bounds__(256) void k_mxfp8_quant(const void* __restrict__ x, int64_t nblocks,
                                                     uint8_t* __restrict__ q, uint8_t* __restrict__ bscale)
{
    constexpr int T = 4, P = 64 / T;
    const int lane = threadIdx.x & 63;
    const int j = lane % T;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t b0 = wave * (U * P) + lane / T;
    Raw8<FT> raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t b = b0 + (int64_t)u * P;
        if (b < nblocks) raw[u] = load8<FT, true>(x, b * 32 + j * 8);
        else raw[u] = Raw8<FT>{};
    }
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
        const uint32_t sb = e8m0_mx8_byte(a);
        const float inv = e8m0_inv(sb);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= inv;
        st8<true>(q + b * 32 + j * 8, make_uint2(e4m3_pack4(v[0], v[1], v[2], v[3]), e4m3_pack4(v[4], v[5], v[6], v[7])));
        if (j == 0) bscale[b] = (uint8_t)sb;
    }
}

// X = 2^(sb - 127) and its exact reciprocal: dequant multiplies by X, the
// STE's dy / X is dy * 2^(127 - sb) (the same correctly rounded quotient).
template <int OP, int FT>
__global__ __launch_bounds__(256) void k_mxfp8_ew(const void* __restrict__ a, const void* __restrict__ b,
                                                  const uint8_t* __restrict__ bscale, int64_t nvec,
                                                  void* __restrict__ out)
{
    if constexpr (OP == OP_DEQ) {
        for (int64_t base = (int64_t)blockIdx.x * 256 * DEQ_V; base < nvec;
             base += (int64_t)gridDim.x * 256 * DEQ_V) {
            uint2 w[DEQ_V];
            uint32_t sb[DEQ_V];
#pragma unroll
            for (int k = 0; k < DEQ_V; ++k) {
                const int64_t vi = base + k * 256 + threadIdx.x;
                if (vi < nvec)
                    w[k] = EW_NT ? ld8<true>(static_cast<const uint8_t*>(a) + vi * 8)
                                 : *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(a) + vi * 8);
            }
#pragma unroll
            for (int k = 0; k < DEQ_V; ++k) {
                const int64_t vi = base + k * 256 + threadIdx.x;
                if (vi < nvec) sb[k] = bscale[vi / 4];
            }
#pragma unroll
            for (int k = 0; k < DEQ_V; ++k) {
                const int64_t vi = base + k * 256 + threadIdx.x;
                if (vi >= nvec) break;
                const float X = e8m0_val(sb[k]);
                float o[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    o[i] = e4m3_val(w[k].x, i) * X;
                    o[4 + i] = e4m3_val(w[k].y, i) * X;
                }
                store8<FT, WT>(out, vi * 8, o);   // device-scope stores: 4% faster than non-temporal here
            }
        }
        return;
    }
    for (int64_t vi = (int64_t)blockIdx.x * 256 + threadIdx.x; vi < nvec; vi += (int64_t)gridDim.x * 256) {
        const int64_t e = vi * 8;
        const uint32_t sb = bscale[e / 32];
        float o[8];
        if constexpr (OP == OP_DQB) {
            const float X = e8m0_val(sb);
            float d[8];
            widen8<FT>(load8<FT, true>(a, e), d);
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = d[i] * X;
        } else {
            const float inv = e8m0_inv(sb);
            float t[8], d[8];
            widen8<FT>(load8<FT, true>(a, e), t);
            widen8<FT>(load8<FT, true>(b, e), d);
#pragma unroll
            for (int i = 0; i < 8; ++i) t[i] *= inv;
            const uint32_t c0 = e4m3_pack4(t[0], t[1], t[2], t[3]);
            const uint32_t c1 = e4m3_pack4(t[4], t[5], t[6], t[7]);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t c = ((i < 4 ? c0 : c1) >> ((i & 3) * 8)) & 0x7fu;
                o[i] = (d[i] * inv) * (c < 0x7eu ? 1.0f : 0.0f);
            }
        }
        store8<FT, OP == OP_DQB ? WT : 1>(out, e, o);
    }
}

// ============================================================ host side

#define TQ_FT_SWITCH(ft, ...)                                     \
    switch (ft) {                                                 \
    case TQ_F32: { constexpr int FTV = F32; __VA_ARGS__; } break; \
    case TQ_F16: { constexpr int FTV = F16; __VA_ARGS__; } break; \
    default: { constexpr int FTV = BF16; __VA_ARGS__; } break;    \
    }

template <int FT, int T, int W, int U>
static void launch_rows(const void* x, int64_t nblocks, uint8_t* q, float* scale, hipStream_t st, int64_t nbc = 1,
                        int64_t ldx = 0)
{
    constexpr int P = 64 / T;
    const int64_t waves = cdiv(nblocks, (int64_t)U * P);
    if (ldx)
        hipLaunchKernelGGL((k_fp8_rows<FT, T, W, U, true>), dim3((unsigned)cdiv(waves, 4)), dim3(256), 0, st, x,
                           nblocks, nbc, ldx, q, scale);
    else
        hipLaunchKernelGGL((k_fp8_rows<FT, T, W, U>), dim3((unsigned)cdiv(waves, 4)), dim3(256), 0, st, x, nblocks,
                           nbc, ldx, q, scale);
}

// 1 x bc blocks of a row-strided input (ldx elements between row starts).
template <int FT>
static bool quant_rows_strided(const void* x, int64_t rows, int64_t cols, int64_t ldx, int64_t bc, uint8_t* q,
                               float* scale, hipStream_t st)
{
    const int64_t nbc = cols / bc, nb = rows * nbc;
    switch (bc) {
    case 16: launch_rows<FT, 2, 1, 8>(x, nb, q, scale, st, nbc, ldx); return true;
    case 32: launch_rows<FT, 4, 1, 8>(x, nb, q, scale, st, nbc, ldx); return true;
    case 64: launch_rows<FT, 8, 1, 8>(x, nb, q, scale, st, nbc, ldx); return true;
    case 128: launch_rows<FT, 8, 2, 1>(x, nb, q, scale, st, nbc, ldx); return true;
    case 256: launch_rows<FT, 16, 2, 4>(x, nb, q, scale, st, nbc, ldx); return true;
    case 512: launch_rows<FT, 64, 1, 8>(x, nb, q, scale, st, nbc, ldx); return true;
    default: return false;
    }
}

template <int FT>
static bool quant_fast(const void* x, int64_t rows, int64_t cols, int64_t br, int64_t bc, uint8_t* q, float* scale,
                       hipStream_t st)
{
    const int64_t nb = (rows / br) * (cols / bc);
    if (br == 1) {
        switch (bc) {
        case 16: launch_rows<FT, 2, 1, 8>(x, nb, q, scale, st); return true;
        case 32: launch_rows<FT, 4, 1, 8>(x, nb, q, scale, st); return true;
        case 64: launch_rows<FT, 8, 1, 8>(x, nb, q, scale, st); return true;
        case 128: launch_rows<FT, 8, 2, 1>(x, nb, q, scale, st); return true;
        case 256: launch_rows<FT, 16, 2, 4>(x, nb, q, scale, st); return true;
        case 512: launch_rows<FT, 64, 1, 8>(x, nb, q, scale, st); return true;
        default: return false;
        }
    }
    const dim3 grid((unsigned)(cols / bc), (unsigned)(rows / br));
    if (rows / br > 65535) return false;
    if (bc == 128 && br == 128) {
        // 512 threads of 4 rows x 8 columns each (52 VGPRs; 256 threads of 8 rows
        // needed 84-89 and ran 1.4% slower)
        hipLaunchKernelGGL((k_fp8_tile<FT, 16, 4, 512>), grid, dim3(512), 0, st, x, cols, cols / bc, q, scale);
        return true;
    }
    if (bc == 128 && br == 64) {
        hipLaunchKernelGGL((k_fp8_tile<FT, 16, 4>), grid, dim3(256), 0, st, x, cols, cols / bc, q, scale);
        return true;
    }
    if (bc == 64 && br == 64) {
        hipLaunchKernelGGL((k_fp8_tile<FT, 8, 2>), grid, dim3(256), 0, st, x, cols, cols / bc, q, scale);
        return true;
    }
    return false;
}

// Any positive block shape; blocks that the shape does not fill are partial.
static tq_status check_blocks(int64_t rows, int64_t cols, int32_t br, int32_t bc)
{
    if (rows < 0 || cols < 0 || br <= 0 || bc <= 0) return TQ_ERR_INVALID;
    return TQ_OK;
}

template <int OP>
static tq_status fp8_elementwise(const void* a, const void* b, int ft, int64_t rows, int64_t cols, int64_t br,
                                 int64_t bc, const float* scale, void* out, hipStream_t st)
{
    const int64_t n = rows * cols;
    if (n == 0) return TQ_OK;
    const int64_t nbc = cdiv(cols, bc);
    if (cols % 8 == 0 && bc % 8 == 0) {
        int shift = -1;
        if (br == 1 && cols % bc == 0 && (bc & (bc - 1)) == 0)
            for (shift = 0; ((int64_t)1 << shift) < bc; ++shift) {}
        const BlkIdx bi = shift >= 0 ? BlkIdx{} : make_blkidx(n, cols, br, bc, nbc);
        TQ_FT_SWITCH(ft, hipLaunchKernelGGL((k_fp8_ew<OP, FTV>), dim3(grid_for(n / 8, 256 * (OP == OP_DEQ ? DEQ_V : OP == OP_STE ? FP8_STE_V : 1))),
                                            dim3(256), 0, st,
                                            a, b, n / 8, cols, br, bc, nbc, shift, bi, scale, out));
    } else {
        TQ_FT_SWITCH(ft, hipLaunchKernelGGL((k_fp8_ew_generic<OP, FTV>), dim3(grid_for(n, 256)), dim3(256), 0, st,
                                            a, b, n, cols, br, bc, nbc, scale, out));
    }
    return launch_status();
}

// ---------------------------------------------------------------- MXFP8
static tq_status check_mx8(int64_t rows, int64_t k)
{
    return (rows < 0 || k < 0 || k % 32) ? TQ_ERR_INVALID : TQ_OK;
}

template <int OP>
static tq_status mx8_elementwise(const void* a, const void* b, int ft, const uint8_t* bscale, int64_t rows, int64_t k,
                                 void* out, hipStream_t st)
{
    const int64_t nvec = rows * k / 8;
    const dim3 grid(grid_for(nvec, 256 * (OP == OP_DEQ ? DEQ_V : 1))), block(256);
    TQ_FT_SWITCH(ft, hipLaunchKernelGGL((k_mxfp8_ew<OP, FTV>), grid, block, 0, st, a, b, bscale, nvec, out));
    return launch_status();
}

}  // namespace tq

using namespace tq;

extern "C" {

tq_status tq_quant_fp8_block(const void* x, int x_dtype, int64_t rows, int64_t cols, int32_t block_rows,
                             int32_t block_cols, uint8_t* q, float* scale, void* stream)
{
    if (!valid_ftype(x_dtype)) return TQ_ERR_INVALID;
    tq_status s = check_blocks(rows, cols, block_rows, block_cols);
    if (s || rows == 0 || cols == 0) return s;
    if (!x || !q || !scale) return TQ_ERR_INVALID;
    if (!aligned16(x) || !aligned16(q)) return TQ_ERR_ALIGN;
    hipStream_t st = as_stream(stream);
    bool done = false;
    if (cols % 8 == 0 && rows % block_rows == 0 && cols % block_cols == 0) {
        TQ_FT_SWITCH(x_dtype, done = quant_fast<FTV>(x, rows, cols, block_rows, block_cols, q, scale, st));
    }
    if (!done) {
        const int64_t nbc = cdiv(cols, block_cols);
        const int64_t nb = cdiv(rows, block_rows) * nbc;
        if (nb > 0x7fffffff) return TQ_ERR_UNSUPPORTED;
        TQ_FT_SWITCH(x_dtype, hipLaunchKernelGGL((k_fp8_generic<FTV>), dim3((unsigned)nb), dim3(256), 0, st, x, rows,
                                                 cols, (int64_t)block_rows, (int64_t)block_cols, nbc, q, scale));
    }
    return launch_status();
}

tq_status tq_dequant_fp8_block(const uint8_t* q, int64_t rows, int64_t cols, int32_t block_rows, int32_t block_cols,
                               const float* scale, void* y, int y_dtype, void* stream)
{
    if (!valid_ftype(y_dtype)) return TQ_ERR_INVALID;
    tq_status s = check_blocks(rows, cols, block_rows, block_cols);
    if (s || rows == 0 || cols == 0) return s;
    if (!q || !scale || !y) return TQ_ERR_INVALID;
    if (!aligned16(q) || !aligned16(y)) return TQ_ERR_ALIGN;
    return fp8_elementwise<OP_DEQ>(q, nullptr, y_dtype, rows, cols, block_rows, block_cols, scale, y, as_stream(stream));
}

tq_status tq_quant_fp8_block_backward(const void* x, int x_dtype, int64_t rows, int64_t cols, int32_t block_rows,
                                      int32_t block_cols, const float* scale, const void* dy, void* dx, void* stream)
{
    if (!valid_ftype(x_dtype)) return TQ_ERR_INVALID;
    tq_status s = check_blocks(rows, cols, block_rows, block_cols);
    if (s || rows == 0 || cols == 0) return s;
    if (!x || !dy || !dx || !scale) return TQ_ERR_INVALID;
    if (!aligned16(x) || !aligned16(dy) || !aligned16(dx)) return TQ_ERR_ALIGN;
    return fp8_elementwise<OP_STE>(x, dy, x_dtype, rows, cols, block_rows, block_cols, scale, dx, as_stream(stream));
}

tq_status tq_dequant_fp8_block_backward(const void* dy, int dy_dtype, int64_t rows, int64_t cols, int32_t block_rows,
                                        int32_t block_cols, const float* scale, void* dq, void* stream)
{
    if (!valid_ftype(dy_dtype)) return TQ_ERR_INVALID;
    tq_status s = check_blocks(rows, cols, block_rows, block_cols);
    if (s || rows == 0 || cols == 0) return s;
    if (!dy || !dq || !scale) return TQ_ERR_INVALID;
    if (!aligned16(dy) || !aligned16(dq)) return TQ_ERR_ALIGN;
    return fp8_elementwise<OP_DQB>(dy, nullptr, dy_dtype, rows, cols, block_rows, block_cols, scale, dq,
                                   as_stream(stream));
}

tq_status tq_quant_mxfp8(const void* x, int x_dtype, int64_t rows, int64_t k, uint8_t* q, uint8_t* block_scale,
                         void* stream)
{
    if (!valid_ftype(x_dtype)) return TQ_ERR_INVALID;
    tq_status s = check_mx8(rows, k);
    if (s || rows * k == 0) return s;
    if (!x || !q || !block_scale) return TQ_ERR_INVALID;
    if (!aligned16(x) || !aligned16(q)) return TQ_ERR_ALIGN;
    constexpr int U = 2;   // 32-element blocks per lane in flight (1 and 4 measured slower)
    const int64_t nb = rows * k / 32;
    const int64_t grid = cdiv(cdiv(nb, U * 16), 4);
    if (grid > 0x7fffffff) return TQ_ERR_UNSUPPORTED;
    TQ_FT_SWITCH(x_dtype, hipLaunchKernelGGL((k_mxfp8_quant<FTV, U>), dim3((unsigned)grid), dim3(256), 0,
                                             as_stream(stream), x, nb, q, block_scale));
    return launch_status();
}

tq_status tq_dequant_mxfp8(const uint8_t* q, const uint8_t* block_scale, int64_t rows, int64_t k, void* y,
                           int y_dtype, void* stream)
{
    if (!valid_ftype(y_dtype)) return TQ_ERR_INVALID;
    tq_status s = check_mx8(rows, k);
    if (s || rows * k == 0) return s;
    if (!q || !block_scale || !y) return TQ_ERR_INVALID;
    if (!aligned16(q) || !aligned16(y)) return TQ_ERR_ALIGN;
    return mx8_elementwise<OP_DEQ>(q, nullptr, y_dtype, block_scale, rows, k, y, as_stream(stream));
}

tq_status tq_quant_mxfp8_backward(const void* x, int x_dtype, const uint8_t* block_scale, int64_t rows, int64_t k,
                                  const void* dy, void* dx, void* stream)
{
    if (!valid_ftype(x_dtype)) return TQ_ERR_INVALID;
    tq_status s = check_mx8(rows, k);
    if (s || rows * k == 0) return s;
    if (!x || !dy || !dx || !block_scale) return TQ_ERR_INVALID;
    if (!aligned16(x) || !aligned16(dy) || !aligned16(dx)) return TQ_ERR_ALIGN;
    return mx8_elementwise<OP_STE>(x, dy, x_dtype, block_scale, rows, k, dx, as_stream(stream));
}

tq_status tq_dequant_mxfp8_backward(const void* dy, int dy_dtype, const uint8_t* block_scale, int64_t rows,
                                    int64_t k, void* dq, void* stream)
{
    if (!valid_ftype(dy_dtype)) return TQ_ERR_INVALID;
    tq_status s = check_mx8(rows, k);
    if (s || rows * k == 0) return s;
    if (!dy || !dq || !block_scale) return TQ_ERR_INVALID;
    if (!aligned16(dy) || !aligned16(dq)) return TQ_ERR_ALIGN;
    return mx8_elementwise<OP_DQB>(dy, nullptr, dy_dtype, block_scale, rows, k, dq, as_stream(stream));
}

tq_status tq_quant_fp8_per_tensor(const void* x, int x_dtype, int64_t numel, int static_scale, uint8_t* q,
                                  float* scale, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!valid_ftype(x_dtype) || numel < 0) return TQ_ERR_INVALID;
    if (numel == 0) return TQ_OK;
    if (!x || !q || !scale) return TQ_ERR_INVALID;
    if (!aligned16(x) || !aligned16(q)) return TQ_ERR_ALIGN;
    hipStream_t st = as_stream(stream);
    const bool vec = numel % 8 == 0;
    const bool small = numel <= 65536;
    const int mode = static_scale ? 1 : small ? 0 : 2;
    int nparts = 0;
    float* ws = static_cast<float*>(workspace);
    if (mode == 2) {
        if (!workspace || workspace_bytes < tq_workspace_bytes(2, numel)) return TQ_ERR_INVALID;
        if (!aligned16(workspace)) return TQ_ERR_ALIGN;
        const int64_t chunk = tensor_chunk(numel, &nparts);
        TQ_FT_SWITCH(x_dtype, {
            if (vec) hipLaunchKernelGGL((k_fp8_tensor_amax<FTV, true>), dim3(nparts), dim3(256), 0, st, x, numel, chunk,
                                        ws);
            else hipLaunchKernelGGL((k_fp8_tensor_amax<FTV, false>), dim3(nparts), dim3(256), 0, st, x, numel, chunk,
                                    ws);
        });
        if (launch_status()) return TQ_ERR_HIP;
    }
    const int vpt = mode == 2 ? FP8_TENSOR_VPT_MERGE : FP8_TENSOR_VPT_STATIC;
    const dim3 grid(mode == 0 ? 1u : vec ? grid_for(numel / 8, 256 * vpt) : grid_for(numel, 256 * 4));
    TQ_FT_SWITCH(x_dtype, {
        if (vec) hipLaunchKernelGGL((k_fp8_tensor_encode<FTV, true>), grid, dim3(256), 0, st, x, numel, mode, ws,
                                    nparts, scale, q);
        else hipLaunchKernelGGL((k_fp8_tensor_encode<FTV, false>), grid, dim3(256), 0, st, x, numel, mode, ws, nparts,
                                scale, q);
    });
    return launch_status();
}

tq_status tq_dequant_fp8_per_tensor(const uint8_t* q, int64_t numel, const float* scale, void* y, int y_dtype,
                                    void* stream)
{
    if (!valid_ftype(y_dtype) || numel < 0) return TQ_ERR_INVALID;
    if (numel == 0) return TQ_OK;
    if (!q || !scale || !y) return TQ_ERR_INVALID;
    if (!aligned16(q) || !aligned16(y)) return TQ_ERR_ALIGN;
    return fp8_elementwise<OP_DEQ>(q, nullptr, y_dtype, 1, numel, 1, numel, scale, y, as_stream(stream));
}

tq_status tq_quant_fp8_rows_strided(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t x_row_stride,
                                    int32_t block_cols, uint8_t* q, float* scale, void* stream)
{
    if (!valid_ftype(x_dtype) || rows < 0 || cols < 0 || block_cols <= 0 || x_row_stride < cols)
        return TQ_ERR_INVALID;
    if (cols % block_cols) return TQ_ERR_INVALID;
    if (rows == 0 || cols == 0) return TQ_OK;
    if (!x || !q || !scale) return TQ_ERR_INVALID;
    const int es = ftype_size(x_dtype);
    if (!aligned16(x) || !aligned16(q) || (x_row_stride * es) % 16 || (cols * es) % 16) return TQ_ERR_ALIGN;
    bool done = false;
    TQ_FT_SWITCH(x_dtype, done = quant_rows_strided<FTV>(x, rows, cols, x_row_stride, block_cols, q, scale,
                                                         as_stream(stream)));
    if (!done) return TQ_ERR_UNSUPPORTED;
    return launch_status();
}

}  // extern "C"
