// tq_int.hip -- integer codes (s8 / u8 / s4 / u4) at per-tensor, per-channel,
// per-token and per-group granularity: quantize, dequantize, STE backward
// and dequantize backward, with their C-ABI entry points.
//
// Definitions: docs.rs baracuda_kernels::quantize (module overview: per-token
// W8A8 rows and GPTQ-style per-group g=128 weights, the STE rule
// dx = (dy / scale) * 1[qmin < q < qmax] recomputed from the saved input;
// module list: dequantize backward dq = dy * scale; default_q_range) and
// teenygrad granularity.rs (enum Granularity).  The readings taken where the
// pages are silent (symmetric range [-qmax, qmax], the affine zero-point,
// scale 0 -> 1) are stated in include/tq.h.
//
// Kernel map (each group is streamed once, 16-byte loads):
//   k_quant_team   contiguous groups of L = 8*T*W elements: a team of T
//                  lanes per group (DPP / bpermute reduction), W vectors of
//                  8 elements per lane held in registers; per-token rows of
//                  512..4096 elements use a whole wave, 128-element GPTQ
//                  groups use 16-lane teams.
//   k_quant_long   contiguous groups of any length multiple of 8: one wave
//                  per group, two passes over the group.
//   k_quant_cols   groups that run down columns ([B, R, C] view: per-channel
//                  on the last axis, per-group along a non-last axis).
//   k_*_generic    any layout (index arithmetic per element), the fallback.
//   k_tensor_*     per-tensor: block partial max, one workgroup publishing the
//                  scale, then encode (small tensors: one single-block launch).
//   k_dequant_vec / k_ste_vec / k_dqb_vec   elementwise streaming.
#include "tq_device.h"
#include "tq_host.h"

namespace tq {

// ------------------------------------------------------------ group params
struct GP {
    float s;     // scale
    float y;     // RN(1 / s) when fast
    float zpf;   // zero-point as a float (0 when symmetric)
    bool fast;   // s inside the range where the FMA division is exact
};

// Scale and zero-point of one group.  yc = RN(1/qmax) (symmetric) or
// RN(1/(qmax - qmin)) (asymmetric), computed once on the host.  amax and mn
// are element values of type FT (or 0); the asymmetric range mx - mn is a
// general binary32 value.
// f16 groups never leave the fast ranges: amax, -mn and mx - mn are 0 or in
// [2^-24, 131008], so with 1 <= qmax, qmax - qmin <= 255 the scale lies in
// [2^-32, 131008] (or is 1) and every guard below is statically true.
template <int FT, bool SYM>
__device__ __forceinline__ GP make_gp(float amax, float mn, float mx, float qmin, float qmax, float yc)
{
    constexpr bool ALWAYS_FAST = FT == F16;
    GP p;
    float s;
    if constexpr (SYM) s = ALWAYS_FAST ? div_q<FT>(amax, qmax, yc) : div_by<FT>(amax, qmax, yc);
    else s = ALWAYS_FAST ? div_q<F32>(mx - mn, qmax - qmin, yc) : div_by<F32>(mx - mn, qmax - qmin, yc);
    s = (s == 0.0f) ? 1.0f : s;
    p.s = s;
    p.fast = ALWAYS_FAST || scale_in_fast_range(s);
    p.y = p.fast ? rcp_rn(s) : 0.0f;
    if constexpr (SYM) {
        p.zpf = 0.0f;
    } else {
        const float t = (ALWAYS_FAST || (p.fast && (value_in_fast_range(mn) || mn == 0.0f))) ? div_q<FT>(mn, s, p.y)
                                                                                              : mn / s;
        p.zpf = __builtin_amdgcn_fmed3f(qmin - __builtin_rintf(t), qmin, qmax);
    }
    return p;
}

// Encode 8 values of one group into code floats (MAGIC + code).  A
// symmetric dynamic scale s = RN(amax / qmax) that is a normal number keeps
// |x / s| below qmax + 0.5 for every element (its relative error is at most
// 2^-24), so fast symmetric groups skip the clamp.  A subnormal scale (amax
// below qmax * 2^-126) carries up to half an ulp of 2^-149 of absolute
// error, so |x / s| can exceed qmax by far (amax = 190 * 2^-149 gives
// s = 2^-149 and x / s = 190 with qmax = 127): such scales lie outside the
// fast range and the slow branch always clamps.
template <int FT, bool FAST, bool CLAMP>
__device__ __forceinline__ void enc8(const float v[8], const GP& p, float lo, float hi, float c[8])
{
    constexpr bool CL = CLAMP || !FAST;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float t = FAST ? div_q<FT>(v[i], p.s, p.y) : v[i] / p.s;
        c[i] = CL ? int_code_f(t, p.zpf, lo, hi) : (t + MAGIC) + p.zpf;
    }
}

template <int BITS, bool NT = false>
__device__ __forceinline__ void store_codes8(uint8_t* q, int64_t e, const float c[8])
{
    if constexpr (BITS == 8)
        st8<NT>(q + e, make_uint2(pack_bytes4(c[0], c[1], c[2], c[3]), pack_bytes4(c[4], c[5], c[6], c[7])));
    else
        st4<NT>(q + (e >> 1), pack_nibbles8(c, true));
}

// Fake quantization writes the round trip instead of the code:
// y = (q - zp) * s, with q - zp = (c - MAGIC) - zp exact (small integers), one
// binary32 rounding for the product, then one for the narrowing to FT.
__device__ __forceinline__ float fake_value(float c, const GP& p)
{
    return ((c - MAGIC) - p.zpf) * p.s;
}

template <int FT>
__device__ __forceinline__ void store_fake8(void* y, int64_t e, const float c[8], const GP& p)
{
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = fake_value(c[i], p);
    store8<FT, true>(y, e, o);
}

// ------------------------------------------------------------ team kernel
// f16 inputs skip the widening pass: the group max / min runs on packed f16
// pairs (v_pk_max_f16 / v_pk_min_f16, exact), and the division widens each
// element inside its two FMAs (v_fma_mix_f32): q0 = fma(x, y, -0) is x * y
// with the same rounding and the same signed zeros, r = fma(q0, s, -x).
// Packed f16 max / min from asm: the builtins would first quiet each loaded
// pair (one more v_pk_max_f16 per dword); NaN inputs are out of contract.
__device__ __forceinline__ uint32_t pk_max_f16(uint32_t a, uint32_t b)
{
    uint32_t r;
    asm("v_pk_max_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ uint32_t pk_min_f16(uint32_t a, uint32_t b)
{
    uint32_t r;
    asm("v_pk_min_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

template <int W, bool SYM>
__device__ __forceinline__ void f16_stats(const Raw8<F16>* raw, float& amax, float& mn, float& mx)
{
    typedef uint16_t u2v __attribute__((ext_vector_type(2)));
    u2v amx = {0, 0};                    // |x| patterns: unsigned order is magnitude order
    uint32_t hmx = 0, hmn = 0;           // two packed f16 zeros
    if constexpr (SYM) {
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const uint32_t d[4] = {raw[w].w[0].x, raw[w].w[0].y, raw[w].w[0].z, raw[w].w[0].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) amx = __builtin_elementwise_max(amx, __builtin_bit_cast(u2v, d[i] & 0x7fff7fffu));
        }
    } else {
        // pairwise tree over the 4W words (independent neighbours, no stalls
        // between dependent packed ops), then the zeros
        uint32_t lo[4 * W], hi[4 * W];
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const uint32_t d[4] = {raw[w].w[0].x, raw[w].w[0].y, raw[w].w[0].z, raw[w].w[0].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) lo[4 * w + i] = hi[4 * w + i] = d[i];
        }
#pragma unroll
        for (int n = 4 * W; n > 1; n /= 2)
#pragma unroll
            for (int i = 0; i < n / 2; ++i) {
                lo[i] = pk_min_f16(lo[2 * i], lo[2 * i + 1]);
                hi[i] = pk_max_f16(hi[2 * i], hi[2 * i + 1]);
            }
        hmn = pk_min_f16(hmn, lo[0]);
        hmx = pk_max_f16(hmx, hi[0]);
    }
    if constexpr (SYM) {
        amax = mx = f16_lo(amx.x > amx.y ? amx.x : amx.y);
        mn = 0.0f;
    } else {
        amax = mx = __builtin_fmaxf(f16_lo(hmx), f16_hi(hmx));
        mn = __builtin_fminf(f16_lo(hmn), f16_hi(hmn));
    }
}

// The binary32 quotient of an f16 dividend (widened inside the FMAs; nz is
// an opaque -0 so the first FMA is not folded back into a multiply).
__device__ __forceinline__ float div_q_mix(float x, float s, float y, float nz)
{
    const float q0 = __builtin_fmaf(x, y, nz);
    const float r = __builtin_fmaf(q0, s, -x);
    return __builtin_fmaf(-r, y, q0);
}

// Per-nibble sum modulo 16 of eight packed nibbles (no carries between them).
__device__ __forceinline__ uint32_t nibble_add(uint32_t a, uint32_t b)
{
    return ((a & 0x77777777u) + (b & 0x77777777u)) ^ ((a ^ b) & 0x88888888u);
}

// Codes of 8 elements of one group, stored.  Asymmetric 4-bit codes clamp
// before the zero-point, med3(t + M, M + qmin - zp, M + qmax - zp), and add
// the zero-point to the eight packed nibbles at once: the result of each is
// in [qmin, qmax] within [0, 15], so the sum modulo 16 is the code itself.
template <int FT, bool FAST, bool SYM, int BITS, bool NT>
__device__ __forceinline__ void encode_store8(const float* v, const Raw8<FT>& raw, const GP& p, float lo, float hi,
                                              float lo_z, float hi_z, uint32_t zn, float nz, uint8_t* q, int64_t e)
{
    float c[8];
    if constexpr (FT == F16) {
        const uint32_t d[4] = {raw.w[0].x, raw.w[0].y, raw.w[0].z, raw.w[0].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = (i & 1) ? f16_hi(d[i >> 1]) : f16_lo(d[i >> 1]);
            const float t = FAST ? div_q_mix(x, p.s, p.y, nz) : x / p.s;
            if constexpr (SYM) c[i] = FAST ? t + MAGIC : __builtin_amdgcn_fmed3f(t + MAGIC, lo, hi);
            else if constexpr (BITS == 4) c[i] = __builtin_amdgcn_fmed3f(t + MAGIC, lo_z, hi_z);
            else c[i] = int_code_f(t, p.zpf, lo, hi);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float t = FAST ? div_q<FT>(v[i], p.s, p.y) : v[i] / p.s;
            if constexpr (SYM) c[i] = FAST ? t + MAGIC : __builtin_amdgcn_fmed3f(t + MAGIC, lo, hi);
            else if constexpr (BITS == 4) c[i] = __builtin_amdgcn_fmed3f(t + MAGIC, lo_z, hi_z);
            else c[i] = int_code_f(t, p.zpf, lo, hi);
        }
    }
    if constexpr (BITS == 4 && !SYM) st4<NT>(q + (e >> 1), nibble_add(pack_nibbles8(c, true), zn));
    else store_codes8<BITS, NT>(q, e, c);
}

// Groups of L = 8*T*W contiguous elements.  Lane j of a team of T lanes
// holds vectors w*T + j (w < W) of its group, so each load instruction of a
// team reads 16*T contiguous bytes; a wave runs U rounds of 64/T groups.
template <int FT, int BITS, bool SYM, int T, int W, int U>
__global__ __launch_bounds__(256) void k_quant_team(const void* __restrict__ x, int64_t G, int64_t ldx,
                                                    float qmin, float qmax, float yc, uint8_t* __restrict__ q,
                                                    float* __restrict__ scale, uint8_t* __restrict__ zp)
{
    constexpr int P = 64 / T;
    constexpr int64_t L = 8 * T * W;
    const int lane = threadIdx.x & 63;
    const int team = lane / T;
    const int j = lane % T;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t g0 = wave * (U * P) + team;

    Raw8<FT> raw[U][W];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t g = g0 + (int64_t)u * P;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            if (g < G) raw[u][w] = load8<FT, (T >= 8)>(x, g * ldx + (int64_t)(w * T + j) * 8);
            else raw[u][w] = Raw8<FT>{};
        }
    }
    float v[U][W][8];
    if constexpr (FT != F16) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int w = 0; w < W; ++w) widen8<FT>(raw[u][w], v[u][w]);
    }

    GP p[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (FT == F16) {
            float a, mn, mx;
            f16_stats<W, SYM>(raw[u], a, mn, mx);
            if constexpr (SYM) p[u] = make_gp<FT, true>(team_max<T>(a), 0.0f, 0.0f, qmin, qmax, yc);
            else p[u] = make_gp<FT, false>(0.0f, team_min<T>(mn), team_max<T>(mx), qmin, qmax, yc);
        } else if constexpr (SYM) {
            float a = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w)
#pragma unroll
                for (int i = 0; i < 8; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[u][w][i]));
            p[u] = make_gp<FT, true>(team_max<T>(a), 0.0f, 0.0f, qmin, qmax, yc);
        } else {
            float mn = 0.0f, mx = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    mn = __builtin_fminf(mn, v[u][w][i]);
                    mx = __builtin_fmaxf(mx, v[u][w][i]);
                }
            p[u] = make_gp<FT, false>(0.0f, team_min<T>(mn), team_max<T>(mx), qmin, qmax, yc);
        }
    }

    const float lo = MAGIC + qmin, hi = MAGIC + qmax;
    const float nz = opaque(-0.0f);
    // Non-temporal code stores where a wave's store instructions cover whole
    // lines: T = 64 (each instruction), T = 8 (the W = 2 instructions of a
    // team together; measured 1% faster on g = 128 4-bit codes).
    constexpr bool CNT = T == 64 || T == 8;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t g = g0 + (int64_t)u * P;
        if (g >= G) continue;
        const float lo_z = lo - p[u].zpf, hi_z = hi - p[u].zpf;          // exact: small integers
        const uint32_t zn = ((uint32_t)(int)p[u].zpf & 0xfu) * 0x11111111u;   // the zero-point in every nibble
        if (p[u].fast) {
#pragma unroll
            for (int w = 0; w < W; ++w)
                encode_store8<FT, true, SYM, BITS, CNT>(v[u][w], raw[u][w], p[u], lo, hi, lo_z, hi_z, zn, nz, q,
                                                             g * L + (int64_t)(w * T + j) * 8);
        } else {
#pragma unroll
            for (int w = 0; w < W; ++w)
                encode_store8<FT, false, SYM, BITS, CNT>(v[u][w], raw[u][w], p[u], lo, hi, lo_z, hi_z, zn, nz, q,
                                                              g * L + (int64_t)(w * T + j) * 8);
        }
        if (j == 0) {
            scale[g] = p[u].s;
            if constexpr (!SYM) zp[g] = (uint8_t)(int)p[u].zpf;
        }
    }
}

// ------------------------------------------------------------ row groups
// One workgroup of NW waves per group of L = 512 * NW * W contiguous
// elements: thread t holds vectors w * 64 * NW + t (w < W), so every load
// instruction of a wave reads 1 KB contiguously and each thread keeps only W
// loads in flight; the group max / min goes through DPP within a wave and
// LDS across the NW waves.
template <int FT, int BITS, bool SYM, int NW, int W>
__global__ __launch_bounds__(64 * NW) void k_quant_rows(const void* __restrict__ x, int64_t ldx, float qmin,
                                                        float qmax, float yc, uint8_t* __restrict__ q,
                                                        float* __restrict__ scale, uint8_t* __restrict__ zp)
{
    constexpr int NT = 64 * NW;
    constexpr int64_t L = 8 * NT * W;
    __shared__ float smx[NW], smn[NW];
    const int64_t g = blockIdx.x;
    const int t = threadIdx.x;
    Raw8<FT> raw[W];
#pragma unroll
    for (int w = 0; w < W; ++w) raw[w] = load8<FT, true>(x, g * ldx + (int64_t)(w * NT + t) * 8);
    float v[W][8];
    float mn = 0.0f, mx = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        widen8<FT>(raw[w], v[w]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (SYM) {
                mx = __builtin_fmaxf(mx, __builtin_fabsf(v[w][i]));
            } else {
                mn = __builtin_fminf(mn, v[w][i]);
                mx = __builtin_fmaxf(mx, v[w][i]);
            }
        }
    }
    mx = team_max<64>(mx);
    if constexpr (!SYM) mn = team_min<64>(mn);
    if ((t & 63) == 0) {
        smx[t >> 6] = mx;
        smn[t >> 6] = mn;
    }
    __syncthreads();
    mx = smx[0];
    mn = smn[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) {
        mx = __builtin_fmaxf(mx, smx[k]);
        mn = __builtin_fminf(mn, smn[k]);
    }
    const GP p = SYM ? make_gp<FT, true>(mx, 0.0f, 0.0f, qmin, qmax, yc) : make_gp<FT, false>(0.0f, mn, mx, qmin, qmax, yc);
    const float lo = MAGIC + qmin, hi = MAGIC + qmax;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        float c[8];
        if (p.fast) enc8<FT, true, !SYM>(v[w], p, lo, hi, c);
        else enc8<FT, false, !SYM>(v[w], p, lo, hi, c);
        store_codes8<BITS, true>(q, g * L + (int64_t)(w * NT + t) * 8, c);
    }
    if (t == 0) {
        scale[g] = p.s;
        if constexpr (!SYM) zp[g] = (uint8_t)(int)p.zpf;
    }
}

// ------------------------------------------------------------ long groups
// One wave per group of L elements (L % 8 == 0); the group is read twice
// (reduce, then encode) in 4-vector strides per lane.
template <int FT, int BITS, bool SYM>
__global__ __launch_bounds__(256) void k_quant_long(const void* __restrict__ x, int64_t G, int64_t L,
                                                    int64_t ldx, float qmin, float qmax, float yc,
                                                    uint8_t* __restrict__ q, float* __restrict__ scale,
                                                    uint8_t* __restrict__ zp)
{
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (g >= G) return;
    const int64_t nvec = L / 8;
    const int64_t base = g * ldx;      // input row; codes go to g * L
    float a = 0.0f, mn = 0.0f, mx = 0.0f;
    for (int64_t v0 = lane; v0 < nvec; v0 += 256) {
        Raw8<FT> raw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (v0 + k * 64 < nvec) raw[k] = load8<FT>(x, base + (v0 + k * 64) * 8);
            else raw[k] = Raw8<FT>{};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float v[8];
            widen8<FT>(raw[k], v);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
                mn = __builtin_fminf(mn, v[i]);
                mx = __builtin_fmaxf(mx, v[i]);
            }
        }
    }
    GP p = SYM ? make_gp<FT, true>(team_max<64>(a), 0.0f, 0.0f, qmin, qmax, yc)
               : make_gp<FT, false>(0.0f, team_min<64>(mn), team_max<64>(mx), qmin, qmax, yc);
    const float lo = MAGIC + qmin, hi = MAGIC + qmax;
    for (int64_t v0 = lane; v0 < nvec; v0 += 256) {
        Raw8<FT> raw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (v0 + k * 64 < nvec) raw[k] = load8<FT>(x, base + (v0 + k * 64) * 8);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (v0 + k * 64 >= nvec) continue;
            float v[8], c[8];
            widen8<FT>(raw[k], v);
            if (p.fast) enc8<FT, true, !SYM>(v, p, lo, hi, c);
            else enc8<FT, false, !SYM>(v, p, lo, hi, c);
            store_codes8<BITS, true>(q, g * L + (v0 + k * 64) * 8, c);
        }
    }
    if (lane == 0) {
        scale[g] = p.s;
        if constexpr (!SYM) zp[g] = (uint8_t)(int)p.zpf;
    }
}

// ------------------------------------------------------------ column groups
// View [B, R, C] (C % 8 == 0); group (b, c) is column c of slab b, R long.
// A block covers 512 columns of one slab; its 4 waves split the rows, merge
// the column partials through LDS, then encode their rows again.  Column
// scales differ inside a vector, so this path divides with IEEE division.
template <int FT, int BITS, bool SYM>
__global__ __launch_bounds__(256) void k_quant_cols(const void* __restrict__ x, int64_t R, int64_t C,
                                                    float qmin, float qmax, float yc, uint8_t* __restrict__ q,
                                                    float* __restrict__ scale, uint8_t* __restrict__ zp)
{
    __shared__ float red[2][4][64 * 8];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t b = blockIdx.y;
    const int64_t c0 = ((int64_t)blockIdx.x * 64 + lane) * 8;
    const bool active = c0 < C;
    const int64_t base = b * R * C;
    float mn[8], mx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) mn[i] = mx[i] = 0.0f;
    if (active) {
        for (int64_t r = wv; r < R; r += 4) {
            float v[8];
            widen8<FT>(load8<FT>(x, base + r * C + c0), v);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (SYM) {
                    mx[i] = __builtin_fmaxf(mx[i], __builtin_fabsf(v[i]));
                } else {
                    mn[i] = __builtin_fminf(mn[i], v[i]);
                    mx[i] = __builtin_fmaxf(mx[i], v[i]);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        red[0][wv][lane * 8 + i] = mn[i];
        red[1][wv][lane * 8 + i] = mx[i];
    }
    __syncthreads();
    GP p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float a = red[0][0][lane * 8 + i], m = red[1][0][lane * 8 + i];
#pragma unroll
        for (int k = 1; k < 4; ++k) {
            a = __builtin_fminf(a, red[0][k][lane * 8 + i]);
            m = __builtin_fmaxf(m, red[1][k][lane * 8 + i]);
        }
        p[i] = SYM ? make_gp<FT, true>(m, 0.0f, 0.0f, qmin, qmax, yc) : make_gp<FT, false>(0.0f, a, m, qmin, qmax, yc);
    }
    if (!active) return;
    if (wv == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            scale[b * C + c0 + i] = p[i].s;
            if constexpr (!SYM) zp[b * C + c0 + i] = (uint8_t)(int)p[i].zpf;
        }
    }
    const float lo = MAGIC + qmin, hi = MAGIC + qmax;
    for (int64_t r = wv; r < R; r += 4) {
        float v[8], c[8];
        widen8<FT>(load8<FT>(x, base + r * C + c0), v);
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = int_code_f(v[i] / p[i].s, p[i].zpf, lo, hi);
        store_codes8<BITS>(q, base + r * C + c0, c);
    }
}

// ------------------------------------------------------------ generic
// Block-wide max of a non-negative value and min of a non-positive value.
__device__ __forceinline__ void block_minmax(float& mn, float& mx)
{
    __shared__ float smn[4], smx[4];
    mn = team_min<64>(mn);
    mx = team_max<64>(mx);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) {
        smn[wv] = mn;
        smx[wv] = mx;
    }
    __syncthreads();
    const int nw = (blockDim.x + 63) >> 6;
    mn = smn[0];
    mx = smx[0];
    for (int k = 1; k < nw; ++k) {
        mn = __builtin_fminf(mn, smn[k]);
        mx = __builtin_fmaxf(mx, smx[k]);
    }
}

template <int FT, bool SYM>
__global__ __launch_bounds__(256) void k_reduce_generic(const void* __restrict__ x, DMap m, float qmin,
                                                        float qmax, float yc, float* __restrict__ scale,
                                                        uint8_t* __restrict__ zp)
{
    const int64_t gid = blockIdx.x;
    const int64_t cnt = m.count();
    float mn = 0.0f, mx = 0.0f;
    for (int64_t j = threadIdx.x; j < cnt; j += blockDim.x) {
        float v = load1<FT>(x, m.elem(gid, j));
        if (SYM) {
            mx = __builtin_fmaxf(mx, __builtin_fabsf(v));
        } else {
            mn = __builtin_fminf(mn, v);
            mx = __builtin_fmaxf(mx, v);
        }
    }
    block_minmax(mn, mx);
    if (threadIdx.x == 0) {
        GP p = SYM ? make_gp<FT, true>(mx, 0.0f, 0.0f, qmin, qmax, yc) : make_gp<FT, false>(0.0f, mn, mx, qmin, qmax, yc);
        scale[gid] = p.s;
        if (!SYM) zp[gid] = (uint8_t)(int)p.zpf;
    }
}

__device__ __forceinline__ float zp_at(const uint8_t* zp, int64_t gid, bool zp_signed)
{
    if (!zp) return 0.0f;
    return zp_signed ? (float)(int8_t)zp[gid] : (float)zp[gid];
}

// One code, IEEE division (generic path).
template <int FT>
__device__ __forceinline__ int code_generic(const void* x, const DMap& m, int64_t e, float qmin,
                                            float qmax, const float* scale, const uint8_t* zp,
                                            bool zp_signed)
{
    const int64_t gid = m.group_of(e);
    const float v = load1<FT>(x, e) / scale[gid];
    const float c = __builtin_amdgcn_fmed3f(__builtin_rintf(v) + zp_at(zp, gid, zp_signed), qmin, qmax);
    return (int)c;
}

template <int FT, int BITS>
__global__ __launch_bounds__(256) void k_encode_generic(const void* __restrict__ x, DMap m, float qmin,
                                                        float qmax, const float* __restrict__ scale,
                                                        const uint8_t* __restrict__ zp, bool zp_signed,
                                                        uint8_t* __restrict__ q, int64_t nbytes)
{
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nbytes;
         b += (int64_t)gridDim.x * blockDim.x) {
        if (BITS == 8) {
            q[b] = (uint8_t)code_generic<FT>(x, m, b, qmin, qmax, scale, zp, zp_signed);
        } else {
            int c0 = code_generic<FT>(x, m, 2 * b, qmin, qmax, scale, zp, zp_signed);
            int c1 = code_generic<FT>(x, m, 2 * b + 1, qmin, qmax, scale, zp, zp_signed);
            q[b] = (uint8_t)((c0 & 0xf) | ((c1 & 0xf) << 4));
        }
    }
}

// ------------------------------------------------------------ per tensor
// Pass 1: each block reduces a contiguous chunk and writes
// ws[b] = max(max |x| or max x, 0) and ws[nblk + b] = |min(min x, 0)|.
// 256 bytes per thread are in flight per step (16 vectors of a 2-byte type,
// 8 of f32): a 32768-element chunk is one step (four vectors per step
// measured 2% slower on the per-token workload's tensor).
template <int FT, bool SYM>
__device__ __forceinline__ void minmax_acc(float v, float& mn, float& mx)
{
    if (SYM) {
        mx = __builtin_fmaxf(mx, __builtin_fabsf(v));
    } else {
        mn = __builtin_fminf(mn, v);
        mx = __builtin_fmaxf(mx, v);
    }
}

template <int FT, bool SYM>
__device__ __forceinline__ void range_minmax(const void* x, int64_t b0, int64_t b1, bool vec, float& mn, float& mx)
{
    constexpr int PL = FT == F32 ? 8 : 16;
    if (vec) {
        for (int64_t e = b0 + (int64_t)threadIdx.x * 8; e < b1; e += (int64_t)blockDim.x * 8 * PL) {
            Raw8<FT> r[PL];
#pragma unroll
            for (int k = 0; k < PL; ++k) {
                const int64_t ek = e + (int64_t)k * blockDim.x * 8;
                if (ek < b1) r[k] = load8<FT>(x, ek);
                else r[k] = Raw8<FT>{};
            }
#pragma unroll
            for (int k = 0; k < PL; ++k) {
                float v[8];
                widen8<FT>(r[k], v);
#pragma unroll
                for (int i = 0; i < 8; ++i) minmax_acc<FT, SYM>(v[i], mn, mx);
            }
        }
    } else {
        for (int64_t e = b0 + threadIdx.x; e < b1; e += blockDim.x) minmax_acc<FT, SYM>(load1<FT>(x, e), mn, mx);
    }
}

template <int FT, bool SYM>
__global__ __launch_bounds__(256) void k_tensor_partial(const void* __restrict__ x, int64_t numel,
                                                        int64_t chunk, float* __restrict__ ws)
{
    const int64_t b0 = (int64_t)blockIdx.x * chunk;
    const int64_t b1 = b0 + chunk < numel ? b0 + chunk : numel;
    float mn = 0.0f, mx = 0.0f;
    range_minmax<FT, SYM>(x, b0, b1, (numel & 7) == 0, mn, mx);
    block_minmax(mn, mx);
    if (threadIdx.x == 0) {
        ws[blockIdx.x] = mx;
        ws[gridDim.x + blockIdx.x] = __builtin_fabsf(mn);
    }
}

// Pass 2, by `mode`:
//   TENSOR_ONE    one block reduces the (small, <= 65536 elements) tensor
//                 itself, publishes scale / zero-point and encodes: one launch;
//   TENSOR_STATIC scale / zero-point are inputs;
//   TENSOR_MERGE  every block merges pass 1's partials (parts[0..nparts) the
//                 maxima, parts[nparts..2 nparts) the |minima|), block 0
//                 publishes scale / zero-point.
enum { TENSOR_ONE = 0, TENSOR_STATIC = 1, TENSOR_MERGE = 2 };
constexpr int TENSOR_EV = 2;   // vectors per thread of the encode pass

template <int FT, int BITS, bool SYM, bool FAKE = false>
__global__ __launch_bounds__(256) void k_tensor_encode(const void* __restrict__ x, int64_t numel, int mode,
                                                       const float* __restrict__ parts, int nparts, float qmin,
                                                       float qmax, float yc, void* __restrict__ out,
                                                       float* __restrict__ scale, uint8_t* __restrict__ zp,
                                                       bool zp_signed)
{
    uint8_t* const q = static_cast<uint8_t*>(out);
    GP p;
    if (mode == TENSOR_MERGE) {
        const Part4 pp = load_partials<!SYM>(parts, nparts);
        float mx, nmn;
        merge_partials<!SYM>(pp, mx, nmn);
        p = SYM ? make_gp<FT, true>(mx, 0.0f, 0.0f, qmin, qmax, yc)
                : make_gp<FT, false>(0.0f, -nmn, mx, qmin, qmax, yc);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            scale[0] = p.s;
            if (!SYM) zp[0] = (uint8_t)(int)p.zpf;
        }
    } else {
        __shared__ GP sp;
        if (mode == TENSOR_ONE) {
            float mn = 0.0f, mx = 0.0f;
            range_minmax<FT, SYM>(x, 0, numel, (numel & 7) == 0, mn, mx);
            block_minmax(mn, mx);
            if (threadIdx.x == 0) {
                GP g = SYM ? make_gp<FT, true>(mx, 0.0f, 0.0f, qmin, qmax, yc)
                           : make_gp<FT, false>(0.0f, mn, mx, qmin, qmax, yc);
                sp = g;
                scale[0] = g.s;
                if (!SYM) zp[0] = (uint8_t)(int)g.zpf;
            }
        } else if (threadIdx.x == 0) {
            GP g;
            g.s = scale[0];
            g.fast = scale_in_fast_range(g.s);
            g.y = g.fast ? rcp_rn(g.s) : 0.0f;
            g.zpf = zp_at(zp, 0, zp_signed);
            sp = g;
        }
        __syncthreads();
        p = sp;
    }
    const bool static_scale = mode == TENSOR_STATIC;
    const float lo = MAGIC + qmin, hi = MAGIC + qmax;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if ((numel & 7) == 0) {
        // EV vectors per thread, all loads before any store (one vector per
        // thread measured 3-5% slower; four, 1-2% slower)
        constexpr int EV = TENSOR_EV;
        const int64_t nvec = numel / 8;
        for (int64_t base = (int64_t)blockIdx.x * 256 * EV + threadIdx.x; base < nvec; base += stride * EV) {
            Raw8<FT> r[EV];
#pragma unroll
            for (int k = 0; k < EV; ++k) {
                const int64_t vi = base + (int64_t)k * 256;
                if (vi < nvec) r[k] = load8<FT, true>(x, vi * 8);
                else r[k] = Raw8<FT>{};
            }
#pragma unroll
            for (int k = 0; k < EV; ++k) {
                const int64_t vi = base + (int64_t)k * 256;
                if (vi >= nvec) continue;
                float v[8], c[8];
                widen8<FT>(r[k], v);
                // a static scale does not bound |x|: keep x / s from overflowing
                const bool fast = p.fast & (!static_scale | codes_fast8(v));
                if (fast) enc8<FT, true, true>(v, p, lo, hi, c);
                else enc8<FT, false, true>(v, p, lo, hi, c);
                if constexpr (FAKE) store_fake8<FT>(out, vi * 8, c, p);
                else store_codes8<BITS, true>(q, vi * 8, c);
            }
        }
    } else {
        const int64_t nbytes = FAKE ? numel : BITS == 8 ? numel : numel / 2;
        for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nbytes; b += stride) {
            if (FAKE) {
                const float c = int_code_f(load1<FT>(x, b) / p.s, p.zpf, lo, hi);
                store1<FT>(out, b, fake_value(c, p));
            } else if (BITS == 8) {
                q[b] = (uint8_t)(int)int_code_f(load1<FT>(x, b) / p.s, p.zpf, lo, hi);
            } else {
                int c0 = (int)int_code_f(load1<FT>(x, 2 * b) / p.s, p.zpf, lo, hi);
                int c1 = (int)int_code_f(load1<FT>(x, 2 * b + 1) / p.s, p.zpf, lo, hi);
                q[b] = (uint8_t)((c0 & 0xf) | ((c1 & 0xf) << 4));
            }
        }
    }
}

// Small tensors (numel % 8 == 0, numel <= 1024 * 8 * SMALL_V): one launch of
// 1024 threads; each thread loads its (up to) SMALL_V vectors once, the block
// reduces through DPP and LDS, and the codes are encoded from registers.
constexpr int SMALL_V = 4;
constexpr int64_t SMALL_MAX = 1024 * 8 * SMALL_V;

template <int FT, int BITS, bool SYM, bool FAKE = false>
__global__ __launch_bounds__(1024) void k_tensor_small(const void* __restrict__ x, int64_t numel, float qmin,
                                                       float qmax, float yc, void* __restrict__ out,
                                                       float* __restrict__ scale, uint8_t* __restrict__ zp)
{
    uint8_t* const q = static_cast<uint8_t*>(out);
    __shared__ float smn[16], smx[16];
    __shared__ GP sp;
    const int t = threadIdx.x;
    const int64_t nvec = numel / 8;
    float v[SMALL_V][8];
    float mn = 0.0f, mx = 0.0f;
#pragma unroll
    for (int k = 0; k < SMALL_V; ++k) {
        const int64_t vi = t + (int64_t)k * 1024;
        Raw8<FT> r = Raw8<FT>{};
        if (vi < nvec) r = load8<FT>(x, vi * 8);
        widen8<FT>(r, v[k]);
#pragma unroll
        for (int i = 0; i < 8; ++i) minmax_acc<FT, SYM>(v[k][i], mn, mx);
    }
    mn = team_min<64>(mn);
    mx = team_max<64>(mx);
    if ((t & 63) == 0) {
        smn[t >> 6] = mn;
        smx[t >> 6] = mx;
    }
    __syncthreads();
    if (t == 0) {
        float a = smn[0], b = smx[0];
        for (int k = 1; k < 16; ++k) {
            a = __builtin_fminf(a, smn[k]);
            b = __builtin_fmaxf(b, smx[k]);
        }
        GP p = SYM ? make_gp<FT, true>(b, 0.0f, 0.0f, qmin, qmax, yc) : make_gp<FT, false>(0.0f, a, b, qmin, qmax, yc);
        sp = p;
        scale[0] = p.s;
        if (!SYM) zp[0] = (uint8_t)(int)p.zpf;
    }
    __syncthreads();
    const GP p = sp;
    const float lo = MAGIC + qmin, hi = MAGIC + qmax;
#pragma unroll
    for (int k = 0; k < SMALL_V; ++k) {
        const int64_t vi = t + (int64_t)k * 1024;
        if (vi >= nvec) break;
        float c[8];
        if (p.fast) enc8<FT, true, !SYM>(v[k], p, lo, hi, c);
        else enc8<FT, false, !SYM>(v[k], p, lo, hi, c);
        if constexpr (FAKE) store_fake8<FT>(out, vi * 8, c, p);
        else store_codes8<BITS>(q, vi * 8, c);
    }
}

// ------------------------------------------------------------ elementwise
// Group ids of a vector of 8 elements starting at e (e % 8 == 0):
//   MAP_CONTIG: groups of L contiguous elements (L % 8 == 0): one group e / L
//               (a shift when L is a power of two: sh >= 0).
//   MAP_COLS  : [B, R, C] column groups (C % 8 == 0): groups
//               (e / (R*C)) * C + e % C + i, i = 0..7.
enum { MAP_CONTIG = 0, MAP_COLS = 1 };

template <int MAPK>
__device__ __forceinline__ int64_t vec_group(int64_t e, int64_t P1, int64_t P2, int sh)
{
    if constexpr (MAPK == MAP_CONTIG) return sh >= 0 ? (e >> sh) : e / P1;
    else return (e / (P1 * P2)) * P2 + e % P2;
}

template <bool SIGNED>
__device__ __forceinline__ float code_f(uint32_t b, int bits)
{
    if (bits == 8) return SIGNED ? (float)(int)(int8_t)b : (float)b;
    return SIGNED ? (float)(int)((b ^ 8u) - 8u) : (float)b;
}

template <bool SIGNED>
__device__ __forceinline__ float zp_f(const uint8_t* zp, int64_t g)
{
    if (!zp) return 0.0f;
    return SIGNED ? (float)(int8_t)zp[g] : (float)zp[g];
}

// Vectors of 8 per thread and grid step in the STE and dequantize-backward
// kernels: one each (two or four, and grids capped at 1024 or 2048
// workgroups, measured slower); the dequantizers take DEQ_V.  8-bit codes come
// through non-temporal loads, 4-bit codes through plain ones (the 4-byte lane
// loads of a 1:4 read:write stream are faster that way).
constexpr int SVPT = 1, DVPT = 1;
constexpr bool DEQ_NT = true;

// One grid-stride pass of the 4-bit dequantizer.  Every code, scale and zero-point
// load of a thread's DEQ_V vectors is issued at a clamped index with no
// branch, and a scheduling barrier keeps all of them ahead of the arithmetic,
// so they are in flight together.  The arithmetic runs on the clamped data
// too and only the stores are guarded: with the arithmetic under
// `if (vi < nvec)` the compiler moved each vector's loads into that branch,
// and each vector's loads were then waited for before the next ones issued
// (u4 g = 128 -> f16 [11008, 4096] 22.4 -> 20.8 us).
template <int MAPK, int YT, bool SIGNED, bool POW2, bool HASZP>
__device__ __forceinline__ void dequant4_pass(const uint8_t* __restrict__ q, int64_t nvec, int64_t P1,
                                                 int64_t P2, int sh, const float* __restrict__ scale,
                                                 const uint8_t* __restrict__ zp, void* __restrict__ y)
{
    constexpr int V = DEQ_V;
    constexpr int NS = MAPK == MAP_CONTIG ? 1 : 8;   // scales per vector
    for (int64_t base = (int64_t)blockIdx.x * 256 * V; base < nvec; base += (int64_t)gridDim.x * 256 * V) {
        uint32_t cw[V];
        float sv[V][NS];
        uint32_t zb[V][NS];
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int64_t vk = base + k * 256 + threadIdx.x;
            const int64_t e = (vk < nvec ? vk : nvec - 1) * 8;
            // plain code loads (measured faster than non-temporal ones for this 1:4
            // read:write shape, where the 4-byte lane loads are a fifth of the bytes)
            cw[k] = *reinterpret_cast<const uint32_t*>(q + (e >> 1));
            int64_t g;
            if constexpr (MAPK == MAP_CONTIG) g = POW2 ? (e >> sh) : e / P1;
            else g = (e / (P1 * P2)) * P2 + e % P2;
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                sv[k][i] = scale[g + i];
                zb[k][i] = HASZP ? zp[g + i] : 0u;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        float out[V][8];
#pragma unroll
        for (int k = 0; k < V; ++k) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t zi = zb[k][NS == 1 ? 0 : i];
                const float z = HASZP ? (SIGNED ? (float)(int8_t)zi : (float)zi) : 0.0f;
                out[k][i] = (code_f<SIGNED>((cw[k] >> (i * 4)) & 0xfu, 4) - z) * sv[k][NS == 1 ? 0 : i];
            }
        }
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int64_t vi = base + k * 256 + threadIdx.x;
            if (vi < nvec) store8<YT, WT>(y, vi * 8, out[k]);
        }
    }
}

template <int MAPK, int YT, int BITS, bool SIGNED>
__global__ __launch_bounds__(256) void k_dequant_vec(const uint8_t* __restrict__ q, int64_t nvec, int64_t P1,
                                                     int64_t P2, int sh, const float* __restrict__ scale,
                                                     const uint8_t* __restrict__ zp, void* __restrict__ y)
{
    if constexpr (BITS == 4) {
        // the shift-or-divide group map and the zero point are uniform: chosen once
        if (MAPK == MAP_CONTIG && sh >= 0) {
            if (zp) dequant4_pass<MAPK, YT, SIGNED, true, true>(q, nvec, P1, P2, sh, scale, zp, y);
            else dequant4_pass<MAPK, YT, SIGNED, true, false>(q, nvec, P1, P2, sh, scale, zp, y);
        } else {
            if (zp) dequant4_pass<MAPK, YT, SIGNED, false, true>(q, nvec, P1, P2, sh, scale, zp, y);
            else dequant4_pass<MAPK, YT, SIGNED, false, false>(q, nvec, P1, P2, sh, scale, zp, y);
        }
    } else {
        // 8-bit codes: this loop already keeps every load of a thread in flight,
        // and the fenced pass measured 3% slower for per-token s8
        constexpr int V = DEQ_V;    // vectors per thread: all their loads before any store
        constexpr int NS = MAPK == MAP_CONTIG ? 1 : 8;   // scales per vector
        for (int64_t base = (int64_t)blockIdx.x * 256 * V; base < nvec; base += (int64_t)gridDim.x * 256 * V) {
            uint32_t cw[V][2];
            float sv[V][NS], zv[V][NS];
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const int64_t vi = base + k * 256 + threadIdx.x;
                cw[k][0] = cw[k][1] = 0;
                if (vi >= nvec) continue;
                const uint2 w = DEQ_NT ? ld8<true>(q + vi * 8) : *reinterpret_cast<const uint2*>(q + vi * 8);
                cw[k][0] = w.x;
                cw[k][1] = w.y;
            }
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const int64_t vi = base + k * 256 + threadIdx.x;
                if (vi >= nvec) continue;
                const int64_t g = vec_group<MAPK>(vi * 8, P1, P2, sh);
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    sv[k][i] = scale[g + i];
                    zv[k][i] = zp_f<SIGNED>(zp, g + i);
                }
            }
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const int64_t vi = base + k * 256 + threadIdx.x;
                if (vi >= nvec) break;
                float out[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t c = (cw[k][i >> 2] >> ((i & 3) * 8)) & 0xffu;
                    out[i] = (code_f<SIGNED>(c, 8) - zv[k][NS == 1 ? 0 : i]) * sv[k][NS == 1 ? 0 : i];
                }
                store8<YT, WT>(y, vi * 8, out);
            }
        }
    }
}

template <int MAPK, int FT>
__global__ __launch_bounds__(256) void k_dqb_vec(const void* __restrict__ dy, int64_t nvec, int64_t P1,
                                                 int64_t P2, int sh, const float* __restrict__ scale,
                                                 void* __restrict__ dq)
{
    for (int64_t base = (int64_t)blockIdx.x * 256 * DVPT; base < nvec; base += (int64_t)gridDim.x * 256 * DVPT) {
        Raw8<FT> raw[DVPT];
#pragma unroll
        for (int k = 0; k < DVPT; ++k) {
            const int64_t vi = base + k * 256 + threadIdx.x;
            if (vi < nvec) raw[k] = load8<FT, true>(dy, vi * 8);
        }
#pragma unroll
        for (int k = 0; k < DVPT; ++k) {
            const int64_t vi = base + k * 256 + threadIdx.x;
            if (vi >= nvec) break;
            const int64_t e = vi * 8;
            const int64_t g = vec_group<MAPK>(e, P1, P2, sh);
            float v[8];
            widen8<FT>(raw[k], v);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = v[i] * scale[MAPK == MAP_CONTIG ? g : g + i];
            store8<FT, WT>(dq, e, v);
        }
    }
}

// STE: q recomputed from x; dx = (dy / s) * 1[qmin < q < qmax].  The code
// needs no clamp here: the mask compares the unclamped code with the range.
template <int MAPK, int FT, bool SIGNED>
__global__ __launch_bounds__(256) void k_ste_vec(const void* __restrict__ x, const void* __restrict__ dy,
                                                 int64_t nvec, int64_t P1, int64_t P2, int sh, float qmin,
                                                 float qmax, const float* __restrict__ scale,
                                                 const uint8_t* __restrict__ zp, void* __restrict__ dx)
{
    const float lo = MAGIC + qmin, hi = MAGIC + qmax;
    for (int64_t base = (int64_t)blockIdx.x * 256 * SVPT; base < nvec; base += (int64_t)gridDim.x * 256 * SVPT) {
        Raw8<FT> rx[SVPT], rd[SVPT];
#pragma unroll
        for (int k = 0; k < SVPT; ++k) {
            const int64_t vi = base + k * 256 + threadIdx.x;
            if (vi < nvec) {
                rx[k] = load8<FT, true>(x, vi * 8);
                rd[k] = load8<FT, true>(dy, vi * 8);
            }
        }
#pragma unroll
        for (int k = 0; k < SVPT; ++k) {
            const int64_t vi = base + k * 256 + threadIdx.x;
            if (vi >= nvec) break;
            const int64_t e = vi * 8;
            const int64_t g = vec_group<MAPK>(e, P1, P2, sh);
            float xv[8], dv[8], out[8];
            widen8<FT>(rx[k], xv);
            widen8<FT>(rd[k], dv);
            if constexpr (MAPK == MAP_CONTIG) {
                const float s = scale[g];
                const float zf = zp_f<SIGNED>(zp, g);
                const bool ok = scale_in_fast_range(s) & values_fast8(dv) & codes_fast8(xv);
                if (ok) {
                    const float yr = rcp_rn(s);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float c = (div_q<FT>(xv[i], s, yr) + MAGIC) + zf;
                        const float m = (c > lo && c < hi) ? 1.0f : 0.0f;
                        out[i] = div_q<FT>(dv[i], s, yr) * m;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float c = int_code_f(xv[i] / s, zf, lo, hi);
                        const float m = (c > lo && c < hi) ? 1.0f : 0.0f;
                        out[i] = (dv[i] / s) * m;
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float s = scale[g + i];
                    const float c = int_code_f(xv[i] / s, zp_f<SIGNED>(zp, g + i), lo, hi);
                    const float m = (c > lo && c < hi) ? 1.0f : 0.0f;
                    out[i] = (dv[i] / s) * m;
                }
            }
            store8<FT, true>(dx, e, out);
        }
    }
}

// Fake-quantize backward (per-tensor): q recomputed from x with the saved
// scale / zero-point, dx = dy * 1[qmin < q < qmax] (dy itself, or a zero with
// dy's sign).  VEC: numel % 8 == 0, 8 elements per thread step.
template <int FT, bool VEC>
__global__ __launch_bounds__(256) void k_fake_ste(const void* __restrict__ x, const void* __restrict__ dy,
                                                  int64_t numel, float qmin, float qmax,
                                                  const float* __restrict__ scale, const uint8_t* __restrict__ zp,
                                                  bool zp_signed, void* __restrict__ dx)
{
    const float lo = MAGIC + qmin, hi = MAGIC + qmax;
    const float s = scale[0];
    const float zf = zp_at(zp, 0, zp_signed);
    const bool sfast = scale_in_fast_range(s);
    const float yr = sfast ? rcp_rn(s) : 0.0f;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if constexpr (VEC) {
        for (int64_t vi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; vi < numel / 8; vi += stride) {
            float xv[8], dv[8], out[8];
            widen8<FT>(load8<FT, true>(x, vi * 8), xv);
            widen8<FT>(load8<FT, true>(dy, vi * 8), dv);
            const bool ok = sfast & codes_fast8(xv);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float t = ok ? div_q<FT>(xv[i], s, yr) : xv[i] / s;
                const float c = int_code_f(t, zf, lo, hi);
                out[i] = dv[i] * ((c > lo && c < hi) ? 1.0f : 0.0f);
            }
            store8<FT, true>(dx, vi * 8, out);
        }
    } else {
        for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < numel; e += stride) {
            const float c = int_code_f(load1<FT>(x, e) / s, zf, lo, hi);
            store1<FT>(dx, e, load1<FT>(dy, e) * ((c > lo && c < hi) ? 1.0f : 0.0f));
        }
    }
}

// Generic elementwise ops (any group layout, one element per thread step).
template <int YT, int BITS, bool SIGNED>
__global__ __launch_bounds__(256) void k_dequant_generic(const uint8_t* __restrict__ q, DMap m,
                                                         const float* __restrict__ scale,
                                                         const uint8_t* __restrict__ zp, void* __restrict__ y)
{
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < m.numel;
         e += (int64_t)gridDim.x * blockDim.x) {
        int c;
        if (BITS == 8) {
            c = SIGNED ? (int)(int8_t)q[e] : (int)q[e];
        } else {
            uint32_t n = (e & 1) ? (q[e >> 1] >> 4) : (q[e >> 1] & 0xfu);
            c = SIGNED ? (int)((n ^ 8u) - 8u) : (int)n;
        }
        const int64_t g = m.group_of(e);
        const float z = zp ? (SIGNED ? (float)(int8_t)zp[g] : (float)zp[g]) : 0.0f;
        store1<YT>(y, e, ((float)c - z) * scale[g]);
    }
}

template <int FT>
__global__ __launch_bounds__(256) void k_dqb_generic(const void* __restrict__ dy, DMap m,
                                                     const float* __restrict__ scale, void* __restrict__ dq)
{
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < m.numel;
         e += (int64_t)gridDim.x * blockDim.x)
        store1<FT>(dq, e, load1<FT>(dy, e) * scale[m.group_of(e)]);
}

template <int FT, bool SIGNED>
__global__ __launch_bounds__(256) void k_ste_generic(const void* __restrict__ x, const void* __restrict__ dy,
                                                     DMap m, float qmin, float qmax,
                                                     const float* __restrict__ scale,
                                                     const uint8_t* __restrict__ zp, void* __restrict__ dx)
{
    const float lo = MAGIC + qmin, hi = MAGIC + qmax;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < m.numel;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t g = m.group_of(e);
        const float s = scale[g];
        const float z = zp ? (SIGNED ? (float)(int8_t)zp[g] : (float)zp[g]) : 0.0f;
        const float c = int_code_f(load1<FT>(x, e) / s, z, lo, hi);
        const float mk = (c > lo && c < hi) ? 1.0f : 0.0f;
        store1<FT>(dx, e, (load1<FT>(dy, e) / s) * mk);
    }
}

// ============================================================ host side

// Dispatch helpers over the runtime (ftype, bits, symmetric) triple.
#define TQ_FT_SWITCH(ft, ...)                                     \
    switch (ft) {                                                 \
    case TQ_F32: { constexpr int FTV = F32; __VA_ARGS__; } break; \
    case TQ_F16: { constexpr int FTV = F16; __VA_ARGS__; } break; \
    default: { constexpr int FTV = BF16; __VA_ARGS__; } break;    \
    }

#define TQ_BITS_SYM_SWITCH(bits, sym, ...)                                                  \
    if (bits == 8 && sym) { constexpr int BV = 8; constexpr bool SV = true; __VA_ARGS__; }  \
    else if (bits == 8) { constexpr int BV = 8; constexpr bool SV = false; __VA_ARGS__; }   \
    else if (sym) { constexpr int BV = 4; constexpr bool SV = true; __VA_ARGS__; }          \
    else { constexpr int BV = 4; constexpr bool SV = false; __VA_ARGS__; }

template <int FT, int BITS, bool SYM, int T, int W, int U>
static void launch_team(const void* x, int64_t G, int64_t ldx, float qmin, float qmax, float yc, uint8_t* q,
                        float* scale, uint8_t* zp, hipStream_t st)
{
    constexpr int P = 64 / T;
    const int64_t waves = cdiv(G, (int64_t)U * P);
    hipLaunchKernelGGL((k_quant_team<FT, BITS, SYM, T, W, U>), dim3((unsigned)cdiv(waves, 4)), dim3(256), 0, st,
                       x, G, ldx, qmin, qmax, yc, q, scale, zp);
}

// Contiguous groups of length L (L % 8 == 0), G groups.  Teams of at least
// 8 lanes read whole 128-byte lines per load instruction; groups of 128 use
// 8 lanes x 2 vectors so the per-group scale arithmetic is shared by 16
// elements per lane.
template <int FT, int BITS, bool SYM>
static void quant_contig(const void* x, int64_t G, int64_t L, int64_t ldx, float qmin, float qmax, float yc,
                         uint8_t* q, float* scale, uint8_t* zp, hipStream_t st)
{
    switch (L) {
    case 16: launch_team<FT, BITS, SYM, 2, 1, 8>(x, G, ldx, qmin, qmax, yc, q, scale, zp, st); return;
    case 32: launch_team<FT, BITS, SYM, 4, 1, 8>(x, G, ldx, qmin, qmax, yc, q, scale, zp, st); return;
    case 64: launch_team<FT, BITS, SYM, 8, 1, 8>(x, G, ldx, qmin, qmax, yc, q, scale, zp, st); return;
    case 128:
        // 8 lanes x 2 vectors per group (16 lanes x 1 vector with 1 or 2 groups per lane measured 9-19% slower)
        launch_team<FT, BITS, SYM, 8, 2, 1>(x, G, ldx, qmin, qmax, yc, q, scale, zp, st);
        return;
    case 256: launch_team<FT, BITS, SYM, 16, 2, 4>(x, G, ldx, qmin, qmax, yc, q, scale, zp, st); return;
    case 512: launch_team<FT, BITS, SYM, 64, 1, 4>(x, G, ldx, qmin, qmax, yc, q, scale, zp, st); return;
    case 1024: launch_team<FT, BITS, SYM, 64, 2, 2>(x, G, ldx, qmin, qmax, yc, q, scale, zp, st); return;
    case 2048: launch_team<FT, BITS, SYM, 64, 4, 1>(x, G, ldx, qmin, qmax, yc, q, scale, zp, st); return;
    case 4096:
        // a 4-wave workgroup per group, 2 loads per thread (8 waves with 1 load and a wave per group with 8
        // measured slower)
        if (G <= 0x7fffffff) {
            hipLaunchKernelGGL((k_quant_rows<FT, BITS, SYM, 4, 2>), dim3((unsigned)G), dim3(256), 0, st, x, ldx, qmin,
                               qmax, yc, q, scale, zp);
        } else {
            launch_team<FT, BITS, SYM, 64, 8, 1>(x, G, ldx, qmin, qmax, yc, q, scale, zp, st);
        }
        return;
    default:
        hipLaunchKernelGGL((k_quant_long<FT, BITS, SYM>), dim3((unsigned)cdiv(G, 4)), dim3(256), 0, st,
                           x, G, L, ldx, qmin, qmax, yc, q, scale, zp);
    }
}

// RN(1/qmax) (symmetric) or RN(1/(qmax - qmin)) (asymmetric), on the host
// in binary32.
static float range_reciprocal(int32_t qmin, int32_t qmax, bool sym)
{
    volatile float one = 1.0f;
    return sym ? one / (float)qmax : one / (float)(qmax - qmin);
}

// Quantize with a group map; picks the contiguous, column or generic path.
static tq_status quant_mapped(const void* x, int xt, const GroupMap& m, int code, int32_t qmin, int32_t qmax,
                              void* q, float* scale, void* zero_point, hipStream_t st)
{
    const bool sym = zero_point == nullptr;
    const int bits = code_bits(code);
    const float fmin = (float)qmin, fmax = (float)qmax;
    const float yc = range_reciprocal(qmin, qmax, sym);
    uint8_t* qb = static_cast<uint8_t*>(q);
    uint8_t* zb = static_cast<uint8_t*>(zero_point);
    if (m.numel == 0) return TQ_OK;
    const int es = ftype_size(xt);
    // contiguous groups: per-token, per-group on the last axis, per-channel on axis 0
    int64_t L = -1, G = 0;
    if (m.kind == KIND_GROUP && m.inner == 1) { L = m.g; G = m.ngroups; }
    if (m.kind == KIND_CHANNEL && m.outer == 1) { L = m.inner; G = m.A; }
    if (L > 0 && L % 8 == 0 && (L * es) % 16 == 0) {
        TQ_FT_SWITCH(xt, TQ_BITS_SYM_SWITCH(bits, sym, quant_contig<FTV, BV, SV>(x, G, L, L, fmin, fmax, yc, qb, scale, zb, st)));
        return launch_status();
    }
    // column groups: per-channel on the last axis, per-group on a non-last axis
    int64_t B = 0, R = 0, C = 0;
    if (m.kind == KIND_CHANNEL && m.inner == 1) { B = 1; R = m.outer; C = m.A; }
    if (m.kind == KIND_GROUP && m.inner > 1) { B = m.outer * (m.A / m.g); R = m.g; C = m.inner; }
    if (C > 0 && C % 8 == 0 && (C * es) % 16 == 0 && B <= 65535) {
        dim3 grid((unsigned)cdiv(C, 512), (unsigned)B);
        TQ_FT_SWITCH(xt, TQ_BITS_SYM_SWITCH(bits, sym,
            hipLaunchKernelGGL((k_quant_cols<FTV, BV, SV>), grid, dim3(256), 0, st, x, R, C, fmin, fmax, yc, qb, scale, zb)));
        return launch_status();
    }
    // generic
    if (m.ngroups > 0x7fffffff) return TQ_ERR_UNSUPPORTED;
    const DMap d = to_dmap(m);
    TQ_FT_SWITCH(xt, {
        if (sym) hipLaunchKernelGGL((k_reduce_generic<FTV, true>), dim3((unsigned)m.ngroups), dim3(256), 0, st,
                                    x, d, fmin, fmax, yc, scale, zb);
        else hipLaunchKernelGGL((k_reduce_generic<FTV, false>), dim3((unsigned)m.ngroups), dim3(256), 0, st,
                                x, d, fmin, fmax, yc, scale, zb);
    });
    const int64_t nbytes = bits == 8 ? m.numel : m.numel / 2;
    const bool zs = code_signed(code);
    TQ_FT_SWITCH(xt, {
        if (bits == 8) hipLaunchKernelGGL((k_encode_generic<FTV, 8>), dim3(grid_for(nbytes, 256)), dim3(256), 0, st,
                                          x, d, fmin, fmax, scale, zb, zs, qb, nbytes);
        else hipLaunchKernelGGL((k_encode_generic<FTV, 4>), dim3(grid_for(nbytes, 256)), dim3(256), 0, st,
                                x, d, fmin, fmax, scale, zb, zs, qb, nbytes);
    });
    return launch_status();
}

// Elementwise ops with a group map.
enum { OP_DEQ = 0, OP_STE = 1, OP_DQB = 2 };

struct EwArgs {
    const void* a;      // q (DEQ), x (STE), dy (DQB)
    const void* b;      // dy (STE)
    void* out;          // y / dx / dq
    int in_type;        // ftype of x / dy
    int out_type;       // ftype of y (DEQ)
    int code;
    float qmin, qmax;
    const float* scale;
    const uint8_t* zp;
};

static int log2_exact(int64_t v)
{
    if (v <= 0 || (v & (v - 1))) return -1;
    int k = 0;
    while ((int64_t(1) << k) < v) ++k;
    return k;
}


template <int MAPK>
static void launch_ew_vec(int op, const EwArgs& a, int64_t nvec, int64_t P1, int64_t P2, hipStream_t st)
{
    const dim3 grid(grid_for(nvec, 256 * DEQ_V)), block(256);
    const bool sg = code_signed(a.code);
    const int bits = code_bits(a.code);
    const int sh = MAPK == MAP_CONTIG ? log2_exact(P1) : -1;
    const uint8_t* q = static_cast<const uint8_t*>(a.a);
    if (op == OP_DEQ) {
        TQ_FT_SWITCH(a.out_type, {
            if (bits == 8 && sg) hipLaunchKernelGGL((k_dequant_vec<MAPK, FTV, 8, true>), grid, block, 0, st, q, nvec, P1, P2, sh, a.scale, a.zp, a.out);
            else if (bits == 8) hipLaunchKernelGGL((k_dequant_vec<MAPK, FTV, 8, false>), grid, block, 0, st, q, nvec, P1, P2, sh, a.scale, a.zp, a.out);
            else if (sg) hipLaunchKernelGGL((k_dequant_vec<MAPK, FTV, 4, true>), grid, block, 0, st, q, nvec, P1, P2, sh, a.scale, a.zp, a.out);
            else hipLaunchKernelGGL((k_dequant_vec<MAPK, FTV, 4, false>), grid, block, 0, st, q, nvec, P1, P2, sh, a.scale, a.zp, a.out);
        });
    } else if (op == OP_STE) {
        TQ_FT_SWITCH(a.in_type, {
            const dim3 sgrid(grid_for(nvec, 256 * SVPT));
            if (sg) hipLaunchKernelGGL((k_ste_vec<MAPK, FTV, true>), sgrid, block, 0, st, a.a, a.b, nvec, P1, P2, sh, a.qmin, a.qmax, a.scale, a.zp, a.out);
            else hipLaunchKernelGGL((k_ste_vec<MAPK, FTV, false>), sgrid, block, 0, st, a.a, a.b, nvec, P1, P2, sh, a.qmin, a.qmax, a.scale, a.zp, a.out);
        });
    } else {
        TQ_FT_SWITCH(a.in_type, hipLaunchKernelGGL((k_dqb_vec<MAPK, FTV>), dim3(grid_for(nvec, 256 * DVPT)), block, 0, st, a.a, nvec, P1, P2, sh, a.scale, a.out));
    }
}

static tq_status elementwise_mapped(int op, const EwArgs& a, const GroupMap& m, hipStream_t st)
{
    if (m.numel == 0) return TQ_OK;
    const int64_t nvec = m.numel / 8;
    const bool vec_ok = m.numel % 8 == 0;
    int64_t L = -1;
    if (m.kind == KIND_TENSOR) L = m.numel;
    if (m.kind == KIND_GROUP && m.inner == 1) L = m.g;
    if (m.kind == KIND_CHANNEL && m.outer == 1) L = m.inner;
    if (vec_ok && L > 0 && L % 8 == 0) {
        launch_ew_vec<MAP_CONTIG>(op, a, nvec, L, 0, st);
        return launch_status();
    }
    int64_t R = 0, C = 0;
    if (m.kind == KIND_CHANNEL && m.inner == 1) { R = m.outer; C = m.A; }
    if (m.kind == KIND_GROUP && m.inner > 1) { R = m.g; C = m.inner; }
    if (vec_ok && C > 0 && C % 8 == 0) {
        launch_ew_vec<MAP_COLS>(op, a, nvec, R, C, st);
        return launch_status();
    }
    const DMap d = to_dmap(m);
    const dim3 grid(grid_for(m.numel, 256)), block(256);
    const bool sg = code_signed(a.code);
    const uint8_t* q = static_cast<const uint8_t*>(a.a);
    if (op == OP_DEQ) {
        const int bits = code_bits(a.code);
        TQ_FT_SWITCH(a.out_type, {
            if (bits == 8 && sg) hipLaunchKernelGGL((k_dequant_generic<FTV, 8, true>), grid, block, 0, st, q, d, a.scale, a.zp, a.out);
            else if (bits == 8) hipLaunchKernelGGL((k_dequant_generic<FTV, 8, false>), grid, block, 0, st, q, d, a.scale, a.zp, a.out);
            else if (sg) hipLaunchKernelGGL((k_dequant_generic<FTV, 4, true>), grid, block, 0, st, q, d, a.scale, a.zp, a.out);
            else hipLaunchKernelGGL((k_dequant_generic<FTV, 4, false>), grid, block, 0, st, q, d, a.scale, a.zp, a.out);
        });
    } else if (op == OP_STE) {
        TQ_FT_SWITCH(a.in_type, {
            if (sg) hipLaunchKernelGGL((k_ste_generic<FTV, true>), grid, block, 0, st, a.a, a.b, d, a.qmin, a.qmax, a.scale, a.zp, a.out);
            else hipLaunchKernelGGL((k_ste_generic<FTV, false>), grid, block, 0, st, a.a, a.b, d, a.qmin, a.qmax, a.scale, a.zp, a.out);
        });
    } else {
        TQ_FT_SWITCH(a.in_type, hipLaunchKernelGGL((k_dqb_generic<FTV>), grid, block, 0, st, a.a, d, a.scale, a.out));
    }
    return launch_status();
}

// ------------------------------------------------------------ validation
// With no elements every pointer may be NULL (empty tensors have no
// storage), so an empty call only needs a range that is valid in some mode.
static tq_status check_quant_args(const void* x, int xt, int code, int32_t qmin, int32_t qmax, const void* q,
                                  const float* scale, const void* zp, int64_t last_dim, int64_t numel)
{
    if (!valid_ftype(xt)) return TQ_ERR_INVALID;
    if (!valid_range(code, qmin, qmax, zp == nullptr) && !(numel == 0 && valid_range(code, qmin, qmax, false)))
        return TQ_ERR_INVALID;
    if (code_bits(code) == 4 && (last_dim & 1)) return TQ_ERR_INVALID;
    if (numel == 0) return TQ_OK;
    if (!x || !q || !scale) return TQ_ERR_INVALID;
    if (!aligned16(x) || !aligned16(q)) return TQ_ERR_ALIGN;
    return TQ_OK;
}

static int64_t shape_numel(int32_t ndim, const int64_t* shape)
{
    int64_t n = 1;
    for (int d = 0; d < ndim; ++d) n *= shape[d];
    return n;
}

static tq_status check_map_args(int32_t ndim, const int64_t* shape, int32_t axis)
{
    if (ndim < 1 || ndim > 8 || !shape) return TQ_ERR_INVALID;
    for (int d = 0; d < ndim; ++d)
        if (shape[d] < 0) return TQ_ERR_INVALID;
    if (axis < 0 || axis >= ndim) return TQ_ERR_INVALID;
    return TQ_OK;
}

// Per-tensor dynamic scale of a large tensor, pass 1: the chunk partials
// (maxima, then |minima|) into the workspace; the encode merges them.
static tq_status tensor_partials(const void* x, int xt, int64_t numel, bool sym, void* workspace,
                                 size_t workspace_bytes, int* nparts, hipStream_t st)
{
    if (!workspace || workspace_bytes < tq_workspace_bytes(0, numel)) return TQ_ERR_INVALID;
    if (!aligned16(workspace)) return TQ_ERR_ALIGN;
    const int64_t chunk = tensor_chunk(numel, nparts);
    float* ws = static_cast<float*>(workspace);
    TQ_FT_SWITCH(xt, {
        if (sym) hipLaunchKernelGGL((k_tensor_partial<FTV, true>), dim3(*nparts), dim3(256), 0, st, x, numel, chunk, ws);
        else hipLaunchKernelGGL((k_tensor_partial<FTV, false>), dim3(*nparts), dim3(256), 0, st, x, numel, chunk, ws);
    });
    return launch_status();
}

}  // namespace tq

using namespace tq;

// ============================================================ C ABI
extern "C" {

tq_status tq_quant_per_token(const void* x, int x_dtype, int64_t rows, int64_t cols, int code, int32_t qmin,
                             int32_t qmax, void* q, float* scale, void* zero_point, void* stream)
{
    if (rows < 0 || cols < 0 || (rows > 0 && cols == 0)) return TQ_ERR_INVALID;
    tq_status s = check_quant_args(x, x_dtype, code, qmin, qmax, q, scale, zero_point, cols, rows * cols);
    if (s || rows == 0) return s;
    return quant_mapped(x, x_dtype, token_map(rows, cols), code, qmin, qmax, q, scale, zero_point,
                        as_stream(stream));
}

tq_status tq_quant_per_token_strided(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t x_row_stride,
                                     int code, int32_t qmin, int32_t qmax, void* q, float* scale, void* zero_point,
                                     void* stream)
{
    if (rows < 0 || cols < 0 || (rows > 0 && cols == 0) || x_row_stride < cols) return TQ_ERR_INVALID;
    tq_status s = check_quant_args(x, x_dtype, code, qmin, qmax, q, scale, zero_point, cols, rows * cols);
    if (s || rows == 0) return s;
    const int es = ftype_size(x_dtype);
    if (cols % 8) return TQ_ERR_UNSUPPORTED;
    if ((cols * es) % 16 || (x_row_stride * es) % 16) return TQ_ERR_ALIGN;
    const bool sym = zero_point == nullptr;
    const int bits = code_bits(code);
    const float fmin = (float)qmin, fmax = (float)qmax, yc = range_reciprocal(qmin, qmax, sym);
    uint8_t* qb = static_cast<uint8_t*>(q);
    uint8_t* zb = static_cast<uint8_t*>(zero_point);
    hipStream_t st = as_stream(stream);
    TQ_FT_SWITCH(x_dtype, TQ_BITS_SYM_SWITCH(bits, sym, quant_contig<FTV, BV, SV>(x, rows, cols, x_row_stride, fmin,
                                                                                   fmax, yc, qb, scale, zb, st)));
    return launch_status();
}

tq_status tq_quant_per_channel(const void* x, int x_dtype, int32_t ndim, const int64_t* host_shape, int32_t axis,
                               int code, int32_t qmin, int32_t qmax, void* q, float* scale, void* zero_point,
                               void* stream)
{
    tq_status s = check_map_args(ndim, host_shape, axis);
    if (s) return s;
    const int64_t numel = shape_numel(ndim, host_shape);
    s = check_quant_args(x, x_dtype, code, qmin, qmax, q, scale, zero_point, host_shape[ndim - 1], numel);
    if (s || numel == 0) return s;
    GroupMap m;
    if (!make_map(KIND_CHANNEL, ndim, host_shape, axis, 1, &m)) return TQ_ERR_INVALID;
    return quant_mapped(x, x_dtype, m, code, qmin, qmax, q, scale, zero_point, as_stream(stream));
}

tq_status tq_quant_per_group(const void* x, int x_dtype, int32_t ndim, const int64_t* host_shape, int32_t axis,
                             int64_t group_size, int code, int32_t qmin, int32_t qmax, void* q, float* scale,
                             void* zero_point, void* stream)
{
    tq_status s = check_map_args(ndim, host_shape, axis);
    if (s) return s;
    const int64_t numel = shape_numel(ndim, host_shape);
    s = check_quant_args(x, x_dtype, code, qmin, qmax, q, scale, zero_point, host_shape[ndim - 1], numel);
    if (s) return s;
    GroupMap m;
    if (!make_map(KIND_GROUP, ndim, host_shape, axis, group_size, &m)) return TQ_ERR_INVALID;
    return quant_mapped(x, x_dtype, m, code, qmin, qmax, q, scale, zero_point, as_stream(stream));
}

size_t tq_workspace_bytes(int op, int64_t numel)
{
    if (op == 0) return numel <= 65536 ? 0 : 2 * 1024 * sizeof(float);
    if (op == 1) return 1024 * sizeof(float);
    if (op == 2) return numel <= 65536 ? 0 : 1024 * sizeof(float);
    if (op == 3) return numel <= 0 ? 0 : 2 * 1024 * sizeof(double);
    return 0;
}

tq_status tq_quant_per_tensor(const void* x, int x_dtype, int64_t numel, int code, int32_t qmin, int32_t qmax,
                              int static_scale, void* q, float* scale, void* zero_point, void* workspace,
                              size_t workspace_bytes, void* stream)
{
    if (numel < 0) return TQ_ERR_INVALID;
    tq_status s = check_quant_args(x, x_dtype, code, qmin, qmax, q, scale, zero_point, numel, numel);
    if (s || numel == 0) return s;
    hipStream_t st = as_stream(stream);
    const bool sym = zero_point == nullptr;
    const int bits = code_bits(code);
    const float fmin = (float)qmin, fmax = (float)qmax, yc = range_reciprocal(qmin, qmax, sym);
    if (!static_scale && numel % 8 == 0 && numel <= SMALL_MAX) {
        uint8_t* qb = static_cast<uint8_t*>(q);
        uint8_t* zb = static_cast<uint8_t*>(zero_point);
        TQ_FT_SWITCH(x_dtype, TQ_BITS_SYM_SWITCH(bits, sym,
            hipLaunchKernelGGL((k_tensor_small<FTV, BV, SV>), dim3(1), dim3(1024), 0, st, x, numel, fmin, fmax, yc, qb,
                               scale, zb)));
        return launch_status();
    }
    const bool small = numel <= 65536;
    uint8_t* qb = static_cast<uint8_t*>(q);
    uint8_t* zb = static_cast<uint8_t*>(zero_point);
    const int mode = static_scale ? TENSOR_STATIC : small ? TENSOR_ONE : TENSOR_MERGE;
    int nparts = 0;
    if (mode == TENSOR_MERGE) {
        s = tensor_partials(x, x_dtype, numel, sym, workspace, workspace_bytes, &nparts, st);
        if (s) return s;
    }
    const float* parts = static_cast<const float*>(workspace);
    const int64_t work = (numel % 8 == 0) ? numel / 8 : numel;
    const dim3 grid(mode != TENSOR_ONE ? grid_for(work, 256 * TENSOR_EV) : 1u);
    const bool zs = code_signed(code);
    TQ_FT_SWITCH(x_dtype, TQ_BITS_SYM_SWITCH(bits, sym,
        hipLaunchKernelGGL((k_tensor_encode<FTV, BV, SV>), grid, dim3(256), 0, st, x, numel, mode, parts, nparts, fmin,
                           fmax, yc, qb, scale, zb, zs)));
    return launch_status();
}

tq_status tq_fake_quant_per_tensor(const void* x, int x_dtype, int64_t numel, int code, int32_t qmin,
                                   int32_t qmax, int static_scale, void* y, float* scale, void* zero_point,
                                   void* workspace, size_t workspace_bytes, void* stream)
{
    if (numel < 0) return TQ_ERR_INVALID;
    tq_status s = check_quant_args(x, x_dtype, code, qmin, qmax, y, scale, zero_point, 0, numel);
    if (s || numel == 0) return s;
    hipStream_t st = as_stream(stream);
    const bool sym = zero_point == nullptr;
    const float fmin = (float)qmin, fmax = (float)qmax, yc = range_reciprocal(qmin, qmax, sym);
    uint8_t* zb = static_cast<uint8_t*>(zero_point);
    if (!static_scale && numel % 8 == 0 && numel <= SMALL_MAX) {
        TQ_FT_SWITCH(x_dtype, {
            if (sym) hipLaunchKernelGGL((k_tensor_small<FTV, 8, true, true>), dim3(1), dim3(1024), 0, st, x, numel,
                                        fmin, fmax, yc, y, scale, zb);
            else hipLaunchKernelGGL((k_tensor_small<FTV, 8, false, true>), dim3(1), dim3(1024), 0, st, x, numel,
                                    fmin, fmax, yc, y, scale, zb);
        });
        return launch_status();
    }
    const bool small = numel <= 65536;
    const int mode = static_scale ? TENSOR_STATIC : small ? TENSOR_ONE : TENSOR_MERGE;
    int nparts = 0;
    if (mode == TENSOR_MERGE) {
        s = tensor_partials(x, x_dtype, numel, sym, workspace, workspace_bytes, &nparts, st);
        if (s) return s;
    }
    const float* parts = static_cast<const float*>(workspace);
    const int64_t work = (numel % 8 == 0) ? numel / 8 : numel;
    const dim3 grid(mode != TENSOR_ONE ? grid_for(work, 256 * TENSOR_EV) : 1u);
    const bool zs = code_signed(code);
    TQ_FT_SWITCH(x_dtype, {
        if (sym) hipLaunchKernelGGL((k_tensor_encode<FTV, 8, true, true>), grid, dim3(256), 0, st, x, numel, mode,
                                    parts, nparts, fmin, fmax, yc, y, scale, zb, zs);
        else hipLaunchKernelGGL((k_tensor_encode<FTV, 8, false, true>), grid, dim3(256), 0, st, x, numel, mode,
                                parts, nparts, fmin, fmax, yc, y, scale, zb, zs);
    });
    return launch_status();
}

tq_status tq_fake_quant_per_tensor_backward(const void* x, int x_dtype, int64_t numel, int code, int32_t qmin,
                                            int32_t qmax, const float* scale, const void* zero_point,
                                            const void* dy, void* dx, void* stream)
{
    if (numel < 0) return TQ_ERR_INVALID;
    tq_status s = check_quant_args(x, x_dtype, code, qmin, qmax, dx, scale, zero_point, 0, numel);
    if (s || numel == 0) return s;
    if (!dy) return TQ_ERR_INVALID;
    if (!aligned16(dy)) return TQ_ERR_ALIGN;
    hipStream_t st = as_stream(stream);
    const uint8_t* zb = static_cast<const uint8_t*>(zero_point);
    const bool zs = code_signed(code);
    const bool vec = numel % 8 == 0;
    const dim3 grid(grid_for(vec ? numel / 8 : numel, 256 * 2));
    TQ_FT_SWITCH(x_dtype, {
        if (vec) hipLaunchKernelGGL((k_fake_ste<FTV, true>), grid, dim3(256), 0, st, x, dy, numel, (float)qmin,
                                    (float)qmax, scale, zb, zs, dx);
        else hipLaunchKernelGGL((k_fake_ste<FTV, false>), grid, dim3(256), 0, st, x, dy, numel, (float)qmin,
                                (float)qmax, scale, zb, zs, dx);
    });
    return launch_status();
}

tq_status tq_dynamic_range_quantize(const void* x, int x_dtype, int32_t ndim, const int64_t* host_shape, int mode,
                                    int scope, int32_t axis, int code, void* q, float* scale, void* zero_point,
                                    void* workspace, size_t workspace_bytes, void* stream)
{
    if (mode != TQ_RANGE_SYMMETRIC && mode != TQ_RANGE_ASYMMETRIC) return TQ_ERR_INVALID;
    const bool sym = mode == TQ_RANGE_SYMMETRIC;
    int32_t qmin, qmax;
    if (tq_default_q_range(code, sym, &qmin, &qmax) != TQ_OK) return TQ_ERR_INVALID;
    tq_status s = check_map_args(ndim, host_shape, scope == TQ_SCOPE_CHANNEL ? axis : 0);
    if (s) return s;
    const int64_t numel = shape_numel(ndim, host_shape);
    if (!sym && !zero_point && numel > 0) return TQ_ERR_INVALID;
    void* zp = sym ? nullptr : zero_point;
    switch (scope) {
    case TQ_SCOPE_TENSOR:
        return tq_quant_per_tensor(x, x_dtype, numel, code, qmin, qmax, 0, q, scale, zp, workspace, workspace_bytes,
                                   stream);
    case TQ_SCOPE_TOKEN: {
        const int64_t cols = host_shape[ndim - 1];
        const int64_t rows = shape_numel(ndim - 1, host_shape);
        return tq_quant_per_token(x, x_dtype, rows, cols, code, qmin, qmax, q, scale, zp, stream);
    }
    case TQ_SCOPE_CHANNEL:
        return tq_quant_per_channel(x, x_dtype, ndim, host_shape, axis, code, qmin, qmax, q, scale, zp, stream);
    default:
        return TQ_ERR_INVALID;
    }
}

// ---------------------------------------------------------------- dequant
static tq_status dequant_common(const void* q, int code, const GroupMap& m, const float* scale,
                                const void* zero_point, void* y, int y_dtype, void* stream)
{
    if (!valid_code(code) || !valid_ftype(y_dtype)) return TQ_ERR_INVALID;
    if (m.numel == 0) return TQ_OK;
    if (!q || !scale || !y) return TQ_ERR_INVALID;
    if (!aligned16(q) || !aligned16(y)) return TQ_ERR_ALIGN;
    EwArgs a{};
    a.a = q;
    a.out = y;
    a.out_type = y_dtype;
    a.code = code;
    a.scale = scale;
    a.zp = static_cast<const uint8_t*>(zero_point);
    return elementwise_mapped(OP_DEQ, a, m, as_stream(stream));
}

tq_status tq_dequant_per_tensor(const void* q, int code, int64_t numel, const float* scale, const void* zero_point,
                                void* y, int y_dtype, void* stream)
{
    if (numel < 0 || (code_bits(code) == 4 && (numel & 1))) return TQ_ERR_INVALID;
    return dequant_common(q, code, tensor_map(numel), scale, zero_point, y, y_dtype, stream);
}

tq_status tq_dequant_per_channel(const void* q, int code, int32_t ndim, const int64_t* host_shape, int32_t axis,
                                 const float* scale, const void* zero_point, void* y, int y_dtype, void* stream)
{
    if (check_map_args(ndim, host_shape, axis)) return TQ_ERR_INVALID;
    if (code_bits(code) == 4 && (host_shape[ndim - 1] & 1)) return TQ_ERR_INVALID;
    GroupMap m;
    if (!make_map(KIND_CHANNEL, ndim, host_shape, axis, 1, &m)) return TQ_ERR_INVALID;
    return dequant_common(q, code, m, scale, zero_point, y, y_dtype, stream);
}

tq_status tq_dequant_per_token(const void* q, int code, int64_t rows, int64_t cols, const float* scale,
                               const void* zero_point, void* y, int y_dtype, void* stream)
{
    if (rows < 0 || cols < 0 || (rows > 0 && cols == 0) || (code_bits(code) == 4 && (cols & 1)))
        return TQ_ERR_INVALID;
    return dequant_common(q, code, token_map(rows, cols), scale, zero_point, y, y_dtype, stream);
}

tq_status tq_dequant_per_group(const void* q, int code, int32_t ndim, const int64_t* host_shape, int32_t axis,
                               int64_t group_size, const float* scale, const void* zero_point, void* y,
                               int y_dtype, void* stream)
{
    if (check_map_args(ndim, host_shape, axis)) return TQ_ERR_INVALID;
    if (code_bits(code) == 4 && (host_shape[ndim - 1] & 1)) return TQ_ERR_INVALID;
    GroupMap m;
    if (!make_map(KIND_GROUP, ndim, host_shape, axis, group_size, &m)) return TQ_ERR_INVALID;
    return dequant_common(q, code, m, scale, zero_point, y, y_dtype, stream);
}

// ---------------------------------------------------------------- STE
static tq_status ste_common(const void* x, int x_dtype, const GroupMap& m, int code, int32_t qmin, int32_t qmax,
                            const float* scale, const void* zero_point, const void* dy, void* dx, void* stream)
{
    if (!valid_ftype(x_dtype)) return TQ_ERR_INVALID;
    if (m.numel == 0) return valid_code(code) && qmin < qmax ? TQ_OK : TQ_ERR_INVALID;
    if (!valid_range(code, qmin, qmax, zero_point == nullptr)) return TQ_ERR_INVALID;
    if (!x || !dy || !dx || !scale) return TQ_ERR_INVALID;
    if (!aligned16(x) || !aligned16(dy) || !aligned16(dx)) return TQ_ERR_ALIGN;
    EwArgs a{};
    a.a = x;
    a.b = dy;
    a.out = dx;
    a.in_type = x_dtype;
    a.code = code;
    a.qmin = (float)qmin;
    a.qmax = (float)qmax;
    a.scale = scale;
    a.zp = static_cast<const uint8_t*>(zero_point);
    return elementwise_mapped(OP_STE, a, m, as_stream(stream));
}

tq_status tq_quant_per_tensor_backward(const void* x, int x_dtype, int64_t numel, int code, int32_t qmin,
                                       int32_t qmax, const float* scale, const void* zero_point, const void* dy,
                                       void* dx, void* stream)
{
    if (numel < 0) return TQ_ERR_INVALID;
    return ste_common(x, x_dtype, tensor_map(numel), code, qmin, qmax, scale, zero_point, dy, dx, stream);
}

tq_status tq_quant_per_channel_backward(const void* x, int x_dtype, int32_t ndim, const int64_t* host_shape,
                                        int32_t axis, int code, int32_t qmin, int32_t qmax, const float* scale,
                                        const void* zero_point, const void* dy, void* dx, void* stream)
{
    if (check_map_args(ndim, host_shape, axis)) return TQ_ERR_INVALID;
    GroupMap m;
    if (!make_map(KIND_CHANNEL, ndim, host_shape, axis, 1, &m)) return TQ_ERR_INVALID;
    return ste_common(x, x_dtype, m, code, qmin, qmax, scale, zero_point, dy, dx, stream);
}

tq_status tq_quant_per_token_backward(const void* x, int x_dtype, int64_t rows, int64_t cols, int code,
                                      int32_t qmin, int32_t qmax, const float* scale, const void* zero_point,
                                      const void* dy, void* dx, void* stream)
{
    if (rows < 0 || cols < 0 || (rows > 0 && cols == 0)) return TQ_ERR_INVALID;
    return ste_common(x, x_dtype, token_map(rows, cols), code, qmin, qmax, scale, zero_point, dy, dx, stream);
}

tq_status tq_quant_per_group_backward(const void* x, int x_dtype, int32_t ndim, const int64_t* host_shape,
                                      int32_t axis, int64_t group_size, int code, int32_t qmin, int32_t qmax,
                                      const float* scale, const void* zero_point, const void* dy, void* dx,
                                      void* stream)
{
    if (check_map_args(ndim, host_shape, axis)) return TQ_ERR_INVALID;
    GroupMap m;
    if (!make_map(KIND_GROUP, ndim, host_shape, axis, group_size, &m)) return TQ_ERR_INVALID;
    return ste_common(x, x_dtype, m, code, qmin, qmax, scale, zero_point, dy, dx, stream);
}

// ---------------------------------------------------------------- dequant backward
static tq_status dqb_common(const void* dy, int dy_dtype, const GroupMap& m, const float* scale, void* dq,
                            void* stream)
{
    if (!valid_ftype(dy_dtype)) return TQ_ERR_INVALID;
    if (m.numel == 0) return TQ_OK;
    if (!dy || !dq || !scale) return TQ_ERR_INVALID;
    if (!aligned16(dy) || !aligned16(dq)) return TQ_ERR_ALIGN;
    EwArgs a{};
    a.a = dy;
    a.out = dq;
    a.in_type = dy_dtype;
    a.code = TQ_S8;
    a.scale = scale;
    return elementwise_mapped(OP_DQB, a, m, as_stream(stream));
}

tq_status tq_dequant_per_tensor_backward(const void* dy, int dy_dtype, int64_t numel, const float* scale, void* dq,
                                         void* stream)
{
    if (numel < 0) return TQ_ERR_INVALID;
    return dqb_common(dy, dy_dtype, tensor_map(numel), scale, dq, stream);
}

tq_status tq_dequant_per_channel_backward(const void* dy, int dy_dtype, int32_t ndim, const int64_t* host_shape,
                                          int32_t axis, const float* scale, void* dq, void* stream)
{
    if (check_map_args(ndim, host_shape, axis)) return TQ_ERR_INVALID;
    GroupMap m;
    if (!make_map(KIND_CHANNEL, ndim, host_shape, axis, 1, &m)) return TQ_ERR_INVALID;
    return dqb_common(dy, dy_dtype, m, scale, dq, stream);
}

tq_status tq_dequant_per_token_backward(const void* dy, int dy_dtype, int64_t rows, int64_t cols,
                                        const float* scale, void* dq, void* stream)
{
    if (rows < 0 || cols < 0 || (rows > 0 && cols == 0)) return TQ_ERR_INVALID;
    return dqb_common(dy, dy_dtype, token_map(rows, cols), scale, dq, stream);
}

tq_status tq_dequant_per_group_backward(const void* dy, int dy_dtype, int32_t ndim, const int64_t* host_shape,
                                        int32_t axis, int64_t group_size, const float* scale, void* dq,
                                        void* stream)
{
    if (check_map_args(ndim, host_shape, axis)) return TQ_ERR_INVALID;
    GroupMap m;
    if (!make_map(KIND_GROUP, ndim, host_shape, axis, group_size, &m)) return TQ_ERR_INVALID;
    return dqb_common(dy, dy_dtype, m, scale, dq, stream);
}

}  // extern "C"
