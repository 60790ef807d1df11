// tq_device.h -- device helpers shared by the gfx950 quantization kernels.
//
// Everything here is wave64 CDNA4 code: 16-byte global loads, DPP / bpermute
// team reductions, v_med3 clamps, and the native FP8 / FP4 / bf16
// conversion instructions.  Arithmetic follows IEEE binary32 with
// round-to-nearest-even (the kernels are built with -ffp-contract=off and
// f32 denormals preserved).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

enum FType { F32 = 0, F16 = 1, BF16 = 2 };
enum Code { S8 = 0, U8 = 1, S4 = 2, U4 = 3 };

typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float as_f(uint32_t b) { return __uint_as_float(b); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// ---------------------------------------------------------------- raw I/O
// Streaming accesses: every input byte is read once and every output byte
// written once.  Kernels mark an access non-temporal (NT) only when each
// wave-wide instruction covers whole 128-byte lines: a non-temporal line
// that an instruction uses only in part is evicted before the next
// instruction needs the rest.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool NT = false>
__device__ __forceinline__ uint4 ld16(const void* p)
{
    u32x4 v;
    if constexpr (NT) v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    else v = *static_cast<const u32x4*>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool NT = false>
__device__ __forceinline__ uint2 ld8(const void* p)
{
    u32x2 v;
    if constexpr (NT) v = __builtin_nontemporal_load(static_cast<const u32x2*>(p));
    else v = *static_cast<const u32x2*>(p);
    return make_uint2(v.x, v.y);
}

// 16-byte stores.  NT = 0: plain; 1: non-temporal; 2 (WT): non-temporal
// with device scope (nt sc1), which passes the L2 on to memory instead of
// leaving dirty lines behind.  Measured per kernel (same code otherwise,
// interleaved runs): WT is 2-7% faster for the 8-bit and 4-bit integer
// dequantize, the FP4 dequantize (with two vectors per thread; with one it
// was slower), the dequantize backward (integer, FP8, MXFP8, FP4), the FP8
// dequantize, row concatenation, the FP4 -> FP8 expansion and the binary64
// dequantize, and 1-3% slower for the binary64 dequantize backward, the byte
// transposes and the fake-quantization kernels, which keep NT = 1.  A store has no output register, so the asm form is safe to
// leave in flight; it only makes the compiler's own vmcnt waits
// conservative.  It does read its data VGPRs after it issues: a store of
// more than 8 bytes needs two wait states before a vector instruction may
// write them (the ISA's store-data hazard), which the compiler inserts after
// its own stores but cannot see inside asm, so the asm carries the s_nop.
constexpr int WT = 2;

template <int NT = 0>
__device__ __forceinline__ void st16(void* p, uint4 w)
{
    const u32x4 v = {w.x, w.y, w.z, w.w};
    if constexpr (NT == WT)
        asm volatile("global_store_dwordx4 %0, %1, off nt sc1\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
    else if constexpr (NT) __builtin_nontemporal_store(v, static_cast<u32x4*>(p));
    else *static_cast<u32x4*>(p) = v;
}

template <bool NT = false>
__device__ __forceinline__ void st8(void* p, uint2 w)
{
    const u32x2 v = {w.x, w.y};
    if constexpr (NT) __builtin_nontemporal_store(v, static_cast<u32x2*>(p));
    else *static_cast<u32x2*>(p) = v;
}

template <bool NT = false>
__device__ __forceinline__ void st4(void* p, uint32_t w)
{
    if constexpr (NT) __builtin_nontemporal_store(w, static_cast<uint32_t*>(p));
    else *static_cast<uint32_t*>(p) = w;
}

// Eight consecutive elements of a float tensor: one 16-byte load for the
// 2-byte types, two for f32.
template <int FT> struct Raw8 { uint4 w[FT == F32 ? 2 : 1]; };

template <int FT, bool NT = false>
__device__ __forceinline__ Raw8<FT> load8(const void* base, int64_t e)
{
    Raw8<FT> r;
    if constexpr (FT == F32) {
        const float* p = static_cast<const float*>(base) + e;
        r.w[0] = ld16<NT>(p);
        r.w[1] = ld16<NT>(p + 4);
    } else {
        r.w[0] = ld16<NT>(static_cast<const uint16_t*>(base) + e);
    }
    return r;
}

__device__ __forceinline__ float f16_lo(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Exact widening to binary32.
template <int FT>
__device__ __forceinline__ void widen8(const Raw8<FT>& r, float v[8])
{
    if constexpr (FT == F32) {
        v[0] = as_f(r.w[0].x); v[1] = as_f(r.w[0].y); v[2] = as_f(r.w[0].z); v[3] = as_f(r.w[0].w);
        v[4] = as_f(r.w[1].x); v[5] = as_f(r.w[1].y); v[6] = as_f(r.w[1].z); v[7] = as_f(r.w[1].w);
    } else if constexpr (FT == BF16) {
        const uint32_t w[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = as_f(w[i] << 16);
            v[2 * i + 1] = as_f(w[i] & 0xffff0000u);
        }
    } else {
        const uint32_t w[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = f16_lo(w[i]);
            v[2 * i + 1] = f16_hi(w[i]);
        }
    }
}

// Makes v opaque to the optimizer.  Used before every narrowing: without it
// the backend folds "round(a * b) to f16" into v_fma_mix*_f16 with a zero
// addend, which rounds the exact product once (not the binary32 product) and
// turns -0 into +0.
__device__ __forceinline__ float opaque(float v)
{
    asm("" : "+v"(v));
    return v;
}

__device__ __forceinline__ uint16_t to_f16_bits(float v)
{
    return __builtin_bit_cast(uint16_t, (_Float16)opaque(v));
}

__device__ __forceinline__ uint16_t to_bf16_bits(float v)
{
    return __builtin_bit_cast(uint16_t, (__bf16)opaque(v));
}

// Round-to-nearest-even narrowing of two binary32 values into one packed
// dword (first value in the low half).
template <int FT>
__device__ __forceinline__ uint32_t narrow2(float a, float b)
{
    if constexpr (FT == BF16) {
        bf2v h = __builtin_convertvector((f2v){opaque(a), opaque(b)}, bf2v);
        return __builtin_bit_cast(uint32_t, h);
    } else {
        uint32_t lo = to_f16_bits(a);
        uint32_t hi = to_f16_bits(b);
        return lo | (hi << 16);
    }
}

// Store eight binary32 values as output type FT at element index e.
template <int FT, int NT = 0>
__device__ __forceinline__ void store8(void* base, int64_t e, const float v[8])
{
    if constexpr (FT == F32) {
        float* p = static_cast<float*>(base) + e;
        st16<NT>(p, make_uint4(as_u(v[0]), as_u(v[1]), as_u(v[2]), as_u(v[3])));
        st16<NT>(p + 4, make_uint4(as_u(v[4]), as_u(v[5]), as_u(v[6]), as_u(v[7])));
    } else {
        uint4 w = make_uint4(narrow2<FT>(v[0], v[1]), narrow2<FT>(v[2], v[3]),
                             narrow2<FT>(v[4], v[5]), narrow2<FT>(v[6], v[7]));
        st16<NT>(static_cast<uint16_t*>(base) + e, w);
    }
}

// Scalar element access (generic paths).
template <int FT>
__device__ __forceinline__ float load1(const void* base, int64_t e)
{
    if constexpr (FT == F32) return static_cast<const float*>(base)[e];
    else {
        uint32_t h = static_cast<const uint16_t*>(base)[e];
        if constexpr (FT == BF16) return as_f(h << 16);
        else return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    }
}

template <int FT>
__device__ __forceinline__ void store1(void* base, int64_t e, float v)
{
    if constexpr (FT == F32) static_cast<float*>(base)[e] = v;
    else if constexpr (FT == BF16) static_cast<uint16_t*>(base)[e] = to_bf16_bits(v);
    else static_cast<uint16_t*>(base)[e] = to_f16_bits(v);
}

// ---------------------------------------------------------------- division
// Correctly rounded binary32 x / s from y = RN(1/s) by FMA corrections
// (Markstein's division; P. Markstein, IBM J. Res. Dev. 34(1), 1990):
//   q0 = x*y,  r = fma(q0, s, -x),  q1 = fma(-r, y, q0)     [one correction]
//   r  = fma(q1, s, -x),  q2 = fma(-r, y, q1)               [second one]
// One correction is exact when x is a bf16 or f16 value: every (dividend
// significand with 7 or 10 fraction bits, binary32 divisor significand)
// pair was checked against IEEE division, and rounding is scale-invariant
// while the intermediates stay normal.  Binary32 dividends take both
// corrections (the first makes the quotient faithful, the second correctly
// rounded).  Written as q + (-r) * y so that x = +-0 returns the zero of x's
// sign, as IEEE division does.
// Exactness range: 2^-40 <= |s| <= 2^40 and 2^-78 <= |x| <= 2^86, or x = 0
// (all intermediates stay normal).  Below 2^-78 the magnitude is still
// below 2^-38, far under every code threshold (>= 2^-10), but its sign can
// be wrong; callers that need that sign restore it with with_sign_of().
template <int FTX>
__device__ __forceinline__ float div_q(float x, float s, float y)
{
    float q0 = x * y;
    float r = __builtin_fmaf(q0, s, -x);
    float q1 = __builtin_fmaf(-r, y, q0);
    if constexpr (FTX == F32) {
        r = __builtin_fmaf(q1, s, -x);
        q1 = __builtin_fmaf(-r, y, q1);
    }
    return q1;
}

__device__ __forceinline__ bool scale_in_fast_range(float s)
{
    float a = __builtin_fabsf(s);
    return a >= 0x1p-40f && a <= 0x1p40f;
}

__device__ __forceinline__ bool value_in_fast_range(float x)
{
    float a = __builtin_fabsf(x);
    return a >= 0x1p-78f && a <= 0x1p86f;
}

// Range guards over a vector of 8 values, reduced branch-free through
// max / min (short-circuit && chains compile into nested exec-mask branches).
// Every |v| <= 2^86 (quotients that only feed a code):
__device__ __forceinline__ bool codes_fast8(const float v[8])
{
    float m = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[0]), __builtin_fabsf(v[1])), __builtin_fabsf(v[2]));
    m = __builtin_fmaxf(__builtin_fmaxf(m, __builtin_fabsf(v[3])), __builtin_fabsf(v[4]));
    m = __builtin_fmaxf(__builtin_fmaxf(m, __builtin_fabsf(v[5])), __builtin_fabsf(v[6]));
    m = __builtin_fmaxf(m, __builtin_fabsf(v[7]));
    return m <= 0x1p86f;
}

// Every v zero or 2^-78 <= |v| <= 2^86 (quotients that are output values):
__device__ __forceinline__ bool values_fast8(const float v[8])
{
    float hi = 0.0f, lo = __builtin_inff();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float a = __builtin_fabsf(v[i]);
        hi = __builtin_fmaxf(hi, a);
        lo = __builtin_fminf(lo, a == 0.0f ? __builtin_inff() : a);
    }
    return (hi <= 0x1p86f) & (lo >= 0x1p-78f);
}

// RN(1/s) for 2^-40 <= |s| <= 2^40: v_rcp_f32 and one Newton step.  On
// gfx950 this equals IEEE 1/s for every binary32 significand (checked
// exhaustively at several exponents; the step is scale-invariant there).
__device__ __forceinline__ float rcp_rn(float s)
{
    const float y0 = __builtin_amdgcn_rcpf(s);
    const float e = __builtin_fmaf(-s, y0, 1.0f);
    return __builtin_fmaf(e, y0, y0);
}

// x / c for a divisor c inside the fast range with yc = RN(1/c): the fast
// sequence when x is in its exact range (or zero), IEEE division otherwise.
template <int FTX>
__device__ __forceinline__ float div_by(float x, float c, float yc)
{
    if (value_in_fast_range(x) || x == 0.0f) return div_q<FTX>(x, c, yc);
    return x / c;
}

// |q| with the sign of x (exact for the fast quotients above, whose sign can
// only be wrong when |q| < 2^-38).
__device__ __forceinline__ float with_sign_of(float q, float x)
{
    return as_f((as_u(q) & 0x7fffffffu) | (as_u(x) & 0x80000000u));
}

// ---------------------------------------------------------------- lanes
// Max / min across a team of T lanes (T = 1..64, power of two) that are
// contiguous and aligned in the wave: DPP quad permutes and row mirrors
// within a 16-lane row, ds_bpermute-based shuffles across rows.  Every lane
// of the team ends with the team's result.
//
// The reductions run on bit patterns.  Every team_max caller reduces values
// >= 0, whose unsigned order is their float order; every team_min caller
// reduces values <= 0 (a minimum that starts at 0), whose float minimum is
// the unsigned maximum (sign bit set, larger magnitude wins; -0 may win over
// +0, which no caller can tell apart).  An integer max needs no NaN
// canonicalization and fuses with the DPP move into one instruction.
// Every control used here reads a valid lane for every lane, so the old
// value is irrelevant (bound_ctrl) and the move folds into the max.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, true);
}

constexpr int DPP_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;

template <int T>
__device__ __forceinline__ uint32_t team_umax(uint32_t u)
{
    if constexpr (T >= 2) u = max(u, dpp<DPP_XOR1>(u));
    if constexpr (T >= 4) u = max(u, dpp<DPP_XOR2>(u));
    if constexpr (T >= 8) u = max(u, dpp<DPP_HALF_MIRROR>(u));
    if constexpr (T >= 16) u = max(u, dpp<DPP_MIRROR>(u));
    if constexpr (T >= 32) u = max(u, (uint32_t)__shfl_xor((int)u, 16, 64));
    if constexpr (T >= 64) u = max(u, (uint32_t)__shfl_xor((int)u, 32, 64));
    return u;
}

// max over the team of values >= 0
template <int T>
__device__ __forceinline__ float team_max(float v)
{
    return as_f(team_umax<T>(as_u(v)));
}

// min over the team of values <= 0
template <int T>
__device__ __forceinline__ float team_min(float v)
{
    return as_f(team_umax<T>(as_u(v)));
}

// Dequantizers take DEQ_V vectors of 8 elements per thread and issue all of
// their loads before any store (workgroup b covers vectors b*256*DEQ_V ..,
// thread j the vectors k*256 + j, so each wave instruction stays contiguous).
// Two measured up to 29% faster than one in the same form (most for the 4-bit
// and FP4 codes, 1:4 read:write streams; MXFP8 unchanged), four no faster.
constexpr int DEQ_V = 2;

// ---------------------------------------------------------------- per-tensor partials
// The encoding pass of a per-tensor scale merges the first pass's partial
// maxima (n of them, n a multiple of 4, at most 1024; all >= 0) in every
// workgroup of 256 threads instead of in a launch of its own: thread t reads
// partials 4t..4t+3 of each of the two arrays (one 16-byte load each, issued
// before the thread's input loads so that their latencies overlap), a DPP
// reduction runs within each wave and LDS across the four.  Every workgroup
// computes the same maxima: max is exact and order-free.
struct Part4 {
    uint4 a, b;
};

template <bool TWO>
__device__ __forceinline__ Part4 load_partials(const float* ws, int n)
{
    Part4 p = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
    const int i = (int)threadIdx.x * 4;
    if (i < n) {
        p.a = ld16<false>(ws + i);
        if constexpr (TWO) p.b = ld16<false>(ws + n + i);
    }
    return p;
}

__device__ __forceinline__ float max4u(uint4 w)
{
    return as_f(max(max(w.x, w.y), max(w.z, w.w)));   // values >= 0: unsigned order is float order
}

// The maxima over the workgroup (ma over the first array, mb over the second
// when TWO).  Contains a workgroup barrier: every thread must call it.
template <bool TWO>
__device__ __forceinline__ void merge_partials(const Part4& p, float& ma, float& mb)
{
    __shared__ float sa[4], sb[4];
    const float a = team_max<64>(max4u(p.a));
    const float b = TWO ? team_max<64>(max4u(p.b)) : 0.0f;
    if ((threadIdx.x & 63) == 0) {
        sa[threadIdx.x >> 6] = a;
        if constexpr (TWO) sb[threadIdx.x >> 6] = b;
    }
    __syncthreads();
    ma = __builtin_fmaxf(__builtin_fmaxf(sa[0], sa[1]), __builtin_fmaxf(sa[2], sa[3]));
    mb = TWO ? __builtin_fmaxf(__builtin_fmaxf(sb[0], sb[1]), __builtin_fmaxf(sb[2], sb[3])) : 0.0f;
}

// ---------------------------------------------------------------- codes
// Integer codes via the 1.5 * 2^23 trick: for |v| < 2^22, v + M rounds v to
// an integer with ties to even (the spacing of binary32 in [2^23, 2^24) is
// 1 and M is even), and the low bits of the sum's pattern hold that
// integer in two's complement.  Adding the (integer) zero-point and
// clamping to [M + qmin, M + qmax] stay exact; for |v| >= 2^22 the clamp
// decides alone.
constexpr float MAGIC = 12582912.0f;   // 1.5 * 2^23

__device__ __forceinline__ float int_code_f(float v, float zpf, float lo, float hi)
{
    return __builtin_amdgcn_fmed3f((v + MAGIC) + zpf, lo, hi);
}

// Pack the low bytes of four code floats into one dword.
__device__ __forceinline__ uint32_t pack_bytes4(float a, float b, float c, float d)
{
    uint32_t ab = __builtin_amdgcn_perm(as_u(b), as_u(a), 0x0c0c0400u);
    uint32_t cd = __builtin_amdgcn_perm(as_u(d), as_u(c), 0x0c0c0400u);
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// Pack eight 4-bit codes (low nibbles of the code floats' patterns) into one
// dword, even index in the low nibble.
__device__ __forceinline__ uint32_t pack_nibbles8(const float c[8], bool mask_high)
{
    uint32_t ev = pack_bytes4(c[0], c[2], c[4], c[6]);
    uint32_t od = pack_bytes4(c[1], c[3], c[5], c[7]);
    if (mask_high) {
        ev &= 0x0f0f0f0fu;
        od &= 0x0f0f0f0fu;
    }
    return ev | (od << 4);
}

// ---------------------------------------------------------------- FP8 / FP4
// OCP E4M3 (gfx950's fp8 format): pre-clamped to +-448 so that the result
// never depends on the instruction's overflow handling; round to nearest
// even.  Four values -> one dword (first value in the low byte).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d)
{
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
    d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ float e4m3_val(uint32_t word, int byte)
{
    switch (byte) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)word, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)word, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)word, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)word, 3);
    }
}

// OCP E2M1, pre-clamped to +-6.  Eight values -> one dword of nibbles
// (first value in the low nibble).
__device__ __forceinline__ uint32_t e2m1_pack8(const float v[8])
{
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_fmed3f(v[i], -6.0f, 6.0f);
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c[0], c[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c[2], c[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c[4], c[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c[6], c[7], 1.0f, 3);
    return w;
}

// Decode one byte of E2M1 pairs: .x = low nibble, .y = high nibble.
__device__ __forceinline__ f2v e2m1_val2(uint32_t word, int byte)
{
    switch (byte) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3);
    }
}

// E8M0 byte -> 2^(b-127) as binary32 (b = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_val(uint32_t b)
{
    return b == 0 ? 0x1p-127f : as_f(b << 23);
}

// 2^(127-b): the exact reciprocal of e8m0_val(b) (b = 254 gives 2^-127).
__device__ __forceinline__ float e8m0_inv(uint32_t b)
{
    return b == 254 ? 0x1p-127f : as_f((254u - b) << 23);
}

// Shared scale byte of an MX block with E4M3 elements (largest exponent 8):
// floor(log2 amax) - 8 + 127, clamped below at 0 (the top clamp at 254 is
// unreachable from a finite binary32 amax); 127 for an all-zero block.
__device__ __forceinline__ uint32_t e8m0_mx8_byte(float amax)
{
    const uint32_t e = as_u(amax) >> 23;   // amax >= 0
    if (amax == 0.0f) return 127;
    return e >= 8 ? e - 8 : 0;
}

// Shared scale byte of an MX block with E2M1 elements:
// floor(log2 amax) - 2 + 127, clamped to [0, 254]; 127 for an all-zero
// block.  floor(log2) of a normal binary32 is its exponent field - 127;
// subnormal amax gives byte 0.
__device__ __forceinline__ uint32_t e8m0_mx_byte(float amax)
{
    uint32_t e = as_u(amax) >> 23;         // amax >= 0
    if (amax == 0.0f) return 127;
    return e >= 2 ? e - 2 : 0;
}

}  // namespace tq
