// tq_f64.hip -- integer-code quantization of binary64 inputs (docs.rs
// baracuda_kernels::quantize overview: f64 among the input types), computed
// in binary64 throughout: scales are binary64, every division, product and
// rounding is a binary64 operation, dequantized values and gradients are
// binary64.
//
//   symmetric : scale = amax / qmax;   asymmetric: mn = min(min x, 0),
//               mx = max(max x, 0), scale = (mx - mn) / (qmax - qmin),
//               zp = clamp(qmin - rne(mn / scale), qmin, qmax);  0 -> 1
//   q  = clamp(rne(x / scale) + zp, qmin, qmax)
//   y  = (q - zp) * scale;   dx = (dy / scale) * 1[qmin < q < qmax];   dq = dy * scale
//
// The divisions are the compiler's correctly rounded binary64 division
// (v_div_scale / v_rcp / FMA refinement / v_div_fmas / v_div_fixup); the
// path stays bound by the 8-byte element stream.
//
// Kernels:
//   k_f64_group_params  one workgroup per group: max / min over the group
//                       (any layout, through the group map), then scale/zp.
//   k_f64_partial + k_f64_finalize   per-tensor: chunk partials, then one
//                       workgroup publishes scale / zp.
//   k_f64_encode / k_f64_ew   two elements per thread (one code byte for
//                       4-bit codes): quantize, dequantize, STE backward,
//                       dequantize backward.
#include "tq_device.h"
#include "tq_host.h"

namespace tq {

// Group index of an element.  Groups along the last axis (inner = 1: per
// token, per group along the last axis, per channel of the last axis) need a
// single division, e / g or e % A; below 2^32 elements it is a multiply-high
// by a host-computed magic number (Granlund and Montgomery's round-up method,
// exact for every 32-bit dividend) instead of the general map's 64-bit
// divisions, which cost more than the whole binary64 encode.
struct FMap {
    DMap m;
    int mode;                 // 0: general map, 1: one group, 2: e / d, 3: e % d
    uint32_t d, mul, sh;      // divisor, magic multiplier, shift (d == 1: identity)

    __device__ __forceinline__ uint32_t div(uint32_t n) const
    {
        if (d == 1) return n;
        const uint32_t t = __umulhi(mul, n);
        return (t + ((n - t) >> 1)) >> sh;
    }
    __device__ __forceinline__ int64_t group_of(int64_t e) const
    {
        switch (mode) {
        case 1: return 0;
        case 2: return div((uint32_t)e);
        case 3: return (uint32_t)e - div((uint32_t)e) * d;
        default: return m.group_of(e);
        }
    }
    // element j of group gid
    __device__ __forceinline__ int64_t elem(int64_t gid, int64_t j) const
    {
        switch (mode) {
        case 2: return gid * (int64_t)d + j;
        case 3: return j * (int64_t)d + gid;
        default: return m.elem(gid, j);
        }
    }
};

static FMap to_fmap(const GroupMap& gm)
{
    FMap f;
    f.m = to_dmap(gm);
    f.mode = 0;
    f.d = 1;
    f.mul = 0;
    f.sh = 0;
    if (gm.kind == KIND_TENSOR) {
        f.mode = 1;
        return f;
    }
    const int64_t dv = gm.kind == KIND_CHANNEL ? gm.A : gm.g;
    if (gm.inner != 1 || gm.numel > 0xffffffffLL || dv < 1 || dv > 0xffffffffLL) return f;
    f.mode = gm.kind == KIND_CHANNEL ? 3 : 2;
    f.d = (uint32_t)dv;
    if (f.d > 1) {
        int l = 0;
        while (((uint64_t)1 << l) < f.d) ++l;                      // ceil(log2 d)
        f.mul = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - f.d)) / f.d + 1);
        f.sh = (uint32_t)(l - 1);
    }
    return f;
}

__device__ __forceinline__ double dmax_team64(double v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ double dmin_team64(double v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmin(v, __shfl_xor(v, o, 64));
    return v;
}

// Block (256 threads) max of mx and min of mn; every thread gets the result.
__device__ __forceinline__ void dblock_minmax(double& mn, double& mx)
{
    __shared__ double smn[4], smx[4];
    mn = dmin_team64(mn);
    mx = dmax_team64(mx);
    if ((threadIdx.x & 63) == 0) {
        smn[threadIdx.x >> 6] = mn;
        smx[threadIdx.x >> 6] = mx;
    }
    __syncthreads();
    mn = fmin(fmin(smn[0], smn[1]), fmin(smn[2], smn[3]));
    mx = fmax(fmax(smx[0], smx[1]), fmax(smx[2], smx[3]));
}

// Scale and zero-point of one group from its max |x| (symmetric: mx holds
// it) or its min / max (asymmetric; both already include 0).
__device__ __forceinline__ void f64_params(bool sym, double mn, double mx, double qmin, double qmax, double* s_out,
                                           int* zp_out)
{
    double s = sym ? mx / qmax : (mx - mn) / (qmax - qmin);
    s = (s == 0.0) ? 1.0 : s;
    *s_out = s;
    if (sym) {
        *zp_out = 0;
    } else {
        const double z = qmin - __builtin_rint(mn / s);
        *zp_out = (int)fmin(fmax(z, qmin), qmax);
    }
}

__global__ __launch_bounds__(256) void k_f64_group_params(const double* __restrict__ x, FMap m, int sym,
                                                          double qmin, double qmax, double* __restrict__ scale,
                                                          uint8_t* __restrict__ zp)
{
    const int64_t gid = blockIdx.x;
    const int64_t n = m.m.count();
    double mn = 0.0, mx = 0.0;
    auto take = [&](double v) {
        if (sym) {
            mx = fmax(mx, fabs(v));
        } else {
            mn = fmin(mn, v);
            mx = fmax(mx, v);
        }
    };
    const double* base = x + gid * (int64_t)m.d;
    if (m.mode == 2 && (m.d & 1) == 0 && ((uintptr_t)base & 15) == 0) {
        // a contiguous group of even length: 16-byte loads
        for (int64_t j = threadIdx.x; 2 * j < n; j += 256) {
            const double2 v = reinterpret_cast<const double2*>(base)[j];
            take(v.x);
            take(v.y);
        }
    } else {
        for (int64_t j = threadIdx.x; j < n; j += 256) take(x[m.elem(gid, j)]);
    }
    dblock_minmax(mn, mx);
    if (threadIdx.x == 0) {
        double s;
        int z;
        f64_params(sym, mn, mx, qmin, qmax, &s, &z);
        scale[gid] = s;
        if (!sym) zp[gid] = (uint8_t)z;
    }
}

// Per-tensor pass 1: chunk maxima of |x| (or of x and -x) into ws.
__global__ __launch_bounds__(256) void k_f64_partial(const double* __restrict__ x, int64_t numel, int64_t chunk,
                                                     int sym, double* __restrict__ ws)
{
    const int64_t b0 = (int64_t)blockIdx.x * chunk;
    const int64_t b1 = b0 + chunk < numel ? b0 + chunk : numel;
    double mn = 0.0, mx = 0.0;
    for (int64_t e = b0 + threadIdx.x; e < b1; e += 256) {
        const double v = x[e];
        if (sym) {
            mx = fmax(mx, fabs(v));
        } else {
            mn = fmin(mn, v);
            mx = fmax(mx, v);
        }
    }
    dblock_minmax(mn, mx);
    if (threadIdx.x == 0) {
        ws[blockIdx.x] = mx;
        ws[gridDim.x + blockIdx.x] = mn;
    }
}

__global__ __launch_bounds__(256) void k_f64_finalize(const double* __restrict__ ws, int nblk, int sym, double qmin,
                                                      double qmax, double* __restrict__ scale,
                                                      uint8_t* __restrict__ zp)
{
    double mn = 0.0, mx = 0.0;
    for (int k = threadIdx.x; k < nblk; k += 256) {
        mx = fmax(mx, ws[k]);
        mn = fmin(mn, ws[nblk + k]);
    }
    dblock_minmax(mn, mx);
    if (threadIdx.x == 0) {
        double s;
        int z;
        f64_params(sym, mn, mx, qmin, qmax, &s, &z);
        scale[0] = s;
        if (!sym) zp[0] = (uint8_t)z;
    }
}

__device__ __forceinline__ double f64_zp(const uint8_t* zp, int64_t g, bool zs)
{
    if (!zp) return 0.0;
    return zs ? (double)(int8_t)zp[g] : (double)zp[g];
}

// clamp(rne(x / s) + zp, qmin, qmax)
__device__ __forceinline__ int f64_code(double x, double s, double z, double qmin, double qmax)
{
    return (int)fmin(fmax(__builtin_rint(x / s) + z, qmin), qmax);
}

// x / s correctly rounded from y = RN(1/s) by two FMA corrections of x * y
// (Markstein's theorem: with y within half an ulp of 1/s, one correction
// step turns a quotient within one ulp into the correctly rounded one; the
// first step makes x * y such a quotient).  Five binary64 operations instead
// of the IEEE sequence's ten, one of them a quarter-rate reciprocal.  Exact
// while the intermediates stay normal, which f64_fast_scale and f64_fast_x
// guarantee; for |x| < 2^-500 the quotient is below 2^-100 in magnitude and
// rounds to a zero code on either path.
__device__ __forceinline__ double f64_quot(double x, double s, double y)
{
    const double q0 = x * y;
    const double q1 = __builtin_fma(-__builtin_fma(s, q0, -x), y, q0);
    return __builtin_fma(-__builtin_fma(s, q1, -x), y, q1);
}

__device__ __forceinline__ bool f64_fast_scale(double s)
{
    const double a = fabs(s);
    return a >= 0x1p-400 && a <= 0x1p400;
}

// Quotients of |x| <= 2^600 by a fast scale stay below 2^1000.
__device__ __forceinline__ bool f64_fast_x(double x)
{
    return fabs(x) <= 0x1p600;
}

__device__ __forceinline__ int f64_code_y(double x, double s, double y, double z, double qmin, double qmax)
{
    return (int)fmin(fmax(__builtin_rint(f64_quot(x, s, y)) + z, qmin), qmax);
}

// Thread t handles elements 2t and 2t+1 (a code byte for 4-bit codes).
template <int BITS>
__global__ __launch_bounds__(256) void k_f64_encode(const double* __restrict__ x, FMap m, double qmin, double qmax,
                                                    const double* __restrict__ scale, const uint8_t* __restrict__ zp,
                                                    bool zs, uint8_t* __restrict__ q)
{
    const int64_t npair = (m.m.numel + 1) / 2;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < npair; t += (int64_t)gridDim.x * 256) {
        int c[2] = {0, 0};
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int64_t e = 2 * t + k;
            if (e < m.m.numel) {
                const int64_t g = m.group_of(e);
                c[k] = f64_code(x[e], scale[g], f64_zp(zp, g, zs), qmin, qmax);
            }
        }
        if (BITS == 4) {
            q[t] = (uint8_t)((c[0] & 0xf) | ((c[1] & 0xf) << 4));
        } else {
            q[2 * t] = (uint8_t)c[0];
            if (2 * t + 1 < m.m.numel) q[2 * t + 1] = (uint8_t)c[1];
        }
    }
}

// Pair-interleaved: a wave-iteration covers 256 element pairs (512
// elements); lane l takes pairs 64 k + l (k < 4), so each 16-byte access
// instruction of the wave covers 1 KB of consecutive pairs.  Needs an even
// element count and 16-byte aligned binary64 buffers.  SAMEG: the 512 share
// a group (one tensor, or groups along the last axis whose length is a
// multiple of 512), so the group index, scale and zero-point are read once.
template <int BITS, bool SAMEG>
__global__ __launch_bounds__(256) void k_f64_encode8(const double* __restrict__ x, FMap m, double qmin, double qmax,
                                                     const double* __restrict__ scale, const uint8_t* __restrict__ zp,
                                                     bool zs, uint8_t* __restrict__ q)
{
    const int64_t npair = m.m.numel / 2;
    const int lane = threadIdx.x & 63;
    const int64_t nwave = (int64_t)gridDim.x * 4;
    for (int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); wv * 256 < npair; wv += nwave) {
        const int64_t p0 = wv * 256 + lane;
        double2 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (p0 + 64 * k < npair) v[k] = reinterpret_cast<const double2*>(x)[p0 + 64 * k];
        double sc = 0.0, z = 0.0, y = 0.0;
        bool fast = false;
        if constexpr (SAMEG) {
            const int64_t g = m.group_of(wv * 512);
            sc = scale[g];
            z = f64_zp(zp, g, zs);
            fast = f64_fast_scale(sc);
            y = 1.0 / sc;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t p = p0 + 64 * k;
            if (p >= npair) break;
            int c0, c1;
            if constexpr (SAMEG) {
                if (fast && f64_fast_x(v[k].x) && f64_fast_x(v[k].y)) {
                    c0 = f64_code_y(v[k].x, sc, y, z, qmin, qmax);
                    c1 = f64_code_y(v[k].y, sc, y, z, qmin, qmax);
                } else {
                    c0 = f64_code(v[k].x, sc, z, qmin, qmax);
                    c1 = f64_code(v[k].y, sc, z, qmin, qmax);
                }
            } else {
                const int64_t g0 = m.group_of(2 * p), g1 = m.group_of(2 * p + 1);
                c0 = f64_code(v[k].x, scale[g0], f64_zp(zp, g0, zs), qmin, qmax);
                c1 = f64_code(v[k].y, scale[g1], f64_zp(zp, g1, zs), qmin, qmax);
            }
            if constexpr (BITS == 4) q[p] = (uint8_t)((c0 & 0xf) | ((c1 & 0xf) << 4));
            else reinterpret_cast<uint16_t*>(q)[p] = (uint16_t)((c0 & 0xff) | ((c1 & 0xff) << 8));
        }
    }
}

// One pass for contiguous groups of even length L <= 2 * V * NT: a workgroup
// of NT threads per group holds it in registers (V pairs per thread,
// non-temporal 16-byte loads, every wave instruction reading 1 KB
// contiguously), reduces its max / min, derives scale and zero-point (every
// thread computes the same values; thread 0 stores them) and encodes from the
// registers.  Measured on rows of 4096: V = 4 (512 threads) beats V = 8 (256)
// by 5% and V = 2 (1024) by 35%.
template <int BITS, int NT, int V>
__global__ __launch_bounds__(NT) void k_f64_rows(const double* __restrict__ x, int64_t L, int sym, double qmin,
                                                 double qmax, double* __restrict__ scale, uint8_t* __restrict__ zp,
                                                 uint8_t* __restrict__ q)
{
    constexpr int NW = NT / 64;
    __shared__ double smn[NW], smx[NW];
    const int64_t g = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t n2 = L / 2;
    const double2* base = reinterpret_cast<const double2*>(x + g * L);
    // every load is issued before the first max (taking each pair's max in
    // the load loop kept one load in flight at a time: 13% slower)
    double2 v[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int64_t j = t + NT * i;
        v[i] = make_double2(0.0, 0.0);
        if (j < n2) {
            const uint4 w = ld16<true>(base + j);
            v[i] = make_double2(__builtin_bit_cast(double, ((uint64_t)w.y << 32) | w.x),
                                __builtin_bit_cast(double, ((uint64_t)w.w << 32) | w.z));
        }
    }
    double mn = 0.0, mx = 0.0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        if (sym) {
            mx = fmax(mx, fmax(fabs(v[i].x), fabs(v[i].y)));
        } else {
            mn = fmin(mn, fmin(v[i].x, v[i].y));
            mx = fmax(mx, fmax(v[i].x, v[i].y));
        }
    }
    mn = dmin_team64(mn);
    mx = dmax_team64(mx);
    if ((t & 63) == 0) {
        smn[t >> 6] = mn;
        smx[t >> 6] = mx;
    }
    __syncthreads();
    mn = smn[0];
    mx = smx[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) {
        mn = fmin(mn, smn[k]);
        mx = fmax(mx, smx[k]);
    }
    double s;
    int zi;
    f64_params(sym, mn, mx, qmin, qmax, &s, &zi);
    if (t == 0) {
        scale[g] = s;
        if (!sym) zp[g] = (uint8_t)zi;
    }
    const double z = sym ? 0.0 : (double)zi;
    // Every element of the group has |x / s| <= qmax - qmin + 1, so only the
    // scale decides between the fast quotient and IEEE division.
    const bool fast = f64_fast_scale(s);
    const double y = 1.0 / s;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int64_t j = t + NT * i;
        if (j >= n2) break;
        int c0, c1;
        if (fast) {
            c0 = f64_code_y(v[i].x, s, y, z, qmin, qmax);
            c1 = f64_code_y(v[i].y, s, y, z, qmin, qmax);
        } else {
            c0 = f64_code(v[i].x, s, z, qmin, qmax);
            c1 = f64_code(v[i].y, s, z, qmin, qmax);
        }
        if constexpr (BITS == 4) q[g * n2 + j] = (uint8_t)((c0 & 0xf) | ((c1 & 0xf) << 4));
        else reinterpret_cast<uint16_t*>(q + g * L)[j] = (uint16_t)((c0 & 0xff) | ((c1 & 0xff) << 8));
    }
}

constexpr int F64_ROW_V = 4;
// Smallest workgroup (64..1024 threads, F64_ROW_V pairs each) that holds a
// group of L elements.
template <int BITS>
static void launch_f64_rows(const double* x, int64_t L, int64_t ngroups, bool sym, double qmin, double qmax,
                            double* scale, uint8_t* zp, uint8_t* q, hipStream_t st)
{
    constexpr int V = F64_ROW_V;
    const int64_t n2 = L / 2;
    const dim3 grid((unsigned)ngroups);
    if (n2 <= 64 * V)
        hipLaunchKernelGGL((k_f64_rows<BITS, 64, V>), grid, dim3(64), 0, st, x, L, (int)sym, qmin, qmax, scale, zp, q);
    else if (n2 <= 128 * V)
        hipLaunchKernelGGL((k_f64_rows<BITS, 128, V>), grid, dim3(128), 0, st, x, L, (int)sym, qmin, qmax, scale, zp, q);
    else if (n2 <= 256 * V)
        hipLaunchKernelGGL((k_f64_rows<BITS, 256, V>), grid, dim3(256), 0, st, x, L, (int)sym, qmin, qmax, scale, zp, q);
    else if (n2 <= 512 * V)
        hipLaunchKernelGGL((k_f64_rows<BITS, 512, V>), grid, dim3(512), 0, st, x, L, (int)sym, qmin, qmax, scale, zp, q);
    else
        hipLaunchKernelGGL((k_f64_rows<BITS, 1024, V>), grid, dim3(1024), 0, st, x, L, (int)sym, qmin, qmax, scale, zp, q);
}

enum { F64_DEQ = 0, F64_STE = 1, F64_DQB = 2 };

template <int OP, int BITS, bool SIGNED>
__global__ __launch_bounds__(256) void k_f64_ew(const void* __restrict__ a, const double* __restrict__ b, FMap m,
                                                double qmin, double qmax, const double* __restrict__ scale,
                                                const uint8_t* __restrict__ zp, double* __restrict__ out)
{
    const int64_t npair = (m.m.numel + 1) / 2;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < npair; t += (int64_t)gridDim.x * 256) {
        uint32_t qb = 0;
        if (OP == F64_DEQ && BITS == 4) qb = static_cast<const uint8_t*>(a)[t];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int64_t e = 2 * t + k;
            if (e >= m.m.numel) break;
            const int64_t g = m.group_of(e);
            const double s = scale[g];
            if constexpr (OP == F64_DEQ) {
                uint32_t c = BITS == 4 ? ((qb >> (4 * k)) & 0xfu) : static_cast<const uint8_t*>(a)[e];
                int v = (int)c;
                if (SIGNED) v = BITS == 4 ? (int)((c ^ 8u) - 8u) : (int)(int8_t)c;
                out[e] = ((double)v - f64_zp(zp, g, SIGNED)) * s;
            } else if constexpr (OP == F64_DQB) {
                out[e] = static_cast<const double*>(a)[e] * s;
            } else {
                const int c = f64_code(static_cast<const double*>(a)[e], s, f64_zp(zp, g, SIGNED), qmin, qmax);
                out[e] = (b[e] / s) * ((qmin < c && c < qmax) ? 1.0 : 0.0);
            }
        }
    }
}

// Pair-interleaved as k_f64_encode8; binary64 outputs leave by non-temporal
// 16-byte stores (whole lines per wave instruction).
template <int OP, int BITS, bool SIGNED, bool SAMEG>
__global__ __launch_bounds__(256) void k_f64_ew8(const void* __restrict__ a, const double* __restrict__ b, FMap m,
                                                 double qmin, double qmax, const double* __restrict__ scale,
                                                 const uint8_t* __restrict__ zp, double* __restrict__ out)
{
    const int64_t npair = m.m.numel / 2;
    const int lane = threadIdx.x & 63;
    const int64_t nwave = (int64_t)gridDim.x * 4;
    for (int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); wv * 256 < npair; wv += nwave) {
        const int64_t p0 = wv * 256 + lane;
        double2 va[4], vb[4];
        uint32_t cw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t p = p0 + 64 * k;
            if (p >= npair) break;
            if constexpr (OP == F64_DEQ) {
                cw[k] = BITS == 4 ? (uint32_t) static_cast<const uint8_t*>(a)[p]
                                  : (uint32_t) reinterpret_cast<const uint16_t*>(a)[p];
            } else {
                va[k] = reinterpret_cast<const double2*>(a)[p];
                if constexpr (OP == F64_STE) vb[k] = reinterpret_cast<const double2*>(b)[p];
            }
        }
        double s1 = 0.0, z1 = 0.0;
        if constexpr (SAMEG) {
            const int64_t g = m.group_of(wv * 512);
            s1 = scale[g];
            z1 = f64_zp(zp, g, SIGNED);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t p = p0 + 64 * k;
            if (p >= npair) break;
            double s[2], z[2];
            if constexpr (SAMEG) {
                s[0] = s[1] = s1;
                z[0] = z[1] = z1;
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int64_t g = m.group_of(2 * p + h);
                    s[h] = scale[g];
                    z[h] = f64_zp(zp, g, SIGNED);
                }
            }
            double o[2];
            if constexpr (OP == F64_DEQ) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t c = BITS == 4 ? (cw[k] >> (4 * h)) & 0xfu : (cw[k] >> (8 * h)) & 0xffu;
                    int v = (int)c;
                    if (SIGNED) v = BITS == 4 ? (int)((c ^ 8u) - 8u) : (int)(int8_t)c;
                    o[h] = ((double)v - z[h]) * s[h];
                }
            } else if constexpr (OP == F64_DQB) {
                o[0] = va[k].x * s[0];
                o[1] = va[k].y * s[1];
            } else {
                const double xa[2] = {va[k].x, va[k].y}, ya[2] = {vb[k].x, vb[k].y};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int c = f64_code(xa[h], s[h], z[h], qmin, qmax);
                    o[h] = (ya[h] / s[h]) * ((qmin < c && c < qmax) ? 1.0 : 0.0);
                }
            }
            const uint64_t b0 = __builtin_bit_cast(uint64_t, o[0]), b1 = __builtin_bit_cast(uint64_t, o[1]);
            st16<OP == F64_DEQ ? WT : 1>(out + 2 * p,
                                         make_uint4((uint32_t)b0, (uint32_t)(b0 >> 32), (uint32_t)b1, (uint32_t)(b1 >> 32)));
        }
    }
}


static bool al(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// The pair-interleaved kernels need an even element count and aligned
// buffers; their SAMEG form needs each wave-iteration's 512 elements inside
// one group.
static bool same_group8(const FMap& d) { return d.mode == 1 || (d.mode == 2 && d.d % 512 == 0); }

template <int BITS>
static void launch_encode(const double* x, const FMap& d, double qmin, double qmax, const double* scale,
                          const uint8_t* zb, bool zs, uint8_t* q, hipStream_t st)
{
    const bool vec = d.m.numel % 2 == 0 && al(x, 16) && (BITS == 4 || al(q, 2));
    if (vec) {
        const dim3 grid(grid_for(d.m.numel / 2, 1024));
        if (same_group8(d))
            hipLaunchKernelGGL((k_f64_encode8<BITS, true>), grid, dim3(256), 0, st, x, d, qmin, qmax, scale, zb, zs, q);
        else
            hipLaunchKernelGGL((k_f64_encode8<BITS, false>), grid, dim3(256), 0, st, x, d, qmin, qmax, scale, zb, zs, q);
        return;
    }
    const dim3 grid(grid_for((d.m.numel + 1) / 2, 256));
    hipLaunchKernelGGL(k_f64_encode<BITS>, grid, dim3(256), 0, st, x, d, qmin, qmax, scale, zb, zs, q);
}

template <int OP, int BITS, bool SIGNED>
static void launch_ew(const void* a, const double* b, const FMap& d, double qmin, double qmax, const double* scale,
                      const uint8_t* zb, double* out, hipStream_t st)
{
    const uintptr_t aa = OP == F64_DEQ ? (BITS == 4 ? 1 : 2) : 16;
    const bool vec = d.m.numel % 2 == 0 && al(a, aa) && (!b || al(b, 16)) && al(out, 16);
    if (vec) {
        const dim3 grid(grid_for(d.m.numel / 2, 1024));
        if (same_group8(d))
            hipLaunchKernelGGL((k_f64_ew8<OP, BITS, SIGNED, true>), grid, dim3(256), 0, st, a, b, d, qmin, qmax, scale, zb,
                               out);
        else
            hipLaunchKernelGGL((k_f64_ew8<OP, BITS, SIGNED, false>), grid, dim3(256), 0, st, a, b, d, qmin, qmax, scale,
                               zb, out);
        return;
    }
    const dim3 grid(grid_for((d.m.numel + 1) / 2, 256));
    hipLaunchKernelGGL((k_f64_ew<OP, BITS, SIGNED>), grid, dim3(256), 0, st, a, b, d, qmin, qmax, scale, zb, out);
}

// Group layout of a call; false for a bad granularity / shape.
static bool f64_map(int32_t ndim, const int64_t* shape, int gran, int32_t axis, int64_t group_size, GroupMap* m)
{
    if (ndim < 1 || ndim > 8 || !shape) return false;
    int64_t numel = 1;
    for (int d = 0; d < ndim; ++d) {
        if (shape[d] < 0) return false;
        numel *= shape[d];
    }
    switch (gran) {
    case TQ_GRAN_TENSOR: *m = tensor_map(numel); return true;
    case TQ_GRAN_TOKEN: {
        const int64_t cols = shape[ndim - 1];
        if (numel > 0 && cols == 0) return false;
        *m = token_map(cols ? numel / cols : 0, cols);
        return true;
    }
    case TQ_GRAN_CHANNEL: return make_map(KIND_CHANNEL, ndim, shape, axis, 1, m);
    case TQ_GRAN_GROUP: return make_map(KIND_GROUP, ndim, shape, axis, group_size, m);
    default: return false;
    }
}

}  // namespace tq

using namespace tq;

extern "C" {

tq_status tq_quant_f64(const double* x, int32_t ndim, const int64_t* host_shape, int gran, int32_t axis,
                       int64_t group_size, int code, int32_t qmin, int32_t qmax, int static_scale, void* q,
                       double* scale, void* zero_point, void* workspace, size_t workspace_bytes, void* stream)
{
    GroupMap m;
    if (!f64_map(ndim, host_shape, gran, axis, group_size, &m)) return TQ_ERR_INVALID;
    const bool sym = zero_point == nullptr;
    if (!valid_range(code, qmin, qmax, sym)) return TQ_ERR_INVALID;
    if (code_bits(code) == 4 && (host_shape[ndim - 1] & 1)) return TQ_ERR_INVALID;
    if (m.numel == 0) return TQ_OK;
    if (!x || !q || !scale) return TQ_ERR_INVALID;
    hipStream_t st = as_stream(stream);
    const double dmin = qmin, dmax = qmax;
    uint8_t* zb = static_cast<uint8_t*>(zero_point);
    const FMap d = to_fmap(m);
    if (!static_scale && d.mode == 2 && d.d % 2 == 0 && d.d <= 2 * 1024 * F64_ROW_V && al(x, 16) && al(q, 2) &&
        m.ngroups <= 0x7fffffff) {
        // contiguous groups that fit a workgroup's registers: one pass
        uint8_t* qb = static_cast<uint8_t*>(q);
        if (code_bits(code) == 4) launch_f64_rows<4>(x, (int64_t)d.d, m.ngroups, sym, dmin, dmax, scale, zb, qb, st);
        else launch_f64_rows<8>(x, (int64_t)d.d, m.ngroups, sym, dmin, dmax, scale, zb, qb, st);
        return launch_status();
    }
    if (!static_scale) {
        if (m.kind == KIND_TENSOR) {
            if (!workspace || workspace_bytes < tq_workspace_bytes(3, m.numel)) return TQ_ERR_INVALID;
            const int64_t chunk = std::max<int64_t>(256 * 16, cdiv(m.numel, 1024));
            const int nblk = (int)cdiv(m.numel, chunk);
            double* ws = static_cast<double*>(workspace);
            hipLaunchKernelGGL(k_f64_partial, dim3(nblk), dim3(256), 0, st, x, m.numel, chunk, (int)sym, ws);
            hipLaunchKernelGGL(k_f64_finalize, dim3(1), dim3(256), 0, st, ws, nblk, (int)sym, dmin, dmax, scale, zb);
        } else {
            if (m.ngroups > 0x7fffffff) return TQ_ERR_UNSUPPORTED;
            hipLaunchKernelGGL(k_f64_group_params, dim3((unsigned)m.ngroups), dim3(256), 0, st, x, d, (int)sym, dmin,
                               dmax, scale, zb);
        }
        if (launch_status()) return TQ_ERR_HIP;
    }
    uint8_t* qb = static_cast<uint8_t*>(q);
    if (code_bits(code) == 4) launch_encode<4>(x, d, dmin, dmax, scale, zb, code_signed(code), qb, st);
    else launch_encode<8>(x, d, dmin, dmax, scale, zb, code_signed(code), qb, st);
    return launch_status();
}

tq_status tq_dequant_f64(const void* q, int code, int32_t ndim, const int64_t* host_shape, int gran, int32_t axis,
                         int64_t group_size, const double* scale, const void* zero_point, double* y, void* stream)
{
    GroupMap m;
    if (!f64_map(ndim, host_shape, gran, axis, group_size, &m) || !valid_code(code)) return TQ_ERR_INVALID;
    if (code_bits(code) == 4 && (host_shape[ndim - 1] & 1)) return TQ_ERR_INVALID;
    if (m.numel == 0) return TQ_OK;
    if (!q || !scale || !y) return TQ_ERR_INVALID;
    const FMap d = to_fmap(m);
    const uint8_t* zb = static_cast<const uint8_t*>(zero_point);
    hipStream_t st = as_stream(stream);
    const bool sg = code_signed(code);
    if (code_bits(code) == 4) {
        if (sg) launch_ew<F64_DEQ, 4, true>(q, nullptr, d, 0.0, 0.0, scale, zb, y, st);
        else launch_ew<F64_DEQ, 4, false>(q, nullptr, d, 0.0, 0.0, scale, zb, y, st);
    } else {
        if (sg) launch_ew<F64_DEQ, 8, true>(q, nullptr, d, 0.0, 0.0, scale, zb, y, st);
        else launch_ew<F64_DEQ, 8, false>(q, nullptr, d, 0.0, 0.0, scale, zb, y, st);
    }
    return launch_status();
}

tq_status tq_quant_f64_backward(const double* x, int32_t ndim, const int64_t* host_shape, int gran, int32_t axis,
                                int64_t group_size, int code, int32_t qmin, int32_t qmax, const double* scale,
                                const void* zero_point, const double* dy, double* dx, void* stream)
{
    GroupMap m;
    if (!f64_map(ndim, host_shape, gran, axis, group_size, &m)) return TQ_ERR_INVALID;
    if (!valid_range(code, qmin, qmax, zero_point == nullptr)) return TQ_ERR_INVALID;
    if (m.numel == 0) return TQ_OK;
    if (!x || !scale || !dy || !dx) return TQ_ERR_INVALID;
    const FMap d = to_fmap(m);
    const uint8_t* zb = static_cast<const uint8_t*>(zero_point);
    hipStream_t st = as_stream(stream);
    if (code_signed(code)) launch_ew<F64_STE, 8, true>(x, dy, d, (double)qmin, (double)qmax, scale, zb, dx, st);
    else launch_ew<F64_STE, 8, false>(x, dy, d, (double)qmin, (double)qmax, scale, zb, dx, st);
    return launch_status();
}

tq_status tq_dequant_f64_backward(const double* dy, int32_t ndim, const int64_t* host_shape, int gran, int32_t axis,
                                  int64_t group_size, const double* scale, double* dq, void* stream)
{
    GroupMap m;
    if (!f64_map(ndim, host_shape, gran, axis, group_size, &m)) return TQ_ERR_INVALID;
    if (m.numel == 0) return TQ_OK;
    if (!dy || !scale || !dq) return TQ_ERR_INVALID;
    const FMap d = to_fmap(m);
    launch_ew<F64_DQB, 8, false>(dy, nullptr, d, 0.0, 0.0, scale, nullptr, dq, as_stream(stream));
    return launch_status();
}

}  // extern "C"
