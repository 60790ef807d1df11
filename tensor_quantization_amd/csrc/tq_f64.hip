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

__global__ __launch_bounds__(256) void k_f64_group_params(const double* __restrict__ x, DMap m, int sym,
                                                          double qmin, double qmax, double* __restrict__ scale,
                                                          uint8_t* __restrict__ zp)
{
    const int64_t gid = blockIdx.x;
    const int64_t n = m.count();
    double mn = 0.0, mx = 0.0;
    for (int64_t j = threadIdx.x; j < n; j += 256) {
        const double v = x[m.elem(gid, j)];
        if (sym) {
            mx = fmax(mx, fabs(v));
        } else {
            mn = fmin(mn, v);
            mx = fmax(mx, v);
        }
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

// Thread t handles elements 2t and 2t+1 (a code byte for 4-bit codes).
template <int BITS>
__global__ __launch_bounds__(256) void k_f64_encode(const double* __restrict__ x, DMap m, double qmin, double qmax,
                                                    const double* __restrict__ scale, const uint8_t* __restrict__ zp,
                                                    bool zs, uint8_t* __restrict__ q)
{
    const int64_t npair = (m.numel + 1) / 2;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < npair; t += (int64_t)gridDim.x * 256) {
        int c[2] = {0, 0};
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int64_t e = 2 * t + k;
            if (e < m.numel) {
                const int64_t g = m.group_of(e);
                c[k] = f64_code(x[e], scale[g], f64_zp(zp, g, zs), qmin, qmax);
            }
        }
        if (BITS == 4) {
            q[t] = (uint8_t)((c[0] & 0xf) | ((c[1] & 0xf) << 4));
        } else {
            q[2 * t] = (uint8_t)c[0];
            if (2 * t + 1 < m.numel) q[2 * t + 1] = (uint8_t)c[1];
        }
    }
}

enum { F64_DEQ = 0, F64_STE = 1, F64_DQB = 2 };

template <int OP, int BITS, bool SIGNED>
__global__ __launch_bounds__(256) void k_f64_ew(const void* __restrict__ a, const double* __restrict__ b, DMap m,
                                                double qmin, double qmax, const double* __restrict__ scale,
                                                const uint8_t* __restrict__ zp, double* __restrict__ out)
{
    const int64_t npair = (m.numel + 1) / 2;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < npair; t += (int64_t)gridDim.x * 256) {
        uint32_t qb = 0;
        if (OP == F64_DEQ && BITS == 4) qb = static_cast<const uint8_t*>(a)[t];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int64_t e = 2 * t + k;
            if (e >= m.numel) break;
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

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

static unsigned grid_for(int64_t work, int64_t per_block)
{
    int64_t g = cdiv(work, per_block);
    if (g < 1) g = 1;
    if (g > (1 << 20)) g = 1 << 20;
    return (unsigned)g;
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
    const DMap d = to_dmap(m);
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
    const dim3 grid(grid_for((m.numel + 1) / 2, 256));
    uint8_t* qb = static_cast<uint8_t*>(q);
    if (code_bits(code) == 4)
        hipLaunchKernelGGL(k_f64_encode<4>, grid, dim3(256), 0, st, x, d, dmin, dmax, scale, zb, code_signed(code), qb);
    else
        hipLaunchKernelGGL(k_f64_encode<8>, grid, dim3(256), 0, st, x, d, dmin, dmax, scale, zb, code_signed(code), qb);
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
    const DMap d = to_dmap(m);
    const dim3 grid(grid_for((m.numel + 1) / 2, 256));
    const uint8_t* zb = static_cast<const uint8_t*>(zero_point);
    hipStream_t st = as_stream(stream);
    const bool sg = code_signed(code);
    if (code_bits(code) == 4) {
        if (sg) hipLaunchKernelGGL((k_f64_ew<F64_DEQ, 4, true>), grid, dim3(256), 0, st, q, nullptr, d, 0.0, 0.0, scale, zb, y);
        else hipLaunchKernelGGL((k_f64_ew<F64_DEQ, 4, false>), grid, dim3(256), 0, st, q, nullptr, d, 0.0, 0.0, scale, zb, y);
    } else {
        if (sg) hipLaunchKernelGGL((k_f64_ew<F64_DEQ, 8, true>), grid, dim3(256), 0, st, q, nullptr, d, 0.0, 0.0, scale, zb, y);
        else hipLaunchKernelGGL((k_f64_ew<F64_DEQ, 8, false>), grid, dim3(256), 0, st, q, nullptr, d, 0.0, 0.0, scale, zb, y);
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
    const DMap d = to_dmap(m);
    const dim3 grid(grid_for((m.numel + 1) / 2, 256));
    const uint8_t* zb = static_cast<const uint8_t*>(zero_point);
    hipStream_t st = as_stream(stream);
    if (code_signed(code))
        hipLaunchKernelGGL((k_f64_ew<F64_STE, 8, true>), grid, dim3(256), 0, st, x, dy, d, (double)qmin, (double)qmax,
                           scale, zb, dx);
    else
        hipLaunchKernelGGL((k_f64_ew<F64_STE, 8, false>), grid, dim3(256), 0, st, x, dy, d, (double)qmin, (double)qmax,
                           scale, zb, dx);
    return launch_status();
}

tq_status tq_dequant_f64_backward(const double* dy, int32_t ndim, const int64_t* host_shape, int gran, int32_t axis,
                                  int64_t group_size, const double* scale, double* dq, void* stream)
{
    GroupMap m;
    if (!f64_map(ndim, host_shape, gran, axis, group_size, &m)) return TQ_ERR_INVALID;
    if (m.numel == 0) return TQ_OK;
    if (!dy || !scale || !dq) return TQ_ERR_INVALID;
    const DMap d = to_dmap(m);
    const dim3 grid(grid_for((m.numel + 1) / 2, 256));
    hipLaunchKernelGGL((k_f64_ew<F64_DQB, 8, false>), grid, dim3(256), 0, as_stream(stream), dy, nullptr, d, 0.0, 0.0,
                       scale, nullptr, dq);
    return launch_status();
}

}  // extern "C"
