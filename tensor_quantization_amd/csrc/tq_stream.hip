// tq_stream.hip -- the streaming ceiling: a kernel that moves bytes in the
// same read : write mix, per-lane widths and store policies as the
// quantization kernels, with no arithmetic beyond folding the loaded words
// into the stored ones.  Measured beside the real kernels, it gives the rate
// the chip reaches for that access pattern at that size, so a kernel's gap
// to the HBM peak splits into what any stream of that shape loses and what
// the kernel's own work adds.
//
// Unit t reads `in` bytes and writes `out` bytes (a lane handles 1, 2 or 4
// units, all loads before all stores):
//   in  = 4, 8, 16: one load at src + t * in
//   in  = 32:       two 16-byte loads, at src + 16 t and src + 16 (n + t)
//                   (two input streams, like x and dy of the STE backward)
//   out = 4, 8, 16: one store at dst + t * out
//   out = 32:       two 16-byte stores at dst + 32 t and dst + 32 t + 16
// Loads of 16 bytes are non-temporal (whole lines per wave instruction);
// stores follow `policy`: 0 plain, 1 non-temporal, 2 non-temporal with
// device scope (16-byte stores only).
#include "tq_device.h"
#include "tq_host.h"

namespace tq {

__device__ __forceinline__ uint32_t fold4(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

template <int IN, int OUT, int POL>
__device__ __forceinline__ void mix_unit(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t n,
                                         int64_t t)
{
    uint4 a;
    if constexpr (IN == 4) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(src + t * 4);
        a = make_uint4(w, w + 1, w + 2, w + 3);
    } else if constexpr (IN == 8) {
        const uint2 w = ld8<false>(src + t * 8);
        a = make_uint4(w.x, w.y, w.x ^ w.y, w.x + w.y);
    } else if constexpr (IN == 16) {
        a = ld16<true>(src + t * 16);
    } else {
        const uint4 u = ld16<true>(src + t * 16);
        const uint4 v = ld16<true>(src + (n + t) * 16);
        a = make_uint4(u.x ^ v.x, u.y ^ v.y, u.z ^ v.z, u.w ^ v.w);
    }
    if constexpr (OUT == 4) {
        const uint32_t w = fold4(a);
        if constexpr (POL) __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(dst + t * 4));
        else *reinterpret_cast<uint32_t*>(dst + t * 4) = w;
    } else if constexpr (OUT == 8) {
        st8<(POL != 0)>(dst + t * 8, make_uint2(a.x ^ a.z, a.y ^ a.w));
    } else if constexpr (OUT == 16) {
        st16<POL>(dst + t * 16, a);
    } else {
        st16<POL>(dst + t * 32, a);
        st16<POL>(dst + t * 32 + 16, make_uint4(a.w, a.z, a.y, a.x));
    }
}

// A workgroup covers V * 256 consecutive units; lane j takes units
// k * 256 + j (k < V), so each wave instruction stays contiguous and a lane
// keeps V loads in flight.
template <int IN, int OUT, int POL, int V>
__global__ __launch_bounds__(256) void k_stream_mix(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                    int64_t n)
{
    const int64_t t0 = (int64_t)blockIdx.x * (256 * V) + threadIdx.x;
    if constexpr (V == 1) {
        if (t0 < n) mix_unit<IN, OUT, POL>(src, dst, n, t0);
    } else {
        // all loads first, then all stores (what the quantizers do); the loads
        // take a clamped index and no branch, so the compiler keeps all V in
        // flight (a load under `if (t < n)` with its transform inside the branch
        // was waited for before the next one was issued)
        uint4 a[V];
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int64_t tk = t0 + (int64_t)k * 256;
            const int64_t t = tk < n ? tk : n - 1;
            {
                if constexpr (IN == 16) a[k] = ld16<true>(src + t * 16);
                else if constexpr (IN == 32) {
                    const uint4 u = ld16<true>(src + t * 16), v = ld16<true>(src + (n + t) * 16);
                    a[k] = make_uint4(u.x ^ v.x, u.y ^ v.y, u.z ^ v.z, u.w ^ v.w);
                } else if constexpr (IN == 8) {
                    const uint2 w = ld8<false>(src + t * 8);
                    a[k] = make_uint4(w.x, w.y, w.x ^ w.y, w.x + w.y);
                } else {
                    const uint32_t w = *reinterpret_cast<const uint32_t*>(src + t * 4);
                    a[k] = make_uint4(w, w + 1, w + 2, w + 3);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int64_t t = t0 + (int64_t)k * 256;
            if (t >= n) continue;
            if constexpr (OUT == 4) {
                const uint32_t w = fold4(a[k]);
                if constexpr (POL) __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(dst + t * 4));
                else *reinterpret_cast<uint32_t*>(dst + t * 4) = w;
            } else if constexpr (OUT == 8) {
                st8<(POL != 0)>(dst + t * 8, make_uint2(a[k].x ^ a[k].z, a[k].y ^ a[k].w));
            } else if constexpr (OUT == 16) {
                st16<POL>(dst + t * 16, a[k]);
            } else {
                st16<POL>(dst + t * 32, a[k]);
                st16<POL>(dst + t * 32 + 16, make_uint4(a[k].w, a[k].z, a[k].y, a[k].x));
            }
        }
    }
}

template <int IN, int OUT, int POL>
static void launch_mix(const void* src, void* dst, int64_t n, int v, hipStream_t st)
{
    const uint8_t* s = static_cast<const uint8_t*>(src);
    uint8_t* d = static_cast<uint8_t*>(dst);
    if (v == 1) hipLaunchKernelGGL((k_stream_mix<IN, OUT, POL, 1>), dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, s, d, n);
    else if (v == 2) hipLaunchKernelGGL((k_stream_mix<IN, OUT, POL, 2>), dim3((unsigned)cdiv(n, 512)), dim3(256), 0, st, s, d, n);
    else hipLaunchKernelGGL((k_stream_mix<IN, OUT, POL, 4>), dim3((unsigned)cdiv(n, 1024)), dim3(256), 0, st, s, d, n);
}

}  // namespace tq

using namespace tq;

extern "C" {

tq_status tq_stream_mix(const void* src, void* dst, int64_t nthreads, int in_bytes, int out_bytes, int policy,
                        int vectors, void* stream)
{
    if (nthreads < 0 || policy < 0 || policy > 2) return TQ_ERR_INVALID;
    if (vectors != 1 && vectors != 2 && vectors != 4) return TQ_ERR_INVALID;
    if (nthreads == 0) return TQ_OK;
    if (!src || !dst) return TQ_ERR_INVALID;
    if (!aligned16(src) || !aligned16(dst)) return TQ_ERR_ALIGN;
    if (cdiv(nthreads, 256) > 0x7fffffff) return TQ_ERR_UNSUPPORTED;
    if (policy == 2 && out_bytes < 16) return TQ_ERR_UNSUPPORTED;
    hipStream_t st = as_stream(stream);
    const int key = in_bytes * 1000 + out_bytes * 10 + policy;
    switch (key) {
#define TQ_MIX(I, O, P) case I * 1000 + O * 10 + P: launch_mix<I, O, P>(src, dst, nthreads, vectors, st); break;
        TQ_MIX(16, 8, 1) TQ_MIX(16, 8, 0)                                   // 8-bit quantize
        TQ_MIX(16, 4, 1) TQ_MIX(16, 4, 0)                                   // 4-bit quantize
        TQ_MIX(8, 16, 2) TQ_MIX(8, 16, 1) TQ_MIX(8, 16, 0)                  // 8-bit dequantize
        TQ_MIX(4, 16, 1) TQ_MIX(4, 16, 2) TQ_MIX(4, 16, 0)                  // 4-bit dequantize
        TQ_MIX(32, 16, 1) TQ_MIX(32, 16, 2) TQ_MIX(32, 16, 0)               // STE backward
        TQ_MIX(16, 16, 2) TQ_MIX(16, 16, 1) TQ_MIX(16, 16, 0)               // copy / dequantize backward
        TQ_MIX(16, 32, 1) TQ_MIX(16, 32, 2)                                 // 1:2 from 16-byte loads
#undef TQ_MIX
    default: return TQ_ERR_UNSUPPORTED;
    }
    return launch_status();
}

}  // extern "C"
