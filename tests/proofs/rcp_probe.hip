// Probe: for every binary32 significand s in [1,2) times 2^k, for every k in
// [-40, 40] (the divisor range of the kernels' fast division), does
// y1 = fma(fma(-s, y0, 1), y0, y0) with y0 = v_rcp_f32(s) equal RN(1/s)?
// One launch per exponent: 2^23 threads exactly, one float each into a
// 2^23-float buffer that the host compares with its own IEEE division.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

__global__ void k(float* out, int ex)
{
    const uint32_t m = blockIdx.x * 256u + threadIdx.x;          // < 2^23
    const float s = __uint_as_float(((uint32_t)(127 + ex) << 23) | m);
    const float y0 = __builtin_amdgcn_rcpf(s);
    const float e = __builtin_fmaf(-s, y0, 1.0f);
    out[m] = __builtin_fmaf(e, y0, y0);
}

int main()
{
    const size_t n = (size_t)1 << 23;
    float* d = nullptr;
    if (hipMalloc(&d, n * 4) != hipSuccess) { printf("hipMalloc failed\n"); return 2; }
    float* h = (float*)malloc(n * 4);
    if (!h) return 2;
    long bad = 0, total = 0;
    int exps = 0;
    for (int ex = -40; ex <= 40; ++ex) {
        hipLaunchKernelGGL(k, dim3((unsigned)(n / 256)), dim3(256), 0, 0, d, ex);
        if (hipMemcpy(h, d, n * 4, hipMemcpyDeviceToHost) != hipSuccess) { printf("copy failed\n"); return 2; }
        for (uint32_t m = 0; m < (1u << 23); ++m) {
            const uint32_t sb = ((uint32_t)(127 + ex) << 23) | m;
            float s;
            memcpy(&s, &sb, 4);
            volatile float one = 1.0f;
            const float want = one / s;
            if (memcmp(&want, &h[m], 4)) {
                if (bad < 5) printf("exp %d m=%06x want %a got %a\n", ex, m, want, h[m]);
                ++bad;
            }
        }
        total += (long)n;
        ++exps;
    }
    printf("rcp+1 Newton over %d exponents (-40..40), %ld divisors: %ld mismatches\n", exps, total, bad);
    (void)hipFree(d);
    free(h);
    return bad ? 1 : 0;
}
