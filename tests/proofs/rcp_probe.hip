// Probe: for every binary32 significand s in [1,2) (times 2^k for a few k), does
// y1 = fma(fma(-s, y0, 1), y0, y0) with y0 = v_rcp_f32(s) equal RN(1/s)?
// Writes one byte per significand and exponent; the host compares with its
// own IEEE division.  Grid: 2^23 threads exactly, out has 4 * 2^23 bytes.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
__global__ void k(float* out) {
    uint32_t m = blockIdx.x * 256u + threadIdx.x;          // < 2^23
    const int ex[4] = {0, -40, 40, 17};
    for (int j = 0; j < 4; ++j) {
        float s = __uint_as_float(((uint32_t)(127 + ex[j]) << 23) | m);
        float y0 = __builtin_amdgcn_rcpf(s);
        float e = __builtin_fmaf(-s, y0, 1.0f);
        float y1 = __builtin_fmaf(e, y0, y0);
        out[(size_t)j * (1u << 23) + m] = y1;
    }
}
int main() {
    const size_t n = (size_t)4 << 23;
    float* d = nullptr;
    if (hipMalloc(&d, n * 4) != hipSuccess) { printf("hipMalloc failed\n"); return 2; }
    hipLaunchKernelGGL(k, dim3((1u << 23) / 256), dim3(256), 0, 0, d);
    float* h = (float*)malloc(n * 4);
    if (hipMemcpy(h, d, n * 4, hipMemcpyDeviceToHost) != hipSuccess) { printf("copy failed\n"); return 2; }
    const int ex[4] = {0, -40, 40, 17};
    long bad[4] = {0, 0, 0, 0};
    for (int j = 0; j < 4; ++j)
        for (uint32_t m = 0; m < (1u << 23); ++m) {
            uint32_t sb = ((uint32_t)(127 + ex[j]) << 23) | m;
            float s; memcpy(&s, &sb, 4);
            volatile float one = 1.0f;
            float want = one / s;
            float got = h[(size_t)j * (1u << 23) + m];
            if (memcmp(&want, &got, 4)) { if (bad[j] < 3) printf("exp %d m=%06x want %a got %a\n", ex[j], m, want, got); bad[j]++; }
        }
    printf("rcp+1 Newton mismatches: exp0 %ld exp-40 %ld exp40 %ld exp17 %ld (of %d each)\n", bad[0], bad[1], bad[2], bad[3], 1 << 23);
    (void)hipFree(d);
    free(h);
    return (bad[0] | bad[1] | bad[2] | bad[3]) ? 1 : 0;
}
