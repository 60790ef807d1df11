// tq_noalloc.hip -- the FP4 block quantize for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts
// that forbid hipMalloc): tq_quant_fp4_block without a workspace argument.
//
// Its only scratch need is the chunk maxima of a dynamic NVFP4 per-tensor
// scale (at most TENSOR_PARTS floats).  They live in `scratch`, a file-scope
// device array of 4 KiB that each GPU the library runs on holds until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host that name is a stand-in, not a device address): the first call on a
// device looks up that device's address of the array with
// hipGetSymbolAddress, with the device current, and every launch takes that
// pointer.  The first launch of a call writes every partial the second one
// reads, so nothing needs to start at zero; calls that overlap on one GPU
// share the array and race.
#include <mutex>

#include "tq_device.h"
#include "tq_host.h"

namespace tq {

static __device__ __align__(256) float scratch[TENSOR_PARTS];

constexpr int MAX_DEVICES = 64;
static std::mutex scratch_mutex;
static float* scratch_ptr[MAX_DEVICES];

// The device address of `scratch` on `dev`, looked up once per device.
static tq_status scratch_on(int dev, float** out)
{
    if (dev < 0 || dev >= MAX_DEVICES) return TQ_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return TQ_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return TQ_ERR_HIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return TQ_ERR_HIP;
        if (e != hipSuccess || !p) return TQ_ERR_HIP;
        scratch_ptr[dev] = static_cast<float*>(p);
    }
    *out = scratch_ptr[dev];
    return TQ_OK;
}

}  // namespace tq

using namespace tq;

extern "C" {

tq_status tq_quant_fp4_block_noalloc(const void* x, int x_dtype, int64_t rows, int64_t k, int kind, uint8_t* packed,
                                     uint8_t* block_scale, float* global_scale, int static_global, void* stream)
{
    tq_status s = check_fp4_quant(x, x_dtype, rows, k, kind, packed, block_scale, global_scale);
    if (s || rows * k == 0) return s;
    hipStream_t st = as_stream(stream);
    float* ws = nullptr;
    if (kind == TQ_NVFP4 && !static_global) {
        int nparts = 0;
        tensor_chunk(rows * k, &nparts);
        if (nparts > TENSOR_PARTS) return TQ_ERR_UNSUPPORTED;     // more partials than the scratch holds
        int dev = 0;
        if (hipStreamGetDevice(st, &dev) != hipSuccess) return TQ_ERR_HIP;
        s = scratch_on(dev, &ws);
        if (s) return s;
    }
    return fp4_quant_launch(x, x_dtype, rows * k, kind, packed, block_scale, global_scale, static_global, ws, st);
}

}  // extern "C"
