// tq_host.h -- host-side helpers shared by the C-ABI entry points:
// argument validation, the group layout of a granularity, launch checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "tq.h"

namespace tq {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool valid_ftype(int t) { return t == TQ_F32 || t == TQ_F16 || t == TQ_BF16; }
inline bool valid_code(int c) { return c == TQ_S8 || c == TQ_U8 || c == TQ_S4 || c == TQ_U4; }
inline int code_bits(int c) { return (c == TQ_S4 || c == TQ_U4) ? 4 : 8; }
inline bool code_signed(int c) { return c == TQ_S8 || c == TQ_S4; }
inline int ftype_size(int t) { return t == TQ_F32 ? 4 : 2; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workgroups for a grid-stride kernel: one per `per_block` units of work,
// at least 1 and at most 2^20.
inline unsigned grid_for(int64_t work, int64_t per_block)
{
    int64_t g = cdiv(work, per_block);
    if (g < 1) g = 1;
    if (g > (1 << 20)) g = 1 << 20;
    return (unsigned)g;
}

// Per-tensor statistics of a large tensor are reduced in two launches: a
// first pass writes one partial per chunk, at most TENSOR_PARTS of them
// (padded to a multiple of 4 with chunks past the end, whose partials are 0),
// and every workgroup of the encoding pass merges them itself.  tensor_chunk
// gives the chunk length (a multiple of 2048 elements, at least 8192) and the
// padded partial count.
constexpr int TENSOR_PARTS = 1024;

// FP4 block quantize (tq_fp4.hip): argument checks, and the launches on
// checked arguments (ws: TENSOR_PARTS floats, 16-byte aligned, used only
// for a dynamic NVFP4 per-tensor scale).
tq_status check_fp4_quant(const void* x, int x_dtype, int64_t rows, int64_t k, int kind, const uint8_t* packed,
                          const uint8_t* block_scale, const float* global_scale);
tq_status fp4_quant_launch(const void* x, int x_dtype, int64_t numel, int kind, uint8_t* packed,
                           uint8_t* block_scale, float* global_scale, int static_global, float* ws, hipStream_t st);

inline int64_t tensor_chunk(int64_t numel, int* nparts)
{
    const int64_t chunk = std::max<int64_t>(256 * 8 * 4, cdiv(cdiv(numel, TENSOR_PARTS), 2048) * 2048);
    *nparts = (int)(cdiv(cdiv(numel, chunk), 4) * 4);
    return chunk;
}

inline tq_status launch_status()
{
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

// Range check of (code, qmin, qmax, symmetric): the range lies inside the
// code's representable range, qmin < qmax, and symmetric mode uses
// [-qmax, qmax] with a signed code.
inline bool valid_range(int code, int32_t qmin, int32_t qmax, bool symmetric)
{
    if (!valid_code(code) || qmin >= qmax) return false;
    int bits = code_bits(code);
    int32_t lo = code_signed(code) ? -(1 << (bits - 1)) : 0;
    int32_t hi = code_signed(code) ? (1 << (bits - 1)) - 1 : (1 << bits) - 1;
    if (qmin < lo || qmax > hi) return false;
    if (symmetric && (qmin != -qmax || !code_signed(code))) return false;
    return true;
}

// Canonical group layout.  The tensor is viewed as [outer, A, inner] around
// the grouped axis.
//   KIND_TENSOR : one group.
//   KIND_CHANNEL: group = index a along A (all outer and inner indices).
//   KIND_GROUP  : group = g consecutive indices along A at fixed (o, i);
//                 group id = (o * (A / g) + a / g) * inner + i.
// Per-token [rows, cols] is KIND_GROUP with outer = rows, A = g = cols,
// inner = 1.
enum { KIND_TENSOR = 0, KIND_CHANNEL = 1, KIND_GROUP = 2 };

struct GroupMap {
    int kind;
    int64_t outer, A, inner, g;
    int64_t numel, ngroups;
};

inline bool make_map(int kind, int32_t ndim, const int64_t* shape, int32_t axis, int64_t g,
                     GroupMap* m)
{
    if (ndim < 1 || ndim > 8 || !shape) return false;
    int64_t numel = 1;
    for (int d = 0; d < ndim; ++d) {
        if (shape[d] < 0) return false;
        numel *= shape[d];
    }
    if (axis < 0 || axis >= ndim) return false;
    m->kind = kind;
    m->numel = numel;
    m->outer = 1;
    m->inner = 1;
    m->A = shape[axis];
    for (int d = 0; d < axis; ++d) m->outer *= shape[d];
    for (int d = axis + 1; d < ndim; ++d) m->inner *= shape[d];
    if (kind == KIND_CHANNEL) {
        m->g = 1;
        m->ngroups = m->A;
    } else {
        if (g <= 0 || m->A % g) return false;
        m->g = g;
        m->ngroups = m->outer * (m->A / g) * m->inner;
    }
    return true;
}

inline GroupMap tensor_map(int64_t numel)
{
    GroupMap m;
    m.kind = KIND_TENSOR;
    m.outer = 1;
    m.A = numel;
    m.inner = 1;
    m.g = numel;
    m.numel = numel;
    m.ngroups = 1;
    return m;
}

inline GroupMap token_map(int64_t rows, int64_t cols)
{
    GroupMap m;
    m.kind = KIND_GROUP;
    m.outer = rows;
    m.A = cols;
    m.inner = 1;
    m.g = cols;
    m.numel = rows * cols;
    m.ngroups = rows;
    return m;
}

// Device copy of a group layout: group id of element e, group size, and the
// j-th element of group gid (index arithmetic for any layout).
struct DMap {
    int kind;
    int64_t outer, A, inner, g, numel;

    __device__ int64_t group_of(int64_t e) const
    {
        if (kind == KIND_TENSOR) return 0;
        const int64_t a = (e / inner) % A;
        if (kind == KIND_CHANNEL) return a;
        const int64_t i = e % inner, o = e / (inner * A);
        return (o * (A / g) + a / g) * inner + i;
    }
    __device__ int64_t count() const
    {
        if (kind == KIND_TENSOR) return numel;
        if (kind == KIND_CHANNEL) return outer * inner;
        return g;
    }
    __device__ int64_t elem(int64_t gid, int64_t j) const
    {
        if (kind == KIND_TENSOR) return j;
        if (kind == KIND_CHANNEL) return (j / inner) * A * inner + gid * inner + j % inner;
        const int64_t i = gid % inner, t = gid / inner;
        const int64_t ab = t % (A / g), o = t / (A / g);
        return (o * A + ab * g + j) * inner + i;
    }
};

inline DMap to_dmap(const GroupMap& m)
{
    DMap d;
    d.kind = m.kind;
    d.outer = m.outer;
    d.A = m.A;
    d.inner = m.inner;
    d.g = m.g;
    d.numel = m.numel;
    return d;
}

}  // namespace tq
