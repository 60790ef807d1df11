/*
 * tq.h -- C ABI of the MI355X (gfx950) scaled-quantization library.
 *
 * Operations: quantize, dequantize, the straight-through-estimator (STE)
 * backward of quantize, and the backward of dequantize, for
 *   - integer codes (s8 / u8 / s4 / u4) at per-tensor, per-channel,
 *     per-token (per-row) and per-group granularity,
 *   - FP8 E4M3 with one fp32 scale per block (1x128 activation groups,
 *     128x128 weight tiles, or any block shape, partial edge blocks
 *     included), per-tensor FP8 with a dynamic or static scale, and MXFP8
 *     (E4M3 with an E8M0 scale per 32 elements),
 *   - FP4 E2M1 packed two per byte with NVFP4 (E4M3 block scale per 16 plus
 *     an fp32 per-tensor scale) or MXFP4 (E8M0 block scale per 32) scales,
 *   - the FP4 transposes to GEMM layout, the concatenations of FP4 weights
 *     and their expansion to FP8 E4M3,
 *   - per-tensor fake quantization (round trip) and its backward, and
 *     dynamic-range quantization by mode and scope,
 *   - integer codes of binary64 inputs computed in binary64,
 *   - the GEMMs that consume the codes: the W8A8 quantized linear, the FP4
 *     weight-only linear and the block-scaled FP8 GEMM.
 *
 * Sources (page titles and sections):
 *   [Q]  docs.rs baracuda_kernels::quantize -- module overview (dtype
 *        coverage; per-token and per-group GPTQ-style g=128 families; the STE
 *        rule dx = (dy / scale) * 1[qmin < q < qmax] with the mask recomputed
 *        from the saved input), the module list (the *_backward plans of the
 *        dequantize ops: dq = dy * scale per group; fake_quantize and its
 *        backward; dynamic_range_quantize; quantized_linear, a fused W8A8
 *        quantized matmul), the re-exports (DynamicRangeMode,
 *        DynamicRangeScope), default_q_range.
 *   [G]  teenygrad granularity.rs -- enum Granularity (PerTensor,
 *        PerChannel{axis}, Group{axis, group_size}).
 *   [W]  metrale QuantizedWeight -- fields (packed E2M1 two per byte
 *        [N, K/2]; block scales E4M3 for NVFP4 / E8M0 for MXFP4; fp32
 *        per-tensor scale; optional static input scale), transpose_for_gemm,
 *        transpose_for_gemm_gs, transpose_concat_for_gemm(_gs, _padded),
 *        concat_rows and predequant_to_fp8.
 *   [S]  smile.llm.quant package summary -- Fp8BlockGemm (E4M3, one fp32 scale
 *        per 1x128 activation group and per 128x128 weight tile),
 *        Fp8BlockDequant, MxFp8 (E8M0 scale per 32 elements), Nvfp4Linear
 *        (an NVFP4 weight-only linear).
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless the argument name starts with
 *     host_.  All buffers are owned by the caller; the library allocates,
 *     caches and frees nothing and keeps no global state, so calls are
 *     thread-safe.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call validates its arguments on the host, enqueues its kernels
 *     on `stream` and returns without synchronizing.  A non-TQ_OK return
 *     means nothing was enqueued, except TQ_ERR_HIP, which reports a launch
 *     failure (hipGetLastError) after an enqueue attempt.
 *   - Tensors are dense, row-major and contiguous (the *_strided calls take a
 *     row stride for their input).  Base pointers must be
 *     16-byte aligned (TQ_ERR_ALIGN otherwise); scale / zero-point arrays need
 *     only their natural alignment.
 *   - Float tensors have a tq_ftype (f32, f16, bf16); arithmetic is IEEE
 *     binary32 with round-to-nearest-even: scale = amax / qmax and
 *     x / scale are correctly rounded binary32 divisions, f16 / bf16 outputs
 *     are rounded once from the binary32 result.
 *   - Integer codes: 8-bit codes take one byte each (s8 as two's
 *     complement); 4-bit codes are packed two per byte along the LAST
 *     dimension, the even index in the low nibble, so the last dimension
 *     must be even.  Zero-points are one byte per group in the code's
 *     unpacked type (u8 for U8/U4, s8 for S8/S4).
 *   - Symmetric mode (zero_point == NULL) requires qmin == -qmax and a signed
 *     code; asymmetric mode requires a zero_point array.
 *   - The input to a quantize call is never modified.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TQ_OK = 0,
    TQ_ERR_INVALID = 1,     /* bad pointer, shape, dtype, range or group size */
    TQ_ERR_UNSUPPORTED = 2, /* well-formed request the library does not implement */
    TQ_ERR_ALIGN = 3,       /* a base pointer is not 16-byte aligned */
    TQ_ERR_HIP = 4          /* the HIP runtime reported a launch error */
} tq_status;

typedef enum { TQ_F32 = 0, TQ_F16 = 1, TQ_BF16 = 2 } tq_ftype;
typedef enum { TQ_S8 = 0, TQ_U8 = 1, TQ_S4 = 2, TQ_U4 = 3 } tq_itype;
typedef enum { TQ_NVFP4 = 0, TQ_MXFP4 = 1 } tq_fp4_kind;
typedef enum { TQ_RANGE_SYMMETRIC = 0, TQ_RANGE_ASYMMETRIC = 1 } tq_range_mode;
typedef enum { TQ_GRAN_TENSOR = 0, TQ_GRAN_CHANNEL = 1, TQ_GRAN_TOKEN = 2, TQ_GRAN_GROUP = 3 } tq_granularity;
typedef enum { TQ_SCOPE_TENSOR = 0, TQ_SCOPE_TOKEN = 1, TQ_SCOPE_CHANNEL = 2 } tq_range_scope;

/* Version of this ABI (bumped on any signature change). */
int tq_abi_version(void);

/* Human-readable name of a status code (static string). */
const char* tq_status_str(int status);

/* default_q_range ([Q], function default_q_range): S8 -> [-128, 127],
 * U8 -> [0, 255], S4 -> [-8, 7], U4 -> [0, 15] for asymmetric use; in
 * symmetric mode the range is [-qmax, qmax] (S8 [-127, 127], S4 [-7, 7]) so
 * the grid is symmetric about zero.  host_qmin / host_qmax are host
 * pointers.  TQ_ERR_INVALID for an unknown code or symmetric unsigned code. */
tq_status tq_default_q_range(int code, int symmetric, int32_t* host_qmin, int32_t* host_qmax);

/* Bytes of device workspace a call needs ([Q] per-tensor scope and the NVFP4
 * per-tensor scale need a grid-wide reduction).  op: 0 = tq_quant_per_tensor
 * with a dynamic scale (0 bytes up to 65536 elements, which one workgroup
 * reduces and encodes in a single launch; tq_fake_quant_per_tensor and the
 * TQ_SCOPE_TENSOR dynamic-range call likewise), 1 = tq_quant_fp4_block with
 * a dynamic global scale, 2 = tq_quant_fp8_per_tensor with a dynamic scale
 * (0 bytes up to 65536 elements), 3 = tq_quant_f64 at TQ_GRAN_TENSOR with a
 * dynamic scale (16 KiB).  numel = elements.  A workspace is device memory,
 * 16-byte aligned (TQ_ERR_ALIGN otherwise), whose contents on entry are
 * ignored; a call in flight owns it (two calls that overlap must not share
 * one).  The first launch of such a call writes up to 1024 partial maxima
 * into it and every workgroup of the second merges them. */
size_t tq_workspace_bytes(int op, int64_t numel);

/* Measurement utility (not a step of the method): the streaming ceiling a
 * kernel is compared with.  `nthreads` units each read `in_bytes` from `src`
 * and write `out_bytes` to `dst`, folding the loaded words into the stored
 * ones and doing nothing else, with the per-lane widths of the quantization
 * kernels: in_bytes 4, 8, 16 (one load at src + t*in_bytes) or 32 (two
 * 16-byte loads, at src + 16 t and src + 16 (nthreads + t): two input
 * streams); out_bytes 4, 8, 16 (one store at dst + t*out_bytes) or 32 (two
 * 16-byte stores).  Each lane takes `vectors` units (1, 2 or 4; a workgroup
 * of 256 lanes covers 256*vectors consecutive units, lane j the units
 * k*256 + j), issuing all its loads before its stores.  16-byte loads are
 * non-temporal; stores follow `policy`: 0 plain, 1 non-temporal, 2
 * non-temporal with device scope (16-byte stores only).  src holds
 * nthreads*in_bytes bytes, dst nthreads*out_bytes; both 16-byte aligned
 * (TQ_ERR_ALIGN).  Supported mixes (in:out) 16:8, 16:4, 8:16, 4:16, 32:16,
 * 16:16, 16:32; others return TQ_ERR_UNSUPPORTED. */
tq_status tq_stream_mix(const void* src, void* dst, int64_t nthreads, int in_bytes, int out_bytes, int policy,
                        int vectors, void* stream);

/* ===================================================================== */
/* Integer codes                                                          */
/* ===================================================================== */
/*
 * Quantize ([Q] module overview; [G] Granularity).  For every group of
 * elements that shares one scale:
 *   symmetric : scale = amax / qmax              (amax = max |x|)
 *   asymmetric: mn = min(min x, 0), mx = max(max x, 0),
 *               scale = (mx - mn) / (qmax - qmin),
 *               zp = clamp(qmin - rne(mn / scale), qmin, qmax)
 *   a scale of exactly 0 (all-zero group) is replaced by 1;
 *   each element: q = clamp(rne(x / scale) + zp, qmin, qmax)
 * (rne = round to nearest integer, ties to even).  Outputs: q (codes),
 * scale (fp32, one per group), zero_point (one byte per group, asymmetric
 * mode only).
 *
 * Group layouts and output shapes:
 *   per_tensor : one group; scale[1], zero_point[1].
 *   per_channel: x of rank ndim with host_shape; one group per index along
 *                `axis`; scale[shape[axis]].
 *   per_token  : x viewed as [rows, cols]; one group per row; scale[rows].
 *   per_group  : `group_size` consecutive indices along `axis` at fixed
 *                indices of the other axes (GPTQ weight [N, K] with axis 1
 *                and group_size 128 -> scale [N, K/128]); the scale tensor
 *                is x's shape with shape[axis] replaced by
 *                shape[axis] / group_size.  shape[axis] % group_size == 0.
 */

/* Per-tensor quantize.  static_scale != 0: scale (and zero_point) are
 * INPUTS (a static activation scale as in [W] field input_scale) and no
 * reduction runs.  Otherwise the grid-wide reduction uses `workspace`
 * (device, >= tq_workspace_bytes(0, numel) bytes, contents ignored; may be
 * NULL when that is 0). */
tq_status tq_quant_per_tensor(const void* x, int x_dtype, int64_t numel,
                              int code, int32_t qmin, int32_t qmax, int static_scale,
                              void* q, float* scale, void* zero_point,
                              void* workspace, size_t workspace_bytes, void* stream);

/* host_shape: host array of ndim (1..8) extents. */
tq_status tq_quant_per_channel(const void* x, int x_dtype, int32_t ndim, const int64_t* host_shape,
                               int32_t axis, int code, int32_t qmin, int32_t qmax,
                               void* q, float* scale, void* zero_point, void* stream);

tq_status tq_quant_per_token(const void* x, int x_dtype, int64_t rows, int64_t cols,
                             int code, int32_t qmin, int32_t qmax,
                             void* q, float* scale, void* zero_point, void* stream);

/* Per-token quantize of a row-strided input: row r of x starts x_row_stride
 * elements after row r-1 (x_row_stride >= cols; a column slice of a wider
 * matrix); q, scale and zero_point are dense as in tq_quant_per_token, and
 * the results are those of tq_quant_per_token on the dense rows.  Needs
 * cols % 8 == 0 (TQ_ERR_UNSUPPORTED otherwise) and 16-byte aligned rows:
 * x aligned, cols and x_row_stride multiples of 16 bytes (TQ_ERR_ALIGN). */
tq_status tq_quant_per_token_strided(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                     int64_t x_row_stride, int code, int32_t qmin, int32_t qmax,
                                     void* q, float* scale, void* zero_point, void* stream);

tq_status tq_quant_per_group(const void* x, int x_dtype, int32_t ndim, const int64_t* host_shape,
                             int32_t axis, int64_t group_size, int code, int32_t qmin, int32_t qmax,
                             void* q, float* scale, void* zero_point, void* stream);

/* Dequantize: y = (q - zp) * scale in binary32, rounded once to y_dtype.
 * zero_point NULL means zp = 0. */
tq_status tq_dequant_per_tensor(const void* q, int code, int64_t numel, const float* scale,
                                const void* zero_point, void* y, int y_dtype, void* stream);
tq_status tq_dequant_per_channel(const void* q, int code, int32_t ndim, const int64_t* host_shape,
                                 int32_t axis, const float* scale, const void* zero_point,
                                 void* y, int y_dtype, void* stream);
tq_status tq_dequant_per_token(const void* q, int code, int64_t rows, int64_t cols,
                               const float* scale, const void* zero_point,
                               void* y, int y_dtype, void* stream);
tq_status tq_dequant_per_group(const void* q, int code, int32_t ndim, const int64_t* host_shape,
                               int32_t axis, int64_t group_size, const float* scale,
                               const void* zero_point, void* y, int y_dtype, void* stream);

/* Quantize backward (STE, [Q] module overview): the code q is recomputed
 * from the saved input x with the saved scale / zero_point (the amax is not
 * recomputed), then
 *   dx = (dy / scale) * (qmin < q < qmax ? 1 : 0)
 * as a binary32 product (a masked element is a zero carrying the sign of
 * dy / scale), rounded once to x_dtype.  dy and dx have x's dtype and shape. */
tq_status tq_quant_per_tensor_backward(const void* x, int x_dtype, int64_t numel,
                                       int code, int32_t qmin, int32_t qmax,
                                       const float* scale, const void* zero_point,
                                       const void* dy, void* dx, void* stream);
tq_status tq_quant_per_channel_backward(const void* x, int x_dtype, int32_t ndim,
                                        const int64_t* host_shape, int32_t axis,
                                        int code, int32_t qmin, int32_t qmax,
                                        const float* scale, const void* zero_point,
                                        const void* dy, void* dx, void* stream);
tq_status tq_quant_per_token_backward(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                      int code, int32_t qmin, int32_t qmax,
                                      const float* scale, const void* zero_point,
                                      const void* dy, void* dx, void* stream);
tq_status tq_quant_per_group_backward(const void* x, int x_dtype, int32_t ndim,
                                      const int64_t* host_shape, int32_t axis, int64_t group_size,
                                      int code, int32_t qmin, int32_t qmax,
                                      const float* scale, const void* zero_point,
                                      const void* dy, void* dx, void* stream);

/* Dequantize backward ([Q] module list): dq = dy * scale of the element's
 * group (straight-through in the code), binary32 product rounded once to
 * dy_dtype; dq has dy's dtype and shape. */
tq_status tq_dequant_per_tensor_backward(const void* dy, int dy_dtype, int64_t numel,
                                         const float* scale, void* dq, void* stream);
tq_status tq_dequant_per_channel_backward(const void* dy, int dy_dtype, int32_t ndim,
                                          const int64_t* host_shape, int32_t axis,
                                          const float* scale, void* dq, void* stream);
tq_status tq_dequant_per_token_backward(const void* dy, int dy_dtype, int64_t rows, int64_t cols,
                                        const float* scale, void* dq, void* stream);
tq_status tq_dequant_per_group_backward(const void* dy, int dy_dtype, int32_t ndim,
                                        const int64_t* host_shape, int32_t axis,
                                        int64_t group_size, const float* scale, void* dq,
                                        void* stream);

/* Fake quantization ([Q] module list: fake_quantize, "per-tensor, FP round
 * trip", and fake_quantize_backward "via STE").  Per-tensor scale and
 * zero-point exactly as tq_quant_per_tensor (dynamic, using `workspace` of
 * tq_workspace_bytes(0, numel) bytes, or static inputs when static_scale != 0),
 * and every element quantized and dequantized at once:
 *   y = (q - zp) * scale,  q = clamp(rne(x / scale) + zp, qmin, qmax)
 * in binary32, rounded once to x_dtype; y has x's dtype and shape, no code is
 * stored.  `code` fixes the allowed range and the zero-point byte's type. */
tq_status tq_fake_quant_per_tensor(const void* x, int x_dtype, int64_t numel, int code,
                                   int32_t qmin, int32_t qmax, int static_scale, void* y,
                                   float* scale, void* zero_point, void* workspace,
                                   size_t workspace_bytes, void* stream);
/* Straight-through backward of the round trip (reading: the round trip is
 * the identity inside the range, so dy passes unscaled):
 *   dx = dy * (qmin < q < qmax ? 1 : 0)
 * with q recomputed from the saved x, scale and zero_point; a masked element
 * is a zero with dy's sign.  dy and dx have x's dtype and shape. */
tq_status tq_fake_quant_per_tensor_backward(const void* x, int x_dtype, int64_t numel, int code,
                                            int32_t qmin, int32_t qmax, const float* scale,
                                            const void* zero_point, const void* dy, void* dx,
                                            void* stream);

/* Dynamic-range quantize ([Q] module list: dynamic_range_quantize, a compose
 * op, with DynamicRangeMode and DynamicRangeScope).  Reading: the range is
 * derived from the data at the scope and the matching quantize above runs
 * with tq_default_q_range(code, mode == TQ_RANGE_SYMMETRIC):
 *   TQ_SCOPE_TENSOR  -> tq_quant_per_tensor (dynamic; workspace as there),
 *   TQ_SCOPE_TOKEN   -> tq_quant_per_token, rows = product of the leading
 *                       extents, cols = the last,
 *   TQ_SCOPE_CHANNEL -> tq_quant_per_channel along `axis` (ignored otherwise).
 * TQ_RANGE_ASYMMETRIC needs zero_point; TQ_RANGE_SYMMETRIC ignores it and
 * rejects unsigned codes.  Outputs as for the routed call. */
tq_status tq_dynamic_range_quantize(const void* x, int x_dtype, int32_t ndim,
                                    const int64_t* host_shape, int mode, int scope, int32_t axis,
                                    int code, void* q, float* scale, void* zero_point,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Binary64 inputs ([Q] module overview: f64 among the input types).
 * Reading: an f64 input is computed in binary64 throughout -- the integer-code
 * definitions above with every division, product and rounding a binary64
 * operation, `scale` arrays of binary64, and binary64 dequantized values and
 * gradients.  One call per operation with the granularity as an argument:
 * gran = TQ_GRAN_TENSOR, TQ_GRAN_TOKEN (rows = product of the leading extents),
 * TQ_GRAN_CHANNEL (along `axis`) or TQ_GRAN_GROUP (`group_size` along `axis`);
 * scale / zero_point have the shapes of the binary32 calls.  Codes, zero-points,
 * ranges and symmetric mode as above.  Pointers need only their natural
 * alignment.  A dynamic TQ_GRAN_TENSOR scale needs `workspace` of
 * tq_workspace_bytes(3, numel) bytes; otherwise it may be NULL. */
tq_status tq_quant_f64(const double* x, int32_t ndim, const int64_t* host_shape, int gran,
                       int32_t axis, int64_t group_size, int code, int32_t qmin, int32_t qmax,
                       int static_scale, void* q, double* scale, void* zero_point,
                       void* workspace, size_t workspace_bytes, void* stream);
/* y = (q - zp) * scale (binary64). */
tq_status tq_dequant_f64(const void* q, int code, int32_t ndim, const int64_t* host_shape,
                         int gran, int32_t axis, int64_t group_size, const double* scale,
                         const void* zero_point, double* y, void* stream);
/* dx = (dy / scale) * (qmin < q < qmax ? 1 : 0), q recomputed from x. */
tq_status tq_quant_f64_backward(const double* x, int32_t ndim, const int64_t* host_shape, int gran,
                                int32_t axis, int64_t group_size, int code, int32_t qmin,
                                int32_t qmax, const double* scale, const void* zero_point,
                                const double* dy, double* dx, void* stream);
/* dq = dy * scale. */
tq_status tq_dequant_f64_backward(const double* dy, int32_t ndim, const int64_t* host_shape,
                                  int gran, int32_t axis, int64_t group_size, const double* scale,
                                  double* dq, void* stream);

/* ===================================================================== */
/* FP8 E4M3 blocks ([S] Fp8BlockGemm, Fp8BlockDequant)                    */
/* ===================================================================== */
/* x is [rows, cols]; blocks are block_rows x block_cols (1 x 128 for
 * activations, 128 x 128 for weights).  scale is [ceil(rows/block_rows),
 * ceil(cols/block_cols)] fp32; when the blocks do not tile the shape, the
 * blocks of the last block row / column are partial and cover only the
 * elements that exist (tiling shapes take the fast kernels):
 *   scale = amax / 448 (1 if that is 0),  q = E4M3(x / scale)
 * with OCP E4M3 (bias 7, max 448), round to nearest even, saturating at
 * +-448 and keeping the sign of zero.  q is [rows, cols] bytes. */
tq_status tq_quant_fp8_block(const void* x, int x_dtype, int64_t rows, int64_t cols,
                             int32_t block_rows, int32_t block_cols,
                             uint8_t* q, float* scale, void* stream);
/* FP8 1 x block_cols quantize of a row-strided input (row r starts
 * x_row_stride elements after row r-1, x_row_stride >= cols); q and scale are
 * dense ([rows, cols] and [rows, cols/block_cols]) and equal those of
 * tq_quant_fp8_block(…, 1, block_cols, …) on the dense rows.  block_cols is
 * 16, 32, 64, 128, 256 or 512 (TQ_ERR_UNSUPPORTED otherwise) and must divide
 * cols; rows need 16-byte alignment as for tq_quant_per_token_strided. */
tq_status tq_quant_fp8_rows_strided(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                    int64_t x_row_stride, int32_t block_cols, uint8_t* q,
                                    float* scale, void* stream);
/* y = val(q) * scale, rounded once to y_dtype. */
tq_status tq_dequant_fp8_block(const uint8_t* q, int64_t rows, int64_t cols,
                               int32_t block_rows, int32_t block_cols, const float* scale,
                               void* y, int y_dtype, void* stream);
/* STE: dx = (dy / scale) * (-448 < val(q) < 448 ? 1 : 0), q recomputed. */
tq_status tq_quant_fp8_block_backward(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                      int32_t block_rows, int32_t block_cols, const float* scale,
                                      const void* dy, void* dx, void* stream);
/* dq = dy * scale. */
tq_status tq_dequant_fp8_block_backward(const void* dy, int dy_dtype, int64_t rows, int64_t cols,
                                        int32_t block_rows, int32_t block_cols,
                                        const float* scale, void* dq, void* stream);

/* FP8 E4M3 with one fp32 scale for the whole tensor ([S] Fp8KvCodec: FP8
 * KV store / load with per-tensor scales).  x has numel elements (any
 * shape, contiguous); q has numel E4M3 bytes.
 *   scale = amax / 448 (1 if that is 0), or when static_scale != 0 the
 *   caller's value in scale[0] (an input; no reduction runs);
 *   q = E4M3(x / scale) as in the block calls.
 * The dynamic scale needs `workspace` of tq_workspace_bytes(2, numel) bytes
 * (may be NULL when that is 0). */
tq_status tq_quant_fp8_per_tensor(const void* x, int x_dtype, int64_t numel, int static_scale,
                                  uint8_t* q, float* scale, void* workspace,
                                  size_t workspace_bytes, void* stream);
/* Load: y = val(q) * scale[0], rounded once to y_dtype. */
tq_status tq_dequant_fp8_per_tensor(const uint8_t* q, int64_t numel, const float* scale, void* y,
                                    int y_dtype, void* stream);

/* MXFP8 ([S] MxFp8: E4M3 elements with one shared E8M0 scale per 32
 * consecutive elements along the reduction dimension).  x is [rows, k],
 * k % 32 == 0; q is [rows, k] E4M3 bytes, block_scale [rows, k/32] bytes.
 * Shared scale by the OCP MX v1.0 rule with E4M3's largest exponent 8:
 *   sb = floor(log2 amax) - 8 + 127 clamped to [0, 254] (127 for an all-zero
 *   block), X = 2^(sb - 127);  q = E4M3(x / X), round to nearest even,
 *   saturating at +-448 (amax / X lies in [256, 512)), keeping the sign of
 *   zero. */
tq_status tq_quant_mxfp8(const void* x, int x_dtype, int64_t rows, int64_t k, uint8_t* q,
                         uint8_t* block_scale, void* stream);
/* y = val(q) * X, rounded once to y_dtype. */
tq_status tq_dequant_mxfp8(const uint8_t* q, const uint8_t* block_scale, int64_t rows, int64_t k,
                           void* y, int y_dtype, void* stream);
/* STE: dx = (dy / X) * (-448 < val(q) < 448 ? 1 : 0), q recomputed from x. */
tq_status tq_quant_mxfp8_backward(const void* x, int x_dtype, const uint8_t* block_scale,
                                  int64_t rows, int64_t k, const void* dy, void* dx, void* stream);
/* dq = dy * X. */
tq_status tq_dequant_mxfp8_backward(const void* dy, int dy_dtype, const uint8_t* block_scale,
                                    int64_t rows, int64_t k, void* dq, void* stream);

/* W8A8 quantized linear ([Q] quantized_linear: a fused W8A8 quantized
 * matmul; the page names the operation only).  qx [M, K] symmetric s8 codes
 * with one fp32 scale per row sx [M] (tq_quant_per_token's output), qw [N, K]
 * symmetric s8 codes with one fp32 scale per output channel sw [N]
 * (tq_quant_per_token on the weight rows); out = x W^T:
 *   acc[m][n] = sum_k qx[m][k] * qw[n][k]           exact, 32-bit
 *   y[m][n]   = ((float)acc * sx[m]) * sw[n]        binary32, in that order
 * rounded once more to y_dtype; y is [M, N].  Bit-exact: the integer sums
 * are exact on the matrix cores.  N and K multiples of 128 and K <= 131071
 * (so every sum fits 32 bits), TQ_ERR_UNSUPPORTED otherwise; any M; qx, qw
 * 16-byte aligned, y aligned to 4 output elements (TQ_ERR_ALIGN otherwise).  K = 0 writes zeros (the code pointers may then be null).
 * Launches only; no allocation. */
tq_status tq_w8a8_linear(const int8_t* qx, const float* sx, const int8_t* qw, const float* sw, int64_t M, int64_t N,
                         int64_t K, void* y, int y_dtype, void* stream);

/* FP4 weight-only linear ([W] the packed E2M1 weight with its block scales
 * and fp32 per-tensor scale, made for a 16-bit-activation tile GEMM;
 * [S] Nvfp4Linear).  x [M, K] bf16 activations times the weight in the
 * quantizer's own layout, packed [N, K/2] (low nibble = even k) and
 * block_scale [N, K/gs] (E4M3 bytes, gs = 16, for kind TQ_NVFP4; E8M0 bytes,
 * gs = 32, for TQ_MXFP4); global_scale (device, one float) is the NVFP4
 * per-tensor scale (ignored for MXFP4).  out = x W^T, y [M, N]:
 *   y[m][n] = s_g * sum_k x[m][k] * E2M1(code(n, k)) * scale(n, k / gs)
 * The weight is expanded to bf16 exactly (E2M1 x block scale), the products
 * are summed on the bf16 matrix cores in 64-wide blocks and the block sums
 * in binary32; the result is within a few 2^-24 of the magnitude sum
 * sum |x w| per block of the exact value, then rounded to y_dtype.  The
 * K-contiguous [N, K/2] layout is the matrix cores' operand order, so no
 * transposed twin is read.  x_dtype must be TQ_BF16, N a multiple of 128 and
 * K of 64 (TQ_ERR_UNSUPPORTED otherwise); any M; x, packed 16-byte aligned,
 * block_scale 4-byte aligned, y aligned to 4 output elements; MXFP4 scale bytes 1 .. 254.  K = 0 writes
 * zeros.  Launches only; no allocation. */
tq_status tq_fp4_linear(const void* x, int x_dtype, const uint8_t* packed, const uint8_t* block_scale,
                        const float* global_scale, int kind, int64_t M, int64_t N, int64_t K, void* y,
                        int y_dtype, void* stream);

/* Block-scaled FP8 GEMM ([S] Fp8BlockGemm: activations E4M3 with one fp32
 * scale per 1 x 128 group, weights E4M3 with one fp32 scale per 128 x 128
 * tile; out = x W^T).  qa [M, K] with sa [M, K/128] (tq_quant_fp8_block with
 * 1 x 128 blocks), qw [N, K] with sw [N/128, K/128] (128 x 128 blocks):
 *   y[m][n] = sum_kb (sa[m][kb] * sw[n/128][kb]) *
 *             sum_{k in kb} val(qa[m][k]) * val(qw[n][k])
 * computed on the matrix cores: each 128-wide K block is one E4M3 matrix-core
 * step of 128 products per output; the block sum is scaled by sa * sw and
 * accumulated in binary32, and the total is rounded once to y_dtype (y is
 * [M, N]).  The
 * matrix core does not add exactly: within each group of 8 consecutive K it
 * cuts every product toward zero to a multiple of 2^(E - 13), E the group's
 * largest operand exponent sum, and it keeps about 24 bits when it combines
 * the group sums and converts toward zero.  So the result is within
 * sum_kb |sa sw| (those cuts) + about 2^-18 of the magnitude sum
 * sum |sa sw val val| of the exact value, not bit-equal to it.  K and N
 * multiples of 128 (TQ_ERR_INVALID otherwise), any M; qa, qw 16-byte
 * aligned, y aligned to 4 output elements.  K = 0 writes zeros (the operand pointers may then be null);
 * M = 0 or N = 0 does nothing.  Launches only; no allocation. */
tq_status tq_fp8_block_gemm(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                            int64_t M, int64_t N, int64_t K, void* y, int y_dtype, void* stream);

/* ===================================================================== */
/* FP4 E2M1 blocks ([W] QuantizedWeight fields; [S] MxFp8 for the E8M0 rule) */
/* ===================================================================== */
/* x is [rows, k]; blocks of gs = 16 (NVFP4) or 32 (MXFP4) consecutive
 * elements along k (k % gs == 0).  Outputs: packed [rows, k/2] (two E2M1
 * codes per byte, even index in the low nibble), block_scale [rows, k/gs]
 * bytes, and for NVFP4 the fp32 per-tensor scale global_scale[1].
 *   NVFP4: s_g = amax_tensor / (6 * 448) (1 if 0), or the caller's value when
 *          static_global != 0 (global_scale is then an input);
 *          sb = E4M3(amax_block / (6 * s_g)), replaced by 0x38 (1.0) if it
 *          encodes to zero; eff = val(sb) * s_g.
 *   MXFP4: sb = E8M0 byte of 2^(floor(log2 amax_block) - 2) (127 if the block
 *          is all zero), eff = 2^(sb - 127); global_scale is unused (may be
 *          NULL).
 *   every element: q = E2M1(x / eff), round to nearest even, saturating at
 *          +-6, keeping the sign of zero.
 * The dynamic NVFP4 scale needs `workspace` (>= tq_workspace_bytes(1, rows*k)
 * bytes); otherwise workspace may be NULL. */
tq_status tq_quant_fp4_block(const void* x, int x_dtype, int64_t rows, int64_t k, int kind,
                             uint8_t* packed, uint8_t* block_scale, float* global_scale,
                             int static_global, void* workspace, size_t workspace_bytes,
                             void* stream);
/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, hosts that forbid hipMalloc):
 * tq_quant_fp4_block without the workspace, same arguments otherwise and the
 * same results bit for bit.  A dynamic NVFP4 per-tensor scale keeps its up
 * to 1024 chunk maxima in a 4 KiB device array of the library's own (one per
 * GPU, held until the process ends, found by hipGetSymbolAddress on the first
 * call on that GPU); nothing is allocated, freed or synchronized.  Any tensor
 * size is taken (the chunks grow so that 1024 partials always suffice;
 * TQ_ERR_UNSUPPORTED if that ever failed).  Calls that overlap on one GPU
 * share that array and race: serialize them (one stream, or events). */
tq_status tq_quant_fp4_block_noalloc(const void* x, int x_dtype, int64_t rows, int64_t k, int kind,
                                     uint8_t* packed, uint8_t* block_scale, float* global_scale,
                                     int static_global, void* stream);
/* y = val(q) * eff, rounded once to y_dtype. */
tq_status tq_dequant_fp4_block(const uint8_t* packed, const uint8_t* block_scale,
                               const float* global_scale, int64_t rows, int64_t k, int kind,
                               void* y, int y_dtype, void* stream);
/* STE: dx = (dy / eff) * (-6 < val(q) < 6 ? 1 : 0), q recomputed from x. */
tq_status tq_quant_fp4_block_backward(const void* x, int x_dtype, const uint8_t* block_scale,
                                      const float* global_scale, int64_t rows, int64_t k, int kind,
                                      const void* dy, void* dx, void* stream);
/* dq = dy * eff. */
tq_status tq_dequant_fp4_block_backward(const void* dy, int dy_dtype, const uint8_t* block_scale,
                                        const float* global_scale, int64_t rows, int64_t k,
                                        int kind, void* dq, void* stream);

/* GEMM layout ([W] transpose_for_gemm / transpose_for_gemm_gs): byte
 * transposes packed [n, k/2] -> packed_t [k/2, n] and block_scale
 * [n, k/group_size] -> block_scale_t [k/group_size, n] into caller-provided
 * buffers (the page's version allocates new buffers; here the caller owns
 * them).  Each byte keeps its two nibbles.  block_scale / block_scale_t may
 * both be NULL to transpose only the codes. */
tq_status tq_fp4_transpose_for_gemm(const uint8_t* packed, const uint8_t* block_scale,
                                    int64_t n, int64_t k, int32_t group_size,
                                    uint8_t* packed_t, uint8_t* block_scale_t, void* stream);

/* [W] transpose_concat_for_gemm / _gs / _padded: several weights sharing k,
 * part i packed [n_i, k/2] with block_scale [n_i, k/group_size], transposed
 * and concatenated along n into one GEMM operand:
 *   packed_t[j][off_i + r] = packed_i[r][j]      (packed_t is [k/2, stride])
 *   block_scale_t[b][off_i + r] = block_scale_i[r][b]   ([k/group_size, stride])
 * with off_i = n_0 + ... + n_(i-1) and stride = n_total rounded up to a
 * multiple of `align` (align = 1: no padding); columns n_total..stride-1 are
 * zero.  host_packed / host_block_scale are HOST arrays of nparts DEVICE
 * pointers, host_n a host array of the n_i; parts need no alignment (16-byte
 * aligned parts with n_i, off_i and stride multiples of 16 take the tiled
 * path).  The stride is written to *host_stride when it is not NULL.
 * block_scale_t == NULL (host_block_scale may then be NULL) transposes only
 * the codes.  nparts <= 0 (an empty list) or align <= 0 is TQ_ERR_INVALID.
 * Per-tensor scales are the caller's business: the page's result carries the
 * first part's and checks nothing. */
tq_status tq_fp4_transpose_concat_for_gemm(int32_t nparts, const uint8_t* const* host_packed,
                                           const uint8_t* const* host_block_scale,
                                           const int64_t* host_n, int64_t k, int32_t group_size,
                                           int64_t align, uint8_t* packed_t,
                                           uint8_t* block_scale_t, int64_t* host_stride,
                                           void* stream);

/* [W] concat_rows: two NVFP4 weights with the same k (k % 16 == 0) stacked
 * by rows, [n1, k/2] + [n2, k/2] -> packed_out [n1+n2, k/2] and
 * [n1, k/16] + [n2, k/16] -> block_scale_out [n1+n2, k/16].  The per-tensor
 * scales (host floats) must be bit-identical, else TQ_ERR_INVALID and nothing
 * is enqueued: the result has one per-tensor scale (either input's).  Device
 * to device copies on `stream`; no alignment requirement. */
tq_status tq_fp4_concat_rows(const uint8_t* packed1, const uint8_t* block_scale1,
                             float host_global_scale1, const uint8_t* packed2,
                             const uint8_t* block_scale2, float host_global_scale2, int64_t n1,
                             int64_t n2, int64_t k, uint8_t* packed_out,
                             uint8_t* block_scale_out, void* stream);

/* [W] predequant_to_fp8: the FP4 weight [rows, k] expanded to E4M3 bytes
 * [rows, k] with the per-tensor scale applied:
 *   fp8_out = E4M3(val(q) * eff),  eff = val(sb) * host_global_scale (NVFP4)
 *                                  or 2^(sb - 127) (MXFP4; the scale is unused)
 * each product rounded once to binary32, then encoded round-to-nearest-even,
 * saturating at +-448, keeping the sign of zero.  packed needs 8-byte
 * alignment, fp8_out 16-byte.  Asynchronous like every call here (the page's
 * version synchronizes because it allocates the output). */
tq_status tq_fp4_predequant_to_fp8(const uint8_t* packed, const uint8_t* block_scale,
                                   float host_global_scale, int64_t rows, int64_t k, int kind,
                                   uint8_t* fp8_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
