/*
 * tq_oracle.c -- plain, slow CPU oracle for scaled quantize / dequantize /
 * straight-through-estimator backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark can compare the HIP library against an
 * obviously correct scalar definition.  It shares no source, header, table
 * or constant with the HIP library.
 *
 * Arithmetic model.  The method fixes fp32 scales and IEEE fp32 division, so
 * every step that the definition states as a binary32 operation is done here
 * in C `float` (x86-64 SSE, round-to-nearest-even), built with
 * -O2 -ffp-contract=off and without -ffast-math, so no a*b+c is fused and no
 * operation is reordered.  Format conversions (minifloat encode/decode,
 * bf16/f16 narrowing) are written from the bit-field definitions and use
 * exact double arithmetic internally.
 *
 * Sources of the definitions (pages of the tensor_quantization reading):
 *  - docs.rs baracuda_kernels::quantize, module overview: dtype coverage
 *    (f32/f16/bf16 in, s8/u8 out), per-token and per-group (GPTQ-style g=128)
 *    families, and the STE rule dx = (dy / scale) * 1[qmin < q < qmax] with
 *    the mask recomputed from the saved input.
 *  - same page, module list: dequantize backward rules dq = dy * scale (per
 *    tensor), dq[i] = dy[i] * scale[c] (per channel), straight-through
 *    dq = dy * scale[n] (per token / per group).
 *  - same page, function default_q_range: S8 -> [-128, 127], U8 -> [0, 255].
 *  - teenygrad granularity.rs, enum Granularity: PerTensor / PerChannel{axis} /
 *    Group{axis, group_size}.
 *  - metrale QuantizedWeight, fields + transpose_for_gemm(_gs): packed E2M1
 *    two per byte [N, K/2], per-group scales (E4M3 for NVFP4 with a host fp32
 *    per-tensor scale, E8M0 for MXFP4), transposes to [K/2, N] / [K/gs, N].
 *  - smile.llm.quant package summary, Fp8BlockGemm / Fp8BlockDequant / MxFp8:
 *    E4M3 with one fp32 scale per 1x128 activation group or 128x128 weight
 *    tile; E8M0 scale per 32 elements for the MX family.
 * Readings of points the pages leave open are listed beside the code that
 * takes them (symmetric s8 range, zero-point formula, NVFP4 two-level scale,
 * MX shared-exponent rule, degenerate groups, nibble order).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ enums */
/* The oracle's own numbering; it is deliberately independent of the
 * library's header (the Python side maps names to these values). */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };
enum { ORC_S8 = 0, ORC_U8 = 1, ORC_S4 = 2, ORC_U4 = 3 };
enum { ORC_TENSOR = 0, ORC_CHANNEL = 1, ORC_TOKEN = 2, ORC_GROUP = 3 };
enum { ORC_NVFP4 = 0, ORC_MXFP4 = 1 };
enum { ORC_OK = 0, ORC_BAD = 1 };

/* --------------------------------------------------------- bit helpers */
static float f_from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t bits_of_f(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

/* Round to the nearest integer, ties to even (the default FE_TONEAREST
 * mode makes nearbyint do exactly that). */
static double rne(double v) { return nearbyint(v); }

/* ------------------------------------------------- widen to binary32 */
/* bfloat16 is the upper half of a binary32 pattern: widening is exact. */
float orc_bf16_to_f32(uint16_t h) { return f_from_bits((uint32_t)h << 16); }

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
float orc_f16_to_f32(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 31) return m ? NAN : (s ? -INFINITY : INFINITY);
    if (e == 0) v = ldexp((double)m, -24);              /* m/1024 * 2^-14 */
    else v = ldexp(1.0 + m / 1024.0, e - 15);
    return (float)(s ? -v : v);                          /* exact */
}

static float widen(const void* p, int dt, int64_t i)
{
    if (dt == ORC_F32) return ((const float*)p)[i];
    if (dt == ORC_F16) return orc_f16_to_f32(((const uint16_t*)p)[i]);
    return orc_bf16_to_f32(((const uint16_t*)p)[i]);
}

/* ------------------------------------------------ narrow from binary32 */
/* Generic round-to-nearest-even encode of |a| (a >= 0, finite, exact in a
 * double) into a binary format with `mb` fraction bits whose smallest
 * normal exponent is `emin`.  Returns the magnitude field (exponent and
 * fraction bits, no sign).  A fraction that rounds up to 2^mb carries into
 * the exponent field through the integer addition, as it should. */
static uint32_t enc_mag(double a, int mb, int emin)
{
    if (a < ldexp(1.0, emin)) {                  /* subnormal range */
        return (uint32_t)rne(a / ldexp(1.0, emin - mb));
    }
    int e;
    frexp(a, &e);                                /* a = f * 2^e, f in [.5,1) */
    e -= 1;                                      /* a = (1+t) * 2^e */
    double t = a / ldexp(1.0, e) - 1.0;          /* exact */
    uint32_t M = (uint32_t)rne(t * ldexp(1.0, mb));
    return ((uint32_t)(e - emin + 1) << mb) + M;
}

/* Value of a magnitude field of the same generic format. */
static double dec_mag(uint32_t field, int mb, int emin)
{
    uint32_t E = field >> mb, M = field & ((1u << mb) - 1);
    if (E == 0) return ldexp((double)M, emin - mb);
    return ldexp(1.0 + (double)M / ldexp(1.0, mb), (int)E - 1 + emin);
}

/* binary32 -> bfloat16, round to nearest even on the bit pattern. */
uint16_t orc_narrow_bf16(float v)
{
    uint32_t b = bits_of_f(v);
    if (isnan(v)) return (uint16_t)((b >> 16) | 0x40);
    uint32_t lsb = (b >> 16) & 1u;
    return (uint16_t)((b + 0x7fffu + lsb) >> 16);
}

/* binary32 -> IEEE binary16, round to nearest even, overflow to inf. */
uint16_t orc_narrow_f16(float v)
{
    uint16_t s = (uint16_t)(signbit(v) ? 0x8000 : 0);
    if (isnan(v)) return 0x7e00;
    double a = fabs((double)v);
    /* largest finite 65504; the midpoint to 2^16 is 65520, whose tie goes
     * to the even neighbour 2^16, i.e. overflow. */
    if (a >= 65520.0) return (uint16_t)(s | 0x7c00);
    return (uint16_t)(s | enc_mag(a, 10, -14));
}

static void store_float(void* p, int dt, int64_t i, float v)
{
    if (dt == ORC_F32) ((float*)p)[i] = v;
    else if (dt == ORC_F16) ((uint16_t*)p)[i] = orc_narrow_f16(v);
    else ((uint16_t*)p)[i] = orc_narrow_bf16(v);
}

/* --------------------------------------------------------- OCP E4M3FN */
/* 1 sign, 4 exponent (bias 7, smallest normal exponent -6), 3 fraction
 * bits; no infinities; S.1111.111 is NaN; largest finite 448 (0x7E).
 * Encoding saturates: magnitudes at or above 448 give 448, keeping the sign;
 * the sign of a zero result is kept (-tiny -> 0x80).  NaN is out of
 * contract. */
uint8_t orc_enc_e4m3(float v)
{
    uint8_t s = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    if (a > 448.0) a = 448.0;
    return (uint8_t)(s | enc_mag(a, 3, -6));
}

float orc_dec_e4m3(uint8_t c)
{
    if ((c & 0x7f) == 0x7f) return NAN;
    double v = dec_mag(c & 0x7fu, 3, -6);
    return (float)((c & 0x80) ? -v : v);
}

/* --------------------------------------------------------- OCP E2M1 */
/* 1 sign, 2 exponent (bias 1, smallest normal exponent 0), 1 fraction bit;
 * values 0, .5, 1, 1.5, 2, 3, 4, 6; no inf/NaN; encoding saturates at 6
 * and keeps the sign of zero. */
uint8_t orc_enc_e2m1(float v)
{
    uint8_t s = signbit(v) ? 0x8 : 0;
    double a = fabs((double)v);
    if (a > 6.0) a = 6.0;
    return (uint8_t)(s | enc_mag(a, 1, 0));
}

float orc_dec_e2m1(uint8_t c)
{
    double v = dec_mag(c & 0x7u, 1, 0);
    return (float)((c & 0x8) ? -v : v);
}

/* --------------------------------------------------------- E8M0 */
/* Unsigned exponent byte, bias 127: value 2^(b-127); 0xFF is NaN. */
float orc_dec_e8m0(uint8_t b) { return (float)ldexp(1.0, (int)b - 127); }

/* Shared scale of an MX block whose elements are E2M1 (largest exponent 2):
 * X = 2^(floor(log2 amax) - 2), clamped to the E8M0 range [2^-127, 2^127].
 * Reading for an all-zero block: X = 1 (byte 127). */
uint8_t orc_enc_e8m0_mx(float amax)
{
    if (amax == 0.0f) return 127;
    int e;
    frexp((double)amax, &e);                     /* amax in [2^(e-1), 2^e) */
    int b = (e - 1) - 2 + 127;
    if (b < 0) b = 0;
    if (b > 254) b = 254;
    return (uint8_t)b;
}

/* ------------------------------------------------- integer code ranges */
/* default_q_range of the docs.rs quantize module gives S8 -> [-128, 127]
 * and U8 -> [0, 255]; the 4-bit rows extend that by width.  Reading for
 * symmetric mode: the range is [-qmax, qmax] so the grid is symmetric
 * about zero (the per-tensor workload clamps to [-127, 127]). */
static int code_bits(int code) { return (code == ORC_S4 || code == ORC_U4) ? 4 : 8; }
static int code_signed(int code) { return code == ORC_S8 || code == ORC_S4; }

int orc_default_q_range(int code, int symmetric, int* qmin, int* qmax)
{
    switch (code) {
    case ORC_S8: *qmin = symmetric ? -127 : -128; *qmax = 127; return ORC_OK;
    case ORC_U8: *qmin = 0; *qmax = 255; return symmetric ? ORC_BAD : ORC_OK;
    case ORC_S4: *qmin = symmetric ? -7 : -8; *qmax = 7; return ORC_OK;
    case ORC_U4: *qmin = 0; *qmax = 15; return symmetric ? ORC_BAD : ORC_OK;
    }
    return ORC_BAD;
}

/* ------------------------------------------------------- granularity */
/* Group membership of element e (row-major index) of a tensor.
 *  PerTensor            -> one group.
 *  PerChannel{axis}     -> the element's index along axis.
 *  per token [rows, C]  -> the row (leading dims flattened into rows).
 *  Group{axis, g}       -> g consecutive indices along axis at fixed indices
 *                          of every other axis; the scale tensor has the
 *                          input's shape with shape[axis] -> shape[axis]/g
 *                          (GPTQ weight [N, K] with axis 1 -> [N, K/g]).
 * Reading: "PerChannel == Group with group_size 1" holds where both
 * definitions agree (1-D tensors, and the identities checked in the tests);
 * PerChannel keeps one scale per index along its axis. */
typedef struct {
    int gran;
    int64_t outer, A, inner, g, ngroups, numel;
} orc_groups;

static int make_groups(int ndim, const int64_t* shape, int gran, int axis, int64_t g,
                       orc_groups* G)
{
    if (ndim < 1) return ORC_BAD;
    int64_t numel = 1;
    for (int d = 0; d < ndim; ++d) { if (shape[d] < 0) return ORC_BAD; numel *= shape[d]; }
    G->gran = gran; G->numel = numel; G->g = 1;
    if (gran == ORC_TENSOR) { G->outer = 1; G->A = numel; G->inner = 1; G->ngroups = 1; return ORC_OK; }
    if (gran == ORC_TOKEN) {
        int64_t cols = shape[ndim - 1];
        G->outer = cols ? numel / cols : 0; G->A = cols; G->inner = 1; G->ngroups = G->outer;
        return ORC_OK;
    }
    if (axis < 0 || axis >= ndim) return ORC_BAD;
    G->outer = 1; G->inner = 1; G->A = shape[axis];
    for (int d = 0; d < axis; ++d) G->outer *= shape[d];
    for (int d = axis + 1; d < ndim; ++d) G->inner *= shape[d];
    if (gran == ORC_CHANNEL) { G->ngroups = G->A; return ORC_OK; }
    if (gran == ORC_GROUP) {
        if (g <= 0 || G->A % g) return ORC_BAD;
        G->g = g; G->ngroups = G->outer * (G->A / g) * G->inner;
        return ORC_OK;
    }
    return ORC_BAD;
}

static int64_t group_of(const orc_groups* G, int64_t e)
{
    switch (G->gran) {
    case ORC_TENSOR: return 0;
    case ORC_TOKEN: return e / G->A;
    case ORC_CHANNEL: return (e / G->inner) % G->A;
    default: {
        int64_t i = e % G->inner, a = (e / G->inner) % G->A, o = e / (G->inner * G->A);
        return (o * (G->A / G->g) + a / G->g) * G->inner + i;
    }
    }
}

/* ------------------------------------------------- code storage */
/* 8-bit codes: one byte each (s8 as two's complement).  4-bit codes: two
 * per byte along the last dimension, the even index in the low nibble
 * (the GPTQ-style workload's "low nibble first"). */
static void put_code(void* q, int code, int64_t e, int v)
{
    uint8_t* b = (uint8_t*)q;
    if (code_bits(code) == 8) { b[e] = (uint8_t)(v & 0xff); return; }
    uint8_t nib = (uint8_t)(v & 0xf);
    if (e & 1) b[e >> 1] = (uint8_t)((b[e >> 1] & 0x0f) | (nib << 4));
    else       b[e >> 1] = (uint8_t)((b[e >> 1] & 0xf0) | nib);
}

static int get_code(const void* q, int code, int64_t e)
{
    const uint8_t* b = (const uint8_t*)q;
    int v;
    if (code_bits(code) == 8) v = b[e];
    else v = (e & 1) ? (b[e >> 1] >> 4) : (b[e >> 1] & 0xf);
    if (code_signed(code)) {
        int bits = code_bits(code);
        if (v >= (1 << (bits - 1))) v -= (1 << bits);
    }
    return v;
}

/* zero-points: one byte each in the code's unpacked type (u8 for U8/U4,
 * s8 for S8/S4). */
static int get_zp(const void* zp, int code, int64_t gidx)
{
    if (!zp) return 0;
    const uint8_t* b = (const uint8_t*)zp;
    return code_signed(code) ? (int)(int8_t)b[gidx] : (int)b[gidx];
}

static void put_zp(void* zp, int64_t gidx, int v) { ((uint8_t*)zp)[gidx] = (uint8_t)(v & 0xff); }

/* ------------------------------------------------- integer quantize */
/* One element's code (round, then add the integer zero-point, then clamp):
 *   q = clamp(rne(x / scale) + zp, qmin, qmax). */
static int encode_int(float x, float scale, int zp, int qmin, int qmax)
{
    float v = x / scale;                         /* IEEE binary32 division */
    double r = rne((double)v) + (double)zp;
    if (r < qmin) r = qmin;
    if (r > qmax) r = qmax;
    return (int)r;
}

/* Scale and zero-point of one group.
 * Symmetric: scale = amax / qmax.
 * Asymmetric (reading for "GPTQ-style" affine quantization; zero is forced
 * into the range so that it is exactly representable):
 *   mn = min(min x, 0), mx = max(max x, 0),
 *   scale = (mx - mn) / (qmax - qmin),
 *   zp = clamp(qmin - rne(mn / scale), qmin, qmax).
 * Degenerate groups (reading): a scale of exactly 0 is replaced by 1. */
static void group_params(float amax, float mn, float mx, int symmetric, int qmin, int qmax,
                         float* scale, int* zp)
{
    float s;
    if (symmetric) {
        s = amax / (float)qmax;
        if (s == 0.0f) s = 1.0f;
        *scale = s; *zp = 0;
        return;
    }
    float range = mx - mn;                       /* binary32 subtraction */
    s = range / (float)(qmax - qmin);
    if (s == 0.0f) s = 1.0f;
    double z = (double)qmin - rne((double)(mn / s));
    if (z < qmin) z = qmin;
    if (z > qmax) z = qmax;
    *scale = s; *zp = (int)z;
}

int orc_quant_int(const void* x, int xt, int ndim, const int64_t* shape, int gran, int axis,
                  int64_t group_size, int code, int qmin, int qmax, int symmetric,
                  int static_scale, void* q, float* scale, void* zp)
{
    orc_groups G;
    if (make_groups(ndim, shape, gran, axis, group_size, &G)) return ORC_BAD;
    if (code_bits(code) == 4 && (shape[ndim - 1] & 1)) return ORC_BAD;
    if (qmin >= qmax || (symmetric && qmin != -qmax)) return ORC_BAD;
    if (!symmetric && !zp) return ORC_BAD;

    int64_t n = G.numel, ng = G.ngroups;
    float* s = (float*)malloc(sizeof(float) * (ng ? ng : 1));
    int* z = (int*)malloc(sizeof(int) * (ng ? ng : 1));
    if (static_scale) {
        for (int64_t gi = 0; gi < ng; ++gi) { s[gi] = scale[gi]; z[gi] = symmetric ? 0 : get_zp(zp, code, gi); }
    } else {
        float* amax = (float*)calloc(ng ? ng : 1, sizeof(float));
        float* mn = (float*)calloc(ng ? ng : 1, sizeof(float));   /* starts at 0: min(.., 0) */
        float* mx = (float*)calloc(ng ? ng : 1, sizeof(float));   /* starts at 0: max(.., 0) */
        for (int64_t e = 0; e < n; ++e) {
            float v = widen(x, xt, e);
            int64_t gi = group_of(&G, e);
            if (fabsf(v) > amax[gi]) amax[gi] = fabsf(v);
            if (v < mn[gi]) mn[gi] = v;
            if (v > mx[gi]) mx[gi] = v;
        }
        for (int64_t gi = 0; gi < ng; ++gi) {
            group_params(amax[gi], mn[gi], mx[gi], symmetric, qmin, qmax, &s[gi], &z[gi]);
            scale[gi] = s[gi];
            if (!symmetric) put_zp(zp, gi, z[gi]);
        }
        free(amax); free(mn); free(mx);
    }
    for (int64_t e = 0; e < n; ++e) {
        int64_t gi = group_of(&G, e);
        put_code(q, code, e, encode_int(widen(x, xt, e), s[gi], z[gi], qmin, qmax));
    }
    free(s); free(z);
    return ORC_OK;
}

/* y = (q - zp) * scale, rounded once to the output type. */
int orc_dequant_int(const void* q, int code, int ndim, const int64_t* shape, int gran, int axis,
                    int64_t group_size, const float* scale, const void* zp, void* y, int yt)
{
    orc_groups G;
    if (make_groups(ndim, shape, gran, axis, group_size, &G)) return ORC_BAD;
    for (int64_t e = 0; e < G.numel; ++e) {
        int64_t gi = group_of(&G, e);
        float d = (float)(get_code(q, code, e) - get_zp(zp, code, gi));
        store_float(y, yt, e, d * scale[gi]);
    }
    return ORC_OK;
}

/* STE backward: q is recomputed from the saved input and the saved scale and
 * zero-point (the amax is not recomputed);
 *   dx = (dy / scale) * (qmin < q < qmax ? 1 : 0)
 * as a literal binary32 product, so a masked element is a zero carrying the
 * sign of dy / scale; dx has the input's type. */
int orc_quant_int_backward(const void* x, int xt, int ndim, const int64_t* shape, int gran,
                           int axis, int64_t group_size, int qmin, int qmax,
                           const float* scale, const void* zp, int code,
                           const void* dy, void* dx)
{
    orc_groups G;
    if (make_groups(ndim, shape, gran, axis, group_size, &G)) return ORC_BAD;
    for (int64_t e = 0; e < G.numel; ++e) {
        int64_t gi = group_of(&G, e);
        int qv = encode_int(widen(x, xt, e), scale[gi], get_zp(zp, code, gi), qmin, qmax);
        float mask = (qmin < qv && qv < qmax) ? 1.0f : 0.0f;
        float g = widen(dy, xt, e) / scale[gi];
        store_float(dx, xt, e, g * mask);
    }
    return ORC_OK;
}

/* Dequantize backward: dq = dy * scale of the element's group, in dy's type. */
int orc_dequant_int_backward(const void* dy, int dyt, int ndim, const int64_t* shape, int gran,
                             int axis, int64_t group_size, const float* scale, void* dq)
{
    orc_groups G;
    if (make_groups(ndim, shape, gran, axis, group_size, &G)) return ORC_BAD;
    for (int64_t e = 0; e < G.numel; ++e)
        store_float(dq, dyt, e, widen(dy, dyt, e) * scale[group_of(&G, e)]);
    return ORC_OK;
}

/* ------------------------------------------------------ FP8 E4M3 blocks */
/* Blocks of br x bc elements of a row-major [rows, cols] tensor (1x128 for
 * activations, 128x128 for weights); scales are [ceil(rows/br),
 * ceil(cols/bc)] fp32, block (i, j) holding element (r, c) with i = r / br,
 * j = c / bc.  Reading for shapes the blocks do not tile: the blocks on the
 * last row / column of blocks are partial and cover only the elements that
 * exist (their amax is over those elements).
 *   scale = amax / 448 (1 if that is 0),  q = E4M3(x / scale). */
static int fp8_dims(int64_t rows, int64_t cols, int64_t br, int64_t bc, int64_t* nbc)
{
    if (rows < 0 || cols < 0 || br <= 0 || bc <= 0) return ORC_BAD;
    *nbc = (cols + bc - 1) / bc;
    return ORC_OK;
}

int orc_quant_fp8_block(const void* x, int xt, int64_t rows, int64_t cols, int64_t br, int64_t bc,
                        uint8_t* q, float* scale)
{
    int64_t nbc;
    if (fp8_dims(rows, cols, br, bc, &nbc)) return ORC_BAD;
    int64_t nb = ((rows + br - 1) / br) * nbc;
    float* amax = (float*)calloc(nb ? nb : 1, sizeof(float));
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int64_t b = (r / br) * nbc + c / bc;
            float a = fabsf(widen(x, xt, r * cols + c));
            if (a > amax[b]) amax[b] = a;
        }
    for (int64_t b = 0; b < nb; ++b) {
        float s = amax[b] / 448.0f;
        scale[b] = (s == 0.0f) ? 1.0f : s;
    }
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int64_t b = (r / br) * nbc + c / bc;
            q[r * cols + c] = orc_enc_e4m3(widen(x, xt, r * cols + c) / scale[b]);
        }
    free(amax);
    return ORC_OK;
}

int orc_dequant_fp8_block(const uint8_t* q, int64_t rows, int64_t cols, int64_t br, int64_t bc,
                          const float* scale, void* y, int yt)
{
    int64_t nbc;
    if (fp8_dims(rows, cols, br, bc, &nbc)) return ORC_BAD;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            store_float(y, yt, r * cols + c,
                        orc_dec_e4m3(q[r * cols + c]) * scale[(r / br) * nbc + c / bc]);
    return ORC_OK;
}

/* STE with the E4M3 saturation bounds: in range means -448 < val(q) < 448. */
int orc_quant_fp8_block_backward(const void* x, int xt, int64_t rows, int64_t cols, int64_t br,
                                 int64_t bc, const float* scale, const void* dy, void* dx)
{
    int64_t nbc;
    if (fp8_dims(rows, cols, br, bc, &nbc)) return ORC_BAD;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int64_t e = r * cols + c;
            float s = scale[(r / br) * nbc + c / bc];
            float qv = orc_dec_e4m3(orc_enc_e4m3(widen(x, xt, e) / s));
            float mask = (-448.0f < qv && qv < 448.0f) ? 1.0f : 0.0f;
            store_float(dx, xt, e, (widen(dy, xt, e) / s) * mask);
        }
    return ORC_OK;
}

int orc_dequant_fp8_block_backward(const void* dy, int dyt, int64_t rows, int64_t cols,
                                   int64_t br, int64_t bc, const float* scale, void* dq)
{
    int64_t nbc;
    if (fp8_dims(rows, cols, br, bc, &nbc)) return ORC_BAD;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            store_float(dq, dyt, r * cols + c,
                        widen(dy, dyt, r * cols + c) * scale[(r / br) * nbc + c / bc]);
    return ORC_OK;
}

/* ------------------------------------------------------ FP4 E2M1 blocks */
/* Row-major [rows, K]; blocks of gs consecutive elements along K (16 for
 * NVFP4, 32 for MXFP4); packed codes [rows, K/2], low nibble = even index;
 * block scales [rows, K/gs], one byte each.
 *
 * NVFP4 (reading of the two-level scale): a per-tensor fp32 scale
 *   s_g = amax_tensor / (6 * 448)   (or the caller's static value; 1 if 0),
 * an E4M3 block scale sb = E4M3(amax_block / (6 * s_g)) (0x38 = 1.0 if it
 * decodes to 0), and the element scale eff = val(sb) * s_g.
 * MXFP4: sb = the E8M0 shared exponent above, eff = 2^(sb - 127).
 * Each element: q = E2M1(x / eff). */
static int fp4_gs(int kind) { return kind == ORC_NVFP4 ? 16 : 32; }

static float fp4_eff(int kind, uint8_t sb, float sg)
{
    if (kind == ORC_NVFP4) return orc_dec_e4m3(sb) * sg;
    return orc_dec_e8m0(sb);
}

static int fp4_dims(int kind, int64_t rows, int64_t k)
{
    if (kind != ORC_NVFP4 && kind != ORC_MXFP4) return ORC_BAD;
    if (rows < 0 || k < 0 || k % fp4_gs(kind)) return ORC_BAD;
    return ORC_OK;
}

int orc_quant_fp4_block(const void* x, int xt, int64_t rows, int64_t k, int kind,
                        uint8_t* packed, uint8_t* bscale, float* global_scale, int static_global)
{
    if (fp4_dims(kind, rows, k)) return ORC_BAD;
    int gs = fp4_gs(kind);
    int64_t nb = k / gs;
    float sg = 1.0f;
    if (kind == ORC_NVFP4) {
        if (static_global) {
            sg = *global_scale;
        } else {
            float amax = 0.0f;
            for (int64_t e = 0; e < rows * k; ++e) {
                float a = fabsf(widen(x, xt, e));
                if (a > amax) amax = a;
            }
            sg = amax / 2688.0f;
            if (sg == 0.0f) sg = 1.0f;
            *global_scale = sg;
        }
    }
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            float amax = 0.0f;
            for (int j = 0; j < gs; ++j) {
                float a = fabsf(widen(x, xt, r * k + b * gs + j));
                if (a > amax) amax = a;
            }
            uint8_t sb;
            if (kind == ORC_NVFP4) {
                sb = orc_enc_e4m3(amax / (6.0f * sg));
                if (orc_dec_e4m3(sb) == 0.0f) sb = 0x38;
            } else {
                sb = orc_enc_e8m0_mx(amax);
            }
            bscale[r * nb + b] = sb;
            float eff = fp4_eff(kind, sb, sg);
            for (int j = 0; j < gs; ++j) {
                int64_t e = r * k + b * gs + j;
                uint8_t c = orc_enc_e2m1(widen(x, xt, e) / eff);
                uint8_t* p = &packed[e >> 1];
                *p = (e & 1) ? (uint8_t)((*p & 0x0f) | (c << 4)) : (uint8_t)((*p & 0xf0) | c);
            }
        }
    return ORC_OK;
}

static uint8_t fp4_code_at(const uint8_t* packed, int64_t e)
{
    return (e & 1) ? (uint8_t)(packed[e >> 1] >> 4) : (uint8_t)(packed[e >> 1] & 0xf);
}

int orc_dequant_fp4_block(const uint8_t* packed, const uint8_t* bscale, const float* global_scale,
                          int64_t rows, int64_t k, int kind, void* y, int yt)
{
    if (fp4_dims(kind, rows, k)) return ORC_BAD;
    int gs = fp4_gs(kind);
    float sg = (kind == ORC_NVFP4) ? *global_scale : 1.0f;
    for (int64_t e = 0; e < rows * k; ++e) {
        int64_t r = e / k, b = (e % k) / gs;
        float eff = fp4_eff(kind, bscale[r * (k / gs) + b], sg);
        store_float(y, yt, e, orc_dec_e2m1(fp4_code_at(packed, e)) * eff);
    }
    return ORC_OK;
}

/* STE with the E2M1 saturation bounds: in range means -6 < val(q) < 6. */
int orc_quant_fp4_block_backward(const void* x, int xt, const uint8_t* bscale,
                                 const float* global_scale, int64_t rows, int64_t k, int kind,
                                 const void* dy, void* dx)
{
    if (fp4_dims(kind, rows, k)) return ORC_BAD;
    int gs = fp4_gs(kind);
    float sg = (kind == ORC_NVFP4) ? *global_scale : 1.0f;
    for (int64_t e = 0; e < rows * k; ++e) {
        int64_t r = e / k, b = (e % k) / gs;
        float eff = fp4_eff(kind, bscale[r * (k / gs) + b], sg);
        float qv = orc_dec_e2m1(orc_enc_e2m1(widen(x, xt, e) / eff));
        float mask = (-6.0f < qv && qv < 6.0f) ? 1.0f : 0.0f;
        store_float(dx, xt, e, (widen(dy, xt, e) / eff) * mask);
    }
    return ORC_OK;
}

int orc_dequant_fp4_block_backward(const void* dy, int dyt, const uint8_t* bscale,
                                   const float* global_scale, int64_t rows, int64_t k, int kind,
                                   void* dq)
{
    if (fp4_dims(kind, rows, k)) return ORC_BAD;
    int gs = fp4_gs(kind);
    float sg = (kind == ORC_NVFP4) ? *global_scale : 1.0f;
    for (int64_t e = 0; e < rows * k; ++e) {
        int64_t r = e / k, b = (e % k) / gs;
        float eff = fp4_eff(kind, bscale[r * (k / gs) + b], sg);
        store_float(dq, dyt, e, widen(dy, dyt, e) * eff);
    }
    return ORC_OK;
}

/* GEMM layout (QuantizedWeight::transpose_for_gemm / _gs): a plain byte
 * transpose; each byte keeps its two nibbles.
 *   packed_t[j][n] = packed[n][j]   ([N, K/2] -> [K/2, N])
 *   scale_t[b][n]  = scale[n][b]    ([N, K/gs] -> [K/gs, N]) */
int orc_fp4_transpose_for_gemm(const uint8_t* packed, const uint8_t* bscale, int64_t n, int64_t k,
                               int64_t gs, uint8_t* packed_t, uint8_t* bscale_t)
{
    if (n < 0 || k < 0 || (k & 1) || gs <= 0 || k % gs) return ORC_BAD;
    int64_t kb = k / 2, nb = k / gs;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < kb; ++j) packed_t[j * n + r] = packed[r * kb + j];
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < nb; ++b) bscale_t[b * n + r] = bscale[r * nb + b];
    return ORC_OK;
}

/* Elementwise access to the scalar primitives for the tests. */
void orc_enc_e4m3_array(const float* v, int64_t n, uint8_t* out)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_enc_e4m3(v[i]); }
void orc_enc_e2m1_array(const float* v, int64_t n, uint8_t* out)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_enc_e2m1(v[i]); }
void orc_narrow_bf16_array(const float* v, int64_t n, uint16_t* out)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_narrow_bf16(v[i]); }
void orc_narrow_f16_array(const float* v, int64_t n, uint16_t* out)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_narrow_f16(v[i]); }
void orc_f16_to_f32_array(const uint16_t* h, int64_t n, float* out)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f32(h[i]); }
void orc_enc_e8m0_mx_array(const float* v, int64_t n, uint8_t* out)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_enc_e8m0_mx(v[i]); }

/* ------------------------------------------------ FP4 layout follow-ons */
/* QuantizedWeight::transpose_concat_for_gemm / _gs / _padded: several
 * weights sharing K, each packed [n_i, K/2] with block scales [n_i, K/gs],
 * transposed and concatenated along N:
 *   packed_t[j][off_i + r] = packed_i[r][j],  scale_t[b][off_i + r] = scale_i[r][b]
 * with off_i = n_0 + ... + n_(i-1), rows of the outputs `stride` bytes long
 * (stride >= sum n_i; the _padded variant rounds it up to a multiple of
 * `align`) and the pad columns zero.  An empty list is an error. */
int orc_fp4_transpose_concat(int nparts, const uint8_t* const* packed, const uint8_t* const* bscale,
                             const int64_t* n, int64_t k, int64_t gs, int64_t stride,
                             uint8_t* packed_t, uint8_t* bscale_t)
{
    if (nparts <= 0 || k < 0 || (k & 1) || gs <= 0 || k % gs) return ORC_BAD;
    int64_t total = 0;
    for (int i = 0; i < nparts; ++i) { if (n[i] < 0) return ORC_BAD; total += n[i]; }
    if (stride < total) return ORC_BAD;
    int64_t kb = k / 2, nb = k / gs;
    memset(packed_t, 0, (size_t)(kb * stride));
    memset(bscale_t, 0, (size_t)(nb * stride));
    int64_t off = 0;
    for (int i = 0; i < nparts; ++i) {
        for (int64_t r = 0; r < n[i]; ++r) {
            for (int64_t j = 0; j < kb; ++j) packed_t[j * stride + off + r] = packed[i][r * kb + j];
            for (int64_t b = 0; b < nb; ++b) bscale_t[b * stride + off + r] = bscale[i][r * nb + b];
        }
        off += n[i];
    }
    return ORC_OK;
}

/* QuantizedWeight::concat_rows: [N1, K/2] + [N2, K/2] -> [N1+N2, K/2] (and the
 * block scales alike) for NVFP4 weights whose per-tensor scales must be
 * bit-identical, else an error (the result carries one scale for every row). */
int orc_fp4_concat_rows(const uint8_t* p1, const uint8_t* s1, float g1, const uint8_t* p2, const uint8_t* s2,
                        float g2, int64_t n1, int64_t n2, int64_t k, uint8_t* pout, uint8_t* sout)
{
    if (n1 < 0 || n2 < 0 || k < 0 || k % 16) return ORC_BAD;
    if (bits_of_f(g1) != bits_of_f(g2)) return ORC_BAD;
    int64_t kb = k / 2, nb = k / 16;
    memcpy(pout, p1, (size_t)(n1 * kb));
    memcpy(pout + n1 * kb, p2, (size_t)(n2 * kb));
    memcpy(sout, s1, (size_t)(n1 * nb));
    memcpy(sout + n1 * nb, s2, (size_t)(n2 * nb));
    return ORC_OK;
}

/* QuantizedWeight::predequant_to_fp8: the weight dequantized with its
 * per-tensor scale applied, stored as E4M3:
 *   out = E4M3(val(q) * eff),  eff = val(sb) * s_g (NVFP4) or 2^(sb-127) (MXFP4)
 * (binary32 products, one rounding each, then the saturating E4M3 encode). */
int orc_fp4_predequant_to_fp8(const uint8_t* packed, const uint8_t* bscale, float sg, int64_t rows, int64_t k,
                              int kind, uint8_t* out)
{
    if (fp4_dims(kind, rows, k)) return ORC_BAD;
    int gs = fp4_gs(kind);
    for (int64_t e = 0; e < rows * k; ++e) {
        int64_t r = e / k, b = (e % k) / gs;
        float eff = fp4_eff(kind, bscale[r * (k / gs) + b], kind == ORC_NVFP4 ? sg : 1.0f);
        out[e] = orc_enc_e4m3(orc_dec_e2m1(fp4_code_at(packed, e)) * eff);
    }
    return ORC_OK;
}

/* ------------------------------------------------ fake quantization */
/* fake_quantize (per-tensor floating-point round trip): every element is
 * quantized with the tensor's scale / zero-point and dequantized at once,
 *   y = narrow_xt((float)(q - zp) * scale),  q = clamp(rne(x / scale) + zp),
 * with scale / zp derived from the data exactly as for per-tensor quantize,
 * or given (static_scale).  y has x's type. */
int orc_fake_quant_per_tensor(const void* x, int xt, int64_t numel, int code, int qmin, int qmax, int symmetric,
                              int static_scale, float* scale, void* zp, void* y)
{
    if (numel < 0 || qmin >= qmax || (symmetric && qmin != -qmax) || (!symmetric && !zp)) return ORC_BAD;
    float s;
    int z;
    if (static_scale) {
        s = *scale;
        z = symmetric ? 0 : get_zp(zp, code, 0);
    } else {
        float amax = 0.0f, mn = 0.0f, mx = 0.0f;
        for (int64_t e = 0; e < numel; ++e) {
            float v = widen(x, xt, e);
            if (fabsf(v) > amax) amax = fabsf(v);
            if (v < mn) mn = v;
            if (v > mx) mx = v;
        }
        group_params(amax, mn, mx, symmetric, qmin, qmax, &s, &z);
        *scale = s;
        if (!symmetric) put_zp(zp, 0, z);
    }
    for (int64_t e = 0; e < numel; ++e) {
        int q = encode_int(widen(x, xt, e), s, z, qmin, qmax);
        store_float(y, xt, e, (float)(q - z) * s);
    }
    return ORC_OK;
}

/* fake_quantize backward, straight-through (reading): the round trip passes
 * the gradient unchanged where the code is strictly inside the range and
 * blocks it at the clamp bounds, q recomputed from the saved x, scale, zp:
 *   dx = narrow_xt(dy * (qmin < q < qmax ? 1 : 0))   (a zero keeps dy's sign). */
int orc_fake_quant_per_tensor_backward(const void* x, int xt, int64_t numel, int code, int qmin, int qmax,
                                       const float* scale, const void* zp, const void* dy, void* dx)
{
    if (numel < 0 || qmin >= qmax) return ORC_BAD;
    int z = get_zp(zp, code, 0);
    for (int64_t e = 0; e < numel; ++e) {
        int q = encode_int(widen(x, xt, e), *scale, z, qmin, qmax);
        float mask = (qmin < q && q < qmax) ? 1.0f : 0.0f;
        store_float(dx, xt, e, widen(dy, xt, e) * mask);
    }
    return ORC_OK;
}

/* ------------------------------------------------ dynamic range quantize */
/* dynamic_range_quantize (compose op; reading of DynamicRangeMode /
 * DynamicRangeScope): the range is taken from the data at the chosen scope
 * and the matching quantize runs with the code's default range for the
 * mode:  mode 0 = symmetric ([-qmax, qmax]), 1 = asymmetric (full range,
 * zero-point);  scope 0 = per tensor, 1 = per token (rows = product of the
 * leading dims), 2 = per channel along `axis`. */
int orc_dynamic_range_quantize(const void* x, int xt, int ndim, const int64_t* shape, int mode, int scope, int axis,
                               int code, void* q, float* scale, void* zp)
{
    int qmin, qmax;
    if (mode != 0 && mode != 1) return ORC_BAD;
    if (orc_default_q_range(code, mode == 0, &qmin, &qmax)) return ORC_BAD;
    int gran = scope == 0 ? ORC_TENSOR : scope == 1 ? ORC_TOKEN : scope == 2 ? ORC_CHANNEL : -1;
    if (gran < 0) return ORC_BAD;
    return orc_quant_int(x, xt, ndim, shape, gran, scope == 2 ? axis : 0, 0, code, qmin, qmax, mode == 0, 0, q,
                         scale, mode == 0 ? NULL : zp);
}

/* ------------------------------------------------------------ MXFP8 */
/* MXFP8 (smile.llm.quant MxFp8: E4M3 elements, one E8M0 scale per 32
 * consecutive elements along the reduction dimension).  Shared scale by the
 * OCP MX v1.0 rule with the element format's largest exponent (8 for E4M3):
 *   X = 2^(floor(log2 amax) - 8), byte = that exponent + 127 clamped to
 *   [0, 254]; reading for an all-zero block: byte 127 (X = 1);
 *   q = E4M3(x / X), saturating at +-448 (amax / X lies in [256, 512)).
 * Row-major [rows, K], K % 32 == 0; q [rows, K] bytes, scales [rows, K/32]. */
uint8_t orc_enc_e8m0_mx8(float amax)
{
    if (amax == 0.0f) return 127;
    int e;
    frexp((double)amax, &e);                     /* amax in [2^(e-1), 2^e) */
    int b = (e - 1) - 8 + 127;
    if (b < 0) b = 0;
    if (b > 254) b = 254;
    return (uint8_t)b;
}

static int mx8_dims(int64_t rows, int64_t k) { return (rows < 0 || k < 0 || k % 32) ? ORC_BAD : ORC_OK; }

int orc_quant_mxfp8(const void* x, int xt, int64_t rows, int64_t k, uint8_t* q, uint8_t* bscale)
{
    if (mx8_dims(rows, k)) return ORC_BAD;
    for (int64_t b = 0; b < rows * k / 32; ++b) {
        float amax = 0.0f;
        for (int j = 0; j < 32; ++j) {
            float a = fabsf(widen(x, xt, b * 32 + j));
            if (a > amax) amax = a;
        }
        uint8_t sb = orc_enc_e8m0_mx8(amax);
        bscale[b] = sb;
        float X = orc_dec_e8m0(sb);
        for (int j = 0; j < 32; ++j) q[b * 32 + j] = orc_enc_e4m3(widen(x, xt, b * 32 + j) / X);
    }
    return ORC_OK;
}

/* y = val(q) * X, rounded once to y's type. */
int orc_dequant_mxfp8(const uint8_t* q, const uint8_t* bscale, int64_t rows, int64_t k, void* y, int yt)
{
    if (mx8_dims(rows, k)) return ORC_BAD;
    for (int64_t e = 0; e < rows * k; ++e) store_float(y, yt, e, orc_dec_e4m3(q[e]) * orc_dec_e8m0(bscale[e / 32]));
    return ORC_OK;
}

/* STE: dx = (dy / X) * (-448 < val(q) < 448 ? 1 : 0), q recomputed from x. */
int orc_quant_mxfp8_backward(const void* x, int xt, const uint8_t* bscale, int64_t rows, int64_t k,
                             const void* dy, void* dx)
{
    if (mx8_dims(rows, k)) return ORC_BAD;
    for (int64_t e = 0; e < rows * k; ++e) {
        float X = orc_dec_e8m0(bscale[e / 32]);
        float qv = orc_dec_e4m3(orc_enc_e4m3(widen(x, xt, e) / X));
        float mask = (-448.0f < qv && qv < 448.0f) ? 1.0f : 0.0f;
        store_float(dx, xt, e, (widen(dy, xt, e) / X) * mask);
    }
    return ORC_OK;
}

/* dq = dy * X. */
int orc_dequant_mxfp8_backward(const void* dy, int dyt, const uint8_t* bscale, int64_t rows, int64_t k, void* dq)
{
    if (mx8_dims(rows, k)) return ORC_BAD;
    for (int64_t e = 0; e < rows * k; ++e) store_float(dq, dyt, e, widen(dy, dyt, e) * orc_dec_e8m0(bscale[e / 32]));
    return ORC_OK;
}
void orc_enc_e8m0_mx8_array(const float* v, int64_t n, uint8_t* out)
{ for (int64_t i = 0; i < n; ++i) out[i] = orc_enc_e8m0_mx8(v[i]); }

/* ------------------------------------------------ FP8 per-tensor */
/* FP8 E4M3 with one fp32 scale for the whole tensor (smile.llm.quant
 * Fp8KvCodec: FP8 KV store / load with per-tensor scales):
 *   scale = amax / 448 (1 if that is 0), or the caller's (static) value;
 *   q = E4M3(x / scale).  Load is the block dequantize with one block. */
int orc_quant_fp8_per_tensor(const void* x, int xt, int64_t numel, int static_scale, float* scale, uint8_t* q)
{
    if (numel < 0) return ORC_BAD;
    float s;
    if (static_scale) {
        s = *scale;
    } else {
        float amax = 0.0f;
        for (int64_t e = 0; e < numel; ++e) {
            float a = fabsf(widen(x, xt, e));
            if (a > amax) amax = a;
        }
        s = amax / 448.0f;
        if (s == 0.0f) s = 1.0f;
        *scale = s;
    }
    for (int64_t e = 0; e < numel; ++e) q[e] = orc_enc_e4m3(widen(x, xt, e) / s);
    return ORC_OK;
}

/* ------------------------------------------------ binary64 inputs */
/* docs.rs quantize overview lists f64 among the input types.  Reading: an
 * f64 input is computed in binary64 throughout -- the same definitions as
 * the binary32 family above with every division, product and rounding done
 * in binary64, scales stored as binary64, outputs (dequantized values and
 * gradients) in binary64:
 *   symmetric : scale = amax / qmax;  asymmetric: mn = min(min x, 0),
 *               mx = max(max x, 0), scale = (mx - mn) / (qmax - qmin),
 *               zp = clamp(qmin - rne(mn / scale), qmin, qmax);  0 -> 1
 *   q  = clamp(rne(x / scale) + zp, qmin, qmax)
 *   y  = (q - zp) * scale
 *   dx = (dy / scale) * 1[qmin < q < qmax]
 *   dq = dy * scale */
static int encode_int64(double x, double scale, int zp, int qmin, int qmax)
{
    double r = rne(x / scale) + (double)zp;
    if (r < qmin) r = qmin;
    if (r > qmax) r = qmax;
    return (int)r;
}

int orc_quant_f64(const double* x, int ndim, const int64_t* shape, int gran, int axis, int64_t group_size, int code,
                  int qmin, int qmax, int symmetric, int static_scale, void* q, double* scale, void* zp)
{
    orc_groups G;
    if (make_groups(ndim, shape, gran, axis, group_size, &G)) return ORC_BAD;
    if (code_bits(code) == 4 && (shape[ndim - 1] & 1)) return ORC_BAD;
    if (qmin >= qmax || (symmetric && qmin != -qmax) || (!symmetric && !zp)) return ORC_BAD;
    int64_t ng = G.ngroups ? G.ngroups : 1;
    int* z = (int*)calloc(ng, sizeof(int));
    if (static_scale) {
        for (int64_t gi = 0; gi < G.ngroups; ++gi) z[gi] = symmetric ? 0 : get_zp(zp, code, gi);
    } else {
        double* amax = (double*)calloc(ng, sizeof(double));
        double* mn = (double*)calloc(ng, sizeof(double));
        double* mx = (double*)calloc(ng, sizeof(double));
        for (int64_t e = 0; e < G.numel; ++e) {
            int64_t gi = group_of(&G, e);
            if (fabs(x[e]) > amax[gi]) amax[gi] = fabs(x[e]);
            if (x[e] < mn[gi]) mn[gi] = x[e];
            if (x[e] > mx[gi]) mx[gi] = x[e];
        }
        for (int64_t gi = 0; gi < G.ngroups; ++gi) {
            double s;
            if (symmetric) {
                s = amax[gi] / (double)qmax;
                if (s == 0.0) s = 1.0;
                z[gi] = 0;
            } else {
                s = (mx[gi] - mn[gi]) / (double)(qmax - qmin);
                if (s == 0.0) s = 1.0;
                double zz = (double)qmin - rne(mn[gi] / s);
                if (zz < qmin) zz = qmin;
                if (zz > qmax) zz = qmax;
                z[gi] = (int)zz;
                put_zp(zp, gi, z[gi]);
            }
            scale[gi] = s;
        }
        free(amax); free(mn); free(mx);
    }
    for (int64_t e = 0; e < G.numel; ++e) {
        int64_t gi = group_of(&G, e);
        put_code(q, code, e, encode_int64(x[e], scale[gi], z[gi], qmin, qmax));
    }
    free(z);
    return ORC_OK;
}

int orc_dequant_f64(const void* q, int code, int ndim, const int64_t* shape, int gran, int axis, int64_t group_size,
                    const double* scale, const void* zp, double* y)
{
    orc_groups G;
    if (make_groups(ndim, shape, gran, axis, group_size, &G)) return ORC_BAD;
    for (int64_t e = 0; e < G.numel; ++e) {
        int64_t gi = group_of(&G, e);
        y[e] = (double)(get_code(q, code, e) - get_zp(zp, code, gi)) * scale[gi];
    }
    return ORC_OK;
}

int orc_quant_f64_backward(const double* x, int ndim, const int64_t* shape, int gran, int axis, int64_t group_size,
                           int code, int qmin, int qmax, const double* scale, const void* zp, const double* dy,
                           double* dx)
{
    orc_groups G;
    if (make_groups(ndim, shape, gran, axis, group_size, &G)) return ORC_BAD;
    for (int64_t e = 0; e < G.numel; ++e) {
        int64_t gi = group_of(&G, e);
        int qv = encode_int64(x[e], scale[gi], get_zp(zp, code, gi), qmin, qmax);
        double mask = (qmin < qv && qv < qmax) ? 1.0 : 0.0;
        dx[e] = (dy[e] / scale[gi]) * mask;
    }
    return ORC_OK;
}

int orc_dequant_f64_backward(const double* dy, int ndim, const int64_t* shape, int gran, int axis,
                             int64_t group_size, const double* scale, double* dq)
{
    orc_groups G;
    if (make_groups(ndim, shape, gran, axis, group_size, &G)) return ORC_BAD;
    for (int64_t e = 0; e < G.numel; ++e) dq[e] = dy[e] * scale[group_of(&G, e)];
    return ORC_OK;
}

/* ------------------------------------------------ FP8 block GEMM */
/* smile.llm.quant Fp8BlockGemm: activations in E4M3 with one fp32 scale per
 * 1 x 128 group, weights in E4M3 with one fp32 scale per 128 x 128 tile;
 * out = x W^T.  With qa [M, K], sa [M, K/128], qw [N, K], sw [N/128, K/128]:
 *   y[m][n] = sum over K-blocks kb of (sa[m][kb] * sw[n/128][kb]) *
 *             sum_{k in kb} val(qa[m][k]) * val(qw[n][k])
 * evaluated in binary64 (each block's sum of fp8 products is exact there).
 * yabs receives the same sum with every product and scale taken in magnitude
 * (the scale of the rounding error of any binary32 evaluation order). */
int orc_fp8_block_gemm(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw, int64_t M, int64_t N,
                       int64_t K, double* y, double* yabs)
{
    if (M < 0 || N < 0 || K < 0 || K % 128 || N % 128) return ORC_BAD;
    int64_t nkb = K / 128;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t kb = 0; kb < nkb; ++kb) {
                double s = 0.0, sabs = 0.0;
                for (int64_t k = kb * 128; k < kb * 128 + 128; ++k) {
                    double p = (double)orc_dec_e4m3(qa[m * K + k]) * (double)orc_dec_e4m3(qw[n * K + k]);
                    s += p;
                    sabs += fabs(p);
                }
                double c = (double)sa[m * nkb + kb] * (double)sw[(n / 128) * nkb + kb];
                acc += c * s;
                aacc += fabs(c) * sabs;
            }
            y[m * N + n] = acc;
            if (yabs) yabs[m * N + n] = aacc;
        }
    return ORC_OK;
}

/* ------------------------------------------------ W8A8 quantized linear */
/* baracuda_kernels::quantize module list, quantized_linear: a fused W8A8
 * quantized matmul.  The page names the operation only.  Reading: the
 * activation codes qx [M, K] are symmetric s8 with one fp32 scale per row
 * (the per-token quantizer's output), the weight codes qw [N, K] symmetric s8
 * with one fp32 scale per output channel (per row of W); out = x W^T with
 *   acc[m][n] = sum_k qx[m][k] * qw[n][k]            exact integer
 *   y[m][n]   = ((float)acc[m][n] * sx[m]) * sw[n]   binary32, in that order
 * rounded once more to yt.  K is limited so that every partial sum fits in
 * 32 bits (|acc| <= 128 * 128 * K < 2^31). */
int orc_w8a8_linear(const int8_t* qx, const float* sx, const int8_t* qw, const float* sw, int64_t M, int64_t N,
                    int64_t K, void* y, int yt)
{
    if (M < 0 || N < 0 || K < 0 || K > 131071 || (yt != ORC_F32 && yt != ORC_F16 && yt != ORC_BF16)) return ORC_BAD;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) acc += (int64_t)qx[m * K + k] * (int64_t)qw[n * K + k];
            float v = (float)acc;
            v = v * sx[m];
            v = v * sw[n];
            store_float(y, yt, m * N + n, v);
        }
    return ORC_OK;
}

/* ------------------------------------------------ FP4 weight-only linear */
/* metrale QuantizedWeight (the packed E2M1 weight [N, K/2] with its block
 * scales and fp32 per-tensor scale, made for a 16-bit-activation tile GEMM,
 * w4a16) and smile.llm.quant Nvfp4Linear (an NVFP4 weight-only linear):
 * out = x W^T with W the dequantized weight,
 *   W[n][k] = E2M1(code(n, k)) * val(bscale[n][k / gs]) * s_g     (NVFP4)
 *   W[n][k] = E2M1(code(n, k)) * 2^(bscale[n][k / 32] - 127)      (MXFP4)
 *   y[m][n] = sum_k x[m][k] * W[n][k]
 * x is bf16 [M, K]; codes low nibble first as in the quantizer.  Evaluated in
 * binary64: each product x * E2M1 * scale * s_g has at most 8 + 2 + 4 + 24
 * significant bits, so it is exact, and only the sum rounds (at 2^-53).
 * yabs receives the same sum of magnitudes. */
int orc_fp4_linear(const uint16_t* x, const uint8_t* packed, const uint8_t* bscale, float global_scale, int kind,
                   int64_t M, int64_t N, int64_t K, double* y, double* yabs)
{
    if (fp4_dims(kind, N, K) || M < 0) return ORC_BAD;
    const int gs = fp4_gs(kind);
    const double sg = (kind == ORC_NVFP4) ? (double)global_scale : 1.0;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const uint8_t sb = bscale[n * (K / gs) + k / gs];
                const double s = (kind == ORC_NVFP4) ? (double)orc_dec_e4m3(sb) : (double)orc_dec_e8m0(sb);
                const double p = (double)orc_bf16_to_f32(x[m * K + k]) *
                                 ((double)orc_dec_e2m1(fp4_code_at(packed + n * (K / 2), k)) * s * sg);
                acc += p;
                aacc += fabs(p);
            }
            y[m * N + n] = acc;
            if (yabs) yabs[m * N + n] = aacc;
        }
    return ORC_OK;
}
