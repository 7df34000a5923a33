/*
 * ggrms_oracle.c -- plain CPU oracle for the fused gated group-RMSNorm.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  The product (the HIP
 * library and its Python binding) never links, loads or calls it, and this
 * file shares no code, header, table or helper with the product.
 *
 * What is computed.  The page "gated_group_rmsnorm" (Mojo module doc,
 * max.modular.com, the math block after the intro) defines, for a row n and
 * a group g of group_size = G contiguous columns, col = g*G + j:
 *
 *     gated = f32(y[n,col]) * silu(f32(gate[n,col]))        in f32
 *     m2    = sum over j of gated^2                        in f32
 *     nf    = rsqrt(m2 / G + eps)                          eps after the mean
 *     out   = cast(f32(w[col]) * f32(cast(gated*nf, y.dtype)), out.dtype)
 *
 * The paragraph after the math block says the intermediate cast to the
 * activation dtype comes before the fp32 weight multiply and that the weight
 * is fp32.  The second mode (round_intermediate = 0) keeps gated*nf in f32
 * and narrows only at the store, as the page "com.microsoft.GatedRMSNorm"
 * (Description section) puts it for its own operator.
 *
 * That page's operator itself normalises before gating: the group's
 * normaliser comes from the input alone, nf = 1/sqrt(mean_j y_j^2 + eps), and
 * out = y * nf * w * silu(gate) with every intermediate in f32, where its
 * weight holds one value per column of a group, shared by every group (Inputs
 * table).  It is available with GGRMS_ORACLE_NORM_BEFORE_GATE and
 * GGRMS_ORACLE_WEIGHT_PER_GROUP (which also applies to the gate-first form).
 *
 * Readings where the pages say nothing (each is listed in the design notes):
 *   - silu(x) = x / (1 + exp(-x)), evaluated in f32 with the C library expf.
 *   - m2 is accumulated in f32 in ascending j, one rounding per product and
 *     one per addition (built with -ffp-contract=off, so no fused multiply-add).
 *   - m2 / G is an f32 division by (float)G, eps is added after it, and
 *     rsqrt is 1.0f / sqrtf(.) with the correctly rounded sqrtf.
 *   - Both casts round to nearest, ties to even (IEEE 754 roundTiesToEven),
 *     with gradual underflow (fp16 and bf16 subnormals are kept) and overflow
 *     to infinity.  A NaN stays a NaN (quiet, sign kept).
 *   - In round_intermediate = 0 mode, and for f32 data in either mode, the
 *     intermediate cast is the identity.
 *
 * The rounding helpers below are written from the IEEE 754 definition:
 * round the exact value to the nearest number that has at most p significant
 * bits and an exponent no smaller than emin, ties to the even one.  Every
 * step of that is exact in f32, so it needs no wider type.
 *
 * Parity is pinned in tests/ (exhaustive cast checks against library casts,
 * the unfused op chain built from library routines in fp64, arbitrary
 * precision brute force on tiny inputs, closed forms and invariants).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "ggrms_oracle.h"

/* ---------------------------------------------------------------- formats */

/* Significant bits, minimum normal exponent and largest finite value. */
#define BF16_P 8
#define BF16_EMIN (-126)
#define F16_P 11
#define F16_EMIN (-14)
#define F16_MAX 65504.0f

static uint32_t f32_bits(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    return u;
}

static float f32_from_bits(uint32_t u) {
    float x;
    memcpy(&x, &u, sizeof x);
    return x;
}

/*
 * Nearest value to x with at most p significant bits and exponent >= emin,
 * ties to even, exponent range unbounded above.  x must be finite.
 *
 * With q = 2^e the spacing of that grid around |x| (e = max(floor(log2|x|),
 * emin) - (p - 1)), |x| / q is exact (a power-of-two scaling that neither
 * overflows nor underflows here), its integer part and fraction are exact,
 * and the rounded integer times q is exact again.
 */
static float round_to_grid(float x, int p, int emin) {
    float ax = fabsf(x);
    if (ax == 0.0f) return x;
    int e2;
    (void)frexpf(ax, &e2); /* ax = m * 2^e2 with m in [0.5, 1) */
    int lead = e2 - 1;     /* exponent of the leading bit */
    if (lead < emin) lead = emin;
    int qexp = lead - (p - 1);
    float n = ldexpf(ax, -qexp); /* in [0, 2^p) */
    float k = floorf(n);
    float frac = n - k;
    if (frac > 0.5f || (frac == 0.5f && fmodf(k, 2.0f) != 0.0f)) k += 1.0f;
    float r = ldexpf(k, qexp);
    return copysignf(r, x);
}

/* f32 -> bf16 bit pattern, round to nearest even. */
static uint16_t rne_bf16(float x) {
    uint32_t u = f32_bits(x);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
    if (isinf(x)) return (uint16_t)(sign | 0x7F80u);
    /* bf16 has f32's exponent range; a result past the largest finite bf16
     * comes out of ldexpf as an f32 infinity, which is bf16's infinity. */
    float r = round_to_grid(x, BF16_P, BF16_EMIN);
    /* r has at most 8 significant bits, so its low 16 f32 bits are zero. */
    return (uint16_t)(f32_bits(r) >> 16);
}

/* f32 -> IEEE binary16 bit pattern, round to nearest even. */
static uint16_t rne_f16(float x) {
    uint16_t sign = (uint16_t)((f32_bits(x) >> 16) & 0x8000u);
    if (isnan(x)) return (uint16_t)(sign | 0x7E00u);
    if (isinf(x)) return (uint16_t)(sign | 0x7C00u);
    float r = fabsf(round_to_grid(x, F16_P, F16_EMIN));
    if (r > F16_MAX) return (uint16_t)(sign | 0x7C00u);
    if (r == 0.0f) return sign;
    if (r < ldexpf(1.0f, F16_EMIN)) {
        /* subnormal: r = mant * 2^-24 */
        uint16_t mant = (uint16_t)ldexpf(r, 24);
        return (uint16_t)(sign | mant);
    }
    int e2;
    float m = frexpf(r, &e2); /* r = m * 2^e2, m in [0.5, 1) */
    int lead = e2 - 1;
    uint16_t biased = (uint16_t)(lead + 15);
    uint16_t mant = (uint16_t)(ldexpf(m, 11) - 1024.0f);
    return (uint16_t)(sign | (uint16_t)(biased << 10) | mant);
}

/* bf16 bit pattern -> f32: a bf16 is the upper half of an f32. */
static float widen_bf16(uint16_t h) {
    return f32_from_bits((uint32_t)h << 16);
}

/* IEEE binary16 bit pattern -> f32 (exact). */
static float widen_f16(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    unsigned expo = (h >> 10) & 0x1Fu;
    unsigned mant = h & 0x3FFu;
    if (expo == 0x1Fu) {
        if (mant == 0) return f32_from_bits(sign | 0x7F800000u);
        return f32_from_bits(sign | 0x7FC00000u | (mant << 13));
    }
    float mag;
    if (expo == 0)
        mag = ldexpf((float)mant, -24);
    else
        mag = ldexpf((float)(1024u + mant), (int)expo - 25);
    return sign ? -mag : mag;
}

static float load_elem(const void* base, int64_t idx, int dtype) {
    switch (dtype) {
    case GGRMS_ORACLE_F32: return ((const float*)base)[idx];
    case GGRMS_ORACLE_F16: return widen_f16(((const uint16_t*)base)[idx]);
    default: return widen_bf16(((const uint16_t*)base)[idx]);
    }
}

static void store_elem(void* base, int64_t idx, int dtype, float v) {
    switch (dtype) {
    case GGRMS_ORACLE_F32: ((float*)base)[idx] = v; break;
    case GGRMS_ORACLE_F16: ((uint16_t*)base)[idx] = rne_f16(v); break;
    default: ((uint16_t*)base)[idx] = rne_bf16(v); break;
    }
}

/* The value a cast to `dtype` and back to f32 leaves. */
static float round_trip(float v, int dtype) {
    switch (dtype) {
    case GGRMS_ORACLE_F32: return v;
    case GGRMS_ORACLE_F16: return widen_f16(rne_f16(v));
    default: return widen_bf16(rne_bf16(v));
    }
}

/* ------------------------------------------------------------ the method */

float ggrms_oracle_silu(float x) {
    return x / (1.0f + expf(-x));
}

/*
 * One (row, group) unit.  `a` is caller scratch of G floats; `w` points at
 * the weight of the unit's first column.
 *
 * Gate first (the "gated_group_rmsnorm" page's math block):
 *     a = y * silu(gate); nf = rsqrt(sum a^2 / G + eps);
 *     out = cast(w * [cast](a * nf)).
 * Norm first (the "com.microsoft.GatedRMSNorm" page, Description section,
 * its product read left to right in f32, every intermediate f32):
 *     nf = rsqrt(sum y^2 / G + eps); out = cast(((y * nf) * w) * silu(gate)).
 */
static void one_unit(const void* y, const void* gate, const float* w, void* out,
                     int64_t yoff, int64_t goff, int64_t ooff, int64_t G, float eps,
                     int dtype, int ri, int norm_first, float* a) {
    for (int64_t j = 0; j < G; ++j) {
        float yf = load_elem(y, yoff + j, dtype);
        a[j] = norm_first ? yf : yf * ggrms_oracle_silu(load_elem(gate, goff + j, dtype));
    }
    float m2 = 0.0f;
    for (int64_t j = 0; j < G; ++j) m2 = m2 + a[j] * a[j];
    float nf = 1.0f / sqrtf(m2 / (float)G + eps);
    for (int64_t j = 0; j < G; ++j) {
        float t = a[j] * nf;
        if (norm_first) {
            t = t * w[j];
            t = t * ggrms_oracle_silu(load_elem(gate, goff + j, dtype));
            store_elem(out, ooff + j, dtype, t);
        } else {
            if (ri) t = round_trip(t, dtype);
            store_elem(out, ooff + j, dtype, w[j] * t);
        }
    }
}

int ggrms_oracle_forward_ex(const void* y, const void* gate, const float* norm_weight,
                            void* out, int64_t rows, int64_t width, int64_t group_size,
                            int64_t y_row_stride, int64_t gate_row_stride,
                            int64_t out_row_stride, float eps, int dtype, int flags,
                            float* scratch) {
    if (rows < 0 || width <= 0 || group_size <= 0 || width % group_size != 0) return 1;
    if (dtype != GGRMS_ORACLE_F32 && dtype != GGRMS_ORACLE_F16 &&
        dtype != GGRMS_ORACLE_BF16)
        return 1;
    if (flags & ~(GGRMS_ORACLE_ROUND_INTERMEDIATE | GGRMS_ORACLE_NORM_BEFORE_GATE |
                  GGRMS_ORACLE_WEIGHT_PER_GROUP))
        return 1;
    int ri = (flags & GGRMS_ORACLE_ROUND_INTERMEDIATE) != 0;
    int norm_first = (flags & GGRMS_ORACLE_NORM_BEFORE_GATE) != 0;
    int per_group = (flags & GGRMS_ORACLE_WEIGHT_PER_GROUP) != 0;
    if (ri && norm_first) return 1; /* the norm-first operator narrows only at the store */
    if (rows == 0) return 0;
    if (!y || !gate || !norm_weight || !out || !scratch) return 1;
    int64_t groups = width / group_size;
    for (int64_t n = 0; n < rows; ++n) {
        for (int64_t g = 0; g < groups; ++g) {
            int64_t col0 = g * group_size;
            one_unit(y, gate, norm_weight + (per_group ? 0 : col0), out,
                     n * y_row_stride + col0, n * gate_row_stride + col0,
                     n * out_row_stride + col0, group_size, eps, dtype, ri, norm_first,
                     scratch);
        }
    }
    return 0;
}

int ggrms_oracle_forward(const void* y, const void* gate, const float* norm_weight,
                         void* out, int64_t rows, int64_t width, int64_t group_size,
                         int64_t y_row_stride, int64_t gate_row_stride,
                         int64_t out_row_stride, float eps, int dtype,
                         int round_intermediate, float* scratch) {
    if (round_intermediate != 0 && round_intermediate != 1) return 1;
    return ggrms_oracle_forward_ex(y, gate, norm_weight, out, rows, width, group_size,
                                   y_row_stride, gate_row_stride, out_row_stride, eps, dtype,
                                   round_intermediate ? GGRMS_ORACLE_ROUND_INTERMEDIATE : 0,
                                   scratch);
}

/* ----------------------------------------------- element-wise casts */

void ggrms_oracle_round_array(const float* in, uint16_t* out, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = dtype == GGRMS_ORACLE_F16 ? rne_f16(in[i]) : rne_bf16(in[i]);
}

void ggrms_oracle_round_bits_range(uint32_t first, int64_t n, uint16_t* out, int dtype) {
    for (int64_t i = 0; i < n; ++i) {
        float x = f32_from_bits(first + (uint32_t)i);
        out[i] = dtype == GGRMS_ORACLE_F16 ? rne_f16(x) : rne_bf16(x);
    }
}

void ggrms_oracle_widen_array(const uint16_t* in, float* out, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = dtype == GGRMS_ORACLE_F16 ? widen_f16(in[i]) : widen_bf16(in[i]);
}

void ggrms_oracle_silu_array(const float* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = ggrms_oracle_silu(in[i]);
}
