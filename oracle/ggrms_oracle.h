/*
 * ggrms_oracle.h -- CPU oracle for the fused gated group-RMSNorm.
 *
 * TEST INFRASTRUCTURE.  Only tests, the smoke check and the benchmark's CPU
 * baseline use this.  It is independent of the product library and shares
 * no declarations with it; its dtype codes are its own.
 *
 * All pointers are host pointers.  Strides are in elements.  16-bit data is
 * passed as raw bit patterns (uint16_t).
 */
#ifndef GGRMS_ORACLE_H
#define GGRMS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { GGRMS_ORACLE_F32 = 0, GGRMS_ORACLE_F16 = 1, GGRMS_ORACLE_BF16 = 2 };

/* Flags of ggrms_oracle_forward_ex. */
enum {
    GGRMS_ORACLE_ROUND_INTERMEDIATE = 1, /* gate-first: cast gated*nf before the weight */
    GGRMS_ORACLE_NORM_BEFORE_GATE = 2,   /* out = y * nf(y) * w * silu(gate), all f32 */
    GGRMS_ORACLE_WEIGHT_PER_GROUP = 4    /* weight has group_size values shared by all groups */
};

/*
 * out[n, g*G + j] for every row n < rows and column < width, following the
 * math block of the "gated_group_rmsnorm" page (see ggrms_oracle.c).
 * y, gate and out share `dtype`; norm_weight is f32 with `width` elements.
 * `scratch` holds group_size floats.  Returns 0, or 1 for bad arguments.
 */
int ggrms_oracle_forward(const void* y, const void* gate, const float* norm_weight,
                         void* out, int64_t rows, int64_t width, int64_t group_size,
                         int64_t y_row_stride, int64_t gate_row_stride,
                         int64_t out_row_stride, float eps, int dtype,
                         int round_intermediate, float* scratch);

/* The same with flags; ROUND_INTERMEDIATE together with NORM_BEFORE_GATE is
 * rejected (that operator narrows only at the store).  Returns 0 or 1. */
int ggrms_oracle_forward_ex(const void* y, const void* gate, const float* norm_weight,
                            void* out, int64_t rows, int64_t width, int64_t group_size,
                            int64_t y_row_stride, int64_t gate_row_stride,
                            int64_t out_row_stride, float eps, int dtype, int flags,
                            float* scratch);

/* silu(x) = x / (1 + expf(-x)) in f32. */
float ggrms_oracle_silu(float x);

/* Element-wise casts used by the method (dtype = F16 or BF16). */
void ggrms_oracle_round_array(const float* in, uint16_t* out, int64_t n, int dtype);
/* Rounds the f32 values whose bit patterns are first, first+1, ... (n of them). */
void ggrms_oracle_round_bits_range(uint32_t first, int64_t n, uint16_t* out, int dtype);
void ggrms_oracle_widen_array(const uint16_t* in, float* out, int64_t n, int dtype);
void ggrms_oracle_silu_array(const float* in, float* out, int64_t n);

#ifdef __cplusplus
}
#endif

#endif
