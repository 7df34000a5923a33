/*
 * synth.c -- counter-based seeded draws for the synthetic workloads.
 *
 * No arithmetic of the normalisation lives here: this only turns
 * (seed, tensor id, element index) into a float32 draw.
 *
 * SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) is used as a hash of the
 * counter; a normal draw is the cosine branch of the Box-Muller transform in
 * double precision, rounded once to float32.
 */
#include <math.h>
#include <stdint.h>

static uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

static uint64_t stream_key(uint64_t seed, uint64_t tensor_id) {
    return mix64(seed * 0x100000001B3ull + tensor_id * 0xD1B54A32D192ED03ull);
}

static uint64_t draw_bits(uint64_t key, uint64_t idx) {
    return mix64(idx * 0x9E3779B97F4A7C15ull + key);
}

/* (0,1) open interval from 32 bits. */
static double unit_open(uint32_t w) {
    return ((double)w + 0.5) * (1.0 / 4294967296.0);
}

void synth_normal_f32(uint64_t seed, uint64_t tensor_id, uint64_t first, int64_t n,
                      double sigma, float* out) {
    const double two_pi = 6.283185307179586476925286766559;
    uint64_t key = stream_key(seed, tensor_id);
    for (int64_t i = 0; i < n; ++i) {
        uint64_t b = draw_bits(key, first + (uint64_t)i);
        double u1 = unit_open((uint32_t)(b >> 32));
        double u2 = unit_open((uint32_t)b);
        out[i] = (float)(sigma * sqrt(-2.0 * log(u1)) * cos(two_pi * u2));
    }
}

void synth_uniform_f32(uint64_t seed, uint64_t tensor_id, uint64_t first, int64_t n,
                       double lo, double hi, float* out) {
    uint64_t key = stream_key(seed, tensor_id);
    for (int64_t i = 0; i < n; ++i) {
        uint64_t b = draw_bits(key, first + (uint64_t)i);
        out[i] = (float)(lo + (hi - lo) * unit_open((uint32_t)(b >> 32)));
    }
}

/* Row-gather variant: rows[r] * row_len + c for c < row_len. */
void synth_rows_f32(uint64_t seed, uint64_t tensor_id, const int64_t* rows, int64_t nrows,
                    int64_t row_len, int kind, double p0, double p1, float* out) {
    for (int64_t r = 0; r < nrows; ++r) {
        uint64_t first = (uint64_t)rows[r] * (uint64_t)row_len;
        if (kind == 0)
            synth_normal_f32(seed, tensor_id, first, row_len, p0, out + r * row_len);
        else
            synth_uniform_f32(seed, tensor_id, first, row_len, p0, p1, out + r * row_len);
    }
}
