/*
 * Seeded synthetic inputs for the BitLinear W1.58A8 layer.
 *
 * This module only draws random numbers and lays them out; it holds none of
 * the layer's arithmetic (no absmean, no ternarization, no quantization, no
 * product).  The same bytes feed both the CPU oracle and the GPU library.
 *
 * Generator: counter-based SplitMix64.  The output for (key, i) is the
 * SplitMix64 finalizer (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014; constants from Vigna's public-domain
 * splitmix64.c) applied to key + (i + 1) * 0x9E3779B97F4A7C15.  A key is
 * derived from (seed, stream) by finalizing seed and stream separately and
 * mixing them, so every tensor of every workload has its own stream id.
 *
 * Normal deviates: Box-Muller in binary64 (Box and Muller, Ann. Math. Statist.
 * 1958).  Deviate i uses the counters 2i and 2i+1 as two uniforms in (0, 1]
 * and returns sqrt(-2 ln u1) * cos(2 pi u2).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static uint64_t sm64_finalize(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static uint64_t stream_key(uint64_t seed, uint64_t stream) {
    return sm64_finalize(sm64_finalize(seed) ^ (sm64_finalize(stream + GOLDEN) + GOLDEN));
}

static uint64_t draw_u64(uint64_t key, uint64_t counter) {
    return sm64_finalize(key + (counter + 1u) * GOLDEN);
}

/* uniform in (0, 1]: 53 random bits, offset by one so that log() is finite */
static double draw_unit(uint64_t key, uint64_t counter) {
    return (double)((draw_u64(key, counter) >> 11) + 1u) * 0x1.0p-53;
}

static double draw_normal(uint64_t key, uint64_t i) {
    const double two_pi = 6.283185307179586476925286766559;
    double u1 = draw_unit(key, 2u * i);
    double u2 = draw_unit(key, 2u * i + 1u);
    return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/* float -> bf16 bit pattern, round to nearest even (inputs are finite) */
static uint16_t f32_to_bf16_bits(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

/* out[i] = (float)(scale * z_i), i in [0, n) */
void dg_normal_f32(uint64_t seed, uint64_t stream, double scale, int64_t n, float* out) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (float)(scale * draw_normal(key, (uint64_t)i));
}

/* rows x cols bf16 matrix, row r column c = bf16(float(z * mult_c)), where
 * mult_c = outlier_mult for the columns listed in outlier_cols and 1 elsewhere. */
void dg_normal_bf16(uint64_t seed, uint64_t stream, int64_t rows, int64_t cols,
                    const int32_t* outlier_cols, int64_t n_outliers, double outlier_mult,
                    uint16_t* out) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            double z = draw_normal(key, (uint64_t)(r * cols + c));
            out[r * cols + c] = f32_to_bf16_bits((float)z);
        }
        for (int64_t o = 0; o < n_outliers; ++o) {
            int64_t c = outlier_cols[o];
            double z = draw_normal(key, (uint64_t)(r * cols + c));
            out[r * cols + c] = f32_to_bf16_bits((float)(z * outlier_mult));
        }
    }
}

/* n_pick distinct column indices in [0, cols), drawn without replacement by
 * rejection, then sorted ascending.  Requires n_pick <= cols. */
int dg_pick_columns(uint64_t seed, uint64_t stream, int64_t cols, int64_t n_pick, int32_t* out) {
    if (n_pick < 0 || n_pick > cols) return -1;
    uint64_t key = stream_key(seed, stream);
    int64_t got = 0;
    for (uint64_t ctr = 0; got < n_pick; ++ctr) {
        int32_t c = (int32_t)(draw_u64(key, ctr) % (uint64_t)cols);
        int dup = 0;
        for (int64_t j = 0; j < got; ++j) dup |= (out[j] == c);
        if (!dup) out[got++] = c;
    }
    for (int64_t i = 1; i < n_pick; ++i)
        for (int64_t j = i; j > 0 && out[j - 1] > out[j]; --j) {
            int32_t t = out[j]; out[j] = out[j - 1]; out[j - 1] = t;
        }
    return 0;
}

/* raw 64-bit draws, for the generator's own statistical checks */
void dg_raw_u64(uint64_t seed, uint64_t stream, int64_t n, uint64_t* out) {
    uint64_t key = stream_key(seed, stream);
    for (int64_t i = 0; i < n; ++i) out[i] = draw_u64(key, (uint64_t)i);
}
