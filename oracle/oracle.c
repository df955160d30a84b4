/*
 * CPU oracle for the BitNet b1.58 BitLinear W1.58A8 layer.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the GPU library never
 * links, calls or includes it, and it shares no code with the GPU library.
 *
 * Every function is the plain definition, written out serially.  OpenMP only
 * splits loops whose iterations are independent (output rows, elements), so
 * results do not depend on the thread count.  Floating point follows IEEE-754
 * binary32 where the method computes in fp32 (built with -ffp-contract=off
 * and without fast-math), and the absmean mean is computed exactly.
 *
 * Sources (the BitNet b1.58 pages):
 *  - bako.co, "BitNet b1.58 and the 1-Bit AI Architecture Revolution",
 *    section "The BitLinear Layer and AbsMean Quantization": gamma is the mean
 *    absolute value of the entire weight matrix; weights are divided by
 *    (gamma + eps), eps = 1e-5, rounded to the nearest integer and clamped to
 *    [-1, 1]; gamma is returned with the ternary tensor.  Same section: the
 *    product of ternary weights and activations needs only additions and
 *    subtractions.
 *  - deepmox.com chapter 8, section "A low-bit model is a whole-stack design":
 *    weights take the values -1, 0, +1; activations use a per-token 8-bit path
 *    (W1.58A8); the GPU path stores four ternary values per 8-bit unit.
 *  - onilabs.co, "A Two-Billion Ternary Bet": activations are quantized
 *    dynamically (per call, from the values themselves).
 *
 * Readings where the pages are silent (listed with reasons in the design notes):
 *  - gamma is the exact mean of |W|, rounded once to fp32 (round to nearest,
 *    ties to even); gamma + eps and W / (gamma + eps) are fp32 operations with
 *    correct rounding; "round" is round-half-to-even (torch.round).
 *  - activation scale s = 127 / max(max_k |x|, 1e-5) in fp32; q = RNE(x * s)
 *    clamped to [-128, 127]; alpha = max_k |x| (absmax) per token.
 *  - output y = acc * gamma * alpha / 127, evaluated in binary64 and rounded
 *    directly to bf16 (nearest, ties to even).
 *  - packed layout: 2-bit code c = q + 1 in {0, 1, 2}; the matrix is cut into
 *    tiles of 16 rows x 64 columns, tiles ordered column-tile fastest, each
 *    tile row-major with 16 bytes per row; inside a row's 16 bytes, the trit
 *    at column offset t (0..63) sits in byte t % 16, bits 2*(t/16) .. +1.
 *    Rows are padded to a multiple of 16 with code 1.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Exact absmean.                                                            */
/* ------------------------------------------------------------------------ */

/* |w| * 2^149 is the integer mant * 2^shift for every finite fp32 w. */
static void abs_times_2p149(float w, uint64_t* mant, int* shift) {
    uint32_t bits;
    memcpy(&bits, &w, sizeof bits);
    bits &= 0x7FFFFFFFu;
    uint32_t biased = bits >> 23, frac = bits & 0x7FFFFFu;
    if (biased == 0) {              /* subnormal: frac * 2^-149 */
        *mant = frac;
        *shift = 0;
    } else {                        /* (2^23 + frac) * 2^(biased - 150) */
        *mant = frac | 0x800000u;
        *shift = (int)biased - 1;
    }
}

/* Non-negative integer in base 2^32 (little-endian digits). 12 digits hold
 * sum(|w|) * 2^149 for up to 2^40 finite elements (< 2^(128+149+40)) and
 * that value times a count below 2^40. */
#define NDIG 14
typedef struct { uint64_t d[NDIG]; } wide;

static void wide_normalize(wide* a) {
    uint64_t carry = 0;
    for (int i = 0; i < NDIG; ++i) {
        uint64_t t = a->d[i] + carry;
        a->d[i] = t & 0xFFFFFFFFu;
        carry = t >> 32;
    }
}

/* a += v * 2^shift, with v < 2^64 (digits may exceed 32 bits until normalized) */
static void wide_add_shifted(wide* a, uint64_t v, int shift) {
    int q = shift / 32, r = shift % 32;
    unsigned __int128 x = (unsigned __int128)v << r;
    for (int i = q; x != 0 && i < NDIG; ++i) {
        a->d[i] += (uint64_t)(x & 0xFFFFFFFFu);
        x >>= 32;
    }
}

static int wide_cmp(const wide* a, const wide* b) {
    for (int i = NDIG - 1; i >= 0; --i) {
        if (a->d[i] != b->d[i]) return a->d[i] < b->d[i] ? -1 : 1;
    }
    return 0;
}

/* f * count * 2^149 as an exact integer, for finite f >= 0 */
static wide scaled_float(float f, uint64_t count) {
    wide r;
    memset(&r, 0, sizeof r);
    uint64_t mant;
    int shift;
    abs_times_2p149(f, &mant, &shift);
    unsigned __int128 p = (unsigned __int128)mant * count;
    wide_add_shifted(&r, (uint64_t)p, shift);
    wide_add_shifted(&r, (uint64_t)(p >> 64), shift + 64);
    wide_normalize(&r);
    return r;
}

static wide wide_sum(const wide* a, const wide* b) {
    wide r;
    for (int i = 0; i < NDIG; ++i) r.d[i] = a->d[i] + b->d[i];
    wide_normalize(&r);
    return r;
}

/* Round X / (count * 2^149) to the nearest fp32, ties to even, by bracketing
 * it between two neighbouring floats and comparing exactly. */
static float round_ratio_to_f32(const wide* X, uint64_t count) {
    double approx = 0.0;
    for (int i = NDIG - 1; i >= 0; --i) approx = approx * 4294967296.0 + (double)X->d[i];
    approx = ldexp(approx, -149) / (double)count;
    float lo = (float)approx;
    if (!(lo <= 3.4028234663852886e38f)) lo = 3.4028234663852886e38f;
    while (lo > 0.0f) {             /* ensure lo <= exact */
        wide s = scaled_float(lo, count);
        if (wide_cmp(&s, X) <= 0) break;
        lo = nextafterf(lo, 0.0f);
    }
    for (;;) {                      /* ensure next(lo) > exact */
        float up = nextafterf(lo, INFINITY);
        if (isinf(up)) return lo;
        wide s = scaled_float(up, count);
        if (wide_cmp(&s, X) > 0) break;
        lo = up;
    }
    wide slo = scaled_float(lo, count);
    if (wide_cmp(&slo, X) == 0) return lo;
    float hi = nextafterf(lo, INFINITY);
    wide shi = scaled_float(hi, count);
    wide twice_x = wide_sum(X, X);
    wide mid2 = wide_sum(&slo, &shi);           /* 2 * midpoint, scaled */
    int c = wide_cmp(&twice_x, &mid2);
    if (c < 0) return lo;
    if (c > 0) return hi;
    uint32_t lo_bits;
    memcpy(&lo_bits, &lo, sizeof lo_bits);
    return (lo_bits & 1u) ? hi : lo;            /* tie: even significand */
}

/* gamma = mean over all `count` elements of |w|, exactly, rounded once to fp32. */
float orc_absmean(const float* w, int64_t count) {
    if (count <= 0) return 0.0f;
    wide total;
    memset(&total, 0, sizeof total);
    const int64_t chunk = (int64_t)1 << 24;     /* digits stay below 2^56 per chunk */
    int64_t nchunks = (count + chunk - 1) / chunk;
#pragma omp parallel for schedule(dynamic)
    for (int64_t c = 0; c < nchunks; ++c) {
        wide part;
        memset(&part, 0, sizeof part);
        int64_t end = (c + 1) * chunk < count ? (c + 1) * chunk : count;
        for (int64_t i = c * chunk; i < end; ++i) {
            uint64_t mant;
            int shift;
            abs_times_2p149(w[i], &mant, &shift);
            wide_add_shifted(&part, mant, shift);
        }
        wide_normalize(&part);
#pragma omp critical
        {
            for (int i = 0; i < NDIG; ++i) total.d[i] += part.d[i];
            wide_normalize(&total);
        }
    }
    return round_ratio_to_f32(&total, (uint64_t)count);
}

/* ------------------------------------------------------------------------ */
/* Ternarization: q = clamp(round(w / (gamma + eps)), -1, 1).                */
/* ------------------------------------------------------------------------ */

void orc_ternarize(const float* w, int64_t count, float gamma, int8_t* q) {
    const float eps = 1e-5f;
    float denom = gamma + eps;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        float scaled = w[i] / denom;
        float r = rintf(scaled);            /* nearest, ties to even */
        if (r > 1.0f) r = 1.0f;
        if (r < -1.0f) r = -1.0f;
        q[i] = (int8_t)r;
    }
}

/* ------------------------------------------------------------------------ */
/* Packed layout (4 ternary values per byte).                                */
/* ------------------------------------------------------------------------ */

int64_t orc_packed_bytes(int64_t n, int64_t k) {
    return ((n + 15) / 16) * 16 * (k / 4);
}

/* byte offset and bit offset of trit (row, col) in a matrix with k columns */
static void trit_position(int64_t row, int64_t col, int64_t k, int64_t* byte, int* bit) {
    int64_t tile_row = row / 16, r = row % 16;
    int64_t tile_col = col / 64, t = col % 64;
    int64_t tiles_per_row = k / 64;
    int64_t tile_start = (tile_row * tiles_per_row + tile_col) * 256;
    *byte = tile_start + r * 16 + t % 16;
    *bit = 2 * (t / 16);
}

/* q is [n][k] with values in {-1, 0, 1}; k must be a multiple of 64.
 * Returns 0, or -1 if k is not a multiple of 64, -2 if a value is not a trit. */
int orc_pack(const int8_t* q, int64_t n, int64_t k, uint8_t* packed) {
    if (k % 64 != 0 || n < 0) return -1;
    memset(packed, 0x55, (size_t)orc_packed_bytes(n, k));   /* code 1 = trit 0 */
    for (int64_t row = 0; row < n; ++row) {
        for (int64_t col = 0; col < k; ++col) {
            int8_t v = q[row * k + col];
            if (v < -1 || v > 1) return -2;
            int64_t byte;
            int bit;
            trit_position(row, col, k, &byte, &bit);
            uint8_t code = (uint8_t)(v + 1);
            packed[byte] = (uint8_t)((packed[byte] & ~(3u << bit)) | (code << bit));
        }
    }
    return 0;
}

/* Inverse of orc_pack for the n real rows.  Returns 0, -1 on a bad k, or -3 if
 * a code 3 (no trit) is found anywhere in the buffer, padding rows included. */
int orc_unpack(const uint8_t* packed, int64_t n, int64_t k, int8_t* q) {
    if (k % 64 != 0 || n < 0) return -1;
    int64_t total = orc_packed_bytes(n, k);
    for (int64_t b = 0; b < total; ++b) {
        uint8_t v = packed[b];
        for (int f = 0; f < 4; ++f)
            if (((v >> (2 * f)) & 3u) == 3u) return -3;
    }
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < n; ++row) {
        for (int64_t col = 0; col < k; ++col) {
            int64_t byte;
            int bit;
            trit_position(row, col, k, &byte, &bit);
            q[row * k + col] = (int8_t)((int)((packed[byte] >> bit) & 3u) - 1);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Denser code: five trits per byte (base 3).                                */
/* ------------------------------------------------------------------------ */
/*
 * Sources: bako.co, "BitNet b1.58 and the 1-Bit AI Architecture Revolution",
 * section "The Information Theory of 1.58 Bits": a weight with three states
 * carries log2(3), about 1.58, bits.  deepmox.com chapter 1, "Why Smaller
 * Weights Are Not the Whole Story", section "A different place to make
 * efficiency decisions": the 2B4T model's non-embedding weights take 0.4 GB,
 * less than two bits per weight.
 * Readings (the pages give no format):
 *  - five trits t_0..t_4 share one byte (3^5 = 243 <= 256): 1.6 bits per
 *    weight.  With codes c_d = t_d + 1 the byte holds v = sum_d c_d * 3^(4-d)
 *    (t_0 the most significant base-3 digit) as b = ceil(256 * v / 243), the
 *    base-3 fraction v / 243 scaled to a byte and rounded up; decoding takes
 *    v = floor(243 * b / 256) and its base-3 digits.  (Rounding up keeps
 *    b / 256 inside [v / 243, (v + 1) / 243), so each digit also equals
 *    floor(3 * ((b * 3^d) mod 256) / 256), which a decoder can use instead.)
 *    13 byte values are no code.
 *  - layout: 16-row x 320-column super-tiles of 1024 bytes, column
 *    super-tile fastest (super-tile (i, s) at byte 1024 * (i * ceil(k/320) + s));
 *    inside one, the 320 columns form four groups of 80; group g of row r
 *    owns bytes 256 g + 16 r .. + 15, and its column 80 g + 16 d + j sits in
 *    byte j (0..15) as digit d (0..4).  So digit d of the 16 bytes of (g, r)
 *    is 16 consecutive columns.  Columns past k (the last super-tile is
 *    partial unless 320 divides k) and rows past n hold trit 0.
 */

int64_t orc_packed_bytes_b3(int64_t n, int64_t k) {
    return ((n + 15) / 16) * 16 * ((k + 319) / 320) * 64;
}

static const int pow3[5] = {81, 27, 9, 3, 1};   /* 3^(4 - d) */

/* byte of the five trits t[0..4] (each in {-1, 0, 1}) */
uint8_t orc_b3_encode(const int8_t* t) {
    int v = 0;
    for (int d = 0; d < 5; ++d) v += (t[d] + 1) * pow3[d];
    return (uint8_t)((256 * v + 242) / 243);    /* ceil(256 v / 243) */
}

/* the five trits of byte b; returns 0, or -1 if b is not the code of any
 * five trits */
int orc_b3_decode(uint8_t b, int8_t* t) {
    int v = (243 * (int)b) / 256;               /* floor(243 b / 256) */
    for (int d = 0; d < 5; ++d) t[d] = (int8_t)((v / pow3[d]) % 3 - 1);
    return orc_b3_encode(t) == b ? 0 : -1;
}

static void b3_position(int64_t row, int64_t col, int64_t k, int64_t* byte, int* digit) {
    int64_t supers = (k + 319) / 320;
    int64_t s = col / 320, t = col % 320;
    int64_t g = t / 80, u = t % 80;
    *digit = (int)(u / 16);
    *byte = ((row / 16) * supers + s) * 1024 + g * 256 + (row % 16) * 16 + u % 16;
}

/* q [n][k] with values in {-1, 0, 1}, k a multiple of 64.  Returns 0, -1 on a
 * bad shape, -2 if a value is not a trit. */
int orc_pack_b3(const int8_t* q, int64_t n, int64_t k, uint8_t* packed) {
    if (k % 64 != 0 || n < 0) return -1;
    int64_t total = orc_packed_bytes_b3(n, k);
    int8_t* trits = (int8_t*)malloc((size_t)(total > 0 ? 5 * total : 1));
    if (!trits) return -1;
    memset(trits, 0, (size_t)(5 * total));     /* padding: trit 0 */
    for (int64_t row = 0; row < n; ++row)
        for (int64_t col = 0; col < k; ++col) {
            int8_t v = q[row * k + col];
            if (v < -1 || v > 1) {
                free(trits);
                return -2;
            }
            int64_t byte;
            int digit;
            b3_position(row, col, k, &byte, &digit);
            trits[5 * byte + digit] = v;
        }
    for (int64_t b = 0; b < total; ++b) packed[b] = orc_b3_encode(trits + 5 * b);
    free(trits);
    return 0;
}

/* Inverse of orc_pack_b3 for the n real rows.  Returns 0, -1 on a bad k, or
 * -3 if any byte of the buffer (padding included) is no code. */
int orc_unpack_b3(const uint8_t* packed, int64_t n, int64_t k, int8_t* q) {
    if (k % 64 != 0 || n < 0) return -1;
    int64_t total = orc_packed_bytes_b3(n, k);
    int8_t t[5];
    for (int64_t b = 0; b < total; ++b)
        if (orc_b3_decode(packed[b], t) != 0) return -3;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < n; ++row) {
        int8_t tt[5];
        for (int64_t col = 0; col < k; ++col) {
            int64_t byte;
            int digit;
            b3_position(row, col, k, &byte, &digit);
            orc_b3_decode(packed[byte], tt);
            q[row * k + col] = tt[digit];
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-token absmax 8-bit activation quantization.                          */
/* ------------------------------------------------------------------------ */

static float bf16_bits_to_float(uint16_t h) {
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

void orc_quant_act(const uint16_t* x, int64_t m, int64_t k, int8_t* q, float* alpha) {
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < m; ++row) {
        float amax = 0.0f;
        for (int64_t col = 0; col < k; ++col) {
            float v = fabsf(bf16_bits_to_float(x[row * k + col]));
            if (v > amax) amax = v;
        }
        float scale = 127.0f / (amax > 1e-5f ? amax : 1e-5f);
        for (int64_t col = 0; col < k; ++col) {
            float prod = bf16_bits_to_float(x[row * k + col]) * scale;
            float r = rintf(prod);
            if (r > 127.0f) r = 127.0f;
            if (r < -128.0f) r = -128.0f;
            q[row * k + col] = (int8_t)r;
        }
        alpha[row] = amax;
    }
}

/* ------------------------------------------------------------------------ */
/* The integer product, two ways.                                           */
/* ------------------------------------------------------------------------ */

/* acc[i][j] = sum_t qx[i][t] * qw[j][t].  Returns -1 if a sum leaves int32. */
int orc_linear_mul(const int8_t* qw, const int8_t* qx, int64_t m, int64_t n, int64_t k, int32_t* acc) {
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t j = 0; j < n; ++j) {
        for (int64_t i = 0; i < m; ++i) {
            int64_t s = 0;
            for (int64_t t = 0; t < k; ++t) s += (int64_t)qx[i * k + t] * (int64_t)qw[j * k + t];
            if (s > INT32_MAX || s < INT32_MIN) bad = 1;
            acc[i * n + j] = (int32_t)s;
        }
    }
    return bad ? -1 : 0;
}

/* Addition-only form: sum of x where w = +1 minus sum of x where w = -1;
 * w = 0 contributes nothing.  Returns -2 on a value outside {-1, 0, 1}. */
int orc_linear_add(const int8_t* qw, const int8_t* qx, int64_t m, int64_t n, int64_t k, int32_t* acc) {
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t j = 0; j < n; ++j) {
        for (int64_t i = 0; i < m; ++i) {
            int64_t plus = 0, minus = 0;
            for (int64_t t = 0; t < k; ++t) {
                int8_t w = qw[j * k + t];
                if (w == 1) plus += qx[i * k + t];
                else if (w == -1) minus += qx[i * k + t];
                else if (w != 0) bad = 1;
            }
            acc[i * n + j] = (int32_t)(plus - minus);
        }
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Rescale to bf16.                                                          */
/* ------------------------------------------------------------------------ */

/* Nearest bf16 (ties to even) of a binary64 value, as a bit pattern. */
uint16_t orc_bf16_from_double(double v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isnan(v)) return 0x7FC0u;
    int e;
    frexp(a, &e);                       /* a in [2^(e-1), 2^e) */
    int ulp_exp = e - 8;                /* 8 significant bits */
    if (ulp_exp < -133) ulp_exp = -133; /* subnormal spacing 2^-133 */
    double r = nearbyint(ldexp(a, -ulp_exp));
    double rounded = ldexp(r, ulp_exp);
    if (rounded >= 0x1p128) return (uint16_t)(sign | 0x7F80u);
    float f = (float)rounded;           /* exact */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(sign | (bits >> 16));
}

/* y[i][j] = bf16(acc[i][j] * gamma * alpha[i] / 127), evaluated in binary64 */
void orc_rescale(const int32_t* acc, int64_t m, int64_t n, float gamma, const float* alpha, uint16_t* y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double v = (double)acc[i * n + j] * (double)gamma * (double)alpha[i] / 127.0;
            y[i * n + j] = orc_bf16_from_double(v);
        }
}

/* ------------------------------------------------------------------------ */
/* Whole layer from packed weights (used to time the CPU baseline).          */
/* ------------------------------------------------------------------------ */

/* y = BitLinear(x) with packed ternary weights: quantize x per token, take the
 * integer product reading each trit from the packed buffer, rescale to bf16.
 * xq, alpha and acc are caller-provided scratch/outputs of sizes m*k, m, m*n. */
int orc_bitlinear_forward(const uint8_t* packed, float gamma, const uint16_t* x, int64_t m, int64_t n,
                          int64_t k, int8_t* xq, float* alpha, int32_t* acc, uint16_t* y) {
    if (k % 64 != 0) return -1;
    orc_quant_act(x, m, k, xq, alpha);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        for (int64_t i = 0; i < m; ++i) {
            int64_t s = 0;
            for (int64_t t = 0; t < k; ++t) {
                int64_t byte;
                int bit;
                trit_position(j, t, k, &byte, &bit);
                int w = (int)((packed[byte] >> bit) & 3u) - 1;
                s += (int64_t)w * xq[i * k + t];
            }
            acc[i * n + j] = (int32_t)s;
        }
    }
    orc_rescale(acc, m, n, gamma, alpha, y);
    return 0;
}

/* y = BitLinear(x) with base-3 packed ternary weights (orc_pack_b3): the same
 * steps as orc_bitlinear_forward, reading each trit from the base-3 buffer. */
int orc_bitlinear_forward_b3(const uint8_t* packed, float gamma, const uint16_t* x, int64_t m, int64_t n,
                             int64_t k, int8_t* xq, float* alpha, int32_t* acc, uint16_t* y) {
    if (k % 64 != 0) return -1;
    orc_quant_act(x, m, k, xq, alpha);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        for (int64_t i = 0; i < m; ++i) {
            int64_t s = 0;
            int8_t t[5];
            for (int64_t c = 0; c < k; ++c) {
                int64_t byte;
                int digit;
                b3_position(j, c, k, &byte, &digit);
                orc_b3_decode(packed[byte], t);
                s += (int64_t)t[digit] * xq[i * k + c];
            }
            acc[i * n + j] = (int32_t)s;
        }
    }
    orc_rescale(acc, m, n, gamma, alpha, y);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Squared-ReLU gating after a fused gate+up BitLinear.                      */
/* ------------------------------------------------------------------------ */
/*
 * Sources: deepmox.com chapter 8, section "A low-bit model is a whole-stack
 * design", and onilabs.co, "A Two-Billion Ternary Bet": the 2B4T model places
 * squared ReLU in its feed-forward block, beside the ternary linear layers.
 * Readings (the pages give no formula):
 *  - the feed-forward block is gated, as the gate and up projections of the
 *    2B-shaped model imply: one BitLinear with 2f output rows (one gamma, the
 *    whole matrix's) whose rows 0..f-1 are the gate and f..2f-1 the up
 *    projection; h = relu(g)^2 * u elementwise;
 *  - g and u are the exact rescaled products acc * gamma * alpha / 127 (no
 *    intermediate rounding); h is evaluated in binary64 and rounded once to
 *    bf16 (nearest, ties to even).
 */

/* h[i][j] = bf16(relu(g)^2 * u), g = acc[i][j] * s_i, u = acc[i][f + j] * s_i,
 * s_i = gamma * alpha[i] / 127; acc is [m][2f] in gate-then-up row order. */
void orc_glu(const int32_t* acc, int64_t m, int64_t f, float gamma, const float* alpha, uint16_t* h) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < f; ++j) {
            double s = (double)gamma * (double)alpha[i] / 127.0;
            double g = (double)acc[i * 2 * f + j] * s;
            double u = (double)acc[i * 2 * f + f + j] * s;
            double r = g > 0.0 ? g : 0.0;
            h[i * f + j] = orc_bf16_from_double(r * r * u);
        }
}

/* Row order of a gate+up matrix in its packed form: 16-row tiles alternate,
 * packed row tile 2t = gate rows 16t..16t+15, packed row tile 2t + 1 = up rows
 * 16t..16t+15 (rows f + 16t .. of the [2f][k] matrix); f % 16 == 0.  Returns
 * the source row of packed row p. */
static int64_t glu_source_row(int64_t p, int64_t f) {
    int64_t tile = p / 16, r = p % 16;
    return (tile % 2 == 0 ? 0 : f) + 16 * (tile / 2) + r;
}

/* Pack a gate+up ternary matrix q [2f][k] in the alternating tile order.
 * Returns 0, -1 on a bad shape, -2 if a value is not a trit. */
int orc_pack_glu(const int8_t* q, int64_t f, int64_t k, uint8_t* packed) {
    if (k % 64 != 0 || f < 0 || f % 16 != 0) return -1;
    int8_t* perm = (int8_t*)malloc((size_t)(2 * f * k > 0 ? 2 * f * k : 1));
    if (!perm) return -1;
    for (int64_t p = 0; p < 2 * f; ++p) memcpy(perm + p * k, q + glu_source_row(p, f) * k, (size_t)k);
    int rc = orc_pack(perm, 2 * f, k, packed);
    free(perm);
    return rc;
}

/* Inverse of orc_pack_glu: q [2f][k] in gate-then-up row order. */
int orc_unpack_glu(const uint8_t* packed, int64_t f, int64_t k, int8_t* q) {
    if (k % 64 != 0 || f < 0 || f % 16 != 0) return -1;
    int8_t* perm = (int8_t*)malloc((size_t)(2 * f * k > 0 ? 2 * f * k : 1));
    if (!perm) return -1;
    int rc = orc_unpack(packed, 2 * f, k, perm);
    if (rc == 0)
        for (int64_t p = 0; p < 2 * f; ++p) memcpy(q + glu_source_row(p, f) * k, perm + p * k, (size_t)k);
    free(perm);
    return rc;
}

/* Feed-forward front half from gate+up weights packed in the alternating
 * order: quantize x per token, take the integer products reading each trit
 * from the packed buffer, gate.  acc [m][2f] is returned in gate-then-up
 * order; xq, alpha, acc and h are caller-provided. */
int orc_bitlinear_glu_forward(const uint8_t* packed, float gamma, const uint16_t* x, int64_t m, int64_t f,
                              int64_t k, int8_t* xq, float* alpha, int32_t* acc, uint16_t* h) {
    if (k % 64 != 0 || f % 16 != 0) return -1;
    orc_quant_act(x, m, k, xq, alpha);
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < 2 * f; ++p) {
        int64_t j = glu_source_row(p, f);
        for (int64_t i = 0; i < m; ++i) {
            int64_t s = 0;
            for (int64_t t = 0; t < k; ++t) {
                int64_t byte;
                int bit;
                trit_position(p, t, k, &byte, &bit);
                int w = (int)((packed[byte] >> bit) & 3u) - 1;
                s += (int64_t)w * xq[i * k + t];
            }
            acc[i * 2 * f + j] = (int32_t)s;
        }
    }
    orc_glu(acc, m, f, gamma, alpha, h);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Straight-through backward of the BitLinear.                               */
/* ------------------------------------------------------------------------ */
/*
 * Source: bako.co, "BitNet b1.58 and the 1-Bit AI Architecture Revolution",
 * section "Training Dynamics: The Straight-Through Estimator": the backward
 * pass treats the rounding step as the identity, so gradients pass through
 * the quantized weights to high-precision shadow weights, which are
 * re-quantized at the next forward pass.
 * Readings: both quantizers (weights and activations, rounding and clipping)
 * are the identity in the backward pass and their scales (gamma, alpha) are
 * constants.  The forward in dequantized form is y = xhat * What^T with
 * xhat[i][t] = alpha_i / 127 * qx[i][t] and What[j][t] = gamma * q[j][t], so
 *   dx[i][t] = gamma * sum_j dy[i][j] * q[j][t]          (gradient for x)
 *   dw[j][t] = sum_i dy[i][j] * alpha_i * qx[i][t] / 127  (gradient for the
 *                                                          shadow weights)
 * dy is bf16 [m][n]; dx [m][k] and dw [n][k] are fp32, each evaluated in
 * binary64 and rounded once.
 */
static double bf16_to_double(uint16_t h) { return (double)bf16_bits_to_float(h); }

/* dx from packed weights (the layout of orc_pack). */
int orc_backward_x(const uint8_t* packed, float gamma, const uint16_t* dy, int64_t m, int64_t n, int64_t k,
                   float* dx) {
    if (k % 64 != 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t t = 0; t < k; ++t) {
            double s = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                int64_t byte;
                int bit;
                trit_position(j, t, k, &byte, &bit);
                int w = (int)((packed[byte] >> bit) & 3u) - 1;
                s += (double)w * bf16_to_double(dy[i * n + j]);
            }
            dx[i * k + t] = (float)((double)gamma * s);
        }
    }
    return 0;
}

/* dw from the int8 activations and their per-token absmax. */
void orc_backward_w(const uint16_t* dy, const int8_t* qx, const float* alpha, int64_t m, int64_t n, int64_t k,
                    float* dw) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        for (int64_t t = 0; t < k; ++t) {
            double s = 0.0;
            for (int64_t i = 0; i < m; ++i)
                s += bf16_to_double(dy[i * n + j]) * (double)alpha[i] * (double)qx[i * k + t];
            dw[j * k + t] = (float)(s / 127.0);
        }
    }
}

/* The packed form of q^T ([k][n], n % 64 == 0) from the packed form of q
 * ([n][k]): the layout the backward product reads, since it contracts over
 * the rows of q. */
int orc_pack_transposed(const uint8_t* packed, int64_t n, int64_t k, uint8_t* packed_t) {
    if (k % 64 != 0 || n % 64 != 0) return -1;
    int8_t* q = (int8_t*)malloc((size_t)(n * k > 0 ? n * k : 1));
    int8_t* qt = (int8_t*)malloc((size_t)(n * k > 0 ? n * k : 1));
    int rc = (q && qt) ? orc_unpack(packed, n, k, q) : -1;
    if (rc == 0) {
        for (int64_t j = 0; j < n; ++j)
            for (int64_t t = 0; t < k; ++t) qt[t * n + j] = q[j * k + t];
        rc = orc_pack(qt, k, n, packed_t);
    }
    free(q);
    free(qt);
    return rc;
}

/* Thread count of the OpenMP loops above (results never depend on it; the
 * benchmark's CPU-baseline leg times the oracle at one thread and at all). */
int orc_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
}
