/*
 * Seeded synthetic inputs for the decode/verify step: weights, KV-cache
 * contents, token ids, Bernoulli coins and uniform integers.
 *
 * This module is an input generator only. It holds none of the step's
 * arithmetic (no normalisation, projection, attention or acceptance). Both
 * the CPU oracle and the GPU path consume the bytes it writes, so the two
 * sides see bit-identical inputs.
 *
 * Every value is a pure function of (seed, stream key, element counter):
 *
 *   raw(key, i)   = SplitMix64 output number i of the generator seeded with
 *                   `key` (Steele, Lea & Flood, "Fast splittable pseudorandom
 *                   number generators", OOPSLA 2014): the state advances by
 *                   the golden-ratio increment 0x9E3779B97F4A7C15 and each
 *                   state is passed through the variant-13 finaliser.
 *   uniform(k,i)  = top 53 bits of raw(k, i) scaled to [0, 1).
 *   normal(k,i)   = Marsaglia's polar method (Marsaglia & Bray, "A convenient
 *                   method for generating normal variables", SIAM Review
 *                   1964) for the pair p = floor(i/2): attempt a = 0, 1, ...
 *                   draws u = 2*uniform(k, 256p + 2a) - 1 and
 *                   v = 2*uniform(k, 256p + 2a + 1) - 1 until
 *                   0 < s = u^2 + v^2 < 1, then the pair is
 *                   (u, v) * sqrt(-2 ln(s) / s); even i takes the u branch.
 *                   (Each attempt fails with probability 1 - pi/4; a pair
 *                   never needs its 128 reserved attempts in practice, and
 *                   the last one is taken as is if it ever came to that.)
 *
 * Element i of a tensor is therefore available without generating
 * elements 0..i-1, which lets a checker regenerate any slice of a very large
 * tensor (a KV page, one layer's weights) on its own.
 *
 * Floating-point outputs are rounded to the requested storage type with
 * round-to-nearest-even (fp32 -> fp16 / bf16 conversions written here from
 * the IEEE-754 binary16 and bfloat16 bit layouts).
 *
 * Build: gcc -O3 -fopenmp -shared -fPIC synth.c -o libsynth.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

enum { SYNTH_F32 = 0, SYNTH_F16 = 1, SYNTH_BF16 = 2 };

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Output number i (0-based) of a SplitMix64 generator whose initial state is key. */
static inline uint64_t raw_at(uint64_t key, uint64_t i) {
    return mix64(key + (i + 1) * GOLDEN_GAMMA);
}

/* Uniform double in [0, 1) with 53 random bits. */
static inline double uniform_at(uint64_t key, uint64_t i) {
    return (double)(raw_at(key, i) >> 11) * (1.0 / 9007199254740992.0);
}

/* Derive a stream key from a seed and a list of small integer tags. */
uint64_t synth_key(uint64_t seed, const uint64_t* tags, int n_tags) {
    uint64_t k = mix64(seed ^ 0x5EED5EED5EED5EEDULL);
    for (int t = 0; t < n_tags; ++t) k = mix64(k ^ mix64(tags[t] + (uint64_t)(t + 1) * GOLDEN_GAMMA));
    return k;
}

uint64_t synth_raw(uint64_t key, uint64_t i) { return raw_at(key, i); }

/* ---- rounding fp32 -> binary16 / bfloat16, round to nearest, ties to even ---- */

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40); /* NaN */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static inline uint16_t f32_to_f16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t sign = (u >> 16) & 0x8000u;
    uint32_t absu = u & 0x7FFFFFFFu;
    if (absu >= 0x7F800000u) return (uint16_t)(sign | 0x7C00u | (absu > 0x7F800000u ? 0x200u : 0u));
    int32_t exp = (int32_t)(absu >> 23) - 127;    /* unbiased exponent */
    uint32_t mant = (absu & 0x7FFFFFu) | 0x800000u; /* 24-bit significand with hidden bit */
    if (absu == 0) return (uint16_t)sign;
    if (exp > 15) return (uint16_t)(sign | 0x7C00u); /* overflow to infinity */
    /* binary16: normal exponents -14..15 keep 10 fraction bits; below -14 the
       value is subnormal with a fixed scale of 2^-24. */
    int shift; /* number of low significand bits to drop */
    uint32_t he;
    if (exp >= -14) {
        shift = 13;
        he = (uint32_t)(exp + 15);
    } else {
        shift = 13 + (-14 - exp);
        he = 0;
        if (shift > 24) return (uint16_t)sign; /* far below half the smallest subnormal */
    }
    uint32_t kept = mant >> shift;
    uint32_t rem = mant & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (kept & 1u))) kept += 1u;
    if (he == 0) {
        /* subnormal: kept counts units of 2^-24; a carry into 0x400 becomes the smallest normal */
        return (uint16_t)(sign | kept);
    }
    /* normal: kept includes the hidden bit at 0x400; a carry to 0x800 bumps the exponent */
    if (kept & 0x800u) {
        kept >>= 1;
        he += 1;
        if (he >= 31) return (uint16_t)(sign | 0x7C00u);
    }
    return (uint16_t)(sign | (he << 10) | (kept & 0x3FFu));
}

static inline void store(void* out, int64_t j, int dtype, double v) {
    float f = (float)v;
    if (dtype == SYNTH_F32) ((float*)out)[j] = f;
    else if (dtype == SYNTH_F16) ((uint16_t*)out)[j] = f32_to_f16_rne(f);
    else ((uint16_t*)out)[j] = f32_to_bf16_rne(f);
}

/* Both normal deviates of pair p (polar method, counter-addressed attempts). */
static inline void normal_pair(uint64_t key, uint64_t p, double* z0, double* z1) {
    double u = 0.0, v = 0.0, s = 0.0;
    for (uint64_t a = 0; a < 128; ++a) {
        u = 2.0 * uniform_at(key, 256 * p + 2 * a) - 1.0;
        v = 2.0 * uniform_at(key, 256 * p + 2 * a + 1) - 1.0;
        s = u * u + v * v;
        if (s > 0.0 && s < 1.0) break;
    }
    if (!(s > 0.0 && s < 1.0)) { /* unreachable in practice; keep the output finite */
        *z0 = 0.0;
        *z1 = 0.0;
        return;
    }
    const double f = sqrt(-2.0 * log(s) / s);
    *z0 = u * f;
    *z1 = v * f;
}

/* out[j] = round(mean + std * normal(key, start + j)) for j in [0, n). */
void synth_normal(uint64_t key, uint64_t start, int64_t n, double mean, double std, int dtype, void* out) {
    if (n <= 0) return;
    uint64_t first_pair = start >> 1;
    uint64_t last_pair = (start + (uint64_t)n - 1) >> 1;
    int64_t n_pairs = (int64_t)(last_pair - first_pair + 1);
#pragma omp parallel for schedule(static)
    for (int64_t pi = 0; pi < n_pairs; ++pi) {
        uint64_t pair = first_pair + (uint64_t)pi;
        double z0, z1;
        normal_pair(key, pair, &z0, &z1);
        uint64_t i0 = 2 * pair;
        if (i0 >= start) store(out, (int64_t)(i0 - start), dtype, mean + std * z0);
        if (i0 + 1 < start + (uint64_t)n) store(out, (int64_t)(i0 + 1 - start), dtype, mean + std * z1);
    }
}

/* out[j] = lo + floor(uniform * (hi - lo)) via a 64x64->128 multiply, j in [0, n). */
void synth_uniform_int(uint64_t key, uint64_t start, int64_t n, int64_t lo, int64_t hi, int32_t* out) {
    uint64_t range = (uint64_t)(hi - lo);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        unsigned __int128 prod = (unsigned __int128)raw_at(key, start + (uint64_t)j) * range;
        out[j] = (int32_t)(lo + (int64_t)(prod >> 64));
    }
}

/* out[j] = uniform(key, start + j) in [0, 1), as doubles. */
void synth_uniform(uint64_t key, uint64_t start, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) out[j] = uniform_at(key, start + (uint64_t)j);
}

/* out[j] = raw 64-bit outputs (used for shuffles by the caller). */
void synth_raw_fill(uint64_t key, uint64_t start, int64_t n, uint64_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) out[j] = raw_at(key, start + (uint64_t)j);
}
