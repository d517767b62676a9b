/*
 * Seeded synthetic inputs, host side.
 *
 * This module produces the inputs of the data-parallel update step (initial
 * master weights and per-replica, per-micro-step gradients).  It holds none of
 * the step's own arithmetic.  A bit-identical device twin lives in
 * synth_gpu.hip; both follow the definition below, written independently.
 *
 * Definition
 *   mix64(z)      : the SplitMix64 output function (Steele, Lea & Flood,
 *                   "Fast splittable pseudorandom number generators", 2014):
 *                   z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
 *                   z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31.
 *   GOLDEN        : 0x9E3779B97F4A7C15.
 *   key(seed, role, step, replica, micro)
 *                 = mix64(mix64(seed + GOLDEN) ^ (role << 56 | step << 32
 *                                                 | replica << 16 | micro))
 *                   with role < 256, step < 2^24, replica, micro < 2^16.
 *   h_i           = mix64(key + (i + 1) * GOLDEN), i.e. output i of a
 *                   SplitMix64 stream whose state starts at key.
 *   z_i           = (sum of the four 16-bit fields of h_i) - 131070, an
 *                   Irwin-Hall(4) integer with variance (65536^2 - 1) / 3.
 *   x_i (binary32) = RNE((float)z_i * c), c a binary32 scale supplied by the
 *                   caller (sigma * sqrt(3) / 65536, times any loss scale).
 *   out_i         = x_i rounded to nearest-even into the output format
 *                   (binary32, binary16 or bfloat16).
 * All arithmetic is integer except one binary32 multiply, so the host and the
 * device produce the same bits.
 */
#include <stdint.h>
#include <string.h>

#define SYN_GOLDEN 0x9E3779B97F4A7C15ULL

enum { SYN_F32 = 0, SYN_F16 = 1, SYN_BF16 = 2 };

static inline uint64_t syn_mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint32_t syn_f32_bits(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    return u;
}

/* binary32 -> bfloat16, round to nearest even; NaN stays a quiet NaN. */
static inline uint16_t syn_to_bf16(float x) {
    uint32_t u = syn_f32_bits(x);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* binary32 -> binary16, round to nearest even, subnormals kept, overflow to
 * infinity, NaN stays a quiet NaN. */
static inline uint16_t syn_to_f16(float x) {
    uint32_t u = syn_f32_bits(x);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t e = (u >> 23) & 0xFFu;
    uint32_t mant = u & 0x007FFFFFu;
    if (e == 0xFFu) return (uint16_t)(sign | 0x7C00u | (mant ? 0x0200u : 0u));
    int32_t ue = (int32_t)e - 127;         /* unbiased exponent */
    if (ue > 15) return (uint16_t)(sign | 0x7C00u);
    if (ue >= -14) {
        /* normal half: 10 kept mantissa bits, 13 dropped */
        uint32_t v = ((uint32_t)(ue + 15) << 10) | (mant >> 13);
        uint32_t rem = mant & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (v & 1u))) v += 1u; /* may carry into inf */
        return (uint16_t)(sign | v);
    }
    if (e == 0) return sign; /* binary32 zero or subnormal: far below half's range */
    /* subnormal half: value = m24 * 2^(ue-23), half ulp = 2^-24 */
    uint32_t m24 = mant | 0x00800000u;
    int32_t shift = -ue - 1;               /* (-14 - ue) + 13, >= 14 */
    if (shift > 24) return sign;
    uint32_t v = m24 >> shift;
    uint32_t rem = m24 & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (v & 1u))) v += 1u;
    return (uint16_t)(sign | v);
}

uint64_t synth_stream_key(uint64_t seed, uint32_t role, uint32_t step,
                          uint32_t replica, uint32_t micro) {
    uint64_t fields = ((uint64_t)(role & 0xFFu) << 56) | ((uint64_t)(step & 0xFFFFFFu) << 32) |
                      ((uint64_t)(replica & 0xFFFFu) << 16) | (uint64_t)(micro & 0xFFFFu);
    return syn_mix64(syn_mix64(seed + SYN_GOLDEN) ^ fields);
}

static inline float syn_value(uint64_t key, int64_t i, float c) {
    uint64_t h = syn_mix64(key + (uint64_t)(i + 1) * SYN_GOLDEN);
    int32_t s = (int32_t)(h & 0xFFFFu) + (int32_t)((h >> 16) & 0xFFFFu) +
                (int32_t)((h >> 32) & 0xFFFFu) + (int32_t)((h >> 48) & 0xFFFFu);
    return (float)(s - 131070) * c;
}

/* Writes out[j] for absolute stream positions i = start + j, j < count. */
void synth_normal_host(uint64_t key, int64_t start, int64_t count, float c, int dtype,
                       void* out, int threads) {
    (void)threads;
    int64_t j;
    if (dtype == SYN_F32) {
        float* o = (float*)out;
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
        for (j = 0; j < count; ++j) o[j] = syn_value(key, start + j, c);
    } else if (dtype == SYN_F16) {
        uint16_t* o = (uint16_t*)out;
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
        for (j = 0; j < count; ++j) o[j] = syn_to_f16(syn_value(key, start + j, c));
    } else {
        uint16_t* o = (uint16_t*)out;
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
        for (j = 0; j < count; ++j) o[j] = syn_to_bf16(syn_value(key, start + j, c));
    }
}

/* Test hook: the raw 64-bit hash at one position. */
uint64_t synth_hash_at(uint64_t key, int64_t i) {
    return syn_mix64(key + (uint64_t)(i + 1) * SYN_GOLDEN);
}
