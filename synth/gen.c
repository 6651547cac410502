/*
 * Seeded synthetic inputs for the decoder-block workloads.
 *
 * This file is the single source of random input bytes.  The same host bytes
 * are handed to the CPU oracle and to the GPU library, so neither side carries
 * a generator of its own and nothing here computes any part of the block.
 *
 * Generator (counter based, stateless, so results do not depend on threads):
 *   mix(z)      SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable
 *               pseudorandom number generators", OOPSLA 2014; constants as in
 *               Vigna's public-domain splitmix64.c).
 *   key         mix(seed ^ mix(tensor_id)).
 *   pair j      h1 = mix(key ^ 2j), h2 = mix(key ^ (2j+1));
 *               u1 = ((h1 >> 11) + 1) * 2^-53 in (0,1], u2 = (h2 >> 11) * 2^-53;
 *               Box-Muller in double: rho = sqrt(-2 ln u1),
 *               n[2j] = rho cos(2 pi u2), n[2j+1] = rho sin(2 pi u2).
 *   value       (float)(sigma * n), then optionally bf16 round-to-nearest-even.
 *   integers    element j: h = mix(key ^ j); lo + (((h >> 32) * (hi-lo+1)) >> 32).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix(uint64_t z) {
    z += 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t tensor_key(uint64_t seed, uint64_t tensor_id) {
    return mix(seed ^ mix(tensor_id));
}

/* fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN. */
static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* n normal(0, sigma) values.  out_f32 receives the value actually stored
 * (the bf16-rounded one, widened exactly, when round_bf16 != 0).
 * out_bf16 (nullable) receives the bf16 bits. */
void synth_normal(uint64_t seed, uint64_t tensor_id, int64_t n, double sigma, int round_bf16,
                  float *out_f32, uint16_t *out_bf16) {
    const uint64_t key = tensor_key(seed, tensor_id);
    const int64_t pairs = (n + 1) / 2;
    const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < pairs; ++j) {
        uint64_t h1 = mix(key ^ (uint64_t)(2 * j));
        uint64_t h2 = mix(key ^ (uint64_t)(2 * j + 1));
        double u1 = (double)((h1 >> 11) + 1) * 0x1.0p-53;
        double u2 = (double)(h2 >> 11) * 0x1.0p-53;
        double rho = sqrt(-2.0 * log(u1));
        double v[2] = {rho * cos(two_pi * u2), rho * sin(two_pi * u2)};
        for (int e = 0; e < 2; ++e) {
            int64_t idx = 2 * j + e;
            if (idx >= n) break;
            float f = (float)(sigma * v[e]);
            if (round_bf16) {
                uint16_t b = f32_to_bf16_rne(f);
                if (out_bf16) out_bf16[idx] = b;
                f = bf16_to_f32(b);
            }
            out_f32[idx] = f;
        }
    }
}

/* n integers uniform in [lo, hi] (inclusive); requires hi - lo + 1 <= 2^32. */
void synth_int(uint64_t seed, uint64_t tensor_id, int64_t n, int64_t lo, int64_t hi, int32_t *out) {
    const uint64_t key = tensor_key(seed, tensor_id);
    const uint64_t span = (uint64_t)(hi - lo + 1);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        uint64_t h = mix(key ^ (uint64_t)j);
        out[j] = (int32_t)(lo + (int64_t)(((h >> 32) * span) >> 32));
    }
}

/* bf16 rounding of an existing fp32 array (used for sentinels and constants). */
void synth_round_bf16(int64_t n, const float *in, uint16_t *out_bits, float *out_f32) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint16_t b = f32_to_bf16_rne(in[i]);
        out_bits[i] = b;
        if (out_f32) out_f32[i] = bf16_to_f32(b);
    }
}

uint64_t synth_mix(uint64_t z) { return mix(z); }
