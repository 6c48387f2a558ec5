/*
 * Seeded synthetic inputs for the decode-step workloads (weights, KV-cache
 * prefill, token ids, positions).  This module holds none of the decode
 * arithmetic: it only turns (seed, tensor name, element index) into numbers.
 *
 * Every element is produced from a counter, so the result does not depend on
 * the order or the number of threads that generate it:
 *
 *   key        = seed XOR FNV-1a-64(name)
 *   raw(k)     = SplitMix64 output number k of a generator started at `key`
 *                (Steele, Lea & Flood, "Fast splittable pseudorandom number
 *                generators", OOPSLA 2014): mix(key + (k+1)*0x9E3779B97F4A7C15)
 *   normal(i)  = Box-Muller (Box & Muller 1958) on two 53-bit uniforms
 *                u1 = raw(2i), u2 = raw(2i+1):  sqrt(-2 ln(1-u1)) cos(2 pi u2)
 *   bf16 value = round-to-nearest-even of (float)(std * normal(i))
 *
 * Integers in [lo, hi] use raw(i) scaled by multiply-shift.
 */
#include <stdint.h>
#include <stddef.h>
#include <math.h>
#include <string.h>

static uint64_t fnv1a64(const char *s) {
    uint64_t h = 0xcbf29ce484222325ull;
    for (; *s; ++s) {
        h ^= (uint8_t)*s;
        h *= 0x100000001b3ull;
    }
    return h;
}

static uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

static uint64_t raw(uint64_t key, uint64_t k) {
    return mix64(key + (k + 1) * 0x9e3779b97f4a7c15ull);
}

static double unit53(uint64_t r) { /* [0, 1) */
    return (double)(r >> 11) * (1.0 / 9007199254740992.0);
}

static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40); /* NaN stays NaN */
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

uint64_t synth_key(uint64_t seed, const char *name) { return seed ^ fnv1a64(name); }

double synth_normal_at(uint64_t seed, const char *name, uint64_t i) {
    uint64_t key = synth_key(seed, name);
    double u1 = unit53(raw(key, 2 * i)), u2 = unit53(raw(key, 2 * i + 1));
    return sqrt(-2.0 * log(1.0 - u1)) * cos(6.283185307179586 * u2);
}

/* out[j] = bf16(std * normal(offset + j)), j < n */
void synth_normal_bf16(uint64_t seed, const char *name, double std_dev, uint64_t offset, uint16_t *out, int64_t n) {
    uint64_t key = synth_key(seed, name);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        uint64_t i = offset + (uint64_t)j;
        double u1 = unit53(raw(key, 2 * i)), u2 = unit53(raw(key, 2 * i + 1));
        double z = sqrt(-2.0 * log(1.0 - u1)) * cos(6.283185307179586 * u2);
        out[j] = f32_to_bf16_rne((float)(std_dev * z));
    }
}

/* out[j] = integer uniform in [lo, hi] (inclusive), j < n */
void synth_uniform_int(uint64_t seed, const char *name, int64_t lo, int64_t hi, uint64_t offset, int32_t *out, int64_t n) {
    uint64_t key = synth_key(seed, name);
    uint64_t span = (uint64_t)(hi - lo) + 1u;
    for (int64_t j = 0; j < n; ++j) {
        uint64_t r = raw(key, offset + (uint64_t)j) >> 32; /* 32 random bits */
        out[j] = (int32_t)(lo + (int64_t)((r * span) >> 32));
    }
}

/* FNV-1a-64 over a byte buffer: a checksum for determinism tests */
uint64_t synth_fnv_bytes(const void *p, int64_t n) {
    const uint8_t *b = (const uint8_t *)p;
    uint64_t h = 0xcbf29ce484222325ull;
    for (int64_t i = 0; i < n; ++i) {
        h ^= b[i];
        h *= 0x100000001b3ull;
    }
    return h;
}
