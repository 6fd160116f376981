/*
 * Seeded, counter-based synthetic input generator.
 *
 * This file holds no part of the attention / eviction method: it only turns
 * (seed, stream, index) triples into numbers.  Both the GPU path and the CPU
 * oracle consume the bytes it writes, so it is the one piece of code the two
 * sides share.
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  The n-th output of a stream
 * with key K is mix(K + (n + 1) * 0x9E3779B97F4A7C15), where mix is the
 * published 64-bit finaliser (shift-xor 30/27/31 with the two odd multipliers).
 * Because every output is a pure function of (key, n), any slice of a stream
 * can be produced independently and in parallel.
 *
 * Uniforms take the top 53 bits: u = (x >> 11 + 0.5) * 2^-53, so u is in (0,1).
 * Normals use the Box-Muller transform (G. Box, M. Muller, 1958) on the pair of
 * uniforms at counters (2i, 2i+1), keeping the cosine branch, in double
 * precision; the result is rounded to float and, for bf16 outputs, to bf16 with
 * round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Key of a stream: the seed and the stream id are mixed separately so that
 * nearby seeds or ids give unrelated keys. */
static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
    return sm64_mix(seed + SM64_GAMMA) ^ sm64_mix(stream * 0xD1B54A32D192ED03ULL + 0x632BE59BD9B4E019ULL);
}

static inline uint64_t sm64_at(uint64_t key, uint64_t n) {
    return sm64_mix(key + (n + 1) * SM64_GAMMA);
}

static inline double u01(uint64_t x) {
    return ((double)(x >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t key, uint64_t i) {
    double u1 = u01(sm64_at(key, 2 * i));
    double u2 = u01(sm64_at(key, 2 * i + 1));
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Outputs n in [start, start + count) of the stream whose key is given
 * directly (key 0 reproduces SplitMix64 seeded with state 0). */
void synth_raw_u64(uint64_t key, uint64_t start, int64_t count, uint64_t* out) {
    for (int64_t i = 0; i < count; ++i) out[i] = sm64_at(key, start + (uint64_t)i);
}

/* Raw 64-bit outputs n in [start, start + count). */
void synth_u64(uint64_t seed, uint64_t stream, uint64_t start, int64_t count, uint64_t* out) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) out[i] = sm64_at(key, start + (uint64_t)i);
}

/* Uniforms in (0,1), double. */
void synth_uniform_f64(uint64_t seed, uint64_t stream, uint64_t start, int64_t count, double* out) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) out[i] = u01(sm64_at(key, start + (uint64_t)i));
}

/* Normals mean + std * N(0,1), element i of the stream uses counters 2i, 2i+1. */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t start, int64_t count,
                      double mean, double std, float* out) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = (float)(mean + std * normal_at(key, start + (uint64_t)i));
}

/* Same values as synth_normal_f32, rounded float -> bf16 (RNE); raw bf16 bits out. */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t start, int64_t count,
                       double mean, double std, uint16_t* out) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = f32_to_bf16_rne((float)(mean + std * normal_at(key, start + (uint64_t)i)));
}

/* Strided bf16 fill: count rows of row_len normals, row r of the stream starting
 * at counter start + r * row_pitch, written to out + r * out_pitch.  Lets a
 * caller pull one head's slice out of a [position][head][dim] stream. */
void synth_normal_bf16_rows(uint64_t seed, uint64_t stream, uint64_t start, int64_t rows,
                            int64_t row_len, int64_t row_pitch, double mean, double std,
                            uint16_t* out, int64_t out_pitch) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < row_len; ++j)
            out[r * out_pitch + j] = f32_to_bf16_rne(
                (float)(mean + std * normal_at(key, start + (uint64_t)(r * row_pitch + j))));
}
