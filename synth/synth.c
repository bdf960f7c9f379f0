/*
 * synth.c - seeded synthetic inputs for the MoE FFN layer.
 *
 * This module only draws numbers. It holds none of the layer's arithmetic
 * (no router, no selection, no dispatch, no FFN): it fills caller-owned host
 * buffers with Gaussian values so that the CPU oracle and the GPU library can
 * be fed the very same bytes.
 *
 * Generator (counter based, so any element can be drawn on its own):
 *   mix64(z)      = the SplitMix64 output function (Steele, Lea, Flood,
 *                   "Fast splittable pseudorandom number generators",
 *                   OOPSLA 2014): z ^= z>>30; z *= 0xBF58476D1CE4E5B9;
 *                   z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31.
 *   key(seed,tid) = mix64(mix64(seed) ^ (tid * 0xD1B54A32D192ED03))
 *   r(i, s)       = mix64(key + (2*i + s + 1) * 0x9E3779B97F4A7C15),  s in {0,1}
 *   u(i, s)       = ((r >> 11) + 1) * 2^-53                 in (0, 1]
 *   z(i)          = sqrt(-2 ln u(i,0)) * cos(2 pi u(i,1))   (Box-Muller,
 *                   cosine branch, in double)
 *   value         = (float)(mean + std * z)   then, for bf16 tensors,
 *                   fp32 -> bf16 round-to-nearest-even on the bit pattern.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define SYNTH_GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z)
{
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tensor_id)
{
    return mix64(mix64(seed) ^ (tensor_id * 0xD1B54A32D192ED03ULL));
}

static inline double unit_open0(uint64_t r)
{
    return (double)((r >> 11) + 1ULL) * (1.0 / 9007199254740992.0);
}

static inline double gauss_at(uint64_t key, uint64_t i)
{
    const double two_pi = 6.283185307179586476925286766559;
    uint64_t r0 = mix64(key + (2ULL * i + 1ULL) * SYNTH_GOLDEN);
    uint64_t r1 = mix64(key + (2ULL * i + 2ULL) * SYNTH_GOLDEN);
    double u0 = unit_open0(r0);
    double u1 = unit_open0(r1);
    return sqrt(-2.0 * log(u0)) * cos(two_pi * u1);
}

/* fp32 -> bf16 bit pattern, round to nearest, ties to even. NaN stays NaN. */
static inline uint16_t f32_to_bf16_rne(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu))
        return (uint16_t)((b >> 16) | 0x0040u);
    uint32_t lsb = (b >> 16) & 1u;
    b += 0x7FFFu + lsb;
    return (uint16_t)(b >> 16);
}

/* Raw 64-bit draw r(i, s); exposed so tests can pin the stream itself. */
uint64_t synth_raw(uint64_t seed, uint64_t tensor_id, uint64_t i, int s)
{
    uint64_t key = stream_key(seed, tensor_id);
    return mix64(key + (2ULL * i + (uint64_t)s + 1ULL) * SYNTH_GOLDEN);
}

uint64_t synth_mix64(uint64_t z) { return mix64(z); }

uint16_t synth_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }

/* Fill out[0..n) with fp32 N(mean, std^2) draws of stream (seed, tensor_id),
 * element i being draw number (offset + i). */
void synth_normal_f32(uint64_t seed, uint64_t tensor_id, uint64_t offset,
                      size_t n, double mean, double std, float* out)
{
    uint64_t key = stream_key(seed, tensor_id);
    long long nn = (long long)n;
#pragma omp parallel for schedule(static)
    for (long long i = 0; i < nn; ++i)
        out[i] = (float)(mean + std * gauss_at(key, offset + (uint64_t)i));
}

/* Same draws, stored as bf16 bit patterns (fp32 value rounded RNE). */
void synth_normal_bf16(uint64_t seed, uint64_t tensor_id, uint64_t offset,
                       size_t n, double mean, double std, uint16_t* out)
{
    uint64_t key = stream_key(seed, tensor_id);
    long long nn = (long long)n;
#pragma omp parallel for schedule(static)
    for (long long i = 0; i < nn; ++i) {
        float v = (float)(mean + std * gauss_at(key, offset + (uint64_t)i));
        out[i] = f32_to_bf16_rne(v);
    }
}
