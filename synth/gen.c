/*
 * Counter-based synthetic input generator, CPU side.
 *
 * Holds no arithmetic of the optimizer step.  The device side (gen.hip)
 * implements the same definition independently; tests check that both give
 * identical bits.
 *
 * Definition.  mix() is the SplitMix64 output function (Steele, Lea & Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014), GAMMA its
 * golden-ratio increment.
 *   key  = h4 where h0 = 0, h_{k+1} = mix(h_k + x_k + GAMMA) over
 *          x = (seed, tag, step, src), all arithmetic mod 2^64
 *   x_j  = mix(key + (6*index + j + 1) * GAMMA),  j = 0..5
 *   S    = sum of the twelve 32-bit halves of x_0..x_5
 *   z    = (S - 6*2^32) * 2^-32   (double, exact; Irwin-Hall with n = 12,
 *          mean 0, variance 1, an approximately normal variate)
 *   f32  = (float)(z * sigma)     (double product, then round to nearest)
 *   bf16 = f32 rounded to nearest even
 * With absval set the result is |f32| (used for second-moment states).
 */
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t tag, uint64_t step, uint64_t src)
{
    uint64_t h = 0;
    h = mix(h + seed + GAMMA);
    h = mix(h + tag + GAMMA);
    h = mix(h + step + GAMMA);
    h = mix(h + src + GAMMA);
    return h;
}

static inline float draw(uint64_t key, uint64_t index, double sigma, int absval)
{
    uint64_t s = 0;
    for (uint64_t j = 0; j < 6; ++j) {
        uint64_t x = mix(key + (6 * index + j + 1) * GAMMA);
        s += (x & 0xffffffffull) + (x >> 32);
    }
    double z = (double)((int64_t)s - (int64_t)(6ull << 32)) * 0x1p-32;
    float f = (float)(z * sigma);
    if (absval && f < 0.0f)
        f = -f;
    return f;
}

static inline uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

void synth_normal_f32(float* out, int64_t n, uint64_t seed, uint64_t tag,
                      uint64_t step, uint64_t src, int64_t index_base,
                      double sigma, int32_t absval)
{
    uint64_t key = synth_key(seed, tag, step, src);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = draw(key, (uint64_t)(index_base + i), sigma, absval);
}

void synth_normal_bf16(uint16_t* out, int64_t n, uint64_t seed, uint64_t tag,
                       uint64_t step, uint64_t src, int64_t index_base,
                       double sigma)
{
    uint64_t key = synth_key(seed, tag, step, src);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = to_bf16(draw(key, (uint64_t)(index_base + i), sigma, 0));
}

/* Raw 16-bit patterns (low half of one mix per element): sentinels. */
void synth_bits16(uint16_t* out, int64_t n, uint64_t seed, uint64_t tag,
                  uint64_t step, uint64_t src, int64_t index_base)
{
    uint64_t key = synth_key(seed, tag, step, src);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint16_t)mix(key + ((uint64_t)(index_base + i) + 1) * GAMMA);
}
