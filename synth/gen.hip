/*
 * Counter-based synthetic input generator, device side, plus two
 * calibration kernels for the benchmark.
 *
 * Holds no arithmetic of the optimizer step.  The generator follows the same
 * definition as the CPU side (gen.c), written separately:
 *   key  = h4 where h0 = 0, h_{k+1} = SplitMix64mix(h_k + x_k + GAMMA) over
 *          x = (seed, tag, step, src), arithmetic mod 2^64
 *   x_j  = mix(key + (6*index + j + 1) * GAMMA), j = 0..5
 *   z    = (sum of the twelve 32-bit halves - 6*2^32) * 2^-32   (exact)
 *   f32  = (float)(z * sigma); bf16 = f32 rounded to nearest even
 * (SplitMix64: Steele, Lea & Flood, OOPSLA 2014.)
 *
 * Calibration kernels (benchmark only):
 *   synth_copy_dev       - plain 16-byte copy of a known byte count, the
 *                          reference for scaling the HBM byte counters;
 *   synth_mix_stream_dev - the optimizer step's exact memory access pattern
 *                          (W bf16 slices + three fp32 arrays read, three
 *                          fp32 arrays + one bf16 array written, 16-byte
 *                          accesses) with only integer XORs in between, the
 *                          achievable bandwidth ceiling for that mix.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#define GAMMA 0x9E3779B97F4A7C15ull

__host__ __device__ static inline uint64_t mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static uint64_t host_key(uint64_t seed, uint64_t tag, uint64_t step,
                         uint64_t src)
{
    uint64_t h = 0;
    h = mix(h + seed + GAMMA);
    h = mix(h + tag + GAMMA);
    h = mix(h + step + GAMMA);
    h = mix(h + src + GAMMA);
    return h;
}

__device__ static inline float draw(uint64_t key, uint64_t index, double sigma,
                                    int absval)
{
    uint64_t s = 0;
#pragma unroll
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

__device__ static inline uint16_t to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__global__ void k_normal_f32(float* out, int64_t n, uint64_t key,
                             int64_t index_base, double sigma, int absval)
{
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += stride)
        out[i] = draw(key, (uint64_t)(index_base + i), sigma, absval);
}

__global__ void k_normal_bf16(uint16_t* out, int64_t n, uint64_t key,
                              int64_t index_base, double sigma)
{
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += stride)
        out[i] = to_bf16(draw(key, (uint64_t)(index_base + i), sigma, 0));
}

__global__ void k_bits16(uint16_t* out, int64_t n, uint64_t key,
                         int64_t index_base)
{
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += stride)
        out[i] = (uint16_t)mix(key + ((uint64_t)(index_base + i) + 1) * GAMMA);
}

static unsigned grid_for(int64_t n)
{
    int64_t b = (n + 255) / 256;
    if (b > 65536) b = 65536;
    if (b < 1) b = 1;
    return (unsigned)b;
}

static int finish(void)
{
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int synth_normal_f32_dev(float* out, int64_t n, uint64_t seed,
                                    uint64_t tag, uint64_t step, uint64_t src,
                                    int64_t index_base, double sigma,
                                    int32_t absval, void* stream)
{
    if (n < 0 || (n > 0 && !out)) return -1;
    if (n == 0) return 0;
    hipLaunchKernelGGL(k_normal_f32, dim3(grid_for(n)), dim3(256), 0,
                       (hipStream_t)stream, out, n,
                       host_key(seed, tag, step, src), index_base, sigma,
                       (int)absval);
    return finish();
}

extern "C" int synth_normal_bf16_dev(uint16_t* out, int64_t n, uint64_t seed,
                                     uint64_t tag, uint64_t step, uint64_t src,
                                     int64_t index_base, double sigma,
                                     void* stream)
{
    if (n < 0 || (n > 0 && !out)) return -1;
    if (n == 0) return 0;
    hipLaunchKernelGGL(k_normal_bf16, dim3(grid_for(n)), dim3(256), 0,
                       (hipStream_t)stream, out, n,
                       host_key(seed, tag, step, src), index_base, sigma);
    return finish();
}

extern "C" int synth_bits16_dev(uint16_t* out, int64_t n, uint64_t seed,
                                uint64_t tag, uint64_t step, uint64_t src,
                                int64_t index_base, void* stream)
{
    if (n < 0 || (n > 0 && !out)) return -1;
    if (n == 0) return 0;
    hipLaunchKernelGGL(k_bits16, dim3(grid_for(n)), dim3(256), 0,
                       (hipStream_t)stream, out, n,
                       host_key(seed, tag, step, src), index_base);
    return finish();
}

/* ---- calibration kernels ------------------------------------------------ */

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_copy16(u32x4* __restrict__ dst,
                                                const u32x4* __restrict__ src,
                                                int64_t n16)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n16)
        dst[i] = __builtin_nontemporal_load(&src[i]);
}

extern "C" int synth_copy_dev(void* dst, const void* src, int64_t nbytes,
                              void* stream)
{
    if (nbytes < 0 || (nbytes % 16) || (nbytes && (!dst || !src))) return -1;
    if (((uintptr_t)dst | (uintptr_t)src) & 15u) return -2;
    int64_t n16 = nbytes / 16;
    if (n16 == 0) return 0;
    int64_t blocks = (n16 + 255) / 256;
    if (blocks > 0x7fffffff) return -3;
    hipLaunchKernelGGL(k_copy16, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, (u32x4*)dst, (const u32x4*)src,
                       n16);
    return finish();
}

/* One thread per group of 8 elements: W x 16 B of bf16 read, 3 x 32 B of
 * fp32 read and written, 16 B of bf16 written. */
__global__ __launch_bounds__(256) void k_mix_stream(
    const u32x4* __restrict__ grads, int64_t stride16, int W,
    u32x4* __restrict__ a, u32x4* __restrict__ b, u32x4* __restrict__ c,
    u32x4* __restrict__ p, int64_t n_groups)
{
    int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gi >= n_groups)
        return;
    u32x4 x = __builtin_nontemporal_load(&grads[gi]);
    for (int s = 1; s < W; ++s)
        x ^= __builtin_nontemporal_load(&grads[(int64_t)s * stride16 + gi]);
    u32x4 a0 = a[2 * gi], a1 = a[2 * gi + 1];
    u32x4 b0 = b[2 * gi], b1 = b[2 * gi + 1];
    u32x4 c0 = c[2 * gi], c1 = c[2 * gi + 1];
    a0 ^= x; a1 ^= x; b0 ^= a0; b1 ^= a1; c0 ^= b0; c1 ^= b1;
    __builtin_nontemporal_store(a0, &a[2 * gi]);
    __builtin_nontemporal_store(a1, &a[2 * gi + 1]);
    __builtin_nontemporal_store(b0, &b[2 * gi]);
    __builtin_nontemporal_store(b1, &b[2 * gi + 1]);
    __builtin_nontemporal_store(c0, &c[2 * gi]);
    __builtin_nontemporal_store(c1, &c[2 * gi + 1]);
    __builtin_nontemporal_store(c0 ^ c1, &p[gi]);
}

extern "C" int synth_mix_stream_dev(const void* grads, int64_t grad_stride,
                                    int32_t W, void* a, void* b, void* c,
                                    void* p, int64_t n, void* stream)
{
    if (W < 1 || n < 0 || (n % 8) || (grad_stride % 8) || grad_stride < n)
        return -1;
    if (n == 0) return 0;
    if (!grads || !a || !b || !c || !p) return -1;
    if (((uintptr_t)grads | (uintptr_t)a | (uintptr_t)b | (uintptr_t)c |
         (uintptr_t)p) & 15u)
        return -2;
    int64_t groups = n / 8;
    int64_t blocks = (groups + 255) / 256;
    if (blocks > 0x7fffffff) return -3;
    hipLaunchKernelGGL(k_mix_stream, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, (const u32x4*)grads,
                       grad_stride / 8, (int)W, (u32x4*)a, (u32x4*)b,
                       (u32x4*)c, (u32x4*)p, groups);
    return finish();
}
