/*
 * synth_gpu.hip -- seeded synthetic inputs (GPU side), the same definition as
 * synth_cpu.c bit for bit (SplitMix64 outputs, Irwin-Hall of four 16-bit
 * uniforms, two binary32 products, optional x100 outliers, truncation to
 * bf16).  Fills device buffers that are too large to draw on the host.  Holds
 * none of the optimizer's arithmetic.  Build with -ffp-contract=off.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ULL
#define OUTLIER_SALT 0x5A5A5A5A5A5A5A5AULL

__device__ __forceinline__ uint64_t finalize64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t at(uint64_t key, uint64_t i)
{
    return finalize64(key + (i + 1) * SM_GAMMA);
}

__device__ __forceinline__ float value(uint64_t key, uint64_t i, float sigma, int outlier_pct)
{
    uint64_t h = at(key, i);
    uint32_t u = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        u += 2u * (uint32_t)((h >> (16 * k)) & 0xFFFFu) + 1u;
    float z = (float)u * 0x1p-17f - 2.0f;
    float x = (z * 1.7320508f) * sigma;
    if (outlier_pct > 0 && at(key ^ OUTLIER_SALT, i) % 100u < (uint64_t)outlier_pct)
        x = x * 100.0f;
    return x;
}

__global__ void fill_f32_kernel(float* out, int64_t n, uint64_t key, uint64_t i0, float sigma, int pct)
{
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
        out[j] = value(key, i0 + (uint64_t)j, sigma, pct);
}

__global__ void fill_bf16_kernel(uint16_t* out, int64_t n, uint64_t key, uint64_t i0, float sigma, int pct)
{
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
        out[j] = (uint16_t)(__float_as_uint(value(key, i0 + (uint64_t)j, sigma, pct)) >> 16);
}

static int grid_for(int64_t n)
{
    int64_t blocks = (n + 255) / 256;
    return (int)(blocks < 16384 ? (blocks > 0 ? blocks : 1) : 16384);
}

extern "C" int synth_gpu_fill_f32(float* out, int64_t n, uint64_t key, uint64_t i0,
                                  float sigma, int outlier_pct, void* stream)
{
    if (n <= 0) return 0;
    if (!out) return 1;
    hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                       out, n, key, i0, sigma, outlier_pct);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int synth_gpu_fill_bf16(uint16_t* out, int64_t n, uint64_t key, uint64_t i0,
                                   float sigma, int outlier_pct, void* stream)
{
    if (n <= 0) return 0;
    if (!out) return 1;
    hipLaunchKernelGGL(fill_bf16_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                       out, n, key, i0, sigma, outlier_pct);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
