// device_common.h -- small device helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16)
{
    return __uint_as_float(bits16 << 16);
}

// fp16 bits -> fp32 (exact; v_cvt_f32_f16 keeps subnormals).
__device__ __forceinline__ float f16_to_f32(uint16_t h)
{
    _Float16 v = __builtin_bit_cast(_Float16, h);
    return (float)v;
}

// fp32 -> bf16 bits, round to nearest even, NaN made quiet.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return (uint16_t)((u >> 16) | 0x40u);
    uint32_t lower = u & 0xffffu, upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

__device__ __forceinline__ double shfl_xor_d(double v, int m)
{
    return __shfl_xor(v, m, 64);
}

__device__ __forceinline__ float wave_max(float v)
{
    for (int m = 32; m >= 1; m >>= 1)
        v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v)
{
    // exact when every partial sum is exactly representable (as it is for the
    // group sums of the projections); otherwise a fixed butterfly order
    for (int m = 32; m >= 1; m >>= 1)
        v += shfl_xor_d(v, m);
    return v;
}

// Block-wide max of a float for blockDim.x == 256 (4 waves).
__device__ __forceinline__ float block_max_256(float v, float *red4)
{
    v = wave_max(v);
    int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0)
        red4[wave] = v;
    __syncthreads();
    float r = fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
    __syncthreads();
    return r;
}

// v_dot4_i32_i8: c + sum of four signed byte products.
__device__ __forceinline__ int sdot4(int a, int b, int c)
{
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

}  // namespace moe
