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

// Cross-block hand-off inside one kernel on a multi-XCD GPU.  Each XCD has its
// own L2; a device-scope release fence would write the whole L2 back.  Instead,
// data that another block reads in the same kernel is stored and loaded with
// relaxed device-scope atomics (they bypass the XCD-local L2), the writer waits
// until its stores have completed (s_waitcnt), and a device-scope counter then
// elects the last block, which reads the data with the same atomic loads.
__device__ __forceinline__ void store_dev(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(double *p, double v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(int32_t *p, int32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double load_dev(const double *p)
{
    return __hip_atomic_load(const_cast<double *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_dev(const int32_t *p)
{
    return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// True in every thread of the block that arrives last of `total` at *ctr.
// Callers store their hand-off data with store_dev first.
__device__ __forceinline__ bool block_arrives_last(uint32_t *ctr, uint32_t total, int *s_flag)
{
    __builtin_amdgcn_s_waitcnt(0);        // this thread's stores have completed
    __syncthreads();
    if (threadIdx.x == 0)
        *s_flag = (__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   total - 1u) ? 1 : 0;
    __syncthreads();
    return *s_flag != 0;
}

// v_dot4_i32_i8: c + sum of four signed byte products.
__device__ __forceinline__ int sdot4(int a, int b, int c)
{
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

}  // namespace moe
