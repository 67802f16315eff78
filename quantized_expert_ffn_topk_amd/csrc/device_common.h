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

// The value of lane l ^ S (S a power of two up to 32) of a wave64.  Strides 1
// and 2 are DPP quad permutes (plain VALU), 4 to 16 ds_swizzle xor masks
// (within each half-wave, no LDS memory access), 32 a ds_bpermute.
template <int S>
__device__ __forceinline__ int xor_lane(int v)
{
    static_assert(S == 1 || S == 2 || S == 4 || S == 8 || S == 16 || S == 32, "lane stride");
    if constexpr (S == 1)
        return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    else if constexpr (S == 2)
        return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
    else if constexpr (S == 32)
        return __shfl_xor(v, 32, 64);
    else
        return __builtin_amdgcn_ds_swizzle(v, (S << 10) | 0x1F);            // and 31, xor S
}

template <int S>
__device__ __forceinline__ float xor_lane_f(float v)
{
    return __int_as_float(xor_lane<S>(__float_as_int(v)));
}

template <int S>
__device__ __forceinline__ double xor_lane_d(double v)
{
    const unsigned long long u = __double_as_longlong(v);
    const int lo = xor_lane<S>((int)(u & 0xffffffffull)), hi = xor_lane<S>((int)(u >> 32));
    return __longlong_as_double(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, xor_lane_f<32>(v));
    v = fmaxf(v, xor_lane_f<16>(v));
    v = fmaxf(v, xor_lane_f<8>(v));
    v = fmaxf(v, xor_lane_f<4>(v));
    v = fmaxf(v, xor_lane_f<2>(v));
    v = fmaxf(v, xor_lane_f<1>(v));
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v)
{
    // exact when every partial sum is exactly representable (as it is for the
    // group sums of the projections); otherwise a fixed butterfly order
    v += xor_lane_d<32>(v);
    v += xor_lane_d<16>(v);
    v += xor_lane_d<8>(v);
    v += xor_lane_d<4>(v);
    v += xor_lane_d<2>(v);
    v += xor_lane_d<1>(v);
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

// 16 bytes of expert weights read once per pass: a global load with the
// non-temporal hint (the stream is not kept in the caches; measured 4-10 %
// faster for the decode and MXFP4 weight streams than plain loads).  Not for
// data other blocks read again soon.
__device__ __forceinline__ uint4 load_stream16(const void *p)
{
    typedef unsigned int gu32x4_t __attribute__((ext_vector_type(4)));
    const gu32x4_t v = __builtin_nontemporal_load((const __attribute__((address_space(1))) gu32x4_t *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// The fp16 group scale that goes with such a stream, read with the same
// non-temporal hint: the scale words are read once per pass like the weights
// they scale (the one-token decode step measured 0.9 us faster than with
// plain loads of them, same bits).
__device__ __forceinline__ uint16_t load_stream2(const uint16_t *p)
{
    return __builtin_nontemporal_load((const __attribute__((address_space(1))) uint16_t *)p);
}

// v_dot4_i32_i8: c + sum of four signed byte products.
__device__ __forceinline__ int sdot4(int a, int b, int c)
{
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

}  // namespace moe
