// kernels_probe.hip -- a streaming read of device memory for measuring the HBM
// read rate on this part, with the same 16-byte non-temporal loads the decode
// kernels use for their expert weights.  Each block reads 64 KiB (512 threads
// x 8 loads of 16 B in flight, consecutive lanes on consecutive 16 B) and
// writes the XOR of the block's 32-bit words, so that nothing it reads can be
// dropped and a test can check every byte was read.
#include "device_common.h"
#include "host_common.h"

#include <climits>

namespace moe {

constexpr int PROBE_T = 512;                      // threads per block
constexpr int PROBE_U = 8;                        // 16-byte loads per thread
constexpr size_t PROBE_BLOCK = (size_t)PROBE_T * PROBE_U * 16;

__global__ __launch_bounds__(PROBE_T) void stream_read_kernel(const uint4 *__restrict__ src,
                                                             uint32_t *__restrict__ sink)
{
    __shared__ uint32_t red[PROBE_T / 64];
    const uint4 *p = src + (size_t)blockIdx.x * (PROBE_T * PROBE_U) + threadIdx.x;
    uint4 v[PROBE_U];
#pragma unroll
    for (int u = 0; u < PROBE_U; ++u)
        v[u] = load_stream16(p + (size_t)u * PROBE_T);
    uint32_t x = 0u;
#pragma unroll
    for (int u = 0; u < PROBE_U; ++u)
        x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    x ^= (uint32_t)xor_lane<32>((int)x);
    x ^= (uint32_t)xor_lane<16>((int)x);
    x ^= (uint32_t)xor_lane<8>((int)x);
    x ^= (uint32_t)xor_lane<4>((int)x);
    x ^= (uint32_t)xor_lane<2>((int)x);
    x ^= (uint32_t)xor_lane<1>((int)x);
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0u;
#pragma unroll
        for (int w = 0; w < PROBE_T / 64; ++w)
            r ^= red[w];
        sink[blockIdx.x] = r;
    }
}

}  // namespace moe

extern "C" moe_status moe_debug_stream_read(const void *src, size_t bytes, uint32_t *sink,
                                            void *stream)
{
    using namespace moe;
    if (!src || !sink)
        return fail(MOE_E_INVAL, "NULL argument");
    if (bytes == 0 || bytes % PROBE_BLOCK != 0)
        return fail(MOE_E_INVAL, "bytes=%zu must be a nonzero multiple of %zu", bytes, PROBE_BLOCK);
    if (reinterpret_cast<uintptr_t>(src) % 16 != 0)
        return fail(MOE_E_INVAL, "src must be 16-byte aligned");
    const size_t blocks = bytes / PROBE_BLOCK;
    if (blocks > (size_t)INT_MAX)
        return fail(MOE_E_INVAL, "bytes=%zu too large", bytes);
    launch(stream_read_kernel, (int)blocks, PROBE_T, 0, static_cast<hipStream_t>(stream),
           static_cast<const uint4 *>(src), sink);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_OK : hip_fail(e, "stream read launch");
}
