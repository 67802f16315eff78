// noalloc.hip -- moe_layer_forward_noalloc: the layer forward of
// moe_layer_forward (no cache) for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, hosts that forbid
// hipMalloc).  Its workspace is one file-scope device array per GPU instead of
// a context's allocations; the kernels and their launch order are those of
// moe_layer_forward, so the results are the same bits.
//
// Layout of the array: a header of counters at fixed offsets (done [4],
// ctr_gu [E+1] at byte 256, ctr_dn [H/32] at byte 4608), cleared by the
// call's first launch, then the data buffers of the workspace plan carved at
// 256-byte boundaries from byte HEADER_BYTES on, for this call's shape and T.
#include <hip/hip_runtime.h>

#include <mutex>

#include "host_common.h"

using namespace moe;

namespace {

constexpr size_t HEADER_BYTES = 16384;
constexpr size_t CTR_GU_OFF = 256;
constexpr size_t CTR_DN_OFF = 4608;
constexpr int MAX_DEVICES = 64;

}  // namespace

// The workspace of every moe_layer_forward_noalloc call on a GPU.  Host code
// never passes this name to a kernel or a copy: on the host it is only a
// stand-in symbol, and the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

struct DeviceScratch {
    unsigned char *ptr = nullptr;   // device address of `scratch` on this GPU
    bool ready = false;
};

DeviceScratch g_dev[MAX_DEVICES];
std::mutex g_mu;

__global__ void clear_u32_kernel(uint32_t *__restrict__ p, int n)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        p[i] = 0u;
}

// Looks up (once per device, with that device current) the address of this
// GPU's copy of the array and checks the device.
moe_status device_scratch(int dev, unsigned char **out)
{
    if (dev < 0 || dev >= MAX_DEVICES)
        return fail(MOE_E_UNSUPPORTED, "device %d: at most %d devices", dev, MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceScratch &d = g_dev[dev];
    if (!d.ready) {
        moe_status st = check_device(dev);
        if (st)
            return st;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p)
            return fail(MOE_E_HIP, "hipGetSymbolAddress(scratch) gave NULL");
        d.ptr = static_cast<unsigned char *>(p);
        d.ready = true;
    }
    *out = d.ptr;
    return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_layer_forward_noalloc(const moe_layer_desc *desc, const void *x,
                                                int32_t T, const moe_layer_weights *w,
                                                int32_t *idx_out, float *gate_w_out, void *out,
                                                void *stream)
{
    moe_status st = validate_desc(desc);
    if (st)
        return st;
    if (T < 0 || T > (1 << 20))
        return fail(MOE_E_INVAL, "T=%d out of range [0, 2^20]", T);
    if (T == 0)
        return MOE_OK;
    if (!x || !w || !out)
        return fail(MOE_E_INVAL, "x/weights/out is NULL");
    if (!w->router_w || !w->router_bias)
        return fail(MOE_E_INVAL, "router weights are NULL");
    if (desc->n_shared && !w->shared)
        return fail(MOE_E_INVAL, "shared expert blob is NULL");
    if (!w->expert_ptrs)
        return fail(MOE_E_INVAL, "expert_ptrs is NULL");
    if ((size_t)(desc->hidden / 32) * 4 > HEADER_BYTES - CTR_DN_OFF)
        return fail(MOE_E_INVAL, "hidden=%d above this entry point's limit", desc->hidden);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    unsigned char *base = nullptr;
    if ((st = device_scratch(dev, &base)) != MOE_OK)
        return st;

    // a context on the stack whose workspace points into the array (its
    // vectors stay empty: nothing here allocates)
    moe_ctx c;
    c.device = dev;
    c.d = *desc;
    c.max_tokens = T;
    c.L = blob_layout(desc->hidden, desc->ffn, desc->group, desc->wfmt);
    c.S = desc->top_k + desc->n_shared;
    size_t off = HEADER_BYTES;
    st = ws_plan(&c, [&](void **p, size_t bytes, int kind) -> moe_status {
        if (kind == WS_DEBUG) {
            *p = nullptr;
            return MOE_OK;
        }
        if (kind == WS_COUNTER) {
            if (p == reinterpret_cast<void **>(&c.done))
                *p = base;
            else if (p == reinterpret_cast<void **>(&c.ctr_gu))
                *p = base + CTR_GU_OFF;
            else
                *p = base + CTR_DN_OFF;
            return MOE_OK;
        }
        const size_t need = off + ((bytes + 255) & ~(size_t)255);
        if (need > MOE_NOALLOC_SCRATCH_BYTES)
            return fail(MOE_E_INVAL,
                        "T=%d at this shape needs more than the %d-byte scratch array of "
                        "moe_layer_forward_noalloc; use moe_layer_forward with a context",
                        T, (int)MOE_NOALLOC_SCRATCH_BYTES);
        *p = base + off;
        off = need;
        return MOE_OK;
    });
    if (st)
        return st;

    // counters start at zero: the kernels that count leave them at zero, but
    // the array keeps whatever the last call on this GPU left
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int n_ctr = (int)((CTR_DN_OFF + (size_t)(desc->hidden / 32) * 4) / 4);
    launch(clear_u32_kernel, 8, 256, 0, s, reinterpret_cast<uint32_t *>(base), n_ctr);
    if ((e = hipGetLastError()) != hipSuccess)
        return hip_fail(e, "counter clear launch");
    return layer_forward_enqueue(&c, x, T, w, nullptr, 0, idx_out, gate_w_out, out, s);
}
