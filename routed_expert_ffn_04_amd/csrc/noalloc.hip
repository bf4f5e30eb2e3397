// moe_layer_noalloc: the fused layer with its scratch in a device array of
// the library instead of a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  The kernels are moe_layer's; only the
// workspace pointer differs.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "moe.h"
#include "internal.h"

namespace {

// Largest layer workspace this entry point serves (moe_layer_workspace_size):
// 64 MiB covers the decode batch of the DeepSeek-V3 layer (H = 7168, 256 + 1
// experts, I = 2048, bf16 weights) up to T = 226 tokens with fp32 outputs
// (36 MiB at T = 128) and up to T = 400 with bf16 outputs.  Every GPU the library runs on holds one copy
// of the array until the process ends.
constexpr size_t kScratchBytes = (size_t)64 << 20;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
std::atomic<void*> g_ptr[kMaxDevices];
std::atomic<int> g_rc[kMaxDevices];

// The device address of this device's copy of the array, looked up once per
// device with that device current (the host-side name of the array is only a
// stand-in: it is never passed to a kernel or a copy).
hipError_t scratch_ptr(int dev, void** out) {
    std::call_once(g_once[dev], [dev] {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev].store(e == hipSuccess ? p : nullptr);
        g_rc[dev].store((int)e);
    });
    *out = g_ptr[dev].load();
    return (hipError_t)g_rc[dev].load();
}

}  // namespace

extern "C" moe_status_t moe_layer_noalloc(const void* x, int32_t x_dt, int32_t T, int32_t H,
                                          const float* w_router, const float* bias, int32_t E, int32_t k,
                                          int32_t score, const moe_experts_t* routed, const moe_experts_t* shared,
                                          void* out, int32_t out_dt, int32_t y_dt,
                                          int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out,
                                          void* stream) {
    if (T < 0 || H <= 0 || E <= 0 || k <= 0 || !routed)
        return (moe_status_t)moe::set_error(MOE_ERR_INVALID, "layer_noalloc: T=%d H=%d E=%d k=%d routed=%p", T, H, E,
                                            k, (const void*)routed);
    const size_t need = moe_layer_workspace_size(T, H, E, k, routed->I, x_dt, routed->dt, shared ? 1 : 0, out_dt, y_dt);
    if (need > kScratchBytes)
        return (moe_status_t)moe::set_error(MOE_ERR_UNSUPPORTED,
                                            "layer_noalloc: the call needs %zu bytes of scratch, more than the "
                                            "%zu-byte static array (use moe_layer with a workspace)",
                                            need, kScratchBytes);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (moe_status_t)moe::set_error(MOE_ERR_HIP, "layer_noalloc: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return (moe_status_t)moe::set_error(MOE_ERR_UNSUPPORTED, "layer_noalloc: device %d >= %d", dev, kMaxDevices);
    if (stream) {
        hipDevice_t sd = 0;
        e = hipStreamGetDevice((hipStream_t)stream, &sd);
        if (e != hipSuccess) return (moe_status_t)moe::set_error(MOE_ERR_HIP, "layer_noalloc: %s", hipGetErrorString(e));
        if (sd != dev)
            return (moe_status_t)moe::set_error(MOE_ERR_INVALID,
                                                "layer_noalloc: the stream belongs to device %d, the current device "
                                                "is %d",
                                                (int)sd, dev);
    }
    void* ws = nullptr;
    e = scratch_ptr(dev, &ws);
    if (e != hipSuccess || !ws)
        return (moe_status_t)moe::set_error(MOE_ERR_HIP, "layer_noalloc: hipGetSymbolAddress: %s",
                                            hipGetErrorString(e));
    return moe_layer(x, x_dt, T, H, w_router, bias, E, k, score, routed, shared, out, out_dt, y_dt, topk_ids_out,
                     topk_w_out, counts_out, ws, kScratchBytes, stream);
}
