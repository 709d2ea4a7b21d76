// Block selection that allocates nothing, for callers that cannot allocate
// device memory: code under HIP graph capture, tight serving loops and
// harnesses that forbid hipMalloc.  sva_select_blocks keeps its block means
// in a workspace the caller brings; sva_select_blocks_noalloc keeps them in
// `scratch`, a fixed array of this library (one copy per GPU, held until
// the process ends), and runs the same kernels on it.
//
// In host code `scratch` names a host-side stand-in, not device memory:
// only the address hipGetSymbolAddress resolves for a device may reach a
// kernel.  That address is resolved once per device at plan creation (the
// device current) and kept in g_scratch; the entry point only reads it.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "plan_dev.h"

namespace sva {

namespace {

// q block means [B,H,nB,nsub,d] then transposed k means [B,H,d,nB·nsub],
// float64: 128 MiB covers the mean scorer up to 48 heads × 1024 blocks of
// d = 128 (the packed 768p shape needs 96 MB).
constexpr size_t kScratchBytes = (size_t)128 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t resolve_select_scratch(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev]) return hipSuccess;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = ptr;
    return hipSuccess;
}

}  // namespace sva

extern "C" int sva_select_blocks_noalloc(sva_plan plan, const void* q_r, const void* k_t,
                                         int32_t* col, void* stream) {
    using sva::set_last_error;
    if (!plan) {
        set_last_error("plan is NULL");
        return SVA_ERR_INVALID_ARG;
    }
    if (plan->host.info.dense) return SVA_OK;
    if (!q_r || !k_t || !col) {
        set_last_error("q_r, k_t and col must be non-NULL");
        return SVA_ERR_INVALID_ARG;
    }
    if (((uintptr_t)q_r & 15u) || ((uintptr_t)k_t & 15u) || ((uintptr_t)col & 3u)) {
        set_last_error("misaligned pointer");
        return SVA_ERR_INVALID_ARG;
    }
    const size_t need = plan->host.info.select_workspace_bytes;
    if (need > sva::kScratchBytes) {
        set_last_error("the selection needs " + std::to_string(need) +
                       " bytes of block means; the fixed scratch holds " +
                       std::to_string(sva::kScratchBytes) + " (use sva_select_blocks)");
        return SVA_ERR_WORKSPACE;
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        set_last_error(std::string("hipGetDevice: ") + hipGetErrorString(e));
        return SVA_ERR_HIP;
    }
    if (dev != plan->device) {
        set_last_error("the current device is not the plan's device");
        return SVA_ERR_INVALID_ARG;
    }
    void* ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(sva::g_scratch_mu);
        ptr = sva::g_scratch[dev];
    }
    if (!ptr) {   // resolved when the plan was created on this device
        set_last_error("select scratch not resolved for this device");
        return SVA_ERR_HIP;
    }
    // pooling writes every mean of the plan before the ranking reads it, so
    // nothing left by an earlier call is read
    e = sva::launch_select(plan->dev, static_cast<const uint16_t*>(q_r),
                           static_cast<const uint16_t*>(k_t), static_cast<double*>(ptr), col,
                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        set_last_error(std::string("select launch: ") + hipGetErrorString(e));
        return SVA_ERR_HIP;
    }
    return SVA_OK;
}
