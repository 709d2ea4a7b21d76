// Streaming device copy: the attainable read + write rate of HBM on this
// part, measured with a kernel of this library (the HBM-bound kernels of the
// path are judged against it beside the 8 TB/s of the data sheet), and a
// kernel of known byte count that scales the profiler's FETCH_SIZE and
// WRITE_SIZE counters.
//
// Each thread moves U 16-byte vectors: the U loads are issued together, then
// the U stores, so a wave keeps U KB in flight; consecutive lanes touch
// consecutive 16-byte words, so every wave access is 1 KB contiguous.  The
// loads and stores carry the non-temporal hint (the data is touched once).
#include <string>

#include "kernels.h"
#include "plan_host.h"

namespace sva {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyU = 4;

__global__ __launch_bounds__(kCopyThreads) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst,
                                                                   int64_t n16) {
    const int64_t base = (int64_t)blockIdx.x * (kCopyThreads * kCopyU) + threadIdx.x;
    u32x4 v[kCopyU];
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
        const int64_t i = base + u * kCopyThreads;
        v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
        const int64_t i = base + u * kCopyThreads;
        if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
    }
}

// The bytes past the last whole 16-byte word, one thread each.
__global__ void copy_tail_kernel(const uint8_t* src, uint8_t* dst, int n) {
    if ((int)threadIdx.x < n) dst[threadIdx.x] = src[threadIdx.x];
}

}  // namespace

}  // namespace sva

extern "C" int sva_stream_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (bytes == 0) return SVA_OK;
    if (!dst || !src || ((uintptr_t)dst & 15u) || ((uintptr_t)src & 15u)) {
        sva::set_last_error("dst and src must be non-NULL and 16-byte aligned");
        return SVA_ERR_INVALID_ARG;
    }
    const uint8_t* s8 = static_cast<const uint8_t*>(src);
    uint8_t* d8 = static_cast<uint8_t*>(dst);
    if ((s8 < d8 + bytes) && (d8 < s8 + bytes)) {
        sva::set_last_error("dst and src must not overlap");
        return SVA_ERR_INVALID_ARG;
    }
    const int64_t n16 = (int64_t)(bytes / 16);
    const int tail = (int)(bytes % 16);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (n16 > 0) {
        const int64_t per = (int64_t)sva::kCopyThreads * sva::kCopyU;
        const int64_t blocks = (n16 + per - 1) / per;
        if (blocks > 0x7fffffff) {
            sva::set_last_error("copy too large");
            return SVA_ERR_INVALID_ARG;
        }
        hipLaunchKernelGGL(sva::stream_copy_kernel, dim3((unsigned)blocks),
                           dim3(sva::kCopyThreads), 0, st,
                           reinterpret_cast<const sva::u32x4*>(src),
                           reinterpret_cast<sva::u32x4*>(dst), n16);
    }
    if (tail > 0)
        hipLaunchKernelGGL(sva::copy_tail_kernel, dim3(1), dim3(16), 0, st,
                           s8 + n16 * 16, d8 + n16 * 16, tail);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        sva::set_last_error(std::string("stream copy launch: ") + hipGetErrorString(e));
        return SVA_ERR_HIP;
    }
    return SVA_OK;
}
