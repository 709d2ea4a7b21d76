// Block means for the compensation of dropped key blocks.
//
// For every key block: the mean key and the mean value over its valid
// tokens (float32 sums of the bf16 inputs, divided by the count, rounded to
// bf16).  They are written as "mean tiles" in the K-tile and V-tile layouts,
// block kb being key kb % 32 of group kb / 32, so the attention kernel
// consumes 32 block means per stage exactly as it consumes 32 keys.  Slots
// past the last block are written as zeros.
//
// Reads the K and V tiles once (2 · Np · d · 2 bytes per head); bound by
// HBM.  One workgroup per (b, h, slot).
#include "kernels.h"

namespace sva {

namespace {

constexpr int kMeanThreads = 256;

__device__ __forceinline__ uint16_t to_bf16(float x) {
    return (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
}

template <int D, int BLK>
__global__ __launch_bounds__(kMeanThreads) void block_means_kernel(DevPlan p, const u32x4* kt,
                                                                   const uint16_t* vt,
                                                                   uint16_t* km, uint16_t* vm) {
    constexpr int NCH = D / 8;     // 8-channel chunks per key
    constexpr int CPT = NCH / 8;   // K chunks per thread
    constexpr int DS = D / 16;     // 16-channel steps of a K tile
    constexpr int NG = BLK / 32;   // 32-token groups per block
    __shared__ float part[32][D + 1];
    const int nslots = p.n_mean_groups * 32;
    const int kb = blockIdx.x % nslots;
    const int64_t bh = blockIdx.x / nslots;
    const int g = kb >> 5, jj = kb & 31;
    // this slot in the mean tiles: K entry (s·64 + hf·32 + jj) of group g for
    // channels 16s + 8hf .. +7; V chunk kc (keys 16(kc/2) + 4(kc%2) +
    // {0..3, 8..11}) slot si, one row per channel
    uint16_t* kmo = km + (bh * p.n_mean_groups + g) * (int64_t)(DS * 64 * 8);
    uint16_t* vmo = vm + (bh * p.n_mean_groups + g) * (int64_t)(4 * D * 8);
    const int kc = 2 * (jj >> 4) + ((jj & 7) >= 4 ? 1 : 0);
    const int si = (jj & 3) + ((jj & 15) >= 8 ? 4 : 0);
    if (kb >= p.nB) {
        for (int c = threadIdx.x; c < D; c += kMeanThreads) {
            kmo[((c >> 4) * 64 + ((c >> 3) & 1) * 32 + jj) * 8 + (c & 7)] = 0;
            vmo[(kc * D + c) * 8 + si] = 0;
        }
        return;
    }
    const int valid = p.blk_valid[kb];

    // K: thread (j, q) sums chunks q, q + 8, ... over tokens j, j + 32, ...
    const int j = threadIdx.x % 32, q = threadIdx.x / 32;
    const u32x4* ksrc = kt + (bh * p.nB + kb) * (int64_t)(BLK * NCH);
    float acc[CPT][8];
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
    for (int tok = j; tok < valid; tok += 32) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const u32x4 v = ksrc[(tok >> 5) * 4 * D + (q + 8 * i) * 32 + (tok & 31)];
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[i][2 * e] += bf16lo(u[e]);
                acc[i][2 * e + 1] += bf16hi(u[e]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) part[j][(q + 8 * i) * 8 + e] = acc[i][e];

    // V: thread c sums channel row c of every chunk of every group
    float vs = 0.f;
    if (threadIdx.x < D) {
        const int c = threadIdx.x;
        const uint16_t* vsrc = vt + (bh * p.nB + kb) * (int64_t)(BLK * D);
        for (int gg = 0; gg < NG; ++gg)
#pragma unroll
            for (int kc2 = 0; kc2 < 4; ++kc2) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(vsrc + ((gg * 4 + kc2) * D + c) * 8);
                const uint32_t u[4] = {w.x, w.y, w.z, w.w};
                const int key0 = gg * 32 + 16 * (kc2 >> 1) + 4 * (kc2 & 1);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int key = key0 + (i & 3) + 8 * (i >> 2);
                    const float x = (i & 1) ? bf16hi(u[i >> 1]) : bf16lo(u[i >> 1]);
                    if (key < valid) vs += x;
                }
            }
    }
    __syncthreads();
    if (threadIdx.x < D) {
        const int c = threadIdx.x;
        float ks = 0.f;
        for (int t = 0; t < 32; ++t) ks += part[t][c];
        kmo[((c >> 4) * 64 + ((c >> 3) & 1) * 32 + jj) * 8 + (c & 7)] = to_bf16(ks / (float)valid);
        vmo[(kc * D + c) * 8 + si] = to_bf16(vs / (float)valid);
    }
}

}  // namespace

hipError_t launch_block_means(const DevPlan& p, const uint16_t* kt, const uint16_t* vt,
                              uint16_t* km, uint16_t* vm, hipStream_t s) {
    dim3 grid((unsigned)((int64_t)p.B * p.H * p.n_mean_groups * 32));
    const u32x4* k4 = reinterpret_cast<const u32x4*>(kt);
    if (p.d == 128 && p.block == 128)
        hipLaunchKernelGGL((block_means_kernel<128, 128>), grid, dim3(kMeanThreads), 0, s, p, k4, vt, km, vm);
    else if (p.d == 128)
        hipLaunchKernelGGL((block_means_kernel<128, 64>), grid, dim3(kMeanThreads), 0, s, p, k4, vt, km, vm);
    else if (p.block == 128)
        hipLaunchKernelGGL((block_means_kernel<64, 128>), grid, dim3(kMeanThreads), 0, s, p, k4, vt, km, vm);
    else
        hipLaunchKernelGGL((block_means_kernel<64, 64>), grid, dim3(kMeanThreads), 0, s, p, k4, vt, km, vm);
    return hipGetLastError();
}

}  // namespace sva
