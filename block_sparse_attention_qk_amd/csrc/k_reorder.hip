// 3D-tile token reorder.
//
// The permutation gathers the raster video tokens tile by tile so each
// block of the sequence is a compact space-time patch (the "Sol Video
// Inference Engine" blog, section 4.2.2, cites Sparse VideoGen2's token
// permutation for GPU layout; the tile order itself is this library's
// reading).  Three directions:
//   forward     raster [B,N,H,d] -> tile order [B,H,Np,d], padding zeroed
//   inverse     tile order -> raster, padding dropped
//   forward_vt  raster -> V tiles [B,H,nB,block/32,d,32]: each block of V
//               as groups of 32 keys stored channel-major (keys
//               interleaved inside groups of 16), the layout the attention
//               kernel streams V in.
//   forward_kt  raster -> K tiles [B,H,nB,block/32,d/16,64,8]: for every
//               32-key group and 16-channel step, the 16-byte operand of
//               each of the 64 lanes of the attention kernel's MFMA, in
//               lane order (lane = 32·hf + j holds key j, channels
//               16s + 8hf .. +8), so one wave-wide load fetches 1 KB.
// All three move every byte once and are bound by HBM bandwidth.  Rows are
// d·2 = 128 or 256 contiguous bytes, so gathers stay at full-line width.
#include "kernels.h"

namespace sva {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 4;

// Forward: one output row (b, h, p) per d/8 lanes.
template <int D>
__global__ __launch_bounds__(kThreads) void reorder_fwd_kernel(DevPlan p, const u32x4* in,
                                                               u32x4* out) {
    constexpr int LPR = D / 8;
    constexpr int RPB = kThreads / LPR;
    const int sub = threadIdx.x % LPR;
    const int64_t rows = (int64_t)p.B * p.H * p.Np;
    const int64_t row0 = (int64_t)blockIdx.x * RPB * kRows + threadIdx.x / LPR;
    u32x4 v[kRows];
    int64_t dst[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int64_t row = row0 + (int64_t)r * RPB;
        dst[r] = row;
        v[r] = u32x4{0u, 0u, 0u, 0u};
        if (row < rows) {
            const int64_t pos = row % p.Np;
            const int64_t bh = row / p.Np;
            const int h = (int)(bh % p.H);
            const int64_t b = bh / p.H;
            const int n = p.inv[pos];
            if (n >= 0) v[r] = in[((b * p.N + n) * p.H + h) * LPR + sub];
        }
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r)
        if (dst[r] < rows) out[dst[r] * LPR + sub] = v[r];
}

// Inverse: one output raster row (b, n, h) per d/8 lanes; writes are
// contiguous, reads gather whole rows.
template <int D>
__global__ __launch_bounds__(kThreads) void reorder_inv_kernel(DevPlan p, const u32x4* in,
                                                               u32x4* out) {
    constexpr int LPR = D / 8;
    constexpr int RPB = kThreads / LPR;
    const int sub = threadIdx.x % LPR;
    const int64_t rows = (int64_t)p.B * p.N * p.H;
    const int64_t row0 = (int64_t)blockIdx.x * RPB * kRows + threadIdx.x / LPR;
    u32x4 v[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int64_t row = row0 + (int64_t)r * RPB;
        if (row < rows) {
            const int h = (int)(row % p.H);
            const int64_t bn = row / p.H;
            const int64_t n = bn % p.N;
            const int64_t b = bn / p.N;
            const int64_t pos = p.perm[n];
            v[r] = in[((b * p.H + h) * p.Np + pos) * LPR + sub];
        }
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int64_t row = row0 + (int64_t)r * RPB;
        if (row < rows) out[row * LPR + sub] = v[r];
    }
}

// Forward into V tiles.  A V tile holds one key block as BLK/32 groups of
// 32 keys; each group is four chunks of 8 keys, each chunk stored as D rows
// of 16 bytes (8 keys of one channel), so the attention kernel copies a
// group as one contiguous span and reads the operand of 32 channels × 8
// keys as 32 consecutive 16-byte slots.  The keys of chunk kc are the ones
// the attention kernel's MFMA operand consumes together: chunk kc holds
// keys 16(kc/2) + 4(kc%2) + {0,1,2,3,8,9,10,11}.
// One workgroup per (b, h, block): thread (kg, dc) gathers the 8 keys of
// chunk kg (over the whole block) for channel chunk dc (8 rows of 16
// bytes), turns the 8×8 bf16 square around in registers and writes
// channels dc*8..dc*8+7 of that chunk (128 contiguous bytes).
template <int D, int BLK>
__global__ __launch_bounds__((D / 8) * (BLK / 8)) void reorder_vt_kernel(DevPlan p,
                                                                       const u32x4* in,
                                                                       u32x4* out) {
    constexpr int DC = D / 8;      // channel chunks per row
    const int dc = threadIdx.x % DC;
    const int kg = threadIdx.x / DC;
    const int kb = blockIdx.x % p.nB;
    const int64_t bh = blockIdx.x / p.nB;
    const int h = (int)(bh % p.H);
    const int64_t b = bh / p.H;
    const int key0 = 16 * (kg >> 1) + 4 * (kg & 1);
    uint32_t m[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int key = key0 + (j & 3) + 8 * (j >> 2);
        const int64_t pos = (int64_t)kb * BLK + key;
        const int n = p.inv[pos];
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (n >= 0) v = in[((b * p.N + n) * p.H + h) * DC + dc];
        m[j][0] = v.x; m[j][1] = v.y; m[j][2] = v.z; m[j][3] = v.w;
    }
    // 32-key group kg/4, chunk kg%4: d rows of 8 keys
    u32x4* dst = out + (((bh * p.nB + kb) * (BLK / 32) + (kg >> 2)) * 4 + (kg & 3)) * D + dc * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t o[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t lo = m[2 * w][e / 2], hi = m[2 * w + 1][e / 2];
            o[w] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                           : ((lo & 0xffffu) | (hi << 16));
        }
        dst[e] = u32x4{o[0], o[1], o[2], o[3]};
    }
}

// Forward into K tiles.  One workgroup per (b, h, block); thread order
// follows the output, so every wave writes 1 KB contiguously and reads 32
// bytes from each of 32 rows (the rest of those rows is read by the
// neighbouring waves of the same workgroup, out of the caches).
template <int D, int BLK>
__global__ __launch_bounds__(256) void reorder_kt_kernel(DevPlan p, const u32x4* in,
                                                        u32x4* out) {
    constexpr int DC = D / 8;              // 16-byte chunks per row
    constexpr int CHUNKS = BLK * DC;       // per block
    const int kb = blockIdx.x % p.nB;
    const int64_t bh = blockIdx.x / p.nB;
    const int h = (int)(bh % p.H);
    const int64_t b = bh / p.H;
    u32x4* dst = out + (bh * p.nB + kb) * (int64_t)CHUNKS;
#pragma unroll
    for (int i = 0; i < CHUNKS / 256; ++i) {
        const int q = threadIdx.x + i * 256;   // (g, s, hf, j) with j fastest
        const int j = q & 31, hf = (q >> 5) & 1, s = (q >> 6) % (D / 16);
        const int g = (q >> 6) / (D / 16);
        const int64_t pos = (int64_t)kb * BLK + g * 32 + j;
        const int n = p.inv[pos];
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (n >= 0) v = in[((b * p.N + n) * p.H + h) * DC + 2 * s + hf];
        dst[q] = v;
    }
}

}  // namespace

hipError_t launch_reorder(const DevPlan& p, const uint16_t* in, uint16_t* out, int direction,
                          hipStream_t s) {
    const u32x4* i4 = reinterpret_cast<const u32x4*>(in);
    u32x4* o4 = reinterpret_cast<u32x4*>(out);
    const int lpr = p.d / 8;
    const int64_t per_block = (int64_t)(kThreads / lpr) * kRows;
    if (direction == 0) {
        const int64_t rows = (int64_t)p.B * p.H * p.Np;
        dim3 grid((unsigned)((rows + per_block - 1) / per_block));
        if (p.d == 128) hipLaunchKernelGGL(reorder_fwd_kernel<128>, grid, dim3(kThreads), 0, s, p, i4, o4);
        else hipLaunchKernelGGL(reorder_fwd_kernel<64>, grid, dim3(kThreads), 0, s, p, i4, o4);
    } else if (direction == 1) {
        const int64_t rows = (int64_t)p.B * p.N * p.H;
        dim3 grid((unsigned)((rows + per_block - 1) / per_block));
        if (p.d == 128) hipLaunchKernelGGL(reorder_inv_kernel<128>, grid, dim3(kThreads), 0, s, p, i4, o4);
        else hipLaunchKernelGGL(reorder_inv_kernel<64>, grid, dim3(kThreads), 0, s, p, i4, o4);
    } else if (direction == 3) {
        dim3 grid((unsigned)((int64_t)p.B * p.H * p.nB));
        if (p.d == 128 && p.block == 128)
            hipLaunchKernelGGL((reorder_kt_kernel<128, 128>), grid, dim3(256), 0, s, p, i4, o4);
        else if (p.d == 128)
            hipLaunchKernelGGL((reorder_kt_kernel<128, 64>), grid, dim3(256), 0, s, p, i4, o4);
        else if (p.block == 128)
            hipLaunchKernelGGL((reorder_kt_kernel<64, 128>), grid, dim3(256), 0, s, p, i4, o4);
        else
            hipLaunchKernelGGL((reorder_kt_kernel<64, 64>), grid, dim3(256), 0, s, p, i4, o4);
    } else {
        dim3 grid((unsigned)((int64_t)p.B * p.H * p.nB));
        const int threads = (p.d / 8) * (p.block / 8);
        if (p.d == 128 && p.block == 128)
            hipLaunchKernelGGL((reorder_vt_kernel<128, 128>), grid, dim3(threads), 0, s, p, i4, o4);
        else if (p.d == 128)
            hipLaunchKernelGGL((reorder_vt_kernel<128, 64>), grid, dim3(threads), 0, s, p, i4, o4);
        else if (p.block == 128)
            hipLaunchKernelGGL((reorder_vt_kernel<64, 128>), grid, dim3(threads), 0, s, p, i4, o4);
        else
            hipLaunchKernelGGL((reorder_vt_kernel<64, 64>), grid, dim3(threads), 0, s, p, i4, o4);
    }
    return hipGetLastError();
}

}  // namespace sva
