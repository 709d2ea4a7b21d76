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

// Forward: one output row (b, h, p) per d/8 lanes.  Loads go out in
// branch-free batches (token indices, then rows from clamped addresses),
// so a thread's rows are in flight together; the row index is below 2^31.
template <int D>
__global__ __launch_bounds__(kThreads) void reorder_fwd_kernel(DevPlan p, const u32x4* in,
                                                               u32x4* out) {
    constexpr int LPR = D / 8;
    constexpr int RPB = kThreads / LPR;
    const int sub = threadIdx.x % LPR;
    const uint32_t rows = (uint32_t)(p.B * p.H * p.Np);
    const uint32_t row0 = blockIdx.x * (uint32_t)(RPB * kRows) + threadIdx.x / LPR;
    int n[kRows];
    uint32_t bh[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const uint32_t row = min(row0 + r * RPB, rows - 1);
        bh[r] = fast_div(row, p.div_Np);
        n[r] = p.inv[row - bh[r] * (uint32_t)p.Np];
        SVA_DCHECK(p, n[r] >= -1 && n[r] < p.N, SVA_DEBUG_TOKEN);
    }
    u32x4 v[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const uint32_t b = fast_div(bh[r], p.div_H);
        const uint32_t h = bh[r] - b * (uint32_t)p.H;
        const int64_t src = ((int64_t)b * p.N + (n[r] >= 0 ? n[r] : 0)) * p.H + h;
        v[r] = in[src * LPR + sub];
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const uint32_t row = row0 + r * RPB;
        if (row < rows) out[(int64_t)row * LPR + sub] = n[r] >= 0 ? v[r] : u32x4{0u, 0u, 0u, 0u};
    }
}

// Inverse: one output raster row (b, n, h) per d/8 lanes; writes are
// contiguous, reads gather whole rows (batched as in the forward kernel).
template <int D>
__global__ __launch_bounds__(kThreads) void reorder_inv_kernel(DevPlan p, const u32x4* in,
                                                               u32x4* out) {
    constexpr int LPR = D / 8;
    constexpr int RPB = kThreads / LPR;
    const int sub = threadIdx.x % LPR;
    const uint32_t rows = (uint32_t)(p.B * p.N * p.H);
    const uint32_t row0 = blockIdx.x * (uint32_t)(RPB * kRows) + threadIdx.x / LPR;
    int pos[kRows];
    uint32_t bh[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const uint32_t row = min(row0 + r * RPB, rows - 1);
        const uint32_t bn = fast_div(row, p.div_H);
        const uint32_t h = row - bn * (uint32_t)p.H;
        const uint32_t b = fast_div(bn, p.div_N);
        pos[r] = p.perm[bn - b * (uint32_t)p.N];
        SVA_DCHECK(p, pos[r] >= 0 && pos[r] < p.Np, SVA_DEBUG_TOKEN);
        bh[r] = b * (uint32_t)p.H + h;
    }
    u32x4 v[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) v[r] = in[((int64_t)bh[r] * p.Np + pos[r]) * LPR + sub];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const uint32_t row = row0 + r * RPB;
        if (row < rows) out[(int64_t)row * LPR + sub] = v[r];
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
// ROWS: the input is already in tile order [B, H, Np, d] (row bh·Np + pos)
// instead of raster; padding positions are still written as zeros.
template <int D, int BLK, bool ROWS>
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
    // branch-free batches: the 8 token indices, then the 8 rows (padding
    // reads token 0 and is zeroed afterwards)
    int n[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        n[j] = p.inv[kb * BLK + key0 + (j & 3) + 8 * (j >> 2)];
        SVA_DCHECK(p, n[j] >= -1 && n[j] < p.N, SVA_DEBUG_TOKEN);
    }
    u32x4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        x[j] = ROWS ? in[(bh * p.Np + kb * BLK + key0 + (j & 3) + 8 * (j >> 2)) * DC + dc]
                    : in[((b * p.N + (n[j] >= 0 ? n[j] : 0)) * p.H + h) * DC + dc];
    uint32_t m[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const u32x4 v = n[j] >= 0 ? x[j] : u32x4{0u, 0u, 0u, 0u};
        m[j][0] = v.x; m[j][1] = v.y; m[j][2] = v.z; m[j][3] = v.w;
    }
    // 32-key group kg/4, chunk kg%4: d rows of 8 keys, i.e. output chunks
    // kg·D + dc·8 + e of the block's tile.  They go through LDS (one padding
    // chunk after every 8, so the 16 lanes of a row group hit distinct
    // banks) and leave as contiguous 1 KB wave stores.
    constexpr int NTH = (D / 8) * (BLK / 8);
    constexpr int TCH = BLK * D / 8;          // 16-byte chunks per block tile
    __shared__ u32x4 tile[TCH + TCH / 8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t o[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t lo = m[2 * w][e / 2], hi = m[2 * w + 1][e / 2];
            o[w] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                           : ((lo & 0xffffu) | (hi << 16));
        }
        const int q = kg * D + dc * 8 + e;
        tile[q + (q >> 3)] = u32x4{o[0], o[1], o[2], o[3]};
    }
    __syncthreads();
    u32x4* dst = out + (bh * p.nB + kb) * (int64_t)TCH;
#pragma unroll
    for (int i = 0; i < TCH / NTH; ++i) {
        const int q = threadIdx.x + i * NTH;
        dst[q] = tile[q + (q >> 3)];
    }
}

// Forward into K tiles.  One workgroup per (b, h, block); thread order
// follows the output, so every wave writes 1 KB contiguously and reads 32
// bytes from each of 32 rows (the rest of those rows is read by the
// neighbouring waves of the same workgroup, out of the caches).
template <int D, int BLK, bool ROWS>
__global__ __launch_bounds__(256) void reorder_kt_kernel(DevPlan p, const u32x4* in,
                                                        u32x4* out) {
    constexpr int DC = D / 8;              // 16-byte chunks per row
    constexpr int CHUNKS = BLK * DC;       // per block
    const int kb = blockIdx.x % p.nB;
    const int64_t bh = blockIdx.x / p.nB;
    const int h = (int)(bh % p.H);
    const int64_t b = bh / p.H;
    u32x4* dst = out + (bh * p.nB + kb) * (int64_t)CHUNKS;
    constexpr int NI = CHUNKS / 256;
    // branch-free batches as in the V-tile kernel
    int n[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int q = threadIdx.x + i * 256;   // (g, s, hf, j) with j fastest
        const int g = (q >> 6) / (D / 16);
        n[i] = p.inv[kb * BLK + g * 32 + (q & 31)];
        SVA_DCHECK(p, n[i] >= -1 && n[i] < p.N, SVA_DEBUG_TOKEN);
    }
    u32x4 x[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int q = threadIdx.x + i * 256;
        const int hf = (q >> 5) & 1, s = (q >> 6) % (D / 16);
        x[i] = ROWS ? in[(bh * p.Np + kb * BLK + ((q >> 6) / (D / 16)) * 32 + (q & 31)) * DC + 2 * s + hf]
                    : in[((b * p.N + (n[i] >= 0 ? n[i] : 0)) * p.H + h) * DC + 2 * s + hf];
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) dst[threadIdx.x + i * 256] = n[i] >= 0 ? x[i] : u32x4{0u, 0u, 0u, 0u};
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
    } else if (direction == 3 || direction == 5) {
        dim3 grid((unsigned)((int64_t)p.B * p.H * p.nB));
        auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, p, i4, o4); };
        const bool rows = direction == 5;
        if (p.d == 128 && p.block == 128)
            rows ? go(reorder_kt_kernel<128, 128, true>) : go(reorder_kt_kernel<128, 128, false>);
        else if (p.d == 128)
            rows ? go(reorder_kt_kernel<128, 64, true>) : go(reorder_kt_kernel<128, 64, false>);
        else if (p.block == 128)
            rows ? go(reorder_kt_kernel<64, 128, true>) : go(reorder_kt_kernel<64, 128, false>);
        else
            rows ? go(reorder_kt_kernel<64, 64, true>) : go(reorder_kt_kernel<64, 64, false>);
    } else {
        dim3 grid((unsigned)((int64_t)p.B * p.H * p.nB));
        const int threads = (p.d / 8) * (p.block / 8);
        auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(threads), 0, s, p, i4, o4); };
        const bool rows = direction == 4;
        if (p.d == 128 && p.block == 128)
            rows ? go(reorder_vt_kernel<128, 128, true>) : go(reorder_vt_kernel<128, 128, false>);
        else if (p.d == 128)
            rows ? go(reorder_vt_kernel<128, 64, true>) : go(reorder_vt_kernel<128, 64, false>);
        else if (p.block == 128)
            rows ? go(reorder_vt_kernel<64, 128, true>) : go(reorder_vt_kernel<64, 128, false>);
        else
            rows ? go(reorder_vt_kernel<64, 64, true>) : go(reorder_vt_kernel<64, 64, false>);
    }
    return hipGetLastError();
}

}  // namespace sva
