// Block selection: mean pooling, block scores, top-k per query block.
//
// Follows "MiniMax-H3 在 8×H200 上基准测试", section "SubBlock 稀疏注意力如何工作":
// a lightweight pooling step scores every key block for each query block
// and head, the best-scored key blocks are kept (sparsity = fraction
// dropped) and their indices go to the block-sparse kernel; rows are ranked
// independently per query block and head.  The score here is the plain
// reading of "mean-pooled Q and K": s(qb, kb) = mean(Q' of qb) · mean(K' of kb).
// The SubBlock scorer of the same section splits each block into runs of
// consecutive tokens, pools each run, and scores a key block by
//   log sum_a sum_b c_a c_b exp(qbar_a · kbar_b / sqrt(d))
// over the runs' valid counts c, an estimate of the key block's
// unnormalised softmax mass for the query block.
//
// Two kernels:
//  pool   one workgroup per (b, h, block) and tensor: float64 sums of the
//         valid rows, divided by the valid count.  Sums of at most 128 bf16
//         values are exact in float64 for the data this sees, so the means
//         do not depend on summation order.  HBM bound (reads Q' in tile
//         order and K' as the attention kernel's K tiles, once each).  q
//         means are stored [B,H,nB,d], k means transposed [B,H,d,nB] so the
//         score loop reads them coalesced.
//  topk   one workgroup per (b, h, R <= 8 query blocks): float64 scores of
//         the R rows against every key block into LDS (each thread walks one
//         key block's transposed mean with 16 loads in flight, the query
//         means broadcast from LDS), then one wave per row
//         finds the r-th largest eligible score by a bitwise search on
//         order-preserving 64-bit keys (ballot + popcount, no sorting),
//         takes equal scores lowest index first, and writes the kept
//         block indices in ascending order with ballot prefix counts.
#include "kernels.h"

namespace sva {

namespace {

constexpr int kPoolThreads = 256;

template <int D>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(DevPlan p, const u32x4* qr,
                                                            double* qmean) {
    constexpr int LPR = D / 8;
    constexpr int RG = kPoolThreads / LPR;   // row groups
    __shared__ double part[RG][D];
    const int kb = blockIdx.x % p.nB;
    const int64_t bh = blockIdx.x / p.nB;
    const int sb = p.block / p.nsub;         // rows per run
    const int s0 = blockIdx.y * sb;          // first row of this run
    const u32x4* src = qr + (bh * p.Np + (int64_t)kb * p.block) * LPR;
    const int dc = threadIdx.x % LPR;
    const int rg = threadIdx.x / LPR;
    const int valid = min(max(p.blk_valid[kb] - s0, 0), sb);
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int r = rg; r < valid; r += RG) {
        const u32x4 v = src[(int64_t)(s0 + r) * LPR + dc];
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += (double)bf16lo(u[e]);
            acc[2 * e + 1] += (double)bf16hi(u[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[rg][dc * 8 + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < D) {
        double s = 0.0;
#pragma unroll 4
        for (int g = 0; g < RG; ++g) s += part[g][threadIdx.x];
        qmean[((bh * p.nB + kb) * p.nsub + blockIdx.y) * D + threadIdx.x] =
            valid > 0 ? s / (double)valid : 0.0;
    }
}

// K means from K tiles: token r = 32g + j of a block sits in entry
// g·4D + c·32 + j of the block's tile for 8-channel chunk c (channels 8c ..
// 8c+7).  One workgroup per (block, run); thread (j, q) sums chunks q, q + 8,
// ... over the run's tokens; the 32 partial sums of a chunk are added
// through LDS.  Output transposed: [B, H, d, nB·nsub].
template <int D, int BLK>
__global__ __launch_bounds__(kPoolThreads) void pool_kt_kernel(DevPlan p, const u32x4* kt,
                                                               double* kmeanT) {
    constexpr int NCH = D / 8;                 // 8-channel chunks
    constexpr int CPT = NCH / 8;               // chunks per thread
    __shared__ double part[32][D + 1];
    const int kb = blockIdx.x % p.nB;
    const int64_t bh = blockIdx.x / p.nB;
    const int sb = BLK / p.nsub;               // tokens per run
    const int s0 = blockIdx.y * sb;
    const u32x4* src = kt + (bh * p.nB + kb) * (int64_t)(BLK * NCH);
    const int j = threadIdx.x % 32, q = threadIdx.x / 32;
    const int valid = min(max(p.blk_valid[kb] - s0, 0), sb);
    double acc[CPT][8];
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = 0.0;
    for (int r = j; r < valid; r += 32) {
        const int tok = s0 + r;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const u32x4 v = src[(tok >> 5) * 4 * D + (q + 8 * i) * 32 + (tok & 31)];
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[i][2 * e] += (double)bf16lo(u[e]);
                acc[i][2 * e + 1] += (double)bf16hi(u[e]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) part[j][(q + 8 * i) * 8 + e] = acc[i][e];
    __syncthreads();
    if (threadIdx.x < D) {
        double s = 0.0;
#pragma unroll 8
        for (int jj = 0; jj < 32; ++jj) s += part[jj][threadIdx.x];
        kmeanT[(bh * D + threadIdx.x) * ((int64_t)p.nB * p.nsub) + (int64_t)kb * p.nsub + blockIdx.y] =
            valid > 0 ? s / (double)valid : 0.0;
    }
}

constexpr int kTopkThreads = 256;
constexpr int kScoreLds = 65536;   // bytes of LDS for the q means and score rows

__device__ __forceinline__ uint64_t order_key(double s) {
    // canonical +0, then flip so unsigned order = numeric order
    const uint64_t u = (uint64_t)__double_as_longlong(s + 0.0);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const uint64_t o = __shfl_xor(v, m, 64);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const uint64_t o = __shfl_xor(v, m, 64);
        v = o < v ? o : v;
    }
    return v;
}

// log of the valid count of run a of block b (-inf for an empty run)
__device__ __forceinline__ double log_count(const DevPlan& p, int b, int a) {
    const int sb = p.block / p.nsub;
    const int c = min(max(p.blk_valid[b] - a * sb, 0), sb);
    return c > 0 ? log((double)c) : -INFINITY;
}

template <int D, int NSLOT, int NSUB>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(DevPlan p, const double* qmean,
                                                            const double* kmeanT, int R,
                                                            int32_t* col) {
    constexpr int RT = 8;              // rows computed per pass over the key means
    constexpr int DB = 16;             // key-mean loads in flight per thread
    constexpr int QW = RT * NSUB;      // query runs held per pass
    extern __shared__ double smem[];
    double* qs = smem;                 // [D][QW], rows past nrows zero
    double* sc = smem + QW * D;        // [R][nB]
    const int nB = p.nB;
    const int groups = (nB + R - 1) / R;
    const int g = blockIdx.x % groups;
    const int64_t bh = blockIdx.x / groups;
    const int qb0 = g * R;
    const int nrows = min(R, nB - qb0);

    for (int i = threadIdx.x; i < QW * D; i += kTopkThreads) {
        const int dd = i / QW, ra = i % QW;
        qs[i] = ra / NSUB < nrows ? qmean[((bh * nB + qb0) * NSUB + ra) * D + dd] : 0.0;
    }
    __syncthreads();

    const double* kt = kmeanT + bh * D * (int64_t)nB * NSUB;
    if (NSUB == 1 && p.scorer == 0) {
        // mean scorer: thread per key block, all RT rows at once; each score
        // is the sequential fma chain over the channels
        for (int kb = threadIdx.x; kb < nB; kb += kTopkThreads) {
            double acc[RT];
#pragma unroll
            for (int r = 0; r < RT; ++r) acc[r] = 0.0;
            for (int d0 = 0; d0 < D; d0 += DB) {
                double kv[DB];
#pragma unroll
                for (int i = 0; i < DB; ++i) kv[i] = kt[(int64_t)(d0 + i) * nB + kb];
#pragma unroll
                for (int i = 0; i < DB; ++i) {
                    const double2* q2 = reinterpret_cast<const double2*>(qs + (d0 + i) * RT);
#pragma unroll
                    for (int r2 = 0; r2 < RT / 2; ++r2) {
                        const double2 qq = q2[r2];
                        acc[2 * r2] = fma(qq.x, kv[i], acc[2 * r2]);
                        acc[2 * r2 + 1] = fma(qq.y, kv[i], acc[2 * r2 + 1]);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < RT; ++r)
                if (r < nrows) sc[r * nB + kb] = acc[r];
        }
    } else {
        // SubBlock scorer: thread per key run (kb, b), the NSUB runs of a key
        // block in adjacent lanes.  Dot products with every query run of the
        // RT rows, then per row the log-sum-exp over query runs (in the
        // thread) and key runs (across the NSUB lanes).
        const double inv_sqrt_d = 1.0 / sqrt((double)D);
        const int nks = nB * NSUB;
        const int iters = (nks + kTopkThreads - 1) / kTopkThreads;
        for (int it = 0; it < iters; ++it) {
            const int ks = it * kTopkThreads + threadIdx.x;
            const bool act = ks < nks;
            const int kcol = act ? ks : nks - 1;
            double acc[QW];
#pragma unroll
            for (int r = 0; r < QW; ++r) acc[r] = 0.0;
            for (int d0 = 0; d0 < D; d0 += DB) {
                double kv[DB];
#pragma unroll
                for (int i = 0; i < DB; ++i) kv[i] = kt[(int64_t)(d0 + i) * nks + kcol];
#pragma unroll
                for (int i = 0; i < DB; ++i) {
                    const double2* q2 = reinterpret_cast<const double2*>(qs + (d0 + i) * QW);
#pragma unroll
                    for (int r2 = 0; r2 < QW / 2; ++r2) {
                        const double2 qq = q2[r2];
                        acc[2 * r2] = fma(qq.x, kv[i], acc[2 * r2]);
                        acc[2 * r2 + 1] = fma(qq.y, kv[i], acc[2 * r2 + 1]);
                    }
                }
            }
            const int kb = kcol / NSUB, b = kcol % NSUB;
            const double lk = log_count(p, kb, b);
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const int qb = qb0 + min(r, nrows - 1);
                double m = -INFINITY;
                double x[NSUB];
#pragma unroll
                for (int a = 0; a < NSUB; ++a) {
                    x[a] = acc[r * NSUB + a] * inv_sqrt_d + log_count(p, qb, a) + lk;
                    m = fmax(m, x[a]);
                }
                double sum = 0.0;
                if (m > -INFINITY) {
#pragma unroll
                    for (int a = 0; a < NSUB; ++a) sum += exp(x[a] - m);
                }
                // combine the NSUB key runs of this key block (adjacent lanes)
#pragma unroll
                for (int off = 1; off < NSUB; off <<= 1) {
                    const double mo = __shfl_xor(m, off, 64);
                    const double so = __shfl_xor(sum, off, 64);
                    const double mn = fmax(m, mo);
                    if (mn > -INFINITY) {
                        sum = (m > -INFINITY ? sum * exp(m - mn) : 0.0) +
                              (mo > -INFINITY ? so * exp(mo - mn) : 0.0);
                        m = mn;
                    }
                }
                if (act && b == 0 && r < nrows) sc[r * nB + kb] = m + log(sum);
            }
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
    for (int r = wave; r < nrows; r += kTopkThreads / 64) {
        const int qb = qb0 + r;
        const int len = p.row_ptr[qb + 1] - p.row_ptr[qb];
        int32_t* out = col + bh * p.nnz_per_head + p.row_ptr[qb];
        if (len >= nB) {                       // dense row
            for (int kb = lane; kb < nB; kb += 64) out[kb] = kb;
            continue;
        }
        const bool vrow = qb < p.nB_video;
        const int tq0 = p.blk_tmin[qb], tq1 = p.blk_tmax[qb];
        uint64_t key[NSLOT];
        uint64_t fbits = 0;
        int nforced = 0;
        uint64_t kmax = 0, kmin = ~0ull;
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
            const int kb = j * 64 + lane;
            bool forced = false;
            key[j] = 0;
            if (kb < nB) {
                forced = kb >= p.nB_video ||
                         (vrow && p.same_frame && tq0 <= p.blk_tmax[kb] && p.blk_tmin[kb] <= tq1);
                if (!forced) {
                    key[j] = order_key(sc[r * nB + kb]);
                    kmax = key[j] > kmax ? key[j] : kmax;
                    kmin = key[j] < kmin ? key[j] : kmin;
                }
            }
            if (forced) fbits |= 1ull << j;
            nforced += __popcll(__ballot(forced));
        }
        const int need = len - nforced;        // blocks to take from the ranking
        uint64_t T = ~0ull;                    // threshold key (r-th largest)
        int need_eq = 0;
        if (need > 0) {
            kmax = wave_max_u64(kmax);
            kmin = wave_min_u64(kmin);
            const uint64_t diff = kmax ^ kmin;
            int top = diff ? 63 - __clzll(diff) : -1;
            T = top >= 0 ? (kmin & ~((2ull << top) - 1)) : kmin;
            if (top == 63) T = 0;
            // largest T with count(key >= T) >= need
            for (int bit = top; bit >= 0; --bit) {
                const uint64_t cand = T | (1ull << bit);
                int cnt = 0;
#pragma unroll
                for (int j = 0; j < NSLOT; ++j) cnt += __popcll(__ballot(key[j] >= cand));
                if (cnt >= need) T = cand;
            }
            int gt = 0;
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) gt += __popcll(__ballot(key[j] > T));
            need_eq = need - gt;
        }
        int base = 0, eq_seen = 0;
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
            const int kb = j * 64 + lane;
            const bool forced = (fbits >> j) & 1ull;
            const bool eq = need > 0 && key[j] == T && kb < nB && !forced;
            const uint64_t em = __ballot(eq);
            const int eq_rank = eq_seen + __popcll(em & lt_mask);
            const bool keep = forced || (need > 0 && key[j] > T) || (eq && eq_rank < need_eq);
            const uint64_t km = __ballot(keep);
            const int slot = base + __popcll(km & lt_mask);
            if (keep && slot < len) out[slot] = kb;
            base += __popcll(km);
            eq_seen += __popcll(em);
        }
    }
}

}  // namespace

hipError_t launch_select(const DevPlan& p, const uint16_t* qr, const uint16_t* kt, double* ws,
                         int32_t* col, hipStream_t s) {
    const int64_t BH = (int64_t)p.B * p.H;
    double* qmean = ws;                                  // [B,H,nB,nsub,d]
    double* kmeanT = ws + BH * p.nB * p.nsub * p.d;      // [B,H,d,nB·nsub]
    if (qr && kt) {
        dim3 grid((unsigned)(BH * p.nB), (unsigned)p.nsub);
        const u32x4* q4 = reinterpret_cast<const u32x4*>(qr);
        const u32x4* k4 = reinterpret_cast<const u32x4*>(kt);
        if (p.d == 128) {
            hipLaunchKernelGGL(pool_kernel<128>, grid, dim3(kPoolThreads), 0, s, p, q4, qmean);
            if (p.block == 128)
                hipLaunchKernelGGL((pool_kt_kernel<128, 128>), grid, dim3(kPoolThreads), 0, s, p, k4, kmeanT);
            else
                hipLaunchKernelGGL((pool_kt_kernel<128, 64>), grid, dim3(kPoolThreads), 0, s, p, k4, kmeanT);
        } else {
            hipLaunchKernelGGL(pool_kernel<64>, grid, dim3(kPoolThreads), 0, s, p, q4, qmean);
            if (p.block == 128)
                hipLaunchKernelGGL((pool_kt_kernel<64, 128>), grid, dim3(kPoolThreads), 0, s, p, k4, kmeanT);
            else
                hipLaunchKernelGGL((pool_kt_kernel<64, 64>), grid, dim3(kPoolThreads), 0, s, p, k4, kmeanT);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // rows per workgroup: up to 8, as many as the score rows' LDS allows
    // next to the query runs (8 rows × nsub runs × d)
    const int qbytes = 8 * p.nsub * p.d * (int)sizeof(double);
    int R = (kScoreLds - qbytes) / (p.nB * (int)sizeof(double));
    R = R < 1 ? 1 : (R > 8 ? 8 : R);
    const int groups = (p.nB + R - 1) / R;
    dim3 grid((unsigned)(BH * groups));
    const size_t lds = (size_t)qbytes + (size_t)R * p.nB * sizeof(double);
    const int nslot = (p.nB + 63) / 64;
#define SVA_TOPK(DD, NS, NSB) \
    hipLaunchKernelGGL((topk_kernel<DD, NS, NSB>), grid, dim3(kTopkThreads), lds, s, p, qmean, kmeanT, R, col)
#define SVA_TOPK_S(DD, NSB)                                                                  \
    do {                                                                                     \
        if (nslot <= 4) SVA_TOPK(DD, 4, NSB);                                                \
        else if (nslot <= 8) SVA_TOPK(DD, 8, NSB);                                           \
        else if (nslot <= 12) SVA_TOPK(DD, 12, NSB);                                         \
        else if (nslot <= 16) SVA_TOPK(DD, 16, NSB);                                         \
        else if (nslot <= 32) SVA_TOPK(DD, 32, NSB);                                         \
        else SVA_TOPK(DD, 64, NSB);                                                          \
    } while (0)
#define SVA_TOPK_D(DD)                                                                       \
    do {                                                                                     \
        if (p.nsub == 1) SVA_TOPK_S(DD, 1);                                                  \
        else if (p.nsub == 2) SVA_TOPK_S(DD, 2);                                             \
        else SVA_TOPK_S(DD, 4);                                                              \
    } while (0)
    if (p.d == 128) SVA_TOPK_D(128);
    else SVA_TOPK_D(64);
#undef SVA_TOPK_D
#undef SVA_TOPK_S
#undef SVA_TOPK
    return hipGetLastError();
}

}  // namespace sva
