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
//         the R rows against every key block into LDS (each thread computes
//         two rows against four consecutive key runs, so one LDS read of the
//         query means feeds four fma; reading them once per fma would make
//         the loop bound by LDS bandwidth), then one wave per row
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
// bytes of LDS for the q means and score rows: up to 8 rows per workgroup
// (each row costs nB·8 bytes); large enough for 4 rows at the plan's
// maximum of 4096 blocks, so a workgroup reads the key means for 4 rows at
// once instead of one
constexpr int kScoreLds = 147456;

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

// valid tokens of run a of block b
__device__ __forceinline__ int run_count(const DevPlan& p, int b, int a) {
    const int sb = p.block / p.nsub;
    return min(max(p.blk_valid[b] - a * sb, 0), sb);
}

template <int D, int NSLOT, int NSUB, bool SUBBLOCK>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(DevPlan p, const double* qmean,
                                                            const double* kmeanT, int R,
                                                            int32_t* col) {
    constexpr int RT = 8;              // rows per workgroup pass (R <= RT)
    constexpr int DB = 4;              // channels of key means loaded per batch
    constexpr int QW = RT * NSUB;      // query runs held in LDS
    constexpr int QT = 2 * NSUB;       // query runs per thread (two rows)
    extern __shared__ double smem[];
    double* qs = smem;                 // [D][QW], rows past nrows zero
    double* sc = smem + QW * D;        // [R][nB]
    double* lgt = sc + R * p.nB;       // [block + 1]: log of a run's valid count
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
    if (SUBBLOCK)
        for (int c = threadIdx.x; c <= p.block; c += kTopkThreads)
            lgt[c] = c > 0 ? log((double)c) : -INFINITY;
    __syncthreads();

    const double* kt = kmeanT + bh * D * (int64_t)nB * NSUB;
    if constexpr (!SUBBLOCK) {
        // Mean scorer: thread per key block, all RT rows at once (its key
        // means are one 512-byte wave load per channel, the query means a
        // broadcast LDS read); each score is the sequential fma chain over
        // the channels.
        constexpr int DBM = 16;
        for (int kb = threadIdx.x; kb < nB; kb += kTopkThreads) {
            double acc[RT];
#pragma unroll
            for (int r = 0; r < RT; ++r) acc[r] = 0.0;
            for (int d0 = 0; d0 < D; d0 += DBM) {
                double kv[DBM];
#pragma unroll
                for (int i = 0; i < DBM; ++i) kv[i] = kt[(int64_t)(d0 + i) * nB + kb];
#pragma unroll
                for (int i = 0; i < DBM; ++i) {
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
        // SubBlock scorer, as a register-blocked product: thread (kg, rp) =
        // (t / 4, t % 4) holds the QT query runs of rows 2rp, 2rp + 1 against
        // the 4 consecutive key runs ks0 .. ks0 + 3 (run ks = kb·NSUB + b of the
        // transposed key means).  Per channel: QT query values from LDS (one
        // address per lane quad), 4 key values, 4·QT fma, each a sequential
        // chain over the channels; one LDS read feeds four fma (one per fma
        // would make the loop bound by LDS bandwidth).  NSUB divides 4, so a
        // thread holds every key run of its key blocks and finishes the estimate
        //   log sum_a sum_b c_a c_b exp(qbar_a · kbar_b / sqrt(d))
        // itself.
        const int nks = nB * NSUB;
        const int rp = threadIdx.x & 3, kg = threadIdx.x >> 2;
        const double inv_sqrt_d = 1.0 / sqrt((double)D);
        double lq[2][NSUB];   // log valid counts of this thread's query runs
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
#pragma unroll
            for (int aa = 0; aa < NSUB; ++aa)
                lq[rr][aa] = lgt[run_count(p, qb0 + min(2 * rp + rr, nrows - 1), aa)];
        for (int ks0 = kg * 4; ks0 < nks; ks0 += kTopkThreads) {
            double acc[QT][4];
#pragma unroll
            for (int a2 = 0; a2 < QT; ++a2)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[a2][j] = 0.0;
            int kcol[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) kcol[j] = min(ks0 + j, nks - 1);
            // key means in batches of DB channels, the next batch loaded
            // while the current one is multiplied
            double kn[DB][4];
#pragma unroll
            for (int i = 0; i < DB; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) kn[i][j] = kt[(int64_t)i * nks + kcol[j]];
            for (int d0 = 0; d0 < D; d0 += DB) {
                double kv[DB][4];
#pragma unroll
                for (int i = 0; i < DB; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) kv[i][j] = kn[i][j];
                if (d0 + DB < D) {
#pragma unroll
                    for (int i = 0; i < DB; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            kn[i][j] = kt[(int64_t)(d0 + DB + i) * nks + kcol[j]];
                }
#pragma unroll
                for (int i = 0; i < DB; ++i) {
                    const double2* q2 = reinterpret_cast<const double2*>(qs + (d0 + i) * QW + rp * QT);
#pragma unroll
                    for (int a2 = 0; a2 < QT / 2; ++a2) {
                        const double2 qq = q2[a2];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            acc[2 * a2][j] = fma(qq.x, kv[i][j], acc[2 * a2][j]);
                            acc[2 * a2 + 1][j] = fma(qq.y, kv[i][j], acc[2 * a2 + 1][j]);
                        }
                    }
                }
            }
#pragma unroll
            for (int kk = 0; kk < 4 / NSUB; ++kk) {
                const int kb = ks0 / NSUB + kk;
                double lk[NSUB];
#pragma unroll
                for (int bb = 0; bb < NSUB; ++bb) lk[bb] = lgt[run_count(p, min(kb, nB - 1), bb)];
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    double x[NSUB][NSUB];
                    double m = -INFINITY;
#pragma unroll
                    for (int aa = 0; aa < NSUB; ++aa)
#pragma unroll
                        for (int bb = 0; bb < NSUB; ++bb) {
                            x[aa][bb] = acc[rr * NSUB + aa][kk * NSUB + bb] * inv_sqrt_d +
                                        lq[rr][aa] + lk[bb];
                            m = fmax(m, x[aa][bb]);
                        }
                    double sum = 0.0;
                    if (m > -INFINITY) {
#pragma unroll
                        for (int aa = 0; aa < NSUB; ++aa)
#pragma unroll
                            for (int bb = 0; bb < NSUB; ++bb) sum += exp(x[aa][bb] - m);
                    }
                    const int r = 2 * rp + rr;
                    if (r < nrows && kb < nB) sc[r * nB + kb] = m + log(sum);
                }
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
            // largest T with count(key >= T) >= need.  Once a candidate
            // leaves exactly `need` keys at or above it, those are the
            // kept ones and every later candidate keeps the same set, so
            // the search stops there (with distinct scores, after the bits
            // that separate the need-th key from the next).
            for (int bit = top; bit >= 0; --bit) {
                const uint64_t cand = T | (1ull << bit);
                int cnt = 0;
#pragma unroll
                for (int j = 0; j < NSLOT; ++j) cnt += __popcll(__ballot(key[j] >= cand));
                if (cnt >= need) {
                    T = cand;
                    if (cnt == need) break;
                }
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
    const size_t lds = (size_t)qbytes + (size_t)R * p.nB * sizeof(double) +
                       (size_t)(p.block + 1) * sizeof(double);
    const int nslot = (p.nB + 63) / 64;
#define SVA_TOPK(DD, NS, NSB, SBK)                                                           \
    hipLaunchKernelGGL((topk_kernel<DD, NS, NSB, SBK>), grid, dim3(kTopkThreads), lds, s, p,  \
                       qmean, kmeanT, R, col)
#define SVA_TOPK_S(DD, NSB, SBK)                                                             \
    do {                                                                                     \
        if (nslot <= 4) SVA_TOPK(DD, 4, NSB, SBK);                                           \
        else if (nslot <= 8) SVA_TOPK(DD, 8, NSB, SBK);                                      \
        else if (nslot <= 12) SVA_TOPK(DD, 12, NSB, SBK);                                    \
        else if (nslot <= 16) SVA_TOPK(DD, 16, NSB, SBK);                                    \
        else if (nslot <= 32) SVA_TOPK(DD, 32, NSB, SBK);                                    \
        else SVA_TOPK(DD, 64, NSB, SBK);                                                     \
    } while (0)
#define SVA_TOPK_D(DD)                                                                       \
    do {                                                                                     \
        if (p.scorer == 0) SVA_TOPK_S(DD, 1, false); /* mean scorer */                 \
        else if (p.nsub == 1) SVA_TOPK_S(DD, 1, true);                                       \
        else if (p.nsub == 2) SVA_TOPK_S(DD, 2, true);                                       \
        else SVA_TOPK_S(DD, 4, true);                                                        \
    } while (0)
    if (p.d == 128) SVA_TOPK_D(128);
    else SVA_TOPK_D(64);
#undef SVA_TOPK_D
#undef SVA_TOPK_S
#undef SVA_TOPK
    return hipGetLastError();
}

}  // namespace sva
