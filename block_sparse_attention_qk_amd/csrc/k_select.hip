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
//  topk   one workgroup per (b, h, R <= 8 query blocks): scores of the R
//         rows against every key block into LDS, then one wave per row
//         finds the r-th largest eligible score by a bitwise search on
//         order-preserving 64-bit keys (ballot + popcount, no sorting),
//         takes equal scores lowest index first, and writes the kept
//         block indices in ascending order with ballot prefix counts.
//         Mean scorer: float64 fma chains, a thread per key block, up to
//         1024 blocks; beyond that the products on the fp64 matrix cores.
//         SubBlock scorer: screened in fp32, decided in float64.  The run
//         products on the fp32 matrix cores and the estimate in fp32 give
//         every score with a bound on its distance from the float64 value
//         (fp32 rounding of a d-term dot product, by Cauchy-Schwarz on the
//         run norms, plus a few ulp for the rest); keys farther than twice
//         the row's largest bound from the row's fp32 cut are decided by
//         the fp32 scores, the few inside are re-scored in float64 and
//         ranked among themselves, so the kept set is the float64 one.
//         Workgroups are laid out so that each XCD works on whole heads
//         (their key means stay in its L2).
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

typedef double f64x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr double kLog2e = 1.4426950408889634;
constexpr double kLn2 = 0.6931471805599453;

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

// v from lane l ^ o (o = 1 or 2: within the lane's quad), by DPP quad permutation
__device__ __forceinline__ float quad_xor_f(float v, int o) {
    const int u = __float_as_int(v);
    return __int_as_float(o == 1 ? __builtin_amdgcn_update_dpp(0, u, 0xB1, 0xF, 0xF, false)
                                 : __builtin_amdgcn_update_dpp(0, u, 0x4E, 0xF, 0xF, false));
}

__device__ __forceinline__ double key_value(uint64_t k) {
    const uint64_t u = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
    return __longlong_as_double((long long)u);
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
    // products on the matrix cores: fp32 for the SubBlock scorer (screened,
    // then the keys near each row's cut re-scored in float64), fp64 for the
    // mean scorer beyond 1024 blocks (below that its fma loop is faster)
    constexpr bool MFMA = SUBBLOCK || NSLOT > 16;
    constexpr int QW = MFMA ? ((RT * NSUB + 15) / 16) * 16 : RT * NSUB;   // query runs in LDS
    constexpr int MT = (RT * NSUB + 15) / 16;   // 16-run query tiles
    constexpr int KS = D / 4;                   // 4-channel steps
    extern __shared__ double smem[];
    double* qs = smem;                 // [D][QW] (fma loop) or the MFMA operands in lane order
    double* sc = smem + QW * D;        // [R][nB]: scores; SubBlock: {fp32 score, its bound}
    double* lgt = sc + R * p.nB;       // [block + 1]: log of a run's valid count
    double* nq2 = lgt + p.block + 1;   // [RT * NSUB] SubBlock: squared norms of the query runs
    const int nB = p.nB;
    const int groups = (nB + R - 1) / R;
    // workgroup b runs on XCD b % 8: give each XCD a contiguous range of
    // (b, h, group) so the workgroups of one head share that XCD's L2
    const int wg = [] {
        const int b = blockIdx.x, G = gridDim.x;
        const int x = b & 7, q = G >> 3, r = G & 7;
        return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + (b >> 3);
    }();
    const int g = wg % groups;
    const int64_t bh = wg / groups;
    const int qb0 = g * R;
    const int nrows = min(R, nB - qb0);

    if constexpr (!MFMA) {
        for (int i = threadIdx.x; i < QW * D; i += kTopkThreads) {
            const int dd = i / QW, ra = i % QW;
            qs[i] = ra / NSUB < nrows ? qmean[((bh * nB + qb0) * NSUB + ra) * D + dd] : 0.0;
        }
    } else if constexpr (!SUBBLOCK) {
        // fp64 operands, entry (mt, s, l) = A[l % 16][l / 16] of step s of
        // query tile mt: run 16mt + 4(m % 4) + m / 4 (m = l % 16), channel
        // 4s + l / 16 (v_mfma_f64_16x16x4f64 hands a lane rows l / 16 + 4i)
        for (int i = threadIdx.x; i < MT * KS * 64; i += kTopkThreads) {
            const int l = i & 63, s = (i >> 6) % KS, mt = i / (64 * KS);
            const int m = l & 15;
            const int ra = mt * 16 + 4 * (m & 3) + (m >> 2);
            qs[i] = ra / NSUB < nrows ? qmean[((bh * nB + qb0) * NSUB + ra) * D + 4 * s + (l >> 4)] : 0.0;
        }
    } else {
        // fp32 operands, entry (mt, s, l) = A[l % 16][l / 16]: run
        // 16mt + l % 16, channel 4s + l / 16 (v_mfma_f32_16x16x4f32 hands a
        // lane rows 4(l / 16) + i, four consecutive runs); the squared norm
        // of every query run, in float64, for the error bound
        float* qs32 = reinterpret_cast<float*>(qs);
        for (int i = threadIdx.x; i < MT * KS * 64; i += kTopkThreads) {
            const int l = i & 63, s = (i >> 6) % KS, mt = i / (64 * KS);
            const int ra = mt * 16 + (l & 15);
            qs32[i] = ra / NSUB < nrows
                          ? (float)qmean[((bh * nB + qb0) * NSUB + ra) * D + 4 * s + (l >> 4)] : 0.f;
        }
        __syncthreads();
        // squared norms of the query runs from the staged values: eight
        // threads per run, D / 8 channels each
        {
            const int ra = threadIdx.x >> 3, part = threadIdx.x & 7;
            double ss = 0.0;
            if (ra < RT * NSUB) {
                const int mt = ra >> 4, m = ra & 15;
                for (int ch = part * (D / 8); ch < (part + 1) * (D / 8); ++ch) {
                    const double v = qs32[(mt * KS + (ch >> 2)) * 64 + (ch & 3) * 16 + m];
                    ss = fma(v, v, ss);
                }
            }
            ss += __shfl_xor(ss, 1, 64);
            ss += __shfl_xor(ss, 2, 64);
            ss += __shfl_xor(ss, 4, 64);
            if (part == 0 && ra < RT * NSUB) nq2[ra] = ss;
        }
    }
    if (SUBBLOCK)
        for (int c = threadIdx.x; c <= p.block; c += kTopkThreads)
            lgt[c] = c > 0 ? log((double)c) : -INFINITY;
    __syncthreads();

    const double* kt = kmeanT + bh * D * (int64_t)nB * NSUB;
    const int nks = nB * NSUB;
    if constexpr (!MFMA) {
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
        // A tile of 16 query runs x 16 key runs (whole blocks for the mean
        // scorer) is a sum of D/4 16x16x4 matrix instructions: lane l
        // supplies A[l % 16][l / 16] and B[l / 16][l % 16] of each 4-channel
        // step and receives four results of column l % 16, so the NSUB key
        // runs of a key block sit in NSUB neighbouring lanes.  The operands
        // of A were staged in LDS in lane order (one conflict-free read per
        // lane and instruction); each wave streams 16-run key tiles from
        // the transposed key means, the next tile loading while the current
        // one is multiplied.
        const int ntile = (nks + 15) / 16;
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int g4 = lane >> 4, n16 = lane & 15;
        const double inv_sqrt_d = 1.0 / sqrt((double)D);
        double lq[MT][4];     // log valid counts of this lane's query runs
        float nqr[MT][4 / NSUB];   // largest norm of the runs of this lane's query blocks
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = mt * 16 + 4 * g4 + i;
                const int row = j / NSUB;
                lq[mt][i] = SUBBLOCK && row < nrows ? lgt[run_count(p, qb0 + row, j % NSUB)] : 0.0;
            }
#pragma unroll
            for (int gr = 0; gr < 4 / NSUB; ++gr) {
                double mx = 0.0;
                if constexpr (SUBBLOCK) {
#pragma unroll
                    for (int a = 0; a < NSUB; ++a) {
                        const int j = mt * 16 + 4 * g4 + gr * NSUB + a;
                        mx = fmax(mx, j < RT * NSUB ? nq2[j] : 0.0);
                    }
                }
                nqr[mt][gr] = (float)sqrt(mx) * 1.0001f;
            }
        }
        // key means of this (b, h) through a buffer resource: per-lane byte
        // offset of (channel l / 16, run), plus a scalar offset per 4-channel step
        const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)kt, (short)0, D * nks * (int)sizeof(double), 0x00020000);
        // the valid count of the lane's key block (SubBlock) is loaded first,
        // with the tile's key means (loads complete in order: a later global
        // read would wait for the whole prefetch)
        auto load_tile = [&](double (&b)[KS], int& nval, int t) {
            const int ksc = min(t * 16 + n16, nks - 1);
            nval = SUBBLOCK ? p.blk_valid[ksc / NSUB] : 0;
            const int voff = (g4 * nks + ksc) * (int)sizeof(double);
#pragma unroll
            for (int s = 0; s < KS; ++s)
                b[s] = __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(
                                                      krs, voff, 4 * s * nks * (int)sizeof(double), 0));
        };
        const int sb = p.block / NSUB;   // tokens per run
        // per-score bound on |fp32 score - float64 score|: the fp32 dot
        // product of a query run and a key run is within
        // (d + 4) 2^-24 |q| |k| of the exact one (operands rounded to fp32
        // included; measured on gfx950: 4.9 2^-24 sum |q_i k_i| at d = 128),
        // the rest of the estimate in fp32 adds a few ulp of its terms
        const float c_dot = (float)((D + 16) * 5.9604644775390625e-08 * inv_sqrt_d);
        const float c_abs = 1.9073486328125e-06f;      // 2^-19
        const float l_sb = (float)log((double)sb);
        auto score_tile = [&](const double (&b)[KS], int nval, int t) {
            const int ks = t * 16 + n16;
            const int kb = ks / NSUB;
            if constexpr (!SUBBLOCK) {
                f64x4_t c[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) c[mt] = f64x4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll
                for (int s = 0; s < KS; ++s)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        c[mt] = __builtin_amdgcn_mfma_f64_16x16x4f64(qs[(mt * KS + s) * 64 + lane],
                                                                     b[s], c[mt], 0, 0, 0);
                // lane (l / 16, l % 16) holds query blocks 4(l / 16) + i
                // against key block kb
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = mt * 16 + 4 * g4 + i;
                        if (row < nrows && kb < nB) sc[row * nB + kb] = c[mt][i];
                    }
            } else {
                const float* qs32 = reinterpret_cast<const float*>(qs);
                f32x4_t c[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) c[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                double kk = 0.0;          // squared norm of this lane's share of the key run
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const float bf = (float)b[s];
                    kk = fma(b[s], b[s], kk);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        c[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(qs32[(mt * KS + s) * 64 + lane],
                                                                     bf, c[mt], 0, 0, 0);
                }
                kk += __shfl_xor(kk, 16, 64);
                kk += __shfl_xor(kk, 32, 64);
                float nk = sqrtf((float)kk);
#pragma unroll
                for (int o = 1; o < NSUB; o <<= 1) nk = fmaxf(nk, quad_xor_f(nk, o));
                nk *= 1.0001f;
                const float lk = (float)lgt[min(max(nval - (ks % NSUB) * sb, 0), sb)];
                float2* sc2 = reinterpret_cast<float2*>(sc);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int gr = 0; gr < 4 / NSUB; ++gr) {
                        float x[NSUB];
                        float m = -INFINITY;
#pragma unroll
                        for (int a = 0; a < NSUB; ++a) {
                            x[a] = c[mt][gr * NSUB + a] * (float)inv_sqrt_d +
                                   ((float)lq[mt][gr * NSUB + a] + lk);
                            m = fmaxf(m, x[a]);
                        }
#pragma unroll
                        for (int o = 1; o < NSUB; o <<= 1) m = fmaxf(m, quad_xor_f(m, o));
                        // every term -inf (no valid token pairs): sum 0, score -inf
                        const float mm = m > -INFINITY ? m : 0.f;
                        float sum = 0.f;
#pragma unroll
                        for (int a = 0; a < NSUB; ++a)
                            sum += __builtin_amdgcn_exp2f((x[a] - mm) * (float)kLog2e);
#pragma unroll
                        for (int o = 1; o < NSUB; o <<= 1) sum += quad_xor_f(sum, o);
                        const float s32 = m + (float)kLn2 * __builtin_amdgcn_logf(sum);
                        // (an empty estimate, -inf, is exact)
                        const float e = s32 > -INFINITY
                                            ? c_dot * nqr[mt][gr] * nk +
                                                  c_abs * (4.f + fabsf(s32) + 2.f * l_sb)
                                            : 0.f;
                        const int row = (mt * 16 + 4 * g4) / NSUB + gr;
                        if (n16 % NSUB == 0 && row < nrows && kb < nB)
                            sc2[row * nB + kb] = make_float2(s32, e);
                    }
            }
        };
        // One tile per iteration: the tile loaded during the previous one is
        // copied out, the next one's loads are issued, then the products.
        // The loads are issued unconditionally (tile index clamped): a load
        // under a condition makes the compiler wait, at the first product,
        // for the loads of the tile after it as well.
        double bn[KS];
        int vn;
        load_tile(bn, vn, min(wave, ntile - 1));
        for (int t = wave; t < ntile; t += 4) {
            double bc[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) bc[s] = bn[s];
            const int vc = vn;
            load_tile(bn, vn, min(t + 4, ntile - 1));
            __builtin_amdgcn_sched_barrier(0);    // keep the prefetch ahead of the products
            score_tile(bc, vc, t);
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
    // the `need`-th largest key T (a prefix of it once the kept set is
    // fixed) and how many keys equal to T are kept, by a bitwise search on
    // order-preserving 64-bit keys (0 = not a candidate)
    // prefix: start below the bits every key shares (a wave max and min
    // first).  Dot-product scores take both signs, so their keys differ in
    // the top bit and the mean scorer starts there; SubBlock estimates
    // (positive, close together) share many leading bits.
    auto threshold = [&](const uint64_t (&key)[NSLOT], int need, uint64_t& T, int& need_eq,
                         bool prefix) {
        int top = 63;
        T = 0;
        if (prefix) {
            uint64_t kmax = 0, kmin = ~0ull;
#pragma unroll
            for (int j = 0; j < NSLOT; ++j)
                if (key[j]) {
                    kmax = key[j] > kmax ? key[j] : kmax;
                    kmin = key[j] < kmin ? key[j] : kmin;
                }
            kmax = wave_max_u64(kmax);
            kmin = wave_min_u64(kmin);
            const uint64_t diff = kmax ^ kmin;
            top = diff ? 63 - __clzll(diff) : -1;
            T = top >= 0 ? (kmin & ~((2ull << top) - 1)) : kmin;
            if (top == 63) T = 0;
        }
        // largest T with count(key >= T) >= need.  Once a candidate leaves
        // exactly `need` keys at or above it, those are the kept ones and
        // every later candidate keeps the same set, so the search stops
        // there (with distinct scores, after the bits that separate the
        // need-th key from the next).
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
    };
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
        float erow = 0.f;                      // SubBlock: largest score bound of the row
        uint64_t fbits = 0;
        int nforced = 0;
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
            const int kb = j * 64 + lane;
            bool forced = false;
            key[j] = 0;
            if (kb < nB) {
                forced = kb >= p.nB_video ||
                         (vrow && p.same_frame && tq0 <= p.blk_tmax[kb] && p.blk_tmin[kb] <= tq1);
                if (!forced) {
                    if constexpr (SUBBLOCK) {
                        const float2 se = reinterpret_cast<const float2*>(sc)[r * nB + kb];
                        key[j] = order_key((double)se.x);
                        erow = fmaxf(erow, se.y);
                    } else {
                        key[j] = order_key(sc[r * nB + kb]);
                    }
                }
            }
            if (forced) fbits |= 1ull << j;
            nforced += __popcll(__ballot(forced));
        }
        const int need = len - nforced;        // blocks to take from the ranking
        uint64_t T = ~0ull;
        int need_eq = 0;
        uint64_t bbits = 0;                    // SubBlock: slots in the band, kept by rescoring
        if (need > 0) {
            threshold(key, need, T, need_eq, SUBBLOCK);
            if constexpr (SUBBLOCK) {
                // The fp32 scores decide every key farther than twice the
                // row's largest bound from the need-th largest fp32 score
                // tv: the float64 scores of keys above tv + 2e all exceed
                // the float64 threshold, those below tv - 2e all fall short
                // of it.  Keys in the band are re-scored in float64
                // (sequential fma, exact log and exp) and ranked among
                // themselves for the remaining places; equal scores keep
                // the lower block index.
                uint64_t tk = ~0ull;           // the need-th largest key
#pragma unroll
                for (int j = 0; j < NSLOT; ++j)
                    if (key[j] && key[j] >= T) tk = key[j] < tk ? key[j] : tk;
                tk = wave_min_u64(tk);
                const double tv = key_value(tk);
                float em = erow;
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) em = fmaxf(em, __shfl_xor(em, o, 64));
                const double band = 2.0 * (double)em;
                const uint64_t k_hi = order_key(tv + band), k_lo = order_key(tv - band);
                int n_hi = 0, n_band = 0;
                uint64_t hbits = 0;            // slots above the band
#pragma unroll
                for (int j = 0; j < NSLOT; ++j) {
                    const bool hi = key[j] && key[j] > k_hi;
                    const bool bd = key[j] && !hi && key[j] >= k_lo;
                    n_hi += __popcll(__ballot(hi));
                    n_band += __popcll(__ballot(bd));
                    if (hi) hbits |= 1ull << j;
                    if (bd) bbits |= 1ull << j;
                }
                const int need_b = need - n_hi;
                // the band keys' float64 estimates, in place of the fp32 keys:
                // one key at a time over the whole wave, lane (pair, quarter)
                // = (l / 4, l % 4) forming the dot product of query run
                // pair / NSUB and key run pair % NSUB over a quarter of the
                // channels in sequential fma
                const double* qm = qmean + (bh * nB + qb) * NSUB * (int64_t)D;
                const int pr = lane >> 2, qt = lane & 3;
                const int pa = (pr / NSUB) % NSUB, pb = pr % NSUB;
                const double lqa = lgt[run_count(p, qb, pa)];
                const double isd = 1.0 / sqrt((double)D);
                auto exact_score = [&](int kb) -> double {
                    double acc = 0.0;
#pragma unroll 8
                    for (int ch = qt * (D / 4); ch < (qt + 1) * (D / 4); ++ch)
                        acc = fma(qm[pa * D + ch], kt[(int64_t)ch * nks + kb * NSUB + pb], acc);
                    acc += __shfl_xor(acc, 1, 64);
                    acc += __shfl_xor(acc, 2, 64);
                    double x = pr < NSUB * NSUB ? acc * isd + lqa + lgt[run_count(p, kb, pb)]
                                                : -INFINITY;
                    double xm = x;
#pragma unroll
                    for (int o = 4; o < 64; o <<= 1) xm = fmax(xm, __shfl_xor(xm, o, 64));
                    double e = (xm > -INFINITY && qt == 0) ? exp(x - xm) : 0.0;
#pragma unroll
                    for (int o = 1; o < 64; o <<= 1) e += __shfl_xor(e, o, 64);
                    return xm + log(e);     // -inf when no run pair has valid tokens
                };
                uint64_t (&key2)[NSLOT] = key;
#pragma unroll
                for (int j = 0; j < NSLOT; ++j) {
                    const bool inb = (bbits >> j) & 1ull;
                    key2[j] = (inb && need_b >= n_band) ? 1ull : 0ull;   // every band key is kept
                    if (need_b < n_band) {
                        uint64_t bm = __ballot(inb);
                        while (bm) {
                            const int L = __ffsll((unsigned long long)bm) - 1;
                            bm &= bm - 1;
                            const uint64_t kx = order_key(exact_score(j * 64 + L));
                            if (lane == L) key2[j] = kx;
                        }
                    }
                }
                uint64_t T2 = 0;
                int need_eq2 = 0;
                if (need_b > 0 && need_b < n_band) threshold(key2, need_b, T2, need_eq2, true);
                // band keys kept: key2 > T2, or equal to T2 in index order
                int eq_seen = 0;
                uint64_t kbits = 0;
#pragma unroll
                for (int j = 0; j < NSLOT; ++j) {
                    const bool inb = (bbits >> j) & 1ull;
                    bool keep = false;
                    if (need_b >= n_band) {
                        keep = inb;
                    } else if (need_b > 0) {
                        const bool eq = inb && key2[j] == T2;
                        const uint64_t emk = __ballot(eq);
                        const int eq_rank = eq_seen + __popcll(emk & lt_mask);
                        keep = inb && (key2[j] > T2 || (eq && eq_rank < need_eq2));
                        eq_seen += __popcll(emk);
                    }
                    if (keep) kbits |= 1ull << j;
                }
                // final: forced, above the band, or kept from the band
                int base = 0;
#pragma unroll
                for (int j = 0; j < NSLOT; ++j) {
                    const int kb = j * 64 + lane;
                    const bool forced = (fbits >> j) & 1ull;
                    const bool keep = forced || ((hbits | kbits) >> j) & 1ull;
                    const uint64_t km = __ballot(keep);
                    const int slot = base + __popcll(km & lt_mask);
                    SVA_DCHECK(p, !keep || kb < nB, SVA_DEBUG_LIST);
                    if (keep && slot < len) out[slot] = kb;
                    base += __popcll(km);
                }
                SVA_DCHECK(p, base == len, SVA_DEBUG_LIST);
                continue;
            }
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
            SVA_DCHECK(p, !keep || kb < nB, SVA_DEBUG_LIST);
            if (keep && slot < len) out[slot] = kb;
            base += __popcll(km);
            eq_seen += __popcll(em);
        }
        SVA_DCHECK(p, base == len, SVA_DEBUG_LIST);
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
    const int nslot = (p.nB + 63) / 64;
    const int qruns = p.scorer == 0 && nslot <= 16 ? 8 : (8 * p.nsub + 15) / 16 * 16;
    const int qbytes = qruns * p.d * (int)sizeof(double);
    int R = (kScoreLds - qbytes) / (p.nB * (int)sizeof(double));
    R = R < 1 ? 1 : (R > 8 ? 8 : R);
    const int groups = (p.nB + R - 1) / R;
    dim3 grid((unsigned)(BH * groups));
    const size_t lds = (size_t)qbytes + (size_t)R * p.nB * sizeof(double) +
                       (size_t)(p.block + 1 + 8 * p.nsub) * sizeof(double);
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
