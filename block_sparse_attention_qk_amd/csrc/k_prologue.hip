// Fused QK-RMSNorm + 3D-RoPE.
//
// Follows "MiniMax-H3 在 8×H200 上基准测试", section "内核层": the QK RMSNorm
// and the 3D RoPE run as one kernel, on the exact rounding path that stores
// the normalised value (bf16) before rotating it.  Per (token, head) row x:
//   y = bf16(x · rsqrt(mean(x²) + eps) · w[h]),  out = bf16(rotate(y)),
// rotate turning channel pairs (2i, 2i+1) of the t/h/w sections by
// coordinate · theta^(-2i/width) (cos/sin from the plan's tables).
//
// The tiled variant writes straight into the attention layouts (Q' in tile
// order, K' as K tiles), so the separate reorders of Q' and K' disappear.
//
// Streaming kernel, bound by HBM: every row is read once and written once
// (4 · rows · d · 2 bytes for Q and K).  d/8 lanes own one row, 16 bytes
// each, so a wave moves 1 KB of contiguous rows per access; the sum of
// squares is reduced across the row's lanes with xor shuffles.  Each
// thread handles kRows rows to keep several loads in flight.  The outputs
// are written with non-temporal stores (no use for them in the caches
// before the next kernel): bit-identical, the raster kernel 2-4 % faster
// (0.618-0.631 -> 0.611 ms at 720p, the pages' per-rank shape 0.050 ->
// 0.048-0.050 ms), the tiled kernel 0.666 -> 0.653 ms at 720p and the V
// reorder that follows it 0.295 -> 0.277 ms.  Non-temporal loads, or
// stores in the V reorder, were slower; so were 2 or 8 rows per thread and
// 128 or 512 threads per block.
#include "kernels.h"

namespace sva {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 4;   // rows per thread
// Tiled kernel: heads per workgroup.  The token indices and every row's
// cos/sin depend on the position only, so a workgroup that serves several
// heads of the same 128 positions computes and loads them once.  Measured
// (bit-identical outputs): 720p 0.718 -> 0.667 ms, 480p 0.137 -> 0.117 ms,
// HunyuanVideo 0.682 -> 0.633 ms; 8 heads no better at 720p and slower at
// 480p (12 heads make groups of 8 and 4); loading the first head's rows
// before the cos/sin work, or the next head's rows before computing the
// current one, was slower (0.745 and 0.743 ms at 720p).
constexpr int kHeadsPerGroup = 4;

// The arithmetic of one row, with every rounding explicit so that the
// raster and the tiled kernels produce the same bits.  HIP's __fmul_rn and
// friends are plain operators here, so contraction into FMA is switched off
// in these helpers: otherwise the compiler may fuse a product into the
// following add differently in each kernel.
__device__ __forceinline__ float rms_scale(float ss, float inv_d, float eps) {
    return rsqrtf(__fmaf_rn(ss, inv_d, eps));
}
__device__ __forceinline__ float norm_val(float v, float rs, float w) {
#pragma clang fp contract(off)
    return (v * rs) * w;
}
__device__ __forceinline__ uint32_t rotate_pair(uint32_t yb, float c, float s) {
#pragma clang fp contract(off)
    const float y0 = bf16lo(yb), y1 = bf16hi(yb);
    const float a = y0 * c, b = y1 * s, e = y0 * s, f = y1 * c;
    return pack_bf16x2(a - b, e + f);
}

struct ProArgs {
    DevPlan p;
    const uint16_t* in[2];
    uint16_t* out[2];
    const float* w[2];
    double* mean[2];   // tiled kernel: block means to write, or NULL
    int hg;            // tiled kernel: heads per workgroup
};

template <int D>
__global__ __launch_bounds__(kThreads) void prologue_kernel(ProArgs a) {
    constexpr int LPR = D / 8;                 // lanes per row
    constexpr int RPB = kThreads / LPR;        // rows per block per step
    const int tensor = blockIdx.y;
    const DevPlan& p = a.p;
    const u32x4* in = reinterpret_cast<const u32x4*>(a.in[tensor]);
    u32x4* out = reinterpret_cast<u32x4*>(a.out[tensor]);
    const float* __restrict__ w = a.w[tensor];
    const int sub = threadIdx.x % LPR;
    // row = (b·N + n)·H + h; the plan guarantees fewer than 2^31 rows
    const uint32_t rows = (uint32_t)(p.B * p.N * p.H);
    const uint32_t row0 = blockIdx.x * (uint32_t)(RPB * kRows) + threadIdx.x / LPR;

    // Loads go out in branch-free batches (rows, weights, cos/sin) from
    // addresses clamped to the last row, so a thread's loads are in flight
    // together; past-the-end rows are computed and not stored.
    u32x4 x[kRows];
    uint32_t hr[kRows], nr[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const uint32_t row = min(row0 + r * RPB, rows - 1);
        x[r] = in[(int64_t)row * LPR + sub];
        const uint32_t tok = fast_div(row, p.div_H);
        hr[r] = row - tok * (uint32_t)p.H;
        nr[r] = tok - fast_div(tok, p.div_N) * (uint32_t)p.N;
    }
    float wv[kRows][8];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        if (w) {
            const float4* wp = reinterpret_cast<const float4*>(w + hr[r] * D + sub * 8);
            const float4 w0 = wp[0], w1 = wp[1];
            wv[r][0] = w0.x; wv[r][1] = w0.y; wv[r][2] = w0.z; wv[r][3] = w0.w;
            wv[r][4] = w1.x; wv[r][5] = w1.y; wv[r][6] = w1.z; wv[r][7] = w1.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) wv[r][e] = 1.f;
        }
    }

    // this lane's four channel pairs: RoPE section (-1: not rotated), the
    // pair's offset in that section's cos/sin table and the section's width
    int pax[4], pbase[4], phalf[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        int pi = sub * 4 + e;
        pax[e] = -1;
        pbase[e] = 0;
        phalf[e] = 0;
#pragma unroll
        for (int ax = 0; ax < 3; ++ax) {
            const int half = p.rope_half[ax];
            if (pax[e] < 0 && pi < half) {
                pax[e] = ax;
                pbase[e] = p.rope_off[ax] + pi;
                phalf[e] = half;
            }
            pi -= half;
        }
    }
    // cos/sin of every row's pairs (grid coordinates (t, h, w) of a video
    // token; extra tokens and pairs past the sections are not rotated; the
    // table always holds entry 0)
    float2 cs[kRows][4];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const bool video = nr[r] < (uint32_t)p.n_video;
        const uint32_t n = video ? nr[r] : 0u;
        const uint32_t pt = fast_div(n, p.div_HW);
        const uint32_t rem = n - pt * (uint32_t)(p.Hh * p.W);
        const uint32_t ph = fast_div(rem, p.div_W);
        const uint32_t pw = rem - ph * (uint32_t)p.W;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t gp = pax[e] == 0 ? pt : (pax[e] == 1 ? ph : pw);
            const bool rot = video && pax[e] >= 0;
            cs[r][e] = p.rope_cs[rot ? pbase[e] + gp * (uint32_t)phalf[e] : 0u];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool rot = video && pax[e] >= 0;
            cs[r][e] = rot ? cs[r][e] : make_float2(1.f, 0.f);
        }
    }
    const float inv_d = 1.0f / D;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const uint32_t row = row0 + r * RPB;
        const uint32_t u[4] = {x[r].x, x[r].y, x[r].z, x[r].w};
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = bf16lo(u[e]);
            v[2 * e + 1] = bf16hi(u[e]);
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
        const float rs = rms_scale(ss, inv_d, p.eps);
        // norm, round to bf16 (the stored value the rotation starts from),
        // rotate
        uint32_t ob[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t yb = pack_bf16x2(norm_val(v[2 * e], rs, wv[r][2 * e]),
                                            norm_val(v[2 * e + 1], rs, wv[r][2 * e + 1]));
            ob[e] = rotate_pair(yb, cs[r][e].x, cs[r][e].y);
        }
        if (row < rows)
            __builtin_nontemporal_store(u32x4{ob[0], ob[1], ob[2], ob[3]}, out + (int64_t)row * LPR + sub);
    }
}

// The prologue written straight into the attention layouts.  A workgroup
// owns PW = 128 consecutive tile positions of kHeadsPerGroup heads of one
// b; position pos holds raster token inv[pos] (or padding).  The token
// indices and the cos/sin values are loaded once, each as one branch-free
// batch (clamped addresses, values discarded afterwards where a row does not
// exist), so a thread's loads are in flight together; then, head by head,
// the rows are loaded and computed exactly as in the raster kernel (d/8
// lanes per row).  Per head,
//  Q' (KT = false): written as tile-order rows, contiguous per workgroup;
//  K' (KT = true): staged in LDS (row stride padded by 16 bytes so the
//     column reads below are free of bank conflicts) and written as K tiles:
//     wave g owns the 32-token group g, lane 32·hf + j reads chunk 2s + hf of
//     token j, so every step s writes one contiguous 1 KB span.
// Padding positions (no raster token) are written as zeros.
//
// With mean != NULL the workgroup also pools what it wrote, for the block
// selection: float64 sums over each run of block/nsub positions (padding
// rows are zeros and add nothing), divided by the run's valid count, stored
// as the selection's q means [B,H,nB,nsub,d] or transposed k means
// [B,H,d,nB·nsub].  Sums of at most 128 bf16 values are exact in float64 for
// the data this sees, so the means equal those of a separate pooling pass.
template <int D, bool KT>
__global__ __launch_bounds__(kThreads) void prologue_tiled_kernel(ProArgs a) {
    constexpr int LPR = D / 8;                 // 16-byte chunks (lanes) per row
    constexpr int DS = D / 16;                 // K-tile steps (chunk pairs)
    constexpr int PW = 128;                    // positions per workgroup
    constexpr int RPP = kThreads / LPR;        // rows per pass
    constexpr int NP = PW / RPP;               // rows per thread
    constexpr int LS = LPR + 1;                // LDS row stride in chunks
    __shared__ u32x4 stage[PW * LS];
    const int tensor = KT ? 1 : 0;
    const DevPlan& p = a.p;
    const u32x4* in = reinterpret_cast<const u32x4*>(a.in[tensor]);
    u32x4* out = reinterpret_cast<u32x4*>(a.out[tensor]);
    const float* __restrict__ w = a.w[tensor];
    double* __restrict__ mean = a.mean[tensor];
    const int per_head = (int)((p.Np + PW - 1) / PW);
    const int n_hg = (p.H + a.hg - 1) / a.hg;
    const int64_t bg = blockIdx.x / per_head;  // (b, head group)
    const int pos0 = (int)(blockIdx.x - bg * per_head) * PW;
    const int64_t b = bg / n_hg;
    const int h0 = (int)(bg - b * n_hg) * a.hg;
    const int h1 = min(h0 + a.hg, p.H);
    const int sub = threadIdx.x % LPR;
    const int r0 = threadIdx.x / LPR;
    const uint32_t hw = (uint32_t)(p.Hh * p.W);

    // The token indices, the RoPE sections and every row's cos/sin depend
    // on the position only: computed once, used for every head of the group.
    int nr[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int pos = pos0 + r0 + i * RPP;
        const int n = p.inv[pos < p.Np ? pos : p.Np - 1];
        SVA_DCHECK(p, pos >= p.Np || (n >= -1 && n < p.N), SVA_DEBUG_TOKEN);
        nr[i] = pos < p.Np ? n : -2;          // -2: past the end, -1: padding
    }
    // this thread's rows (raster offsets of head 0, clamped to a valid row)
    int64_t roff[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int n = nr[i] >= 0 ? nr[i] : 0;
        roff[i] = ((b * p.N + n) * p.H) * LPR + sub;
    }
    // this lane's channel pairs: RoPE section (-1: none), offset in its
    // table and the section's width
    int pax[4], pbase[4], phalf[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        int pi = sub * 4 + e;
        pax[e] = -1;
        pbase[e] = 0;
        phalf[e] = 0;
#pragma unroll
        for (int ax = 0; ax < 3; ++ax) {
            const int half = p.rope_half[ax];
            if (pax[e] < 0 && pi < half) {
                pax[e] = ax;
                pbase[e] = p.rope_off[ax] + pi;
                phalf[e] = half;
            }
            pi -= half;
        }
    }
    // every row's cos/sin (the table always holds entry 0; the identity
    // rotation is substituted where a pair is not rotated)
    float2 cs[NP][4];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int n = nr[i];
        const bool video = n >= 0 && n < p.n_video;
        const uint32_t un = video ? (uint32_t)n : 0u;
        const uint32_t pt = fast_div(un, p.div_HW);
        const uint32_t rem = un - pt * hw;
        const uint32_t ph = fast_div(rem, p.div_W);
        const uint32_t pw = rem - ph * (uint32_t)p.W;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t gp = pax[e] == 0 ? pt : (pax[e] == 1 ? ph : pw);
            const bool rot = video && pax[e] >= 0;
            cs[i][e] = p.rope_cs[rot ? pbase[e] + gp * (uint32_t)phalf[e] : 0u];
        }
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const bool valid = nr[i] >= 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool rot = valid && nr[i] < p.n_video && pax[e] >= 0;
            cs[i][e] = rot ? cs[i][e] : make_float2(1.f, 0.f);
        }
    }
    const float inv_d = 1.0f / D;

    for (int h = h0; h < h1; ++h) {
        const int64_t bh = b * p.H + h;
        if (h > h0 && (KT || mean)) __syncthreads();   // the previous head's LDS reads are done
        float wv[8];
        if (w) {
            const float4* wp = reinterpret_cast<const float4*>(w + h * D + sub * 8);
            const float4 w0 = wp[0], w1 = wp[1];
            wv[0] = w0.x; wv[1] = w0.y; wv[2] = w0.z; wv[3] = w0.w;
            wv[4] = w1.x; wv[5] = w1.y; wv[6] = w1.z; wv[7] = w1.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) wv[e] = 1.f;
        }
        u32x4 x[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) x[i] = in[roff[i] + (int64_t)h * LPR];
#pragma unroll
        for (int i = 0; i < NP; ++i) x[i] = nr[i] >= 0 ? x[i] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int r = r0 + i * RPP;
            const uint32_t u[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = bf16lo(u[e]);
                v[2 * e + 1] = bf16hi(u[e]);
            }
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
#pragma unroll
            for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
            u32x4 res = u32x4{0u, 0u, 0u, 0u};
            if (nr[i] >= 0) {
                const float rs = rms_scale(ss, inv_d, p.eps);
                uint32_t ob[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t yb = pack_bf16x2(norm_val(v[2 * e], rs, wv[2 * e]),
                                                    norm_val(v[2 * e + 1], rs, wv[2 * e + 1]));
                    ob[e] = rotate_pair(yb, cs[i][e].x, cs[i][e].y);
                }
                res = u32x4{ob[0], ob[1], ob[2], ob[3]};
            }
            if (KT || mean) stage[r * LS + sub] = res;
            if (!KT && nr[i] != -2)
                __builtin_nontemporal_store(res, out + (bh * p.Np + pos0 + r) * LPR + sub);
        }
        if (!KT && !mean) continue;
        __syncthreads();
        if constexpr (KT) {
            const int g = threadIdx.x >> 6;        // 32-token group of this wave
            const int lane = threadIdx.x & 63;
            const int j = lane & 31, hf = lane >> 5;
            const int gpos = pos0 + g * 32;        // Np is a multiple of 32
            if (gpos < p.Np) {
                const int kb = gpos / p.block, t = gpos - kb * p.block;
                u32x4* dst = out + ((bh * p.nB + kb) * (p.block / 32) + (t >> 5)) * (DS * 64) + lane;
#pragma unroll
                for (int s2 = 0; s2 < DS; ++s2)
                    __builtin_nontemporal_store(stage[(g * 32 + j) * LS + 2 * s2 + hf], dst + s2 * 64);
            }
        }
        if (!mean) continue;

        // Pooling.  Thread (slice sl, chunk c) sums 8-channel chunk c over the
        // slice's SR rows; a run (block/nsub >= 16 rows) is a whole number of
        // slices.  The slice sums go through LDS (over the staged rows, once
        // every wave has read them), then one thread per (run, channel) adds
        // its run's slices.
        constexpr int NSL = kThreads / LPR;        // slices
        constexpr int SR = PW / NSL;               // rows per slice (8 or 4)
        const int sl = threadIdx.x / LPR, c = threadIdx.x % LPR;
        double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int rr = 0; rr < SR; ++rr) {
            const u32x4 vv = stage[(sl * SR + rr) * LS + c];
            const uint32_t u[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += (double)bf16lo(u[e]);
                acc[2 * e + 1] += (double)bf16hi(u[e]);
            }
        }
        __syncthreads();
        double* part = reinterpret_cast<double*>(stage);   // [NSL][D]
#pragma unroll
        for (int e = 0; e < 8; ++e) part[sl * D + c * 8 + e] = acc[e];
        __syncthreads();
        const int RL = p.block / p.nsub;           // rows per run
        const int spr = RL / SR;                   // slices per run
        for (int it = threadIdx.x; it < (PW / RL) * D; it += kThreads) {
            const int run = it / D, ch = it - run * D;
            const int rpos = pos0 + run * RL;
            if (rpos >= p.Np) break;
            double sum = 0.0;
            for (int k2 = 0; k2 < spr; ++k2) sum += part[(run * spr + k2) * D + ch];
            const int kb = rpos / p.block;
            const int rib = (rpos - kb * p.block) / RL;   // run within the block
            const int valid = min(max(p.blk_valid[kb] - rib * RL, 0), RL);
            const double m = valid > 0 ? sum / (double)valid : 0.0;
            if constexpr (KT)
                mean[(bh * D + ch) * ((int64_t)p.nB * p.nsub) + (int64_t)kb * p.nsub + rib] = m;
            else
                mean[((bh * p.nB + kb) * p.nsub + rib) * D + ch] = m;
        }
    }
}

}  // namespace

hipError_t launch_prologue(const DevPlan& p, const uint16_t* q, const uint16_t* k,
                           const float* wq, const float* wk, uint16_t* qo, uint16_t* ko,
                           bool tiled, double* means, hipStream_t s) {
    ProArgs a;
    a.p = p;
    a.in[0] = q;
    a.in[1] = k;
    a.out[0] = qo;
    a.out[1] = ko;
    a.w[0] = wq;
    a.w[1] = wk;
    a.mean[0] = means;
    a.mean[1] = means ? means + (int64_t)p.B * p.H * p.nB * p.nsub * p.d : nullptr;
    a.hg = 1;
    if (tiled) {
        a.hg = kHeadsPerGroup < p.H ? kHeadsPerGroup : p.H;
        const int64_t n_hg = (p.H + a.hg - 1) / a.hg;
        dim3 gt((unsigned)((int64_t)p.B * n_hg * ((p.Np + 127) / 128)));
        if (p.d == 128) {
            hipLaunchKernelGGL((prologue_tiled_kernel<128, false>), gt, dim3(kThreads), 0, s, a);
            hipLaunchKernelGGL((prologue_tiled_kernel<128, true>), gt, dim3(kThreads), 0, s, a);
        } else {
            hipLaunchKernelGGL((prologue_tiled_kernel<64, false>), gt, dim3(kThreads), 0, s, a);
            hipLaunchKernelGGL((prologue_tiled_kernel<64, true>), gt, dim3(kThreads), 0, s, a);
        }
        return hipGetLastError();
    }
    const int64_t rows = (int64_t)p.B * p.N * p.H;
    const int lpr = p.d / 8;
    const int64_t per_block = (int64_t)(kThreads / lpr) * kRows;
    const int64_t blocks = (rows + per_block - 1) / per_block;
    dim3 grid((unsigned)blocks, 2);
    if (p.d == 128)
        hipLaunchKernelGGL(prologue_kernel<128>, grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(prologue_kernel<64>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace sva
