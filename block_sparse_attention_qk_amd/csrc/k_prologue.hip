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
// thread handles kRows rows to keep several loads in flight.
#include "kernels.h"

namespace sva {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 4;   // rows per thread

struct ProArgs {
    DevPlan p;
    const uint16_t* in[2];
    uint16_t* out[2];
    const float* w[2];
};

// TILED = false: Q', K' in raster order, like the inputs.  TILED = true:
// straight into the attention layouts, Q' in tile order [B,H,Np,d] and K'
// as K tiles (the reorders of Q' and K' fused away); the padding rows are
// zeroed by pad_zero_kernel.
template <int D, bool TILED>
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

    u32x4 x[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const uint32_t row = row0 + r * RPB;
        x[r] = row < rows ? in[(int64_t)row * LPR + sub] : u32x4{0u, 0u, 0u, 0u};
    }

    // this lane's four channel pairs: RoPE section (-1: not rotated) and the
    // pair's offset in that section's cos/sin table
    int pax[4], pbase[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        int pi = sub * 4 + e;
        pax[e] = -1;
        pbase[e] = 0;
#pragma unroll
        for (int ax = 0; ax < 3; ++ax) {
            const int half = p.rope_half[ax];
            if (pax[e] < 0 && pi < half) {
                pax[e] = ax;
                pbase[e] = p.rope_off[ax] + pi;
            }
            pi -= half;
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
        if (row >= rows) continue;
        const uint32_t tok = fast_div(row, p.div_H);
        const uint32_t h = row - tok * (uint32_t)p.H;
        const uint32_t n = tok - fast_div(tok, p.div_N) * (uint32_t)p.N;
        const float rs = rsqrtf(ss * inv_d + p.eps);
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
        // norm, then round to bf16 (the stored value the rotation starts from)
        uint32_t yb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            yb[e] = pack_bf16x2(v[2 * e] * rs * wv[2 * e], v[2 * e + 1] * rs * wv[2 * e + 1]);
        // grid coordinates (t, h, w) of a video token; extra tokens get none
        const bool video = n < (uint32_t)p.n_video;
        const uint32_t pt = fast_div(n, p.div_HW);
        const uint32_t rem = n - pt * (uint32_t)(p.Hh * p.W);
        const uint32_t ph = fast_div(rem, p.div_W);
        const uint32_t pw = rem - ph * (uint32_t)p.W;
        uint32_t ob[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float y0 = bf16lo(yb[e]), y1 = bf16hi(yb[e]);
            float c = 1.f, s = 0.f;
            if (video && pax[e] >= 0) {
                const uint32_t pos = pax[e] == 0 ? pt : (pax[e] == 1 ? ph : pw);
                const float2 cs = p.rope_cs[pbase[e] + pos * p.rope_half[pax[e]]];
                c = cs.x;
                s = cs.y;
            }
            ob[e] = pack_bf16x2(y0 * c - y1 * s, y0 * s + y1 * c);
        }
        const u32x4 res = u32x4{ob[0], ob[1], ob[2], ob[3]};
        if constexpr (!TILED) {
            out[(int64_t)row * LPR + sub] = res;
        } else {
            // tile position of token n of batch b; head h
            const uint32_t b = fast_div(tok, p.div_N);
            const int64_t bh = (int64_t)b * p.H + h;
            const int pos = p.perm[n];
            if (tensor == 0) {
                out[(bh * p.Np + pos) * LPR + sub] = res;
            } else {
                // K tile entry of token t = pos mod block, 16-byte chunk sub:
                // group t/32, step sub/2, lane half sub%2, key t%32
                const int kb = pos / p.block, t = pos - kb * p.block;
                const int64_t e = ((bh * p.nB + kb) * (p.block / 32) + (t >> 5)) * (D / 16 * 64) +
                                  (sub >> 1) * 64 + (sub & 1) * 32 + (t & 31);
                out[e] = res;
            }
        }
    }
}

// Zero rows of the padding positions [n_video, n_video_pad) of every
// (b, h): Q' rows in tile order and K'-tile entries.  One workgroup per
// (b, h), grid.y = tensor.
template <int D>
__global__ __launch_bounds__(kThreads) void pad_zero_kernel(DevPlan p, u32x4* qr, u32x4* kt) {
    constexpr int LPR = D / 8;
    const int64_t bh = blockIdx.x;
    const int npad = (int)(p.n_video_pad - p.n_video);
    for (int i = threadIdx.x; i < npad * LPR; i += kThreads) {
        const int pos = (int)p.n_video + i / LPR, sub = i % LPR;
        if (blockIdx.y == 0) {
            qr[(bh * p.Np + pos) * LPR + sub] = u32x4{0u, 0u, 0u, 0u};
        } else {
            const int kb = pos / p.block, t = pos - kb * p.block;
            kt[((bh * p.nB + kb) * (p.block / 32) + (t >> 5)) * (D / 16 * 64) + (sub >> 1) * 64 +
               (sub & 1) * 32 + (t & 31)] = u32x4{0u, 0u, 0u, 0u};
        }
    }
}

}  // namespace

hipError_t launch_prologue(const DevPlan& p, const uint16_t* q, const uint16_t* k,
                           const float* wq, const float* wk, uint16_t* qo, uint16_t* ko,
                           bool tiled, hipStream_t s) {
    ProArgs a;
    a.p = p;
    a.in[0] = q;
    a.in[1] = k;
    a.out[0] = qo;
    a.out[1] = ko;
    a.w[0] = wq;
    a.w[1] = wk;
    const int64_t rows = (int64_t)p.B * p.N * p.H;
    const int lpr = p.d / 8;
    const int64_t per_block = (int64_t)(kThreads / lpr) * kRows;
    const int64_t blocks = (rows + per_block - 1) / per_block;
    dim3 grid((unsigned)blocks, 2);
    if (tiled && p.n_video_pad > p.n_video) {
        dim3 gz((unsigned)((int64_t)p.B * p.H), 2);
        u32x4* q4 = reinterpret_cast<u32x4*>(qo);
        u32x4* k4 = reinterpret_cast<u32x4*>(ko);
        if (p.d == 128) hipLaunchKernelGGL(pad_zero_kernel<128>, gz, dim3(kThreads), 0, s, p, q4, k4);
        else hipLaunchKernelGGL(pad_zero_kernel<64>, gz, dim3(kThreads), 0, s, p, q4, k4);
    }
    if (p.d == 128) {
        if (tiled) hipLaunchKernelGGL((prologue_kernel<128, true>), grid, dim3(kThreads), 0, s, a);
        else hipLaunchKernelGGL((prologue_kernel<128, false>), grid, dim3(kThreads), 0, s, a);
    } else {
        if (tiled) hipLaunchKernelGGL((prologue_kernel<64, true>), grid, dim3(kThreads), 0, s, a);
        else hipLaunchKernelGGL((prologue_kernel<64, false>), grid, dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace sva
