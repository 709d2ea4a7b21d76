// Block-sparse flash attention (non-causal), bf16 MFMA on gfx950.
//
// For each (b, h, query block qb) the kernel walks the row's list of kept
// key blocks ("MiniMax-H3 在 8×H200 上基准测试", section "SubBlock 稀疏注意力如何工作":
// the kept indices drive a block-sparse kernel and the full attention
// matrix is never formed) and keeps an online softmax per query row: a
// running max m, running sum l and an fp32 output accumulator, rescaled
// when m grows.  A dense plan walks every block and is exact dense
// attention ("SVA_DENSE", the dense warm-up steps of the same page).
//
// Work split: one workgroup per (b, h, qb); one wave per 32 query rows
// (BLK/32 waves).  Per key block the workgroup stages K (row-major) and V
// (transposed tile, as written by the V-tile reorder) in LDS, then each
// wave computes
//   S^T = K · Q^T    v_mfma_f32_32x32x16_bf16, M = keys, N = queries
//   softmax on S^T   each lane owns one query column: row max and sums are
//                    lane-local plus one exchange between the two lane halves
//   O^T += V^T · P^T v_mfma_f32_32x32x16_bf16, M = channels, N = queries;
//                    P^T comes straight from the S^T accumulators, with the
//                    contraction order of the keys matched on the V side.
// Logits are scaled by log2(e)/sqrt(d) and exponentiated with exp2.
//
// LDS layouts avoid bank conflicts with XOR swizzles: K rows (keys) of d
// bf16 in 16-byte chunks, chunk c of row r at c ^ (r mod 16); V^T rows
// (channels) of BLK keys in 8-byte units, unit u of row r at u ^ (r mod
// BLK/4).  Each lane of an MFMA operand read then hits its own banks.
//
// Roofline: 4·BLK²·d flops per (query block, key block) pair on the MFMA
// pipe (8.4 MFLOP at BLK = d = 128) against 2·BLK·d·2 bytes of K and V
// staged (64 KB): 128 flop/byte, which L2 / Infinity Cache reuse across
// neighbouring query blocks of a head has to serve.
#include "kernels.h"

namespace sva {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct AttnArgs {
    DevPlan p;
    const uint4* q;      // [B,H,Np,d]
    const uint4* k;      // [B,H,Np,d]
    const uint4* vt;     // [B,H,nB,d,BLK]
    const int32_t* col;  // [B,H,nnz_per_head]
    uint2* o;            // [B,H,Np,d]
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ float lane_swap_max(float x) {
    // v_permlane32_swap: both outputs hold {x[l mod 32], x[l mod 32 + 32]}
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_swap_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs;
// give each XCD one contiguous range of (b, h, qb) so the query blocks that
// share an L2 at a time are neighbours of one head.
__device__ __forceinline__ int64_t xcd_remap(int64_t wg, int64_t n) {
    const int64_t per = n / 8, rem = n % 8;
    const int64_t x = wg % 8, idx = wg / 8;
    return x * per + (x < rem ? x : rem) + idx;
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void attn_kernel(AttnArgs a) {
    constexpr int NT = BLK * 2;        // threads (BLK/32 waves)
    constexpr int KCH = D / 8;         // 16-byte chunks per K row
    constexpr int VU = BLK / 4;        // 8-byte units per V^T row
    constexpr int KT = BLK / 32;       // 32-key tiles per block
    constexpr int DS = D / 16;         // 16-channel steps (S^T contraction)
    constexpr int DT = D / 32;         // 32-channel tiles (O^T rows)
    __shared__ uint4 sK[BLK * KCH];
    __shared__ uint2 sV[D * VU];

    const DevPlan& p = a.p;
    const int64_t wg = xcd_remap(blockIdx.x, gridDim.x);
    const int qb = (int)(wg % p.nB);
    const int64_t bh = wg / p.nB;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, hf = lane >> 5;
    const int qrow = wave * 32 + j;    // query row within the block

    // Q^T operand: lane (j, hf) holds channels 16s + 8hf .. +8 of row qrow
    bf16x8_t qop[DS];
    {
        const uint4* qp = a.q + ((bh * p.Np) + (int64_t)qb * BLK + qrow) * KCH;
#pragma unroll
        for (int s = 0; s < DS; ++s) qop[s] = as_bf16x8(qp[2 * s + hf]);
    }

    f32x16_t o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[t][v] = 0.f;
    float m = -INFINITY, l = 0.f;
    const float c = 1.4426950408889634f / sqrtf((float)D);   // log2(e)/sqrt(d)

    const bool dense = p.dense != 0;
    const int64_t r0 = p.row_ptr[qb];
    const int len = dense ? p.nB : (int)(p.row_ptr[qb + 1] - r0);
    const int32_t* cl = dense ? nullptr : a.col + bh * p.nnz_per_head + r0;
    const int last_video = p.nB_video - 1;
    const int last_valid = p.blk_valid[last_video];

    for (int it = 0; it < len; ++it) {
        const int kb = dense ? it : cl[it];
        if (kb < 0 || kb >= p.nB) continue;           // ignore out-of-range entries
        __syncthreads();                              // LDS free from the last block
        {
            const uint4* gk = a.k + (bh * p.Np + (int64_t)kb * BLK) * KCH;
#pragma unroll
            for (int i = 0; i < BLK * KCH / NT; ++i) {
                const int cidx = tid + i * NT;
                const int r = cidx / KCH, ch = cidx % KCH;
                sK[r * KCH + (ch ^ (r & (KCH - 1) & 15))] = gk[cidx];
            }
            const uint4* gv = a.vt + (bh * p.nB + kb) * (int64_t)(D * BLK / 8);
#pragma unroll
            for (int i = 0; i < D * BLK / 8 / NT; ++i) {
                const int cidx = tid + i * NT;
                const int r = cidx / (BLK / 8), ch = cidx % (BLK / 8);
                const uint4 v = gv[cidx];
                const int x = r & (VU - 1);
                sV[r * VU + ((2 * ch) ^ x)] = make_uint2(v.x, v.y);
                sV[r * VU + ((2 * ch + 1) ^ x)] = make_uint2(v.z, v.w);
            }
        }
        __syncthreads();

        // S^T = K Q^T: tile kt covers keys kt*32..+32; lane (j, hf) gets
        // keys kt*32 + 8*(v/4) + 4*hf + v%4 of query column qrow.
        f32x16_t st[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) st[kt][v] = 0.f;
            const int r = kt * 32 + j;
#pragma unroll
            for (int s = 0; s < DS; ++s) {
                const uint4 kv = sK[r * KCH + ((2 * s + hf) ^ (r & (KCH - 1) & 15))];
                st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), qop[s], st[kt],
                                                                 0, 0, 0);
            }
        }
        if (kb == last_video && last_valid < BLK) {   // padding keys of the last video block
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = kt * 32 + 8 * (v / 4) + 4 * hf + (v % 4);
                    if (key >= last_valid) st[kt][v] = -INFINITY;
                }
        }
        // online softmax (log2 domain)
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int v = 0; v < 16; ++v) mx = fmaxf(mx, st[kt][v]);
        mx = lane_swap_max(mx) * c;
        const float m_new = fmaxf(m, mx);
        const float alpha = exp2f(m - m_new);
        m = m_new;
        float rs = 0.f;
        bf16x8_t pb[KT][2];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float e = exp2f(fmaf(st[kt][v], c, -m_new));
                st[kt][v] = e;
                rs += e;
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                uint4 u;
                u.x = pack_bf16x2(st[kt][8 * s2 + 0], st[kt][8 * s2 + 1]);
                u.y = pack_bf16x2(st[kt][8 * s2 + 2], st[kt][8 * s2 + 3]);
                u.z = pack_bf16x2(st[kt][8 * s2 + 4], st[kt][8 * s2 + 5]);
                u.w = pack_bf16x2(st[kt][8 * s2 + 6], st[kt][8 * s2 + 7]);
                pb[kt][s2] = as_bf16x8(u);
            }
        }
        l = l * alpha + rs;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[t][v] *= alpha;

        // O^T += V^T P^T.  Step (kt, s2) contracts keys
        // kt*32 + 16*s2 + {4hf..4hf+3, 8+4hf..8+4hf+3} for lane half hf,
        // which are 8-byte units u0 = kt*8 + 4*s2 + hf and u0 + 2 of a V^T row.
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            const int r = t * 32 + j;
            const int x = r & (VU - 1);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int u0 = kt * 8 + 4 * s2 + hf;
                    const uint2 lo = sV[r * VU + (u0 ^ x)];
                    const uint2 hi = sV[r * VU + ((u0 + 2) ^ x)];
                    const uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
                    o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vv), pb[kt][s2],
                                                                   o[t], 0, 0, 0);
                }
        }
    }

    // epilogue: O = O^T / l, padding query rows zero
    const float lt = lane_swap_sum(l);
    const bool row_ok = qrow < p.blk_valid[qb];
    const float inv = (row_ok && lt > 0.f) ? 1.f / lt : 0.f;
    uint2* op = a.o + ((bh * p.Np) + (int64_t)qb * BLK + qrow) * (D / 4);
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            // channels t*32 + 8g + 4hf + 0..3
            uint2 w;
            w.x = pack_bf16x2(o[t][4 * g + 0] * inv, o[t][4 * g + 1] * inv);
            w.y = pack_bf16x2(o[t][4 * g + 2] * inv, o[t][4 * g + 3] * inv);
            op[(t * 32 + 8 * g + 4 * hf) / 4] = w;
        }
}

}  // namespace

hipError_t launch_attention(const DevPlan& p, const uint16_t* qr, const uint16_t* kr,
                            const uint16_t* vt, const int32_t* col, uint16_t* o, hipStream_t s) {
    AttnArgs a;
    a.p = p;
    a.q = reinterpret_cast<const uint4*>(qr);
    a.k = reinterpret_cast<const uint4*>(kr);
    a.vt = reinterpret_cast<const uint4*>(vt);
    a.col = col;
    a.o = reinterpret_cast<uint2*>(o);
    dim3 grid((unsigned)((int64_t)p.B * p.H * p.nB));
    dim3 block(p.block * 2);
    if (p.d == 128 && p.block == 128)
        hipLaunchKernelGGL((attn_kernel<128, 128>), grid, block, 0, s, a);
    else if (p.d == 128)
        hipLaunchKernelGGL((attn_kernel<128, 64>), grid, block, 0, s, a);
    else if (p.block == 128)
        hipLaunchKernelGGL((attn_kernel<64, 128>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((attn_kernel<64, 64>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace sva
