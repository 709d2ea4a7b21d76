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
// Work split: one workgroup per (b, h, qb), one wave per 32 query rows
// (BLK/32 waves), two workgroups per CU (64 KB of LDS and <= 256 registers
// per wave each), so every SIMD holds two waves whose MFMA and softmax
// phases interleave.  A row's key blocks are consumed in stages of 64
// keys; the workgroup keeps two LDS stage buffers and issues the global
// loads of stage s+1 into registers before computing stage s, writing them
// to the other buffer afterwards (one barrier per stage).  Per stage each
// wave computes
//   S^T = K · Q^T    v_mfma_f32_32x32x16_bf16, M = keys, N = queries
//   softmax on S^T   each lane owns one query column: row max and sums are
//                    lane-local plus one exchange between the two lane halves
//   O^T += V^T · P^T v_mfma_f32_32x32x16_bf16, M = channels, N = queries;
//                    P^T comes straight from the S^T accumulators; the V
//                    tiles store keys in the order that accumulator layout
//                    hands them over (see the V-tile reorder), so each V
//                    operand is one 16-byte LDS read.
// Logits are scaled by log2(e)/sqrt(d) and exponentiated with v_exp_f32.
// The running max is raised only when a row's new max exceeds it by more
// than 8 (log2 units); in between, probabilities are taken against the
// stale max (at most 2^8, exact in the final division), which skips most
// rescales of the accumulator.
//
// LDS layouts avoid bank conflicts with XOR swizzles of 16-byte chunks: a
// row of 256 bytes puts chunk c at c ^ (r mod 16), a row of 128 bytes at
// c ^ ((r/2) mod 8), so the 16 lanes served together read 16 different bank
// groups.
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
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

struct AttnArgs {
    DevPlan p;
    const u32x4_t* q;    // [B,H,Np,d]
    const u32x4_t* k;    // [B,H,Np,d]
    const u32x4_t* vt;   // [B,H,nB,d,BLK]
    const int32_t* col;  // [B,H,nnz_per_head]
    uint2* o;            // [B,H,Np,d]
};

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

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

// 16-byte chunk slot of chunk c in LDS row r (rows of RB bytes).
template <int RB>
__device__ __forceinline__ int swz(int c, int r) {
    if constexpr (RB == 256) return c ^ (r & 15);
    else return c ^ ((r >> 1) & 7);
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_kernel(AttnArgs a) {
    constexpr int NT = BLK * 2;          // threads (BLK/32 waves)
    constexpr int SK = 64;               // keys per stage
    constexpr int SPB = BLK / SK;        // stages per block
    constexpr int KCH = D / 8;           // 16-byte chunks per K row
    constexpr int KRB = D * 2;           // bytes per K row
    constexpr int VCH = SK / 8;          // 16-byte chunks per V^T stage row
    constexpr int KPT = SK * KCH / NT;   // K chunks per thread per stage
    constexpr int VPT = D * VCH / NT;    // V chunks per thread per stage
    constexpr int DS = D / 16;           // 16-channel steps (S^T contraction)
    constexpr int DT = D / 32;           // 32-channel tiles (O^T rows)
    constexpr float kTau = 8.0f;         // lazy-rescale threshold (log2 units)
    __shared__ u32x4_t sK[2][SK * KCH];
    __shared__ u32x4_t sV[2][D * VCH];

    const DevPlan& p = a.p;
    const int64_t wg = xcd_remap(blockIdx.x, gridDim.x);
    const int qb = (int)(wg % p.nB);
    const int64_t bh = wg / p.nB;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, hf = lane >> 5;
    const int qrow = wave * 32 + j;      // query row within the block

    // Q^T operand: lane (j, hf) holds channels 16s + 8hf .. +8 of row qrow
    bf16x8_t qop[DS];
    {
        const u32x4_t* qp = a.q + ((bh * p.Np) + (int64_t)qb * BLK + qrow) * KCH;
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
    const u32x4_t* kbase = a.k + bh * p.Np * KCH;
    const u32x4_t* vbase = a.vt + bh * (int64_t)p.nB * (D * BLK / 8);
    const int nstage = len * SPB;

    u32x4_t pk[KPT], pv[VPT];
#define SVA_STAGE_KB(st) \
    ([&] { const int kb_ = dense ? (st) / SPB : cl[(st) / SPB]; \
           return (kb_ >= 0 && kb_ < p.nB) ? kb_ : -1; }())
#define SVA_LOAD_STAGE(st)                                                            \
    do {                                                                              \
        const int kb_ = SVA_STAGE_KB(st);                                             \
        const int kbc_ = kb_ < 0 ? 0 : kb_;                                           \
        const int half_ = (st) % SPB;                                                 \
        const u32x4_t* gk_ = kbase + ((int64_t)kbc_ * BLK + half_ * SK) * KCH;          \
        const u32x4_t* gv_ = vbase + (int64_t)kbc_ * (D * BLK / 8) + half_ * VCH;       \
        _Pragma("unroll") for (int i = 0; i < KPT; ++i) pk[i] = gk_[tid + i * NT];    \
        _Pragma("unroll") for (int i = 0; i < VPT; ++i) {                             \
            const int q_ = tid + i * NT;                                              \
            pv[i] = gv_[(q_ / VCH) * (BLK / 8) + (q_ % VCH)];                         \
        }                                                                             \
    } while (0)
#define SVA_STORE_STAGE(buf)                                                          \
    do {                                                                              \
        _Pragma("unroll") for (int i = 0; i < KPT; ++i) {                             \
            const int q_ = tid + i * NT;                                              \
            const int r_ = q_ / KCH, ch_ = q_ % KCH;                                  \
            sK[buf][r_ * KCH + swz<KRB>(ch_, r_)] = pk[i];                            \
        }                                                                             \
        _Pragma("unroll") for (int i = 0; i < VPT; ++i) {                             \
            const int q_ = tid + i * NT;                                              \
            const int r_ = q_ / VCH, ch_ = q_ % VCH;                                  \
            sV[buf][r_ * VCH + swz<128>(ch_, r_)] = pv[i];                            \
        }                                                                             \
    } while (0)

    if (nstage > 0) {
        SVA_LOAD_STAGE(0);
        SVA_STORE_STAGE(0);
    }
    __syncthreads();

    for (int st = 0; st < nstage; ++st) {
        const int buf = st & 1;
        if (st + 1 < nstage) SVA_LOAD_STAGE(st + 1);
        const int kb = SVA_STAGE_KB(st);
        if (kb >= 0) {
            const int half = st % SPB;
            // S^T = K Q^T: tile kt covers stage keys kt*32..+32; lane (j, hf)
            // gets keys kt*32 + 8*(v/4) + 4*hf + v%4 of query column qrow.
            f32x16_t sc[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int v = 0; v < 16; ++v) sc[kt][v] = 0.f;
                const int r = kt * 32 + j;
#pragma unroll
                for (int s = 0; s < DS; ++s) {
                    const u32x4_t kv = sK[buf][r * KCH + swz<KRB>(2 * s + hf, r)];
                    sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), qop[s],
                                                                     sc[kt], 0, 0, 0);
                }
            }
            if (kb == last_video && last_valid < BLK) {   // padding keys
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int key = half * SK + kt * 32 + 8 * (v / 4) + 4 * hf + (v % 4);
                        if (key >= last_valid) sc[kt][v] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[kt][v]);
            mx = lane_swap_max(mx) * c;
            if (__any(mx > m + kTau)) {
                const float m_new = fmaxf(m, mx);
                const float alpha = __builtin_amdgcn_exp2f(m - m_new);
                m = m_new;
                l *= alpha;
#pragma unroll
                for (int t = 0; t < DT; ++t)
#pragma unroll
                    for (int v = 0; v < 16; ++v) o[t][v] *= alpha;
            }
            bf16x8_t pb[2][2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float e = __builtin_amdgcn_exp2f(fmaf(sc[kt][v], c, -m));
                    sc[kt][v] = e;
                    l += e;
                }
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    u32x4_t u;
                    u.x = pack_bf16x2(sc[kt][8 * s2 + 0], sc[kt][8 * s2 + 1]);
                    u.y = pack_bf16x2(sc[kt][8 * s2 + 2], sc[kt][8 * s2 + 3]);
                    u.z = pack_bf16x2(sc[kt][8 * s2 + 4], sc[kt][8 * s2 + 5]);
                    u.w = pack_bf16x2(sc[kt][8 * s2 + 6], sc[kt][8 * s2 + 7]);
                    pb[kt][s2] = as_bf16x8(u);
                }
            }
            // O^T += V^T P^T.  Step (kt, s2) contracts the 16 stage keys
            // kt*32 + 16*s2 + ..; lane half hf's 8 of them are V^T storage
            // chunk 2*(2kt + s2) + hf of the row.
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                const int r = t * 32 + j;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        const u32x4_t vv = sV[buf][r * VCH + swz<128>(2 * (2 * kt + s2) + hf, r)];
                        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vv), pb[kt][s2],
                                                                       o[t], 0, 0, 0);
                    }
            }
        }
        if (st + 1 < nstage) SVA_STORE_STAGE(buf ^ 1);
        __syncthreads();
    }
#undef SVA_STAGE_KB
#undef SVA_LOAD_STAGE
#undef SVA_STORE_STAGE

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
    a.q = reinterpret_cast<const u32x4_t*>(qr);
    a.k = reinterpret_cast<const u32x4_t*>(kr);
    a.vt = reinterpret_cast<const u32x4_t*>(vt);
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
