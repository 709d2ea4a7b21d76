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
// (BLK/32 waves), two workgroups per CU.  A dense plan, whose rows all walk
// every block, gives a workgroup two query blocks, so one copy of each K/V
// stage feeds twice the waves.  With a partials workspace, a sparse plan's
// rows that are much longer than the others (extra-token rows keep every
// block) are cut into pieces, one workgroup each, each writing its
// unnormalised O, running max and sum; a merge kernel combines them.  A row's key blocks are consumed
// in stages of 32 keys.  Both operand streams come in MFMA-ready tile
// layouts written by the reorder kernels (K tiles, V tiles), in which one
// stage of K and one stage of V are each a contiguous span of 32·d bf16.
// They are copied into LDS as they are, with global_load_lds_dwordx4 (each
// wave-level load moves 1 KB, lane l to byte 16 l), into rotating K and V
// buffers (four of each with 128-token blocks, three and two with 64): the
// copies for later stages are issued before a stage is computed; with
// 64-token blocks an iteration ends by waiting only for the stages the next
// iteration reads (vmcnt; later copies stay in flight) and one barrier,
// with 128-token blocks every second iteration waits for its copies and
// ends with a barrier.  Per stage each wave computes
//   S^T = K · Q^T    v_mfma_f32_32x32x16_bf16, M = keys, N = queries; the
//                    operand of lane l for channel step s is the 16 bytes at
//                    (s·64 + l)·16 of the K stage
//   softmax on S^T   each lane owns one query column: sums are lane-local;
//                    a row max, when one is needed, is lane-local plus one
//                    exchange between the two lane halves (v_permlane32_swap)
//   O^T += V^T · P^T v_mfma_f32_32x32x16_bf16, M = channels, N = queries;
//                    P^T comes straight from the S^T accumulators; the V
//                    stage holds four chunks of 8 keys, each chunk as d rows
//                    of 16 bytes, with the keys in the order that accumulator
//                    layout hands them over (see the V-tile reorder).
// Lanes 0-31 and 32-63 of every LDS read touch 32 consecutive 16-byte slots
// each, which the LDS serves without bank conflicts; every read address is
// one per-lane base plus an immediate offset, and the copies need no
// per-lane address arithmetic beyond base + 16 l.
// Logits are scaled by log2(e)/sqrt(d) and exponentiated with v_exp_f32.
// The running max is raised only when a row's new max exceeds it by more
// than 8 (log2 units); in between, probabilities are taken against the
// stale max (at most 2^8, exact in the final division), which skips most
// rescales of the accumulator.  The row's first stage sets the max; later
// stages are exponentiated against it first, and only a wave in which some
// lane's 16 probabilities sum to 2^8 or more takes the stage max and
// applies the rule, so the common stage needs no max at all.
//
// Roofline: 4·BLK²·d flops per (query block, key block) pair on the MFMA
// pipe (8.4 MFLOP at BLK = d = 128) against 2·BLK·d·2 bytes of K and V
// (64 KB): 128 flop/byte, which L2 / Infinity Cache reuse across
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
    const u32x4_t* k;    // K tiles [B,H,nB,BLK/32,d/16,64,8]
    const u32x4_t* vt;   // V tiles [B,H,nB,BLK/32,4,d,8]
    const int32_t* col;  // [B,H,nnz_per_head]
    const u32x4_t* km;   // block-mean K tiles [B,H,n_mean_groups,d/16,64,8], or NULL
    const u32x4_t* vm;   // block-mean V tiles [B,H,n_mean_groups,4,d,8]
    uint2* o;            // [B,H,Np,d], or [B,N,H,d] with o_raster
    int o_raster;
    float* part;         // partials of split rows, or NULL (no row is split)
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

// XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs.
// Consecutive chunks of C (b, h, qb) go to consecutive XCDs: the query
// blocks that share one XCD's L2 at a time are neighbours of one head, and
// the 8 XCDs together work on neighbouring chunks of the same head, so the
// key and value blocks they miss in L2 are few enough (one head's, about
// 38 MB at the 720p shape) to stay in the Infinity Cache.  (One contiguous
// range per XCD put 8 different heads, about 300 MB, in flight at once.)
// C = 32 for 128-token blocks; with 64-token blocks (four workgroups per
// CU, 128 per XCD) C = 128, so the workgroups resident on an XCD are one
// run of consecutive query blocks (sparse 480p: 1.99 -> 1.56 ms), since
// those kernels move twice the K/V bytes per flop through L2.
// Full rounds of 8 chunks are permuted, the remainder keeps its order.
template <int BLK>
__device__ __forceinline__ int64_t xcd_remap(int64_t wg, int64_t n) {
    constexpr int64_t C = BLK == 64 ? 128 : 32;
    const int64_t full = n / (8 * C) * (8 * C);
    if (wg >= full) return wg;
    const int64_t x = wg % 8, l = wg / 8;
    return (8 * (l / C) + x) * C + l % C;
}

// One 16-byte-per-lane global -> LDS load (global_load_lds_dwordx4): lane l
// writes LDS bytes [lds + 16 l, lds + 16 l + 16).  Issued from asm so the
// compiler's wait-count pass does not track it: that pass cannot tell the
// rotating stage buffers apart across the unrolled loop and would wait for
// every stage in flight before each LDS read.  The kernel waits for these
// loads itself (vmcnt, in issue order).  No register outputs; M0 is set in
// the same block, with one wait state before the load reads it.  The
// compiler treats M0 as reserved and does not honour the clobber; nothing
// else in these kernels uses M0 (gfx950 LDS instructions do not read it).
// tests/test_codegen.py compiles this file and fails if the compiler ever
// keeps a value in M0 or emits another instruction that reads it.  (The
// compiler's own builtin for these copies, which manages M0 itself, moves a
// 64-bit address per lane and measured 7.8 % slower.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// The address is a wave-uniform base in SGPRs plus this lane's byte offset
// (saddr form), so no per-lane 64-bit address arithmetic is spent on it.
// `base` and `off` must be the same in every lane; readfirstlane keeps the
// offset (and so the sum) in SGPRs.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t off, uint32_t lane_off,
                                          uint32_t lds_addr) {
    const uint64_t sb = (uint64_t)(uintptr_t)base + __builtin_amdgcn_readfirstlane(off);
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(lane_off), "s"(sb), "s"(lds_addr)
        : "memory", "m0");
}
// The same copy from a wave-uniform base pointer (SGPRs) and this lane's
// byte offset.  The LDS destination is a wave-uniform base plus a constant,
// added into M0 in the same block; the load still needs one wait state
// after that M0 write (the s_nop).  `imm` must fold to a constant once the
// caller's loops are unrolled.
__device__ __forceinline__ void lds_dma16_at(const void* base, uint32_t lane_off,
                                             uint32_t lds_base, uint32_t imm) {
    asm volatile(
        "s_add_u32 m0, %2, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(lane_off), "s"(base), "s"(lds_base), "i"(imm)
        : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt left unconstrained.
constexpr int kWaitVmcnt0 = (0x7 << 4) | (0xF << 8);

// Stage buffers of K and of V (32·d bf16 each).  K of stage st+1 and V of
// stage st-1 are read in iteration st, so with K copies at least one
// iteration ahead of their use K needs three buffers, and V two (a stage's
// V copied in its own iteration, read in the next).  With 128-token
// blocks: four of each (two workgroups of four waves fill a CU's
// registers).  With 64-token blocks a workgroup has
// only two waves: three K and two V buffers (40 KB at d = 128) let four
// workgroups, the register limit, share a CU (three with 48 KB).
constexpr int attn_k_buffers(int, int blk) { return blk == 64 ? 3 : 4; }
constexpr int attn_v_buffers(int, int blk) { return blk == 64 ? 2 : 4; }
// Workgroup barrier every BP stages.  With 128-token blocks, one barrier
// per two stages (K copies three stages ahead, V copies one, every copy
// landed at each barrier) keeps the four K and four V buffers safe: a wave
// starting iteration i knows every wave has finished iteration i-2 (odd
// i) or i-1 (even i), and the buffers a copy overwrites were last read in
// iteration i-2 or earlier.  Measured against a barrier per stage
// (bit-identical output): 720p 24.70 -> 24.55 ms, dense HunyuanVideo
// 143.1 -> 140.7 ms.  The barrier costs little either way (none at all,
// with wrong results, 24.03 ms); five K buffers with the K copies of the
// last iteration left in flight were slower (24.68 ms).  64-token blocks
// keep one barrier per stage: the same scheme needs eight buffers there,
// which would cost a workgroup per CU.
constexpr int attn_barrier_period(int, int blk) { return blk == 64 ? 1 : 2; }
constexpr int attn_gcd(int a, int b) { return b == 0 ? a : attn_gcd(b, a % b); }
// waves per SIMD the register budget is sized for (LDS decides the rest):
// two, i.e. at most 256 registers.  Allowed more, the 64-token-block kernel
// spreads into AGPRs (238 registers) and runs 3 % slower.
constexpr int attn_min_waves(int, int) { return 2; }

// QPW query blocks per workgroup: 1, or 2 for dense plans, whose rows all
// walk the same list, so one copy of each K/V stage feeds twice the waves.
template <int D, int BLK, bool DENSE, bool COMP, int QPW>
__global__ __launch_bounds__(BLK * 2 * QPW)
__attribute__((amdgpu_waves_per_eu(attn_min_waves(D, BLK), 2)))
void attn_kernel(AttnArgs a) {
    static_assert(QPW == 1 || DENSE, "only dense rows share one walk");
    constexpr int NT = BLK * 2 * QPW;    // threads (QPW·BLK/32 waves)
    constexpr int NWV = NT / 64;
    constexpr int WPB = BLK / 32;        // waves per query block
    constexpr int SK = 32;               // keys per stage (one 32-key MFMA tile)
    constexpr int SPB = BLK / SK;        // stages per block
    constexpr int KCH = D / 8;           // 16-byte chunks per Q row
    constexpr int CPS = SK * D / 8;      // 16-byte chunks per stage, of K and of V
    constexpr int LPW = CPS / (64 * NWV);// wave-level copies per wave and operand
    constexpr int DS = D / 16;           // 16-channel steps (S^T contraction)
    constexpr int DT = D / 32;           // 32-channel tiles (O^T rows)
    constexpr float kTau = 8.0f;         // lazy-rescale threshold (log2 units)
    constexpr float kPmax = 256.0f;      // 2^kTau: the largest probability it allows
    static_assert(LPW >= 1 && LPW * 64 * NWV == CPS, "stage copy split");
    constexpr int NBK = attn_k_buffers(D, BLK);   // K copies run NBK-1 stages ahead
    constexpr int NBV = attn_v_buffers(D, BLK);   // V copies run NBV-1 stages ahead
    static_assert(NBK >= 3 && NBV >= 2 && NBV <= NBK, "stage buffers");
    constexpr int BP = attn_barrier_period(D, BLK);
    static_assert(BP == 1 || BP == 2, "barrier period");
    // stages the K and V copies run ahead of the iteration that issues them
    constexpr int KLEAD = NBK - 1;
    constexpr int VLEAD = BP == 1 ? NBV - 2 : 1;
    static_assert(BP == 1 || (NBK == 4 && NBV == 4), "buffer schedule of the two-stage barrier");
    constexpr int NU0 = NBK / attn_gcd(NBK, NBV) * NBV;
    constexpr int NU1 = NU0 / attn_gcd(NU0, SPB) * SPB;
    constexpr int NU = NU1 / attn_gcd(NU1, BP) * BP;   // loop unrolling: buffer indices constant
    static_assert(NU % SPB == 0 && NU % BP == 0, "a loop body covers whole blocks");
    // list entries a loop body touches (its stages and the copies it issues)
    constexpr int NE = (NU - 1 + KLEAD) / SPB + 1;
    // At each barrier, K of stage st+2 and V of stage st must have landed.
    // One barrier per stage: they were issued in iterations st+3-NBK and
    // st+2-NBV, so the copies of the min(NBK-3, NBV-2) latest iterations
    // may stay in flight.  One per two stages: every copy lands first.
    constexpr int kInFlight = BP == 1 ? (NBK - 3 < NBV - 2 ? NBK - 3 : NBV - 2) * 2 * LPW : 0;
    static_assert(kInFlight < 64, "vmcnt range");
    constexpr int kWaitNext = (kInFlight & 15) | ((kInFlight >> 4) << 14) | (0x7 << 4) | (0xF << 8);
    __shared__ u32x4_t sK[NBK][CPS];
    __shared__ u32x4_t sV[NBV][CPS];
    extern __shared__ int32_t s_col[];   // compensation: this row's block list,
                                         // then a bitmap of it

    const DevPlan& p = a.p;
    const int64_t wg = xcd_remap<BLK>(blockIdx.x, gridDim.x);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, hf = lane >> 5;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform copy
    int64_t bh;
    int qfirst;
    // a work item of a split launch: list entries [e0, e1) of the row,
    // partials into slot `slot` (-1: the whole row, output as usual)
    int e0 = 0, e1 = -1, slot = -1;
    if (QPW == 1 && a.part != nullptr) {
        const int item = (int)(wg % p.n_items);
        bh = wg / p.n_items;
        const __attribute__((address_space(4))) int32_t* it =
            (const __attribute__((address_space(4))) int32_t*)(p.items + 4 * item);
        qfirst = it[0];
        e0 = it[1];
        e1 = it[2];
        slot = it[3];
    } else {
        // First query block of the group.  Sparse plans start each head with
        // the blocks of extra tokens: their rows keep every block and are the
        // longest, so they must not be the last to begin.
        const int ngrp = (p.nB + QPW - 1) / QPW;
        const int qg = (int)(wg % ngrp);     // group of QPW query blocks
        bh = wg / ngrp;
        const int nx = p.nB - p.nB_video;
        qfirst = QPW == 1 ? (qg < nx ? p.nB_video + qg : qg - nx) : qg * QPW;
    }
    // this wave's query block; past the last block (odd nB, QPW = 2) the
    // wave computes on the last block's rows and stores nothing
    // (wave-uniform; readfirstlane tells the compiler, so the row's pointers
    // and lengths stay scalar)
    const bool q_ok = qfirst + wave_u / WPB < p.nB;
    const int qb = __builtin_amdgcn_readfirstlane(q_ok ? qfirst + wave_u / WPB : p.nB - 1);
    const int qrow = (wave % WPB) * 32 + j;   // query row within the block
    SVA_DCHECK(p, qfirst >= 0 && qfirst < p.nB, SVA_DEBUG_ROW);

    // Q^T operand: lane (j, hf) holds channels 16s + 8hf .. +8 of row qrow
    bf16x8_t qop[DS];
    {
        const u32x4_t* qp = a.q + ((bh * p.Np) + (int64_t)qb * BLK + qrow) * KCH;
#pragma unroll
        for (int s = 0; s < DS; ++s) qop[s] = as_bf16x8(qp[2 * s + hf]);
    }
    // Drain the Q loads here: vmcnt retires in order, so a wait for Q placed
    // inside the loop would also wait for the stage copies issued before it.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    f32x16_t o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[t][v] = 0.f;
    // -1e30 instead of -inf keeps exp2(m_old - m_new) and fully masked
    // stages free of inf - inf.
    float m = -1e30f, l = 0.f;
    const float c = 1.4426950408889634f / sqrtf((float)D);   // log2(e)/sqrt(d)

    const int full_len = DENSE ? p.nB : (int)(p.row_ptr[qb + 1] - p.row_ptr[qb]);
    const int64_t r0 = p.row_ptr[qb] + e0;
    const int len = e1 >= 0 ? e1 - e0 : full_len;
    SVA_DCHECK(p, DENSE || (full_len >= 0 && full_len <= p.max_row_len), SVA_DEBUG_ROW);
    // a work item of a split launch: a piece [e0, e1) of the row with a
    // partial slot, or the whole row with slot -1
    SVA_DCHECK(p, e1 < 0 || (e0 >= 0 && e0 <= e1 && e1 <= full_len && slot < p.n_slots &&
                             (slot >= 0 || (e0 == 0 && e1 == full_len))),
               SVA_DEBUG_ROW);
    const int32_t* cl = DENSE ? nullptr : a.col + bh * p.nnz_per_head + r0;
    // the same list through the constant address space: wave-uniform
    // lookups become scalar loads, which do not count against vmcnt (a
    // vector load would make every wait for it wait for the copies too)
    const __attribute__((address_space(4))) int32_t* cls =
        (const __attribute__((address_space(4))) int32_t*)cl;
    const int last_video = p.nB_video - 1;
    const int last_valid = p.blk_valid[last_video];
    // this lane's 16 bytes of every wave-level copy
    // this head's K and V tiles (wave-uniform) and this lane's byte offset
    // in every wave-level copy
    const u32x4_t* kbase = a.k + bh * (int64_t)p.nB * (SPB * CPS);
    const u32x4_t* vbase = a.vt + bh * (int64_t)p.nB * (SPB * CPS);
    const uint32_t lane_off = (uint32_t)lane * 16u;
    const int nstage = len * SPB;
    // the block list is read from global memory (wave-uniform lookups, a few
    // per loop body); only compensation keeps a copy in LDS for its bitmap
    if constexpr (COMP) {
        for (int i = tid; i < len; i += NT) s_col[i] = cl[i];
        __syncthreads();
    }
    // The row is walked from its first block at or after qb rounded down to
    // a multiple of 64, wrapping around (the softmax does not depend on the
    // order).  The query blocks resident on one XCD at a time are about 64
    // neighbours; starting them at the same key block lets them stream the
    // blocks they share through L2 together (27 % fewer bytes from beyond L2
    // than walking every row from block 0 on the 75.6k-token workload).
    int rot = 0;
    {
        const int kstart = qfirst & ~63;   // the same for every wave
        if (DENSE) {
            rot = kstart < len ? kstart : 0;
        } else {
            int cnt = 0;
            for (int i = lane; i < len; i += 64) cnt += __popcll(__ballot(cl[i] < kstart));
            rot = __builtin_amdgcn_readfirstlane(cnt);
            if (rot >= len) rot = 0;
        }
    }

    // List entry w of the walk (w = 0 .. len-1 is list index (rot + w) mod
    // len): the byte offset of its block in this head's K and V tiles, and
    // its number of valid keys.  Entries past the end of the row and
    // out-of-range list entries have no valid keys; their copies read block
    // 0 into buffers that are never read, so every iteration issues the same
    // copies and the copy data always stays inside the head's tiles.
    struct Ent { uint32_t off; int nv; };
    auto entry = [&](int w) {
        const bool in = w < len;
        int li = rot + (in ? w : len - 1);
        li = li >= len ? li - len : li;
        const int kq = DENSE ? li : cls[li];
        const bool ok = in && kq >= 0 && kq < p.nB;
        Ent r;
        r.off = (uint32_t)(ok ? kq : 0) * (uint32_t)(SPB * CPS * 16);
        r.nv = ok ? (kq == last_video ? last_valid : BLK) : 0;
        return r;
    };
    // this lane's byte offset in copy i of stage q of a block (constants)
    uint32_t loff[SPB][LPW];
#pragma unroll
    for (int q = 0; q < SPB; ++q)
#pragma unroll
        for (int i = 0; i < LPW; ++i)
            loff[q][i] = (uint32_t)((q * CPS + (i * NWV + wave_u) * 64) * 16) + lane_off;
    const uint32_t kl0 = lds_addr(&sK[0][0]) + (uint32_t)wave_u * 1024u;
    const uint32_t vl0 = lds_addr(&sV[0][0]) + (uint32_t)wave_u * 1024u;
    // copies of stage Q_ of the block at PTR_ into K buffer BUF_ (resp. V)
#define SVA_COPY_K(PTR_, Q_, BUF_)                                                   \
    do {                                                                             \
        _Pragma("unroll") for (int i = 0; i < LPW; ++i)                              \
            lds_dma16_at(PTR_, loff[Q_][i], kl0,                                   \
                         (uint32_t)(((BUF_) * CPS + i * NWV * 64) * 16));            \
    } while (0)
#define SVA_COPY_V(PTR_, Q_, BUF_)                                                   \
    do {                                                                             \
        _Pragma("unroll") for (int i = 0; i < LPW; ++i)                              \
            lds_dma16_at(PTR_, loff[Q_][i], vl0,                                   \
                         (uint32_t)(((BUF_) * CPS + i * NWV * 64) * 16));            \
    } while (0)
    // S^T of stage st into SC from the K buffer KB_
#define SVA_SCORE(KB_, SC)                                                           \
    do {                                                                             \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) SC[v] = 0.f;                  \
        _Pragma("unroll") for (int s = 0; s < DS; ++s)                               \
            SC = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(KB_[s * 64 + lane]), \
                                                         qop[s], SC, 0, 0, 0);       \
    } while (0)
    // row max of SC over every key
#define SVA_MAX(SC, MX)                                                              \
    do {                                                                             \
        MX = -INFINITY;                                                              \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) MX = fmaxf(MX, SC[v]);        \
    } while (0)
    // keys from LIM on to -inf and the row max again (rare: the last video
    // block, out-of-range list entries, stages past the end).  The masked
    // max is at most the unmasked one; taking the min keeps the unmasked max
    // live on both paths, so it stays before the branch, beside the PV
    // matrix instructions, instead of being merged into one max after it.
#define SVA_MASK(LIM, SC, MX)                                                        \
    do {                                                                             \
        if (LIM < SK) {                                                              \
            /* lane (j, hf) holds stage keys 8*(v/4) + 4*hf + v%4 of column qrow */  \
            _Pragma("unroll") for (int v = 0; v < 16; ++v) {                         \
                const int key_ = 8 * (v / 4) + 4 * hf + (v % 4);                     \
                if (key_ >= LIM) SC[v] = -INFINITY;                                  \
            }                                                                        \
            float mm_;                                                               \
            SVA_MAX(SC, mm_);                                                        \
            MX = fminf(MX, mm_);                                                     \
        }                                                                            \
    } while (0)
    // raise the running max when MX exceeds it by more than kTau
#define SVA_RESCALE(MX)                                                              \
    do {                                                                             \
        if (__any(MX > m + kTau)) {                                                  \
            const float mn_ = fmaxf(m, MX);                                          \
            const float al_ = __builtin_amdgcn_exp2f(m - mn_);                       \
            m = mn_;                                                                 \
            l *= al_;                                                                \
            _Pragma("unroll") for (int t = 0; t < DT; ++t)                           \
            _Pragma("unroll") for (int v = 0; v < 16; ++v) o[t][v] *= al_;           \
        }                                                                            \
    } while (0)
    // probabilities of SC against m, summed into l and packed to bf16 in PB
#define SVA_EXP(SC, PB)                                                              \
    do {                                                                             \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) {                             \
            const float e_ = __builtin_amdgcn_exp2f(fmaf(SC[v], c, -m));             \
            SC[v] = e_;                                                              \
            l += e_;                                                                 \
        }                                                                            \
        _Pragma("unroll") for (int s2 = 0; s2 < 2; ++s2) {                           \
            u32x4_t u_;                                                              \
            u_.x = pack_bf16x2(SC[8 * s2 + 0], SC[8 * s2 + 1]);                      \
            u_.y = pack_bf16x2(SC[8 * s2 + 2], SC[8 * s2 + 3]);                      \
            u_.z = pack_bf16x2(SC[8 * s2 + 4], SC[8 * s2 + 5]);                      \
            u_.w = pack_bf16x2(SC[8 * s2 + 6], SC[8 * s2 + 7]);                      \
            PB[s2] = as_bf16x8(u_);                                                  \
        }                                                                            \
    } while (0)
    // keys from LIM on to -inf (rare; see SVA_MASK), no max
#define SVA_MASK_ONLY(LIM, SC)                                                       \
    do {                                                                             \
        if (LIM < SK) {                                                              \
            _Pragma("unroll") for (int v = 0; v < 16; ++v) {                         \
                const int key_ = 8 * (v / 4) + 4 * hf + (v % 4);                     \
                if (key_ >= LIM) SC[v] = -INFINITY;                                  \
            }                                                                        \
        }                                                                            \
    } while (0)
    // probabilities of SC against m into PB and their sum into LS
#define SVA_EXP_SUM(SC, PB, LS)                                                      \
    do {                                                                             \
        float e_[16];                                                                \
        _Pragma("unroll") for (int v = 0; v < 16; ++v)                               \
            e_[v] = __builtin_amdgcn_exp2f(fmaf(SC[v], c, -m));                      \
        u32x4_t u_[2];                                                               \
        _Pragma("unroll") for (int s2 = 0; s2 < 2; ++s2) {                           \
            u_[s2].x = pack_bf16x2(e_[8 * s2 + 0], e_[8 * s2 + 1]);                  \
            u_[s2].y = pack_bf16x2(e_[8 * s2 + 2], e_[8 * s2 + 3]);                  \
            u_[s2].z = pack_bf16x2(e_[8 * s2 + 4], e_[8 * s2 + 5]);                  \
            u_[s2].w = pack_bf16x2(e_[8 * s2 + 6], e_[8 * s2 + 7]);                  \
            PB[s2] = as_bf16x8(u_[s2]);                                              \
        }                                                                            \
        LS = e_[0];                                                                  \
        _Pragma("unroll") for (int v = 1; v < 16; ++v) LS += e_[v];                  \
    } while (0)
    // Probabilities of stage SC with the lazy rescale decided after the
    // fact: every probability is at most 2^kTau (up to rounding) when no logit
    // exceeds the running max by more than kTau, and a probability above
    // 2^kTau makes the lane's sum exceed it, so only a wave with such a sum
    // takes the max of the stage, raises m by the usual rule and recomputes.
#define SVA_EXP_CHECKED(SC, PB)                                                      \
    do {                                                                             \
        float ls_;                                                                   \
        SVA_EXP_SUM(SC, PB, ls_);                                                    \
        if (__any(ls_ >= kPmax)) {                                                   \
            float mx_;                                                               \
            SVA_MAX(SC, mx_);                                                        \
            mx_ = lane_swap_max(mx_) * c;                                            \
            SVA_RESCALE(mx_);                                                        \
            SVA_EXP_SUM(SC, PB, ls_);                                                \
        }                                                                            \
        l += ls_;                                                                    \
    } while (0)
    // O^T += V^T P^T from the V buffer VB_.  Step s2 contracts stage keys
    // 16*s2 + ..; lane half hf's 8 of them are V chunk 2*s2 + hf.
#define SVA_PV(VB_, PB)                                                              \
    do {                                                                             \
        _Pragma("unroll") for (int t = 0; t < DT; ++t)                               \
        _Pragma("unroll") for (int s2 = 0; s2 < 2; ++s2) {                           \
            const u32x4_t vv_ = VB_[(2 * s2 + hf) * D + t * 32 + j];                 \
            o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vv_), PB[s2],   \
                                                           o[t], 0, 0, 0);           \
        }                                                                            \
    } while (0)

    // Software pipeline, one wave: iteration st computes S^T of stage st+1
    // and O^T += V^T P^T of stage st-1 (16 matrix instructions) while it
    // turns S^T of stage st into probabilities; none of the three depends
    // on another, so the vector work spreads over all 16 matrix
    // instructions.  (A rescale of the accumulators in iteration st comes
    // after the product of stage st-1 in program order, which was taken
    // against the old max.)  The first iteration's product reads a zeroed
    // V buffer with P = 0; the last stage's product follows the loop.
    // K copies run KLEAD and V copies VLEAD stages ahead; at each barrier,
    // the K and V stages the iterations up to the next barrier read have
    // landed.  The loop has no ordinary LDS stores,
    // only copies: after this wave's wait, a bare s_barrier makes every
    // wave's part visible and orders every wave's reads of the oldest
    // buffers before the copies into them.  (__syncthreads() would add a
    // workgroup release fence, which waits for every outstanding load, the
    // copies still ahead included.)
    f32x16_t sc, sn;
    float mx;
    bf16x8_t pb[2];
    constexpr int NUE = NU / SPB;        // list entries per loop body
    constexpr int NC = NE - NUE;         // entries a body hands to the next
    static_assert(NC >= 1, "entry carry");
    const char* kb8 = reinterpret_cast<const char*>(kbase);
    const char* vb8 = reinterpret_cast<const char*>(vbase);
    Ent C[NC];
#pragma unroll
    for (int e = 0; e < NC; ++e) C[e] = entry(e);
    if (nstage > 0) {
        Ent E[NE];
#pragma unroll
        for (int e = 0; e < NE; ++e) E[e] = e < NC ? C[e] : entry(e);
#pragma unroll
        for (int u = 0; u < KLEAD; ++u) SVA_COPY_K(kb8 + E[u / SPB].off, u % SPB, u);
#pragma unroll
        for (int u = 0; u < VLEAD; ++u) SVA_COPY_V(vb8 + E[u / SPB].off, u % SPB, u);
        // the V buffer the first iteration's product reads (with P = 0)
        for (int i = tid; i < CPS; i += NT) sV[NBV - 1][i] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) pb[s2] = as_bf16x8(u32x4_t{0u, 0u, 0u, 0u});
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        SVA_SCORE(sK[0], sc);
        SVA_MAX(sc, mx);
        SVA_MASK(E[0].nv, sc, mx);
        mx = lane_swap_max(mx) * c;
        SVA_RESCALE(mx);
        // with a barrier every second stage, iteration 1 may copy into the
        // buffer this first score read: every wave finishes reading it first
        if (BP == 2) __builtin_amdgcn_s_barrier();
    }
    // A body covers NUE whole list entries (NU stages, a multiple of NBK,
    // NBV and SPB, so every buffer index is a constant).  It needs the
    // entries w .. w+NE-1: the first NC come from the previous body, the
    // rest are looked up (scalar loads) once.
    for (int w = 0; w < len; w += NUE) {
        Ent E[NE];
#pragma unroll
        for (int e = 0; e < NE; ++e) E[e] = e < NC ? C[e] : entry(w + e);
#pragma unroll
        for (int e = 0; e < NC; ++e) C[e] = E[e + NUE];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            // a body's later entries may lie past the end of the row
            if (u > 0 && u % SPB == 0 && w + u / SPB >= len) break;
            const int ck = u + KLEAD, cv = u + VLEAD, cs = u + 1;
            SVA_COPY_K(kb8 + E[ck / SPB].off, ck % SPB, ck % NBK);
            SVA_COPY_V(vb8 + E[cv / SPB].off, cv % SPB, cv % NBV);
            const int lim = E[cs / SPB].nv - (cs % SPB) * SK;
            // one straight-line region: the scheduler interleaves the
            // matrix instructions and the vector work
            SVA_SCORE(sK[cs % NBK], sn);
            SVA_PV(sV[(u + NBV - 1) % NBV], pb);
            SVA_EXP_CHECKED(sc, pb);
            SVA_MASK_ONLY(lim, sn);
            // the compiler's small-GEMM interleave of LDS reads and matrix
            // instructions for this region (bit-identical; 720p 24.60 ->
            // 24.43 ms, sparse 480p 1.62 -> 1.57 ms, dense HunyuanVideo
            // 137.8 -> 134.7 ms; its exp-interleave strategies were slower)
            __builtin_amdgcn_iglp_opt(0);
            sc = sn;
            // (a body starts at a multiple of BP stages, so u & 1 is the
            // stage's parity)
            if (BP == 1 || (u & 1)) {
                __builtin_amdgcn_s_waitcnt(kWaitNext);
                __builtin_amdgcn_s_barrier();
            }
        }
    }
    // the last stage's product (its V landed before the loop's last barrier)
    if (nstage > 0) SVA_PV(sV[(nstage - 1) % NBV], pb);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // no copy left in flight at exit

    // Compensation (sparse rows that drop blocks): every block the row does
    // not list enters the softmax as one extra key, its mean key with logit
    // bias log2|B| and its mean value (the mean tiles hold block kb as key
    // kb % 32 of group kb / 32).  One stage per group of 32 means, after the
    // kept stages, two buffer pairs alternating.
    if constexpr (COMP) {
        const int ng = p.n_mean_groups;
        if (slot < 0 && full_len < p.nB) {
            uint32_t* s_kept = reinterpret_cast<uint32_t*>(s_col + p.max_row_len);
            for (int i = tid; i < ng; i += NT) s_kept[i] = 0u;
            // every wave's copies have landed and every read of the stage
            // buffers is done before they are reused
            __syncthreads();
            for (int i = tid; i < len; i += NT) {
                const int kb = s_col[i];
                if (kb >= 0 && kb < p.nB) atomicOr(&s_kept[kb >> 5], 1u << (kb & 31));
            }
            const u32x4_t* kmb = a.km + bh * (int64_t)ng * CPS;
            const u32x4_t* vmb = a.vm + bh * (int64_t)ng * CPS;
            const float bias_blk = __log2f((float)BLK) / c;
            const float bias_last = __log2f((float)last_valid) / c;
            auto copy = [&](int cg, u32x4_t* KB, u32x4_t* VB) {
#pragma unroll
                for (int i = 0; i < LPW; ++i) {
                    const int e = (i * NWV + wave_u) * 64;
                    lds_dma16(kmb, (uint32_t)(cg * CPS + e) * 16u, lane_off, lds_addr(KB + e));
                    lds_dma16(vmb, (uint32_t)(cg * CPS + e) * 16u, lane_off, lds_addr(VB + e));
                }
            };
            auto stage = [&](int cg, const u32x4_t* KB, const u32x4_t* VB) {
                f32x16_t sm;
                SVA_SCORE(KB, sm);
                const uint32_t kept = s_kept[cg];
                float mm = -INFINITY;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    // lane (j, hf) holds stage keys 8*(v/4) + 4*hf + v%4
                    const int key = 8 * (v / 4) + 4 * hf + (v % 4);
                    const int kb = cg * 32 + key;
                    const bool in = kb < p.nB && !((kept >> key) & 1u);
                    sm[v] = in ? sm[v] + (kb == last_video ? bias_last : bias_blk) : -INFINITY;
                    mm = fmaxf(mm, sm[v]);
                }
                mm = lane_swap_max(mm) * c;
                SVA_RESCALE(mm);
                bf16x8_t pm[2];
                SVA_EXP(sm, pm);
                SVA_PV(VB, pm);
            };
            copy(0, sK[0], sV[0]);
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();          // copies of group 0 and the bitmap visible
            for (int cg = 0; cg < ng; cg += 2) {
                if (cg + 1 < ng) copy(cg + 1, sK[1], sV[1]);
                stage(cg, sK[0], sV[0]);
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                __builtin_amdgcn_s_barrier();
                if (cg + 1 < ng) {
                    if (cg + 2 < ng) copy(cg + 2, sK[0], sV[0]);
                    stage(cg + 1, sK[1], sV[1]);
                    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                    __builtin_amdgcn_s_barrier();
                }
            }
        }
    }
#undef SVA_PV
#undef SVA_EXP
#undef SVA_EXP_SUM
#undef SVA_EXP_CHECKED
#undef SVA_MASK_ONLY
#undef SVA_RESCALE
#undef SVA_MASK
#undef SVA_MAX
#undef SVA_SCORE
#undef SVA_COPY_K
#undef SVA_COPY_V

    // epilogue: O = O^T / l.  Tile order: padding query rows are written as
    // zeros.  Raster order: row qrow goes to raster token inv[qb·BLK + qrow]
    // (the inverse reorder fused away); padding rows have none.
    if (!q_ok) return;
    const float lt = lane_swap_sum(l);
    if (slot >= 0) {
        // a piece of a split row: the unnormalised O^T, m and l of row qrow
        // into the piece's partial slot (O rows of d floats, then m, then l)
        float* pp = a.part + (bh * p.n_slots + slot) * (int64_t)(BLK * (D + 2));
        float4* po = reinterpret_cast<float4*>(pp + (int64_t)qrow * D);
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                po[(t * 32 + 8 * g + 4 * hf) / 4] =
                    make_float4(o[t][4 * g], o[t][4 * g + 1], o[t][4 * g + 2], o[t][4 * g + 3]);
        if (hf == 0) {
            pp[BLK * D + qrow] = m;
            pp[BLK * D + BLK + qrow] = lt;
        }
        return;
    }
    const bool row_ok = qrow < p.blk_valid[qb];
    const float inv = (row_ok && lt > 0.f) ? 1.f / lt : 0.f;
    uint2* op;
    if (a.o_raster) {
        if (!row_ok) return;
        const int n = p.inv[qb * BLK + qrow];
        SVA_DCHECK(p, n >= 0 && n < p.N, SVA_DEBUG_TOKEN);
        const int64_t b = bh / p.H, h = bh - b * p.H;
        op = a.o + ((b * p.N + n) * p.H + h) * (D / 4);
    } else {
        op = a.o + ((bh * p.Np) + (int64_t)qb * BLK + qrow) * (D / 4);
    }
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            // channels t*32 + 8g + 4hf + 0..3
            uint2 w = {0u, 0u};
            if (row_ok) {
                w.x = pack_bf16x2(o[t][4 * g + 0] * inv, o[t][4 * g + 1] * inv);
                w.y = pack_bf16x2(o[t][4 * g + 2] * inv, o[t][4 * g + 3] * inv);
            }
            op[(t * 32 + 8 * g + 4 * hf) / 4] = w;
        }
}

// Merge of a split row's pieces: per query row, M = max of the pieces'
// running maxima, o = sum 2^(m_i - M) O_i / sum 2^(m_i - M) l_i (m in log2
// units), written like the unsplit rows (tile order with zero padding rows,
// or raster order).  One workgroup per (b, h, split row).
template <int D, int BLK>
__global__ __launch_bounds__(256) void attn_merge_kernel(DevPlan p, const float* part, uint2* o,
                                                         int o_raster) {
    constexpr int C4 = D / 4;                   // float4 chunks per row
    const int sr = (int)(blockIdx.x % (unsigned)p.n_split);
    const int64_t bh = blockIdx.x / (unsigned)p.n_split;
    const int qb = p.split_rows[3 * sr];
    const int s0 = p.split_rows[3 * sr + 1];
    const int np = p.split_rows[3 * sr + 2];
    const int64_t ss = (int64_t)BLK * (D + 2);  // floats per slot
    const float* base = part + (bh * p.n_slots + s0) * ss;
    const int valid = p.blk_valid[qb];
    const int64_t b = bh / p.H, h = bh - b * p.H;
    SVA_DCHECK(p, qb >= 0 && qb < p.nB && s0 >= 0 && np >= 1 && s0 + np <= p.n_slots, SVA_DEBUG_ROW);
    for (int idx = threadIdx.x; idx < BLK * C4; idx += 256) {
        const int row = idx / C4, c4 = idx - row * C4;
        float M = -INFINITY;
        for (int q = 0; q < np; ++q) M = fmaxf(M, base[q * ss + BLK * D + row]);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        float L = 0.f;
        for (int q = 0; q < np; ++q) {
            const float* sp = base + q * ss;
            const float w = __builtin_amdgcn_exp2f(sp[BLK * D + row] - M);
            L += w * sp[BLK * D + BLK + row];
            const float4 v = reinterpret_cast<const float4*>(sp + (int64_t)row * D)[c4];
            acc.x += w * v.x;
            acc.y += w * v.y;
            acc.z += w * v.z;
            acc.w += w * v.w;
        }
        const bool row_ok = row < valid;
        const float inv = (row_ok && L > 0.f) ? 1.f / L : 0.f;
        uint2 wv = {0u, 0u};
        if (row_ok) {
            wv.x = pack_bf16x2(acc.x * inv, acc.y * inv);
            wv.y = pack_bf16x2(acc.z * inv, acc.w * inv);
        }
        if (o_raster) {
            if (!row_ok) continue;
            const int n = p.inv[qb * BLK + row];
            SVA_DCHECK(p, n >= 0 && n < p.N, SVA_DEBUG_TOKEN);
            o[((b * p.N + n) * p.H + h) * C4 + c4] = wv;
        } else {
            o[((bh * p.Np) + (int64_t)qb * BLK + row) * C4 + c4] = wv;
        }
    }
}

}  // namespace

hipError_t launch_attention(const DevPlan& p, const uint16_t* qr, const uint16_t* kr,
                            const uint16_t* vt, const int32_t* col, const uint16_t* km,
                            const uint16_t* vm, uint16_t* o, bool o_raster, float* part,
                            hipStream_t s) {
    AttnArgs a;
    a.p = p;
    a.q = reinterpret_cast<const u32x4_t*>(qr);
    a.k = reinterpret_cast<const u32x4_t*>(kr);
    a.vt = reinterpret_cast<const u32x4_t*>(vt);
    a.col = col;
    a.km = reinterpret_cast<const u32x4_t*>(km);
    a.vm = reinterpret_cast<const u32x4_t*>(vm);
    a.o = reinterpret_cast<uint2*>(o);
    a.o_raster = o_raster ? 1 : 0;
    // long rows split only for sparse plans that have split rows
    const bool split = part != nullptr && !p.dense && p.n_items > 0;
    a.part = split ? part : nullptr;
    // dense plans: two query blocks per workgroup, except d = 64 with
    // 128-token blocks, whose stage copy (256 chunks) cannot be split over
    // eight waves
    const int qpw = (p.dense && !(p.d == 64 && p.block == 128)) ? 2 : 1;
    const int64_t per_head = split ? p.n_items : (p.nB + qpw - 1) / qpw;
    dim3 grid((unsigned)((int64_t)p.B * p.H * per_head));
    dim3 block(p.block * 2 * qpw);
    // dynamic LDS: compensation's copy of the block list and its bitmap
    const size_t lds = km ? (size_t)(p.max_row_len + p.n_mean_groups) * sizeof(int32_t) : 0;
    auto launch = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, lds, s, a); };
    // dense plans have nothing to compensate; compensation is its own
    // instantiation so the plain kernels carry none of it
    if (p.dense) {
        if (p.d == 128 && p.block == 128) launch(attn_kernel<128, 128, true, false, 2>);
        else if (p.d == 128) launch(attn_kernel<128, 64, true, false, 2>);
        else if (p.block == 128) launch(attn_kernel<64, 128, true, false, 1>);
        else launch(attn_kernel<64, 64, true, false, 2>);
    } else if (!km) {
        if (p.d == 128 && p.block == 128) launch(attn_kernel<128, 128, false, false, 1>);
        else if (p.d == 128) launch(attn_kernel<128, 64, false, false, 1>);
        else if (p.block == 128) launch(attn_kernel<64, 128, false, false, 1>);
        else launch(attn_kernel<64, 64, false, false, 1>);
    } else {
        if (p.d == 128 && p.block == 128) launch(attn_kernel<128, 128, false, true, 1>);
        else if (p.d == 128) launch(attn_kernel<128, 64, false, true, 1>);
        else if (p.block == 128) launch(attn_kernel<64, 128, false, true, 1>);
        else launch(attn_kernel<64, 64, false, true, 1>);
    }
    if (split) {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        dim3 mg((unsigned)((int64_t)p.B * p.H * p.n_split));
        uint2* o2 = reinterpret_cast<uint2*>(o);
        if (p.d == 128 && p.block == 128)
            hipLaunchKernelGGL((attn_merge_kernel<128, 128>), mg, dim3(256), 0, s, p, part, o2, a.o_raster);
        else if (p.d == 128)
            hipLaunchKernelGGL((attn_merge_kernel<128, 64>), mg, dim3(256), 0, s, p, part, o2, a.o_raster);
        else if (p.block == 128)
            hipLaunchKernelGGL((attn_merge_kernel<64, 128>), mg, dim3(256), 0, s, p, part, o2, a.o_raster);
        else
            hipLaunchKernelGGL((attn_merge_kernel<64, 64>), mg, dim3(256), 0, s, p, part, o2, a.o_raster);
    }
    return hipGetLastError();
}

}  // namespace sva
