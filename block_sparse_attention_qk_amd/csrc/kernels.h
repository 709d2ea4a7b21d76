// Internal: device view of a plan and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "sva.h"

namespace sva {

// Exact unsigned division by a plan constant: for 0 <= x < 2^31,
// x / d == (x · m) >> s with l = ceil(log2 d), s = 31 + l and
// m = ceil(2^s / d) < 2^32 (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994, theorem 4.2 with N = 31).
struct FastDiv {
    uint32_t m;
    int s;
};

inline FastDiv make_fastdiv(uint32_t d) {
    int l = 0;
    while ((1ull << l) < d) ++l;
    const uint64_t two_s = 1ull << (31 + l);
    return FastDiv{(uint32_t)((two_s + d - 1) / d), 31 + l};
}

__device__ __forceinline__ uint32_t fast_div(uint32_t x, FastDiv f) {
    return (uint32_t)(((uint64_t)x * f.m) >> f.s);
}

// Everything a kernel needs to know about a plan, passed by value.
struct DevPlan {
    int B, H, d, block;
    int T, Hh, W;
    int64_t n_video, N, n_video_pad, Np;
    int nB, nB_video, k;
    int dense;          // every block kept
    int same_frame;     // SVA_KEEP_SAME_FRAME
    int scorer;         // SVA_SCORER_*
    int nsub;           // runs per block (1 for the mean scorer)
    int n_mean_groups;  // ceil(nB / 32)
    float eps;
    int rope_off[3];    // offsets (in cos/sin pairs) of the t, h, w tables
    int rope_half[3];   // rotated pairs per section
    const float2* rope_cs;
    const int32_t* perm;       // [N]
    const int32_t* inv;        // [Np]
    const int32_t* blk_valid;  // [nB]
    const int32_t* blk_tmin;   // [nB]
    const int32_t* blk_tmax;   // [nB]
    const int32_t* row_ptr;    // [nB+1]
    int64_t nnz_per_head;
    int max_row_len;
    // split long rows (attention with a workspace): n_items work items of
    // 4 ints (qb, first entry, end entry, partial slot or -1) per (b, h),
    // n_split split rows of 3 ints (qb, first slot, pieces), n_slots
    // partial slots per (b, h); n_items == 0 when no row is split
    const int32_t* items;
    const int32_t* split_rows;
    int n_items, n_split, n_slots;
    // divisions of (token, head) row indices, all below 2^31
    FastDiv div_H, div_N, div_HW, div_W, div_Np;
#ifdef SVA_DEBUG
    uint32_t* dbg;      // the plan's debug word (SVA_DEBUG_* bits)
#endif
};

// Debug builds: a failed check ORs its SVA_DEBUG_* bit into the plan's
// debug word and the kernel goes on.  Release builds compile it away.
#ifdef SVA_DEBUG
#define SVA_DCHECK(P, COND, BIT)                                          \
    do {                                                                  \
        if (!(COND)) atomicOr((P).dbg, (uint32_t)(BIT));                  \
    } while (0)
#else
#define SVA_DCHECK(P, COND, BIT) \
    do {                         \
    } while (0)
#endif

// debug builds: one kernel whose check fails on purpose (sva_debug_selftest)
hipError_t launch_debug_selftest(const DevPlan& p, hipStream_t s);

// tiled: qo = Q' in tile order [B,H,Np,d], ko = K' tiles (padding zeroed);
// otherwise both raster [B,N,H,d].  means (tiled only, may be NULL): the
// selection's block means, laid out as launch_select's workspace
hipError_t launch_prologue(const DevPlan& p, const uint16_t* q, const uint16_t* k,
                           const float* wq, const float* wk, uint16_t* qo, uint16_t* ko,
                           bool tiled, double* means, hipStream_t s);

hipError_t launch_reorder(const DevPlan& p, const uint16_t* in, uint16_t* out, int direction,
                          hipStream_t s);

// qr: Q' in tile order; kt: K' as K tiles; both NULL: ws already holds the
// means (written by the tiled prologue), only the ranking runs.
// ws: [B,H,nB,nsub,d] q means followed by [B,H,d,nB·nsub] k means (float64)
hipError_t launch_select(const DevPlan& p, const uint16_t* qr, const uint16_t* kt, double* ws,
                         int32_t* col, hipStream_t s);

// km, vm: mean tiles (NULL: no compensation); o_raster: O in raster order
// [B,N,H,d] instead of tile order [B,H,Np,d]; part (NULL: no split): the
// partials of split rows, then their merge into o
hipError_t launch_attention(const DevPlan& p, const uint16_t* qr, const uint16_t* kr,
                            const uint16_t* vt, const int32_t* col, const uint16_t* km,
                            const uint16_t* vm, uint16_t* o, bool o_raster, float* part,
                            hipStream_t s);

hipError_t launch_block_means(const DevPlan& p, const uint16_t* kt, const uint16_t* vt,
                              uint16_t* km, uint16_t* vm, hipStream_t s);

// ---- small device helpers shared by the kernels ----

// Native clang vectors (not HIP's uint4 struct): arrays of them stay in
// registers where arrays of the struct can end up in scratch or LDS.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two floats -> two bf16 (round to nearest even, hardware conversion).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t v = {lo, hi};
    bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, b);
}

}  // namespace sva
