// Host-side planning: validation, token permutation, block metadata, block
// budget and row offsets, RoPE tables.  Pure C++ (no HIP), so the same code
// serves the host-only query calls and the device plan.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/sva.h"

namespace sva {

struct HostPlan {
    sva_plan_desc desc{};       // with defaults resolved
    sva_plan_info info{};
    std::vector<int32_t> perm;  // [N]   raster token -> tile-order row
    std::vector<int32_t> inv;   // [Np]  tile-order row -> raster token, -1 = pad
    std::vector<int32_t> blk_valid;  // [nB] valid tokens per block
    std::vector<int32_t> blk_tmin;   // [nB] first frame of the valid tokens (-1 extra)
    std::vector<int32_t> blk_tmax;   // [nB] last frame (-1 extra)
    std::vector<int32_t> row_ptr;    // [nB+1]
    // Attention work items when long rows are split (sva_attention_ws):
    // 4 ints per item (qb, first list entry, end entry, partial slot or -1),
    // the pieces of the split rows first; split rows: 3 ints per row (qb,
    // first slot, pieces).
    std::vector<int32_t> items;
    std::vector<int32_t> split_rows;
    int32_t n_slots = 0;     // partial slots per (b, h)
    // RoPE cos/sin per axis section: entry (pos, i) of axis a at
    // rope_off[a] + pos * rope_half[a] + i, as (cos, sin) pairs.
    std::vector<float> rope_cs;
    int32_t rope_off[3] = {0, 0, 0};
    int32_t rope_half[3] = {0, 0, 0};
};

// Fills `plan` from `desc`; on failure returns an SVA_ERR_* code and sets `err`.
int build_host_plan(const sva_plan_desc& desc, HostPlan& plan, std::string& err,
                    bool with_tables = true);

// True when key block kb is always kept for query block qb (video rows only).
inline bool forced_pair(const HostPlan& p, int qb, int kb) {
    const int nBv = p.info.nB_video;
    if (kb >= nBv) return true;                       // extra-token columns
    if (qb >= nBv) return true;                       // (extra rows are dense)
    if (p.desc.flags & SVA_KEEP_SAME_FRAME)
        return p.blk_tmin[qb] <= p.blk_tmax[kb] && p.blk_tmin[kb] <= p.blk_tmax[qb];
    return false;
}

void set_last_error(const std::string& msg);

}  // namespace sva
