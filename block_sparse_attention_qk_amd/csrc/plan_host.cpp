// Host-side planning (see plan_host.h).
//
// Readings of the pages that fix these tables:
//  - tokens are permuted into 3D tiles so a block is a local space-time
//    patch ("Sol Video Inference Engine" blog, 4.2.2, on Sparse VideoGen2's
//    permutation for GPU layout); tiles are visited in (t, h, w) order,
//    edge tiles are clipped, tokens inside a tile go in (t, h, w) order and
//    the sequence is padded once at the tail to a multiple of the block;
//  - the block budget follows the definition of sparsity as the fraction of
//    key blocks dropped ("MiniMax-H3 在 8×H200 上基准测试", section
//    "SubBlock 稀疏注意力如何工作"): k = ceil((1 - sparsity)·nB), optionally
//    rounded up to a multiple of budget_multiple (that section rounds the
//    SubBlock router's budget in units of 8 blocks), clamped to [1, nB];
//  - forced blocks (extra-token columns, same-frame blocks) count toward
//    the budget, so a row keeps max(k, forced) blocks; extra-token rows are
//    dense.  Row lengths therefore depend only on the geometry and the
//    row offsets are fixed at plan time.
#include "plan_host.h"

#include <cmath>
#include <cstring>
#include <sstream>

namespace sva {

namespace {
int fail(std::string& err, int code, const std::string& msg) {
    err = msg;
    return code;
}
}  // namespace

int build_host_plan(const sva_plan_desc& in, HostPlan& p, std::string& err, bool with_tables) {
    sva_plan_desc d = in;
    if (d.B < 1 || d.H < 1 || d.T < 1 || d.Hh < 1 || d.W < 1)
        return fail(err, SVA_ERR_INVALID_ARG, "B, H, T, Hh, W must all be >= 1");
    if (d.d != 64 && d.d != 128)
        return fail(err, SVA_ERR_UNSUPPORTED, "head dim must be 64 or 128");
    if (d.block != 64 && d.block != 128)
        return fail(err, SVA_ERR_UNSUPPORTED, "block must be 64 or 128");
    if (!(d.sparsity >= 0.0 && d.sparsity < 1.0))
        return fail(err, SVA_ERR_INVALID_ARG, "sparsity must be in [0, 1)");
    if (d.flags & ~(SVA_DENSE | SVA_KEEP_SAME_FRAME | SVA_COMPENSATE))
        return fail(err, SVA_ERR_INVALID_ARG, "unknown flag bits");
    if (d.tile_t == 0 && d.tile_h == 0 && d.tile_w == 0) {
        if (d.block == 64) { d.tile_t = 4; d.tile_h = 4; d.tile_w = 4; }
        else { d.tile_t = 2; d.tile_h = 8; d.tile_w = 8; }
    }
    if (d.tile_t < 1 || d.tile_h < 1 || d.tile_w < 1)
        return fail(err, SVA_ERR_INVALID_ARG, "tile extents must be >= 1");
    if (d.n_extra < 0 || d.n_extra % d.block != 0)
        return fail(err, SVA_ERR_INVALID_ARG, "n_extra must be >= 0 and a multiple of block");
    if (d.rope_theta == 0.0) d.rope_theta = 10000.0;
    if (!(d.rope_theta > 1.0) || !std::isfinite(d.rope_theta))
        return fail(err, SVA_ERR_INVALID_ARG, "rope_theta must be > 1");
    if (d.rope_split[0] == 0 && d.rope_split[1] == 0 && d.rope_split[2] == 0) {
        if (d.d == 64) { d.rope_split[0] = 16; d.rope_split[1] = 24; d.rope_split[2] = 24; }
        else { d.rope_split[0] = 44; d.rope_split[1] = 42; d.rope_split[2] = 42; }
    }
    int split_sum = 0;
    for (int a = 0; a < 3; ++a) {
        if (d.rope_split[a] < 0 || d.rope_split[a] % 2 != 0)
            return fail(err, SVA_ERR_INVALID_ARG, "RoPE sections must be even and >= 0");
        split_sum += d.rope_split[a];
    }
    if (split_sum > d.d)
        return fail(err, SVA_ERR_INVALID_ARG, "RoPE sections exceed the head dim");
    if (d.scorer != SVA_SCORER_MEAN && d.scorer != SVA_SCORER_SUBBLOCK)
        return fail(err, SVA_ERR_INVALID_ARG, "unknown scorer");
    if (d.subblocks == 0) d.subblocks = d.scorer == SVA_SCORER_SUBBLOCK ? 4 : 1;
    if (d.scorer == SVA_SCORER_MEAN && d.subblocks != 1)
        return fail(err, SVA_ERR_INVALID_ARG, "the mean scorer has one run per block");
    if (d.subblocks != 1 && d.subblocks != 2 && d.subblocks != 4)
        return fail(err, SVA_ERR_UNSUPPORTED, "subblocks must be 1, 2 or 4");
    if (d.budget_multiple == 0) d.budget_multiple = 1;
    if (d.budget_multiple < 1)
        return fail(err, SVA_ERR_INVALID_ARG, "budget_multiple must be >= 0");
    if (d.eps == 0.0) d.eps = 1e-6;
    if (!(d.eps > 0.0) || !std::isfinite(d.eps))
        return fail(err, SVA_ERR_INVALID_ARG, "eps must be > 0");

    const int64_t n_video = (int64_t)d.T * d.Hh * d.W;
    const int64_t N = n_video + d.n_extra;
    const int64_t nvp = (n_video + d.block - 1) / d.block * d.block;
    const int64_t Np = nvp + d.n_extra;
    const int64_t nB = Np / d.block;
    if (nB > 4096)
        return fail(err, SVA_ERR_INVALID_ARG, "more than 4096 blocks per head");
    if ((int64_t)d.B * d.H * Np >= ((int64_t)1 << 31))
        return fail(err, SVA_ERR_INVALID_ARG, "tensor too large (2^31 or more rows of d)");

    p.desc = d;
    sva_plan_info& I = p.info;
    std::memset(&I, 0, sizeof(I));
    I.n_video = n_video;
    I.N = N;
    I.n_video_pad = nvp;
    I.Np = Np;
    I.nB = (int32_t)nB;
    I.nB_video = (int32_t)(nvp / d.block);
    I.dense = ((d.flags & SVA_DENSE) || d.sparsity == 0.0) ? 1 : 0;
    if (I.dense) {
        I.k = (int32_t)nB;
    } else {
        double kk = std::ceil((1.0 - d.sparsity) * (double)nB - 1e-9);
        int64_t k = (int64_t)kk;
        if (d.budget_multiple > 1)
            k = (k + d.budget_multiple - 1) / d.budget_multiple * d.budget_multiple;
        if (k < 1) k = 1;
        if (k > nB) k = nB;
        I.k = (int32_t)k;
    }
    I.tile[0] = d.tile_t; I.tile[1] = d.tile_h; I.tile[2] = d.tile_w;
    I.scorer = d.scorer;
    I.subblocks = d.subblocks;
    I.budget_multiple = d.budget_multiple;
    I.n_mean_groups = (int32_t)((nB + 31) / 32);
    for (int a = 0; a < 3; ++a) I.rope_split[a] = d.rope_split[a];

    // --- permutation ---
    p.perm.assign(N, 0);
    p.inv.assign(Np, -1);
    {
        int64_t pos = 0;
        for (int t0 = 0; t0 < d.T; t0 += d.tile_t)
            for (int h0 = 0; h0 < d.Hh; h0 += d.tile_h)
                for (int w0 = 0; w0 < d.W; w0 += d.tile_w) {
                    const int t1 = std::min(t0 + d.tile_t, d.T);
                    const int h1 = std::min(h0 + d.tile_h, d.Hh);
                    const int w1 = std::min(w0 + d.tile_w, d.W);
                    for (int t = t0; t < t1; ++t)
                        for (int h = h0; h < h1; ++h)
                            for (int w = w0; w < w1; ++w) {
                                const int64_t n = ((int64_t)t * d.Hh + h) * d.W + w;
                                p.perm[n] = (int32_t)pos;
                                p.inv[pos] = (int32_t)n;
                                ++pos;
                            }
                }
        for (int64_t e = 0; e < d.n_extra; ++e) {
            p.perm[n_video + e] = (int32_t)(nvp + e);
            p.inv[nvp + e] = (int32_t)(n_video + e);
        }
    }

    // --- block metadata ---
    p.blk_valid.assign(nB, 0);
    p.blk_tmin.assign(nB, INT32_MAX);
    p.blk_tmax.assign(nB, -1);
    for (int64_t pos = 0; pos < n_video; ++pos) {
        const int64_t n = p.inv[pos];
        const int t = (int)(n / ((int64_t)d.Hh * d.W));
        const int64_t b = pos / d.block;
        p.blk_valid[b] += 1;
        p.blk_tmin[b] = std::min(p.blk_tmin[b], t);
        p.blk_tmax[b] = std::max(p.blk_tmax[b], t);
    }
    for (int64_t b = I.nB_video; b < nB; ++b) {
        p.blk_valid[b] = d.block;
        p.blk_tmin[b] = -1;
        p.blk_tmax[b] = -1;
    }

    // --- row lengths and offsets ---
    p.row_ptr.assign(nB + 1, 0);
    int32_t max_len = 0;
    for (int qb = 0; qb < nB; ++qb) {
        int32_t len;
        if (I.dense || qb >= I.nB_video) {
            len = (int32_t)nB;
        } else {
            int32_t nf = 0;
            for (int kb = 0; kb < nB; ++kb) nf += forced_pair(p, qb, kb) ? 1 : 0;
            len = std::max(I.k, nf);
        }
        p.row_ptr[qb + 1] = p.row_ptr[qb] + len;
        max_len = std::max(max_len, len);
    }
    I.max_row_len = max_len;
    I.nnz_per_head = p.row_ptr[nB];
    I.nnz = I.nnz_per_head * d.B * d.H;
    // workspace: q block means [B,H,nB,d] and transposed k block means
    // [B,H,d,nB], float64
    I.select_workspace_bytes =
        I.dense ? 0 : (size_t)2 * d.B * d.H * nB * d.subblocks * d.d * sizeof(double);

    // --- split of long rows ---
    // A sparse plan's extra-token rows keep every block and can be many
    // times longer than the video rows; walked by one workgroup each, they
    // bound the step of a grid with few heads.  With an attention workspace
    // every row longer than 1.5 times the longest video row is cut into
    // pieces of at most that many list entries; each piece is a workgroup
    // of its own writing (m, l, O) partials, merged afterwards.
    p.items.clear();
    p.split_rows.clear();
    p.n_slots = 0;
    if (!I.dense) {
        int32_t chunk = 16;
        for (int qb = 0; qb < I.nB_video; ++qb)
            chunk = std::max(chunk, p.row_ptr[qb + 1] - p.row_ptr[qb]);
        std::vector<char> split(nB, 0);
        for (int qb = 0; qb < nB; ++qb) {
            const int32_t len = p.row_ptr[qb + 1] - p.row_ptr[qb];
            if (2 * len <= 3 * chunk) continue;
            const int32_t pieces = (len + chunk - 1) / chunk;
            split[qb] = 1;
            p.split_rows.insert(p.split_rows.end(), {qb, p.n_slots, pieces});
            for (int32_t q = 0; q < pieces; ++q) {
                const int32_t e0 = (int32_t)((int64_t)len * q / pieces);
                const int32_t e1 = (int32_t)((int64_t)len * (q + 1) / pieces);
                p.items.insert(p.items.end(), {qb, e0, e1, p.n_slots + q});
            }
            p.n_slots += pieces;
        }
        if (p.n_slots > 0) {
            for (int qb = 0; qb < nB; ++qb)
                if (!split[qb])
                    p.items.insert(p.items.end(),
                                   {qb, 0, p.row_ptr[qb + 1] - p.row_ptr[qb], -1});
        } else {
            p.items.clear();
        }
    }
    // partials: per slot, O (block x d), then m and l (block each), float32
    I.attention_workspace_bytes =
        (size_t)d.B * d.H * p.n_slots * d.block * (d.d + 2) * sizeof(float);

    // --- RoPE tables ---
    if (with_tables) {
        const int len[3] = {d.T, d.Hh, d.W};
        int32_t off = 0;
        p.rope_cs.clear();
        for (int a = 0; a < 3; ++a) {
            const int width = d.rope_split[a];
            const int half = width / 2;
            p.rope_off[a] = off;
            p.rope_half[a] = half;
            for (int pos = 0; pos < len[a]; ++pos)
                for (int i = 0; i < half; ++i) {
                    const double ang = (double)pos * std::pow(d.rope_theta, -2.0 * i / width);
                    p.rope_cs.push_back((float)std::cos(ang));
                    p.rope_cs.push_back((float)std::sin(ang));
                }
            off += len[a] * half;
        }
        if (p.rope_cs.empty()) { p.rope_cs.push_back(1.f); p.rope_cs.push_back(0.f); }
    }
    return SVA_OK;
}

}  // namespace sva
