// The host planner under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// tests/test_host_asan.py compiles this file together with
// block_sparse_attention_qk_amd/csrc/plan_host.cpp (pure C++, no HIP) using
// g++ -fsanitize=address,undefined and runs it.  It builds plans for a seeded
// spread of descriptors, among them the video shapes the library is measured
// on, checks the structural invariants of every plan it accepts, and checks
// that each class of invalid descriptor is refused with its error code.
// Prints "ok <accepted> <refused>" and exits 0 when every check holds; a
// sanitizer report ends the process with a non-zero status.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "../block_sparse_attention_qk_amd/csrc/plan_host.h"

namespace sva {
void set_last_error(const std::string&) {}
}  // namespace sva

namespace {

int g_failures = 0;

#define CHECK(c)                                                                  \
    do {                                                                          \
        if (!(c)) {                                                               \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);  \
            ++g_failures;                                                         \
            return false;                                                         \
        }                                                                         \
    } while (0)

// 64-bit linear congruential generator (Knuth's MMIX constants); the top
// bits are used.
struct Lcg {
    uint64_t s;
    uint32_t next() {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        return (uint32_t)(s >> 33);
    }
    int in(int lo, int hi) { return lo + (int)(next() % (uint32_t)(hi - lo + 1)); }
};

sva_plan_desc make(int B, int H, int T, int Hh, int W, int d, int block, double sparsity,
                   unsigned flags) {
    sva_plan_desc desc{};
    desc.B = B; desc.H = H; desc.T = T; desc.Hh = Hh; desc.W = W;
    desc.d = d; desc.block = block; desc.sparsity = sparsity; desc.flags = flags;
    return desc;
}

// Invariants of an accepted plan that hold for every descriptor.
bool check_plan(const sva_plan_desc& in, const sva::HostPlan& p) {
    const sva_plan_desc& d = p.desc;
    const sva_plan_info& I = p.info;
    const int64_t nB = I.nB;
    CHECK(d.B == in.B && d.H == in.H && d.d == in.d && d.block == in.block);
    CHECK(I.n_video == (int64_t)d.T * d.Hh * d.W);
    CHECK(I.N == I.n_video + d.n_extra);
    CHECK(I.n_video_pad % d.block == 0 && I.n_video_pad >= I.n_video &&
          I.n_video_pad - I.n_video < d.block);
    CHECK(I.Np == I.n_video_pad + d.n_extra && I.Np == nB * d.block);

    // permutation: a bijection from raster tokens onto the non-padding rows
    CHECK((int64_t)p.perm.size() == I.N && (int64_t)p.inv.size() == I.Np);
    for (int64_t n = 0; n < I.N; ++n) {
        const int64_t pos = p.perm[n];
        CHECK(pos >= 0 && pos < I.Np);
        CHECK(p.inv[pos] == n);
        CHECK((n < I.n_video) == (pos < I.n_video));
    }
    int64_t pads = 0;
    for (int64_t pos = 0; pos < I.Np; ++pos) pads += p.inv[pos] < 0 ? 1 : 0;
    CHECK(pads == I.n_video_pad - I.n_video);

    // block metadata
    CHECK((int64_t)p.blk_valid.size() == nB);
    int64_t valid = 0;
    for (int64_t b = 0; b < nB; ++b) {
        CHECK(p.blk_valid[b] >= 1 && p.blk_valid[b] <= d.block);
        CHECK(b >= I.nB_video || (p.blk_tmin[b] <= p.blk_tmax[b] && p.blk_tmax[b] < d.T));
        valid += p.blk_valid[b];
    }
    CHECK(valid == I.N);

    // budget and row offsets
    CHECK(I.k >= 1 && I.k <= nB);
    CHECK(I.budget_multiple >= 1);
    CHECK(I.dense || I.k == nB || I.k % I.budget_multiple == 0);
    CHECK((int64_t)p.row_ptr.size() == nB + 1 && p.row_ptr[0] == 0);
    int32_t longest = 0;
    for (int64_t qb = 0; qb < nB; ++qb) {
        const int32_t len = p.row_ptr[qb + 1] - p.row_ptr[qb];
        CHECK(len >= I.k && len <= nB);
        CHECK(!(I.dense || qb >= I.nB_video) || len == nB);
        longest = len > longest ? len : longest;
    }
    CHECK(longest == I.max_row_len);
    CHECK(p.row_ptr[nB] == I.nnz_per_head && I.nnz == I.nnz_per_head * d.B * d.H);
    CHECK(I.dense || I.select_workspace_bytes ==
                         (size_t)2 * d.B * d.H * nB * I.subblocks * d.d * sizeof(double));

    // split rows: the pieces of every row cover its list once, in order
    if (p.n_slots > 0) {
        CHECK(p.items.size() % 4 == 0 && p.split_rows.size() % 3 == 0);
        std::vector<int32_t> covered(nB, 0);
        std::vector<char> slot_used(p.n_slots, 0);
        for (size_t i = 0; i < p.items.size(); i += 4) {
            const int32_t qb = p.items[i], e0 = p.items[i + 1], e1 = p.items[i + 2],
                          slot = p.items[i + 3];
            CHECK(qb >= 0 && qb < nB);
            CHECK(e0 == covered[qb] && e1 > e0);
            CHECK(e1 <= p.row_ptr[qb + 1] - p.row_ptr[qb]);
            covered[qb] = e1;
            if (slot >= 0) {
                CHECK(slot < p.n_slots && !slot_used[slot]);
                slot_used[slot] = 1;
            }
        }
        for (int64_t qb = 0; qb < nB; ++qb)
            CHECK(covered[qb] == p.row_ptr[qb + 1] - p.row_ptr[qb]);
        for (int32_t s = 0; s < p.n_slots; ++s) CHECK(slot_used[s]);
        CHECK(I.attention_workspace_bytes ==
              (size_t)d.B * d.H * p.n_slots * d.block * (d.d + 2) * sizeof(float));
    } else {
        CHECK(p.items.empty() && I.attention_workspace_bytes == 0);
    }

    // RoPE tables: one (cos, sin) pair per position and pair of each section
    const int len[3] = {d.T, d.Hh, d.W};
    size_t pairs = 0;
    for (int a = 0; a < 3; ++a) {
        CHECK(p.rope_half[a] * 2 == d.rope_split[a]);
        CHECK(p.rope_off[a] == (int32_t)pairs);
        pairs += (size_t)len[a] * p.rope_half[a];
    }
    CHECK(p.rope_cs.size() == 2 * (pairs > 0 ? pairs : 1));
    for (size_t i = 0; i < p.rope_cs.size(); i += 2) {
        const double c = p.rope_cs[i], s = p.rope_cs[i + 1];
        CHECK(std::fabs(c * c + s * s - 1.0) < 1e-6);
    }
    return true;
}

bool accept(const sva_plan_desc& desc) {
    sva::HostPlan p;
    std::string err;
    const int rc = sva::build_host_plan(desc, p, err, true);
    if (rc != SVA_OK) {
        std::fprintf(stderr, "refused a valid descriptor: %s\n", err.c_str());
        ++g_failures;
        return false;
    }
    return check_plan(desc, p);
}

bool refuse(const sva_plan_desc& desc, int code) {
    sva::HostPlan p;
    std::string err;
    const int rc = sva::build_host_plan(desc, p, err, true);
    CHECK(rc == code);
    CHECK(!err.empty());
    return true;
}

}  // namespace

int main() {
    int accepted = 0, refused = 0;

    // the measured video shapes: 480p and 720p latents, HunyuanVideo 720p,
    // the packed video + audio sequence and the 4096-block size limit
    const sva_plan_desc shapes[] = {
        make(1, 12, 21, 30, 52, 128, 64, 0.75, SVA_KEEP_SAME_FRAME),
        make(1, 40, 21, 45, 80, 128, 128, 0.75, SVA_KEEP_SAME_FRAME),
        make(1, 24, 33, 45, 80, 128, 128, 0.8, 0u),
        make(1, 2, 16, 128, 128, 64, 64, 0.9, 0u),
    };
    for (const auto& s : shapes) accepted += accept(s) ? 1 : 0;
    {
        sva_plan_desc s = make(1, 48, 20, 48, 80, 128, 128, 0.8, SVA_KEEP_SAME_FRAME);
        s.n_extra = 256;
        accepted += accept(s) ? 1 : 0;
        s = make(1, 1, 1, 1, 1, 64, 64, 0.5, 0u);   // one token
        accepted += accept(s) ? 1 : 0;
    }

    // a seeded spread over every option
    Lcg rng{20251};
    for (int it = 0; it < 400; ++it) {
        const int d = rng.in(0, 1) ? 128 : 64;
        const int block = rng.in(0, 1) ? 128 : 64;
        const double sparsities[] = {0.0, 0.3, 0.5, 0.75, 0.9, 0.99};
        sva_plan_desc s = make(rng.in(1, 2), rng.in(1, 3), rng.in(1, 12), rng.in(1, 40),
                               rng.in(1, 60), d, block, sparsities[rng.in(0, 5)], 0u);
        if (rng.in(0, 6) == 0) s.flags |= SVA_DENSE;
        if (rng.in(0, 1)) s.flags |= SVA_KEEP_SAME_FRAME;
        if (rng.in(0, 3) == 0) s.flags |= SVA_COMPENSATE;
        if (rng.in(0, 2) == 0) {
            s.tile_t = rng.in(1, 5); s.tile_h = rng.in(1, 9); s.tile_w = rng.in(1, 17);
        }
        s.n_extra = block * rng.in(0, 2) * (rng.in(0, 2) == 0 ? 1 : 0);
        if (rng.in(0, 3) == 0) {
            const int a = 2 * rng.in(0, d / 8), b = 2 * rng.in(0, d / 8), c = 2 * rng.in(0, d / 8);
            s.rope_split[0] = a; s.rope_split[1] = b; s.rope_split[2] = c;
        }
        if (rng.in(0, 2) == 0) {
            s.scorer = SVA_SCORER_SUBBLOCK;
            const int subs[] = {0, 1, 2, 4};
            s.subblocks = subs[rng.in(0, 3)];
            s.budget_multiple = rng.in(0, 1) ? 8 : 0;
        }
        if (rng.in(0, 4) == 0) s.rope_theta = 500.0 + rng.in(0, 100000);
        accepted += accept(s) ? 1 : 0;
    }

    // every class of invalid descriptor
    const sva_plan_desc ok = make(1, 2, 4, 8, 8, 64, 64, 0.5, 0u);
    struct Bad {
        sva_plan_desc desc;
        int code;
    };
    std::vector<Bad> bad;
    auto with = [&](auto edit, int code) {
        sva_plan_desc s = ok;
        edit(s);
        bad.push_back({s, code});
    };
    with([](sva_plan_desc& s) { s.B = 0; }, SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.H = -1; }, SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.W = 0; }, SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.d = 96; }, SVA_ERR_UNSUPPORTED);
    with([](sva_plan_desc& s) { s.block = 32; }, SVA_ERR_UNSUPPORTED);
    with([](sva_plan_desc& s) { s.sparsity = 1.0; }, SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.sparsity = -0.1; }, SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.sparsity = std::nan(""); }, SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.flags = 1u << 7; }, SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.tile_t = 0; s.tile_h = 4; s.tile_w = 4; }, SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.n_extra = 32; }, SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.n_extra = -64; }, SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.rope_theta = 0.5; }, SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.rope_theta = INFINITY; }, SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.rope_split[0] = 3; }, SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.rope_split[0] = 32; s.rope_split[1] = 32; s.rope_split[2] = 2; },
         SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.scorer = 2; }, SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.subblocks = 2; }, SVA_ERR_INVALID_ARG);   // mean scorer
    with([](sva_plan_desc& s) { s.scorer = SVA_SCORER_SUBBLOCK; s.subblocks = 3; },
         SVA_ERR_UNSUPPORTED);
    with([](sva_plan_desc& s) { s.budget_multiple = -8; }, SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.eps = -1e-6; }, SVA_ERR_INVALID_ARG);
    with([](sva_plan_desc& s) { s.T = 64; s.Hh = 128; s.W = 128; }, SVA_ERR_INVALID_ARG);  // > 4096 blocks
    with([](sva_plan_desc& s) { s.B = 8; s.H = 1024; s.T = 16; s.Hh = 128; s.W = 128; },
         SVA_ERR_INVALID_ARG);   // 2^31 rows
    for (const auto& b : bad) refused += refuse(b.desc, b.code) ? 1 : 0;

    if (g_failures) {
        std::fprintf(stderr, "%d check(s) failed\n", g_failures);
        return 1;
    }
    std::printf("ok %d %d\n", accepted, refused);
    return 0;
}
