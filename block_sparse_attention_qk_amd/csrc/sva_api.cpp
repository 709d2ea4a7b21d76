// C ABI of the library (declared in include/sva.h): argument checks, plan
// lifetime and the launch calls.  Every check runs on the host before any
// work is enqueued; compute calls never synchronise.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "plan_dev.h"

namespace sva {

namespace {
thread_local std::string g_last_error;

int set_err(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

int hip_err(hipError_t e, const char* what) {
    return set_err(SVA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }
}  // namespace

void set_last_error(const std::string& msg) { g_last_error = msg; }

}  // namespace sva

using sva::set_err;

extern "C" {

int sva_plan_desc_init(sva_plan_desc* desc, int B, int H, int T, int Hh, int W, int d,
                       int block, double sparsity, unsigned flags) {
    if (!desc) return set_err(SVA_ERR_INVALID_ARG, "desc is NULL");
    std::memset(desc, 0, sizeof(*desc));
    desc->B = B;
    desc->H = H;
    desc->T = T;
    desc->Hh = Hh;
    desc->W = W;
    desc->d = d;
    desc->block = block;
    desc->sparsity = sparsity;
    desc->flags = flags;
    return SVA_OK;
}

int sva_plan_query(const sva_plan_desc* desc, sva_plan_info* info) {
    if (!desc || !info) return set_err(SVA_ERR_INVALID_ARG, "desc or info is NULL");
    sva::HostPlan hp;
    std::string err;
    const int rc = sva::build_host_plan(*desc, hp, err, false);
    if (rc != SVA_OK) return set_err(rc, err);
    *info = hp.info;
    return SVA_OK;
}

int sva_plan_host_tables(const sva_plan_desc* desc, int32_t* perm, int32_t* row_ptr,
                         uint8_t* forced) {
    if (!desc) return set_err(SVA_ERR_INVALID_ARG, "desc is NULL");
    sva::HostPlan hp;
    std::string err;
    const int rc = sva::build_host_plan(*desc, hp, err, false);
    if (rc != SVA_OK) return set_err(rc, err);
    if (perm) std::memcpy(perm, hp.perm.data(), hp.perm.size() * sizeof(int32_t));
    if (row_ptr) std::memcpy(row_ptr, hp.row_ptr.data(), hp.row_ptr.size() * sizeof(int32_t));
    if (forced) {
        const int nB = hp.info.nB;
        for (int qb = 0; qb < nB; ++qb) {
            const bool dense_row = hp.info.dense || qb >= hp.info.nB_video;
            for (int kb = 0; kb < nB; ++kb)
                forced[(size_t)qb * nB + kb] =
                    (dense_row || sva::forced_pair(hp, qb, kb)) ? 1 : 0;
        }
    }
    return SVA_OK;
}

int sva_plan_create_ex(sva_plan* out, const sva_plan_desc* desc) {
    if (!out || !desc) return set_err(SVA_ERR_INVALID_ARG, "out or desc is NULL");
    *out = nullptr;
    sva_plan_s* plan = new (std::nothrow) sva_plan_s();
    if (!plan) return set_err(SVA_ERR_HIP, "out of host memory");
    std::string err;
    int rc = sva::build_host_plan(*desc, plan->host, err, true);
    if (rc != SVA_OK) {
        delete plan;
        return set_err(rc, err);
    }
    const sva::HostPlan& h = plan->host;
    hipError_t e = hipGetDevice(&plan->device);
    if (e != hipSuccess) {
        delete plan;
        return sva::hip_err(e, "hipGetDevice");
    }
    // set-up of this device for sva_select_blocks_noalloc
    e = sva::resolve_select_scratch(plan->device);
    if (e != hipSuccess) {
        delete plan;
        return sva::hip_err(e, "hipGetSymbolAddress(select scratch)");
    }
    // one device buffer: perm, inv, valid, tmin, tmax, row_ptr, rope table
    auto align = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t s_perm = align(h.perm.size() * 4), s_inv = align(h.inv.size() * 4);
    const size_t s_blk = align(h.blk_valid.size() * 4), s_rp = align(h.row_ptr.size() * 4);
    const size_t s_rope = align(h.rope_cs.size() * 4);
    const size_t s_items = align(h.items.size() * 4), s_split = align(h.split_rows.size() * 4);
#ifdef SVA_DEBUG
    const size_t s_dbg = 256;   // the debug word
#else
    const size_t s_dbg = 0;
#endif
    const size_t total = s_perm + s_inv + 3 * s_blk + s_rp + s_rope + s_items + s_split + s_dbg;
    e = hipMalloc(&plan->dmem, total);
    if (e != hipSuccess) {
        delete plan;
        return sva::hip_err(e, "hipMalloc(plan tables)");
    }
    char* base = static_cast<char*>(plan->dmem);
    size_t off = 0;
    auto put = [&](const void* src, size_t bytes, size_t slot) -> void* {
        void* dst = base + off;
        off += slot;
        if (bytes && e == hipSuccess) e = hipMemcpy(dst, src, bytes, hipMemcpyHostToDevice);
        return dst;
    };
    sva::DevPlan& d = plan->dev;
    d.perm = static_cast<const int32_t*>(put(h.perm.data(), h.perm.size() * 4, s_perm));
    d.inv = static_cast<const int32_t*>(put(h.inv.data(), h.inv.size() * 4, s_inv));
    d.blk_valid = static_cast<const int32_t*>(put(h.blk_valid.data(), h.blk_valid.size() * 4, s_blk));
    d.blk_tmin = static_cast<const int32_t*>(put(h.blk_tmin.data(), h.blk_tmin.size() * 4, s_blk));
    d.blk_tmax = static_cast<const int32_t*>(put(h.blk_tmax.data(), h.blk_tmax.size() * 4, s_blk));
    d.row_ptr = static_cast<const int32_t*>(put(h.row_ptr.data(), h.row_ptr.size() * 4, s_rp));
    d.rope_cs = static_cast<const float2*>(put(h.rope_cs.data(), h.rope_cs.size() * 4, s_rope));
    d.items = static_cast<const int32_t*>(put(h.items.data(), h.items.size() * 4, s_items));
    d.split_rows = static_cast<const int32_t*>(put(h.split_rows.data(), h.split_rows.size() * 4, s_split));
#ifdef SVA_DEBUG
    d.dbg = static_cast<uint32_t*>(static_cast<void*>(base + off));
    off += s_dbg;
    if (e == hipSuccess) e = hipMemset(d.dbg, 0, sizeof(uint32_t));
#endif
    d.n_items = (int)(h.items.size() / 4);
    d.n_split = (int)(h.split_rows.size() / 3);
    d.n_slots = h.n_slots;
    if (e != hipSuccess) {
        (void)hipFree(plan->dmem);   // the copy error is the one reported
        delete plan;
        return sva::hip_err(e, "hipMemcpy(plan tables)");
    }
    const sva_plan_desc& ds = h.desc;
    const sva_plan_info& I = h.info;
    d.B = ds.B; d.H = ds.H; d.d = ds.d; d.block = ds.block;
    d.T = ds.T; d.Hh = ds.Hh; d.W = ds.W;
    d.n_video = I.n_video; d.N = I.N; d.n_video_pad = I.n_video_pad; d.Np = I.Np;
    d.nB = I.nB; d.nB_video = I.nB_video; d.k = I.k;
    d.dense = I.dense;
    d.same_frame = (ds.flags & SVA_KEEP_SAME_FRAME) ? 1 : 0;
    d.scorer = I.scorer;
    d.nsub = I.subblocks;
    d.n_mean_groups = I.n_mean_groups;
    d.eps = (float)ds.eps;
    for (int a = 0; a < 3; ++a) {
        d.rope_off[a] = h.rope_off[a];
        d.rope_half[a] = h.rope_half[a];
    }
    d.nnz_per_head = I.nnz_per_head;
    d.max_row_len = I.max_row_len;
    d.div_H = sva::make_fastdiv((uint32_t)ds.H);
    d.div_N = sva::make_fastdiv((uint32_t)I.N);
    d.div_HW = sva::make_fastdiv((uint32_t)(ds.Hh * ds.W));
    d.div_W = sva::make_fastdiv((uint32_t)ds.W);
    d.div_Np = sva::make_fastdiv((uint32_t)I.Np);
    *out = plan;
    return SVA_OK;
}

int sva_plan_create(sva_plan* out, int B, int H, int T, int Hh, int W, int d, int block,
                    double sparsity, unsigned dense_flag) {
    sva_plan_desc desc;
    sva_plan_desc_init(&desc, B, H, T, Hh, W, d, block, sparsity, dense_flag);
    return sva_plan_create_ex(out, &desc);
}

int sva_plan_get_info(sva_plan plan, sva_plan_info* info) {
    if (!plan || !info) return set_err(SVA_ERR_INVALID_ARG, "plan or info is NULL");
    *info = plan->host.info;
    return SVA_OK;
}

int sva_destroy(sva_plan plan) {
    if (!plan) return SVA_OK;
    hipError_t e = hipSuccess;
    if (plan->dmem) e = hipFree(plan->dmem);
    delete plan;
    if (e != hipSuccess) return sva::hip_err(e, "hipFree(plan tables)");
    return SVA_OK;
}

int sva_qk_norm_rope(sva_plan plan, const void* q, const void* k, const float* wq,
                     const float* wk, void* q_out, void* k_out, void* stream) {
    if (!plan) return set_err(SVA_ERR_INVALID_ARG, "plan is NULL");
    if (!q || !k || !q_out || !k_out)
        return set_err(SVA_ERR_INVALID_ARG, "q, k, q_out and k_out must be non-NULL");
    if (!sva::aligned16(q) || !sva::aligned16(k) || !sva::aligned16(q_out) ||
        !sva::aligned16(k_out) || !sva::aligned16(wq) || !sva::aligned16(wk))
        return set_err(SVA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    hipError_t e = sva::launch_prologue(plan->dev, static_cast<const uint16_t*>(q),
                                        static_cast<const uint16_t*>(k), wq, wk,
                                        static_cast<uint16_t*>(q_out),
                                        static_cast<uint16_t*>(k_out), false, nullptr,
                                        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return sva::hip_err(e, "qk_norm_rope launch");
    return SVA_OK;
}

int sva_qk_norm_rope_tiled(sva_plan plan, const void* q, const void* k, const float* wq,
                           const float* wk, void* q_r, void* k_t, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (!plan) return set_err(SVA_ERR_INVALID_ARG, "plan is NULL");
    if (!q || !k || !q_r || !k_t)
        return set_err(SVA_ERR_INVALID_ARG, "q, k, q_r and k_t must be non-NULL");
    if (!sva::aligned16(q) || !sva::aligned16(k) || !sva::aligned16(q_r) ||
        !sva::aligned16(k_t) || !sva::aligned16(wq) || !sva::aligned16(wk) ||
        !sva::aligned16(workspace))
        return set_err(SVA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    if (q_r == q || q_r == k || k_t == q || k_t == k)
        return set_err(SVA_ERR_INVALID_ARG, "outputs must not alias the inputs");
    double* means = nullptr;
    if (workspace && !plan->host.info.dense) {
        if (workspace_bytes < plan->host.info.select_workspace_bytes)
            return set_err(SVA_ERR_WORKSPACE, "workspace smaller than select_workspace_bytes");
        means = static_cast<double*>(workspace);
    }
    hipError_t e = sva::launch_prologue(plan->dev, static_cast<const uint16_t*>(q),
                                        static_cast<const uint16_t*>(k), wq, wk,
                                        static_cast<uint16_t*>(q_r),
                                        static_cast<uint16_t*>(k_t), true, means,
                                        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return sva::hip_err(e, "qk_norm_rope_tiled launch");
    return SVA_OK;
}

int sva_reorder(sva_plan plan, const void* in, void* out, int direction, void* stream) {
    if (!plan) return set_err(SVA_ERR_INVALID_ARG, "plan is NULL");
    if (!in || !out) return set_err(SVA_ERR_INVALID_ARG, "in and out must be non-NULL");
    if (!sva::aligned16(in) || !sva::aligned16(out))
        return set_err(SVA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    if (direction != SVA_FORWARD && direction != SVA_INVERSE && direction != SVA_FORWARD_VT &&
        direction != SVA_FORWARD_KT && direction != SVA_ROWS_TO_VT && direction != SVA_ROWS_TO_KT)
        return set_err(SVA_ERR_INVALID_ARG, "unknown reorder direction");
    if (in == out) return set_err(SVA_ERR_INVALID_ARG, "reorder cannot run in place");
    hipError_t e = sva::launch_reorder(plan->dev, static_cast<const uint16_t*>(in),
                                       static_cast<uint16_t*>(out), direction,
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return sva::hip_err(e, "reorder launch");
    return SVA_OK;
}

int sva_select_blocks(sva_plan plan, const void* q_r, const void* k_t, void* workspace,
                      size_t workspace_bytes, int32_t* col, void* stream) {
    if (!plan) return set_err(SVA_ERR_INVALID_ARG, "plan is NULL");
    if (plan->host.info.dense) return SVA_OK;
    if (!col || !workspace)
        return set_err(SVA_ERR_INVALID_ARG, "workspace and col must be non-NULL");
    if ((q_r == nullptr) != (k_t == nullptr))
        return set_err(SVA_ERR_INVALID_ARG,
                       "q_r and k_t must both be given, or both be NULL (means in the workspace)");
    if (!sva::aligned16(q_r) || !sva::aligned16(k_t) || !sva::aligned16(workspace) ||
        ((uintptr_t)col & 3u))
        return set_err(SVA_ERR_INVALID_ARG, "misaligned pointer");
    if (workspace_bytes < plan->host.info.select_workspace_bytes)
        return set_err(SVA_ERR_WORKSPACE, "workspace smaller than select_workspace_bytes");
    hipError_t e = sva::launch_select(plan->dev, static_cast<const uint16_t*>(q_r),
                                      static_cast<const uint16_t*>(k_t),
                                      static_cast<double*>(workspace), col,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return sva::hip_err(e, "select launch");
    return SVA_OK;
}

int sva_attention_ws(sva_plan plan, const void* q_r, const void* k_t, const void* v_t,
                     const int32_t* col, const void* km_t, const void* vm_t, void* o,
                     int o_layout, void* workspace, size_t workspace_bytes, void* stream) {
    if (!plan) return set_err(SVA_ERR_INVALID_ARG, "plan is NULL");
    if (!q_r || !k_t || !v_t || !o)
        return set_err(SVA_ERR_INVALID_ARG, "q_r, k_t, v_t and the output must be non-NULL");
    if ((km_t == nullptr) != (vm_t == nullptr))
        return set_err(SVA_ERR_INVALID_ARG, "km_t and vm_t must both be given or both be NULL");
    if (o_layout != SVA_LAYOUT_TILE && o_layout != SVA_LAYOUT_RASTER)
        return set_err(SVA_ERR_INVALID_ARG, "unknown output layout");
    if (!plan->host.info.dense && !col)
        return set_err(SVA_ERR_INVALID_ARG, "col must be non-NULL for a sparse plan");
    if (!sva::aligned16(q_r) || !sva::aligned16(k_t) || !sva::aligned16(v_t) ||
        !sva::aligned16(o) || !sva::aligned16(km_t) || !sva::aligned16(vm_t) ||
        ((uintptr_t)col & 3u) || !sva::aligned16(workspace))
        return set_err(SVA_ERR_INVALID_ARG, "misaligned pointer");
    float* part = nullptr;
    if (workspace && plan->host.info.attention_workspace_bytes > 0) {
        if (workspace_bytes < plan->host.info.attention_workspace_bytes)
            return set_err(SVA_ERR_WORKSPACE, "workspace smaller than attention_workspace_bytes");
        part = static_cast<float*>(workspace);
    }
    hipError_t e = sva::launch_attention(plan->dev, static_cast<const uint16_t*>(q_r),
                                         static_cast<const uint16_t*>(k_t),
                                         static_cast<const uint16_t*>(v_t), col,
                                         static_cast<const uint16_t*>(km_t),
                                         static_cast<const uint16_t*>(vm_t),
                                         static_cast<uint16_t*>(o),
                                         o_layout == SVA_LAYOUT_RASTER, part,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return sva::hip_err(e, "attention launch");
    return SVA_OK;
}

int sva_attention_ex(sva_plan plan, const void* q_r, const void* k_t, const void* v_t,
                     const int32_t* col, const void* km_t, const void* vm_t, void* o,
                     int o_layout, void* stream) {
    return sva_attention_ws(plan, q_r, k_t, v_t, col, km_t, vm_t, o, o_layout, nullptr, 0,
                            stream);
}

int sva_attention(sva_plan plan, const void* q_r, const void* k_t, const void* v_t,
                  const int32_t* col, void* o_r, void* stream) {
    return sva_attention_ex(plan, q_r, k_t, v_t, col, nullptr, nullptr, o_r, SVA_LAYOUT_TILE,
                            stream);
}

int sva_block_means(sva_plan plan, const void* k_t, const void* v_t, void* km_t, void* vm_t,
                    void* stream) {
    if (!plan) return set_err(SVA_ERR_INVALID_ARG, "plan is NULL");
    if (!k_t || !v_t || !km_t || !vm_t)
        return set_err(SVA_ERR_INVALID_ARG, "k_t, v_t, km_t and vm_t must be non-NULL");
    if (!sva::aligned16(k_t) || !sva::aligned16(v_t) || !sva::aligned16(km_t) ||
        !sva::aligned16(vm_t))
        return set_err(SVA_ERR_INVALID_ARG, "misaligned pointer");
    hipError_t e = sva::launch_block_means(plan->dev, static_cast<const uint16_t*>(k_t),
                                           static_cast<const uint16_t*>(v_t),
                                           static_cast<uint16_t*>(km_t),
                                           static_cast<uint16_t*>(vm_t),
                                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return sva::hip_err(e, "block means launch");
    return SVA_OK;
}

int sva_attention_compensated(sva_plan plan, const void* q_r, const void* k_t,
                              const void* v_t, const int32_t* col, const void* km_t,
                              const void* vm_t, void* o_r, void* stream) {
    if (!km_t || !vm_t) return set_err(SVA_ERR_INVALID_ARG, "km_t and vm_t must be non-NULL");
    return sva_attention_ex(plan, q_r, k_t, v_t, col, km_t, vm_t, o_r, SVA_LAYOUT_TILE, stream);
}

int sva_forward(sva_plan plan, const sva_step_buffers* b, void* const* marks, void* stream) {
    using sva::aligned16;
    if (!plan || !b) return set_err(SVA_ERR_INVALID_ARG, "plan or buffers is NULL");
    const sva_plan_info& I = plan->host.info;
    const bool sparse = !I.dense;
    const bool comp = sparse && (plan->host.desc.flags & SVA_COMPENSATE);
    // every check of the calls below, before anything is enqueued
    if (!b->q || !b->k || !b->v || !b->q_r || !b->k_t || !b->v_t || !b->o)
        return set_err(SVA_ERR_INVALID_ARG, "q, k, v, q_r, k_t, v_t and o must be non-NULL");
    if (!aligned16(b->q) || !aligned16(b->k) || !aligned16(b->v) || !aligned16(b->wq) ||
        !aligned16(b->wk) || !aligned16(b->q_r) || !aligned16(b->k_t) || !aligned16(b->v_t) ||
        !aligned16(b->o) || !aligned16(b->select_ws) || !aligned16(b->attn_ws) ||
        ((uintptr_t)b->col & 3u) || (comp && (!aligned16(b->km_t) || !aligned16(b->vm_t))))
        return set_err(SVA_ERR_INVALID_ARG, "misaligned pointer");
    if (b->q_r == b->q || b->q_r == b->k || b->k_t == b->q || b->k_t == b->k || b->v_t == b->v)
        return set_err(SVA_ERR_INVALID_ARG, "outputs must not alias the inputs");
    if (sparse) {
        if (!b->col || !b->select_ws)
            return set_err(SVA_ERR_INVALID_ARG, "a sparse plan needs col and select_ws");
        if (b->select_ws_bytes < I.select_workspace_bytes)
            return set_err(SVA_ERR_WORKSPACE, "select_ws smaller than select_workspace_bytes");
    }
    if (comp && (!b->km_t || !b->vm_t))
        return set_err(SVA_ERR_INVALID_ARG, "a compensated plan needs km_t and vm_t");
    if (b->attn_ws && I.attention_workspace_bytes > 0 &&
        b->attn_ws_bytes < I.attention_workspace_bytes)
        return set_err(SVA_ERR_WORKSPACE, "attn_ws smaller than attention_workspace_bytes");
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto mark = [&](int i) -> hipError_t {
        return (marks && marks[i]) ? hipEventRecord(static_cast<hipEvent_t>(marks[i]), s)
                                   : hipSuccess;
    };
    hipError_t e = hipSuccess;
    int rc = SVA_OK;
#define SVA_MARK(I_)                                                           \
    do {                                                                       \
        if ((e = mark(I_)) != hipSuccess) return sva::hip_err(e, "hipEventRecord(mark)"); \
    } while (0)
#define SVA_CALL(X_)                                                           \
    do {                                                                       \
        if ((rc = (X_)) != SVA_OK) return rc;                                  \
    } while (0)
    SVA_MARK(0);
    SVA_CALL(sva_qk_norm_rope_tiled(plan, b->q, b->k, b->wq, b->wk, b->q_r, b->k_t,
                                    sparse ? b->select_ws : nullptr, b->select_ws_bytes, stream));
    SVA_MARK(1);
    SVA_CALL(sva_reorder(plan, b->v, b->v_t, SVA_FORWARD_VT, stream));
    SVA_MARK(2);
    if (sparse)
        SVA_CALL(sva_select_blocks(plan, nullptr, nullptr, b->select_ws, b->select_ws_bytes,
                                   b->col, stream));
    SVA_MARK(3);
    if (comp) SVA_CALL(sva_block_means(plan, b->k_t, b->v_t, b->km_t, b->vm_t, stream));
    SVA_MARK(4);
    SVA_CALL(sva_attention_ws(plan, b->q_r, b->k_t, b->v_t, sparse ? b->col : nullptr,
                              comp ? b->km_t : nullptr, comp ? b->vm_t : nullptr, b->o,
                              SVA_LAYOUT_RASTER, b->attn_ws, b->attn_ws_bytes, stream));
    SVA_MARK(5);
#undef SVA_CALL
#undef SVA_MARK
    return SVA_OK;
}

int sva_debug_flags(sva_plan plan, unsigned* flags) {
    if (!plan || !flags) return set_err(SVA_ERR_INVALID_ARG, "plan or flags is NULL");
    *flags = 0u;
#ifdef SVA_DEBUG
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return sva::hip_err(e, "hipDeviceSynchronize");
    uint32_t w = 0;
    e = hipMemcpy(&w, plan->dev.dbg, sizeof w, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return sva::hip_err(e, "hipMemcpy(debug word)");
    e = hipMemset(plan->dev.dbg, 0, sizeof w);
    if (e != hipSuccess) return sva::hip_err(e, "hipMemset(debug word)");
    *flags = w;
    return SVA_OK;
#else
    return set_err(SVA_ERR_UNSUPPORTED, "release build: the kernels carry no debug checks");
#endif
}

int sva_debug_selftest(sva_plan plan, void* stream) {
    if (!plan) return set_err(SVA_ERR_INVALID_ARG, "plan is NULL");
#ifdef SVA_DEBUG
    hipError_t e = sva::launch_debug_selftest(plan->dev, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return sva::hip_err(e, "debug selftest launch");
    return SVA_OK;
#else
    (void)stream;
    return set_err(SVA_ERR_UNSUPPORTED, "release build: the kernels carry no debug checks");
#endif
}

const char* sva_status_string(int status) {
    switch (status) {
        case SVA_OK: return "ok";
        case SVA_ERR_INVALID_ARG: return "invalid argument";
        case SVA_ERR_UNSUPPORTED: return "unsupported shape";
        case SVA_ERR_WORKSPACE: return "workspace too small";
        case SVA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* sva_last_error(void) { return sva::g_last_error.c_str(); }

}  // extern "C"
