// api.hip -- host side of the C ABI declared in include/moe.h: argument
// validation, workspace layout, and the order of kernel launches.
#include <string.h>

#include <mutex>
#include <vector>

#include "common.h"

using namespace moe;

namespace {

thread_local hipError_t g_last_hip = hipSuccess;

int hip_fail(hipError_t e) {
    g_last_hip = e;
    return MOE_ERR_HIP;
}

// ---- stage timing -----------------------------------------------------------
struct Profiler {
    bool on = false;
    int cap = 0, used = 0;
    std::vector<hipEvent_t> ev;
    std::vector<int> stage;
} g_prof;

struct StageScope {
    hipStream_t s;
    int idx = -1;
    StageScope(int stage, hipStream_t st) : s(st) {
        if (!g_prof.on || g_prof.used >= g_prof.cap) return;
        idx = g_prof.used++;
        g_prof.stage[idx] = stage;
        (void)hipEventRecord(g_prof.ev[2 * idx], s);
    }
    ~StageScope() {
        if (idx >= 0) (void)hipEventRecord(g_prof.ev[2 * idx + 1], s);
    }
};

// The GEMMs move 16-byte chunks of every activation and weight row (rows
// are multiples of 64 elements), and the combine 16 bytes of x and h.
bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

// ---- validation ----------------------------------------------------------------
int validate(const moe_config *c) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (c->T < 1 || c->d_model < 1 || c->n_routed < 1 || c->n_routed > 1024) return MOE_ERR_INVALID_ARG;
    if (c->top_k < 1 || c->top_k > c->n_routed || c->top_k > 16) return MOE_ERR_INVALID_ARG;
    if (c->n_shared < 0 || c->n_shared > 64 || c->d_ff < 1) return MOE_ERR_INVALID_ARG;
    if (c->n_shared > 0 && c->d_ff_shared < 1) return MOE_ERR_INVALID_ARG;
    if (c->scoring < MOE_SCORE_SOFTMAX || c->scoring > MOE_ROUTE_HASH) return MOE_ERR_INVALID_ARG;
    if (c->renorm != 0 && c->renorm != 1) return MOE_ERR_INVALID_ARG;
    if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
    if (c->flags & ~(MOE_LOGITS_IN | MOE_LOGITS_OUT)) return MOE_ERR_INVALID_ARG;
    if ((c->flags & MOE_LOGITS_IN) && (c->flags & MOE_LOGITS_OUT)) return MOE_ERR_INVALID_ARG;
    if (c->scoring == MOE_ROUTE_HASH && (c->top_k != 1 || c->flags)) return MOE_ERR_INVALID_ARG;
    if (c->n_groups < 0 || c->n_groups > 64) return MOE_ERR_INVALID_ARG;
    if (c->n_groups > 0) {
        if (c->scoring == MOE_ROUTE_HASH || c->n_routed % c->n_groups) return MOE_ERR_INVALID_ARG;
        if (c->topk_groups < 1 || c->topk_groups > c->n_groups) return MOE_ERR_INVALID_ARG;
        if ((long long)c->topk_groups * (c->n_routed / c->n_groups) < c->top_k)
            return MOE_ERR_INVALID_ARG;
    } else if (c->topk_groups != 0) {
        return MOE_ERR_INVALID_ARG;
    }
    if (c->d_model % 64 || c->d_ff % 64) return MOE_ERR_UNSUPPORTED;
    if (c->n_shared > 0 && c->d_ff_shared % 64) return MOE_ERR_UNSUPPORTED;
    const long long P = (long long)c->T * c->top_k;
    if (P > (1ll << 22)) return MOE_ERR_UNSUPPORTED;
    // the expert GEMMs address rows with 32-bit element offsets
    if ((long long)c->T * c->d_model >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
    if (2ll * c->d_ff * c->d_model >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
    if (2ll * c->n_shared * c->d_ff_shared * c->d_model >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// Route workspace (learned routing): the select blocks' expert histograms,
// int32 [select_blocks][N'], then, when the router GEMM runs, its output,
// [splits][T][N'] fp32 -- the logits themselves when it does not split d
// (unless the caller asked for them in its own buffer), else one partial
// sum per split, which the select kernel adds up as it reads them.
size_t route_logits_bytes(const moe_config &c) {
    return ((size_t)c.T * c.n_routed * sizeof(float) + 255) & ~(size_t)255;
}
size_t route_hist_bytes(const moe_config &c) {
    return ((size_t)select_blocks(c) * c.n_routed * sizeof(int32_t) + 255) & ~(size_t)255;
}
size_t route_ws(const moe_config &c) {
    if (c.scoring == MOE_ROUTE_HASH) return 0;
    const size_t gemm = (c.flags & MOE_LOGITS_IN) ? 0 : route_logits_bytes(c) * router_splits(c);
    return route_hist_bytes(c) + gemm;
}

// p_partial: one row of score sums per select block, then the batch's sums.
size_t pstat_bytes(const moe_config &c) {
    if (c.scoring == MOE_ROUTE_HASH) return 0;
    return (size_t)(select_blocks(c) + 1) * c.n_routed * sizeof(double);
}

// ---- library-owned scratch of moe_forward_static -------------------------------
// For callers that cannot allocate device memory.  Each GPU the library runs
// on holds its own copy of this array until the process ends.  In host code
// the name `scratch` is only a host-side stand-in symbol, never a device
// address: host code uses the per-device address from hipGetSymbolAddress,
// taken once per device with that device current.
constexpr size_t kStaticScratchBytes = 64ull << 20;   // MOE_STATIC_SCRATCH_BYTES
static_assert(kStaticScratchBytes == (size_t)MOE_STATIC_SCRATCH_BYTES, "header and library agree");
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

// Argument checks shared by moe_forward and moe_forward_static (not the
// workspace).
int check_forward_args(const moe_config *cfg, const void *x, const int32_t *topk_idx,
                       const float *topk_w, const void *w13, const void *w2,
                       const void *w13_shared, const void *w2_shared, const void *h) {
    int rc = validate(cfg);
    if (rc) return rc;
    const moe_config &c = *cfg;
    if (!x || !topk_idx || !topk_w || !w13 || !w2 || !h) return MOE_ERR_INVALID_ARG;
    if (c.n_shared > 0 && (!w13_shared || !w2_shared)) return MOE_ERR_INVALID_ARG;
    if (h == x) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w13) || !aligned16(w2) || !aligned16(h) ||
        (c.n_shared > 0 && (!aligned16(w13_shared) || !aligned16(w2_shared))))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int forward_impl(const moe_config &c, const void *x, const int32_t *topk_idx, const float *topk_w,
                 const void *w13, const void *w2, const void *w13_shared, const void *w2_shared,
                 void *h, char *ws, hipStream_t s);

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_config *cfg, int which) {
    if (validate(cfg) != MOE_OK) return 0;
    switch (which) {
        case MOE_WS_ROUTE: return route_ws(*cfg);
        case MOE_WS_FORWARD: return fwd_layout(*cfg).total;
        case MOE_WS_PSTAT: return pstat_bytes(*cfg);
        case MOE_WS_SEQSTAT: return cfg->scoring == MOE_ROUTE_HASH ? 0 : route_logits_bytes(*cfg);
        default: return 0;
    }
}

int moe_route(const moe_config *cfg, const void *x, const void *w_gate, const float *logit_offset,
              const float *bias, const uint32_t *token_ids, float *logits, int32_t *topk_idx,
              float *topk_w, int32_t *expert_counts, void *p_partial, void *workspace,
              size_t ws_bytes, void *stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    const moe_config &c = *cfg;
    if (!topk_idx || !topk_w || !expert_counts) return MOE_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (c.scoring == MOE_ROUTE_HASH) {
        if (!token_ids || p_partial || logits) return MOE_ERR_INVALID_ARG;
        StageScope sc(MOE_STAGE_SELECT, s);
        if ((e = launch_fill_i32(expert_counts, c.n_routed, 0, s)) != hipSuccess) return hip_fail(e);
        if ((e = launch_hash_route(c, token_ids, topk_idx, topk_w, expert_counts, s)) != hipSuccess)
            return hip_fail(e);
        return MOE_OK;
    }
    if (!workspace) return MOE_ERR_INVALID_ARG;
    const float *src = logits;   // what the select kernel reads
    int splits = 1;
    float *lg_out = nullptr;     // where the select kernel writes the summed logits
    int32_t *hist_part = (int32_t *)workspace;
    if (c.flags & MOE_LOGITS_IN) {
        if (!logits) return MOE_ERR_INVALID_ARG;
        if (ws_bytes < route_ws(c)) return MOE_ERR_WORKSPACE;
    } else {
        if (!x || !w_gate) return MOE_ERR_INVALID_ARG;
        if (!aligned16(x) || !aligned16(w_gate)) return MOE_ERR_UNSUPPORTED;
        // the router GEMM addresses W_g rows with 32-bit byte offsets
        if ((long long)c.n_routed * c.d_model >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
        if (c.flags & MOE_LOGITS_OUT) {
            if (!logits) return MOE_ERR_INVALID_ARG;
        } else if (logits) {
            return MOE_ERR_INVALID_ARG;
        }
        if (ws_bytes < route_ws(c)) return MOE_ERR_WORKSPACE;
        splits = router_splits(c);
        float *gemm_out = (float *)((char *)workspace + route_hist_bytes(c));
        if (splits == 1 && (c.flags & MOE_LOGITS_OUT)) gemm_out = logits;
        else if (c.flags & MOE_LOGITS_OUT) lg_out = logits;
        src = gemm_out;
        StageScope sc(MOE_STAGE_ROUTER_GEMM, s);
        if ((e = launch_router_logits(c, x, w_gate, gemm_out, route_logits_bytes(c) / sizeof(float),
                                      s)) != hipSuccess)
            return hip_fail(e);
    }
    StageScope sc(MOE_STAGE_SELECT, s);
    if ((e = launch_select(c, src, splits, route_logits_bytes(c) / sizeof(float), lg_out,
                           logit_offset, bias, topk_idx, topk_w, expert_counts,
                           (double *)p_partial, hist_part, s)) != hipSuccess)
        return hip_fail(e);
    return MOE_OK;
}

int moe_forward(const moe_config *cfg, const void *x, const int32_t *topk_idx, const float *topk_w,
                const void *w13, const void *w2, const void *w13_shared, const void *w2_shared,
                void *h, void *workspace, size_t ws_bytes, void *stream) {
    int rc = check_forward_args(cfg, x, topk_idx, topk_w, w13, w2, w13_shared, w2_shared, h);
    if (rc) return rc;
    if (!workspace) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < fwd_layout(*cfg).total) return MOE_ERR_WORKSPACE;
    return forward_impl(*cfg, x, topk_idx, topk_w, w13, w2, w13_shared, w2_shared, h,
                        (char *)workspace, (hipStream_t)stream);
}

int moe_forward_static(const moe_config *cfg, const void *x, const int32_t *topk_idx,
                       const float *topk_w, const void *w13, const void *w2,
                       const void *w13_shared, const void *w2_shared, void *h, void *stream) {
    int rc = check_forward_args(cfg, x, topk_idx, topk_w, w13, w2, w13_shared, w2_shared, h);
    if (rc) return rc;
    if (fwd_layout(*cfg).total > kStaticScratchBytes) return MOE_ERR_UNSUPPORTED;
    void *ws = nullptr;
    if ((rc = static_scratch(&ws)) != MOE_OK) return rc;
    return forward_impl(*cfg, x, topk_idx, topk_w, w13, w2, w13_shared, w2_shared, h, (char *)ws,
                        (hipStream_t)stream);
}

}  // extern "C"

namespace {

// The launch sequence of the layer's expert part on a validated config and
// a workspace of at least fwd_layout(c).total bytes (the caller's, or the
// library-owned scratch).  The permutation clears the work counters the
// GEMMs start from, so no workspace content survives from one call into
// the next.
int forward_impl(const moe_config &c, const void *x, const int32_t *topk_idx, const float *topk_w,
                 const void *w13, const void *w2, const void *w13_shared, const void *w2_shared,
                 void *h, char *ws, hipStream_t s) {
    const FwdLayout L = fwd_layout(c);
    hipError_t e;
    {
        StageScope sc(MOE_STAGE_PERMUTE, s);
        if ((e = launch_permute(c, L, topk_idx, topk_w, ws, s)) != hipSuccess) return hip_fail(e);
    }
    const MetaIdx mi = meta_index(L.G);
    const int32_t *meta = (const int32_t *)(ws + L.off_meta);
    GroupedArgs a;
    a.T = c.T;
    a.d = c.d_model;
    a.top_k = c.top_k;
    a.n_routed = c.n_routed;
    a.n_shared = c.n_shared;
    a.f = c.d_ff;
    a.fs = c.n_shared > 0 ? c.d_ff_shared : 64;
    a.G = L.G;
    a.split_r = z_split_routed(c) ? 1 : 0;
    a.split_s = z_split_shared(c) ? 1 : 0;
    a.group_off = meta + mi.group_off;
    a.group_cnt = meta + mi.group_cnt;
    a.mt_base = meta + mi.mt;
    a.rtd = (const RowTileDesc *)(ws + L.off_rtd);
    a.nt_routed = a.nt_shared = 1;
    a.perm = (const int32_t *)(ws + L.off_perm);
    a.gsort = (const float *)(ws + L.off_gsort);
    a.x = x;
    a.w13 = w13;
    a.w2 = w2;
    a.w13s = w13_shared;
    a.w2s = w2_shared;
    a.zr = ws + L.off_zr;
    a.zs = ws + L.off_zs;
    a.yr = (float *)(ws + L.off_yr);
    a.ys = (float *)(ws + L.off_ys);
    a.yrh = (uint16_t *)(ws + L.off_yrh);
    a.ysh = (uint16_t *)(ws + L.off_ysh);
    a.shared_f16 = shared_f16(c) ? 1 : 0;
    a.zs16 = (uint16_t *)(ws + L.off_zs16);
    a.w2s16 = (const uint16_t *)(ws + L.off_w2s16);
    a.f16bad = (int32_t *)meta + mi.f16bad;
    {
        StageScope sc(MOE_STAGE_GATE_UP, s);
        a.tile_base = meta + mi.tile1;
        a.xsplit = meta + mi.xs1;
        a.queue = (int32_t *)meta + mi.q1;
        if ((e = launch_gate_up(c, a, s)) != hipSuccess) return hip_fail(e);
    }
    {
        StageScope sc(MOE_STAGE_DOWN, s);
        a.tile_base = meta + mi.tile2;
        a.xsplit = meta + mi.xs2;
        a.queue = (int32_t *)meta + mi.q2;
        if ((e = launch_down(c, a, s)) != hipSuccess) return hip_fail(e);
    }
    {
        StageScope sc(MOE_STAGE_COMBINE, s);
        if ((e = launch_combine(c, x, topk_idx, a.yr, a.ys, a.yrh, a.ysh, h, s)) != hipSuccess) return hip_fail(e);
    }
    return MOE_OK;
}


}  // namespace

extern "C" {

int moe_balance_stats(const moe_config *cfg, const int32_t *expert_counts, const void *p_partial,
                      float alpha1, float *f, float *P, float *loss, void *stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    const moe_config &c = *cfg;
    if (!expert_counts || !f) return MOE_ERR_INVALID_ARG;
    if ((P || loss) && (!p_partial || c.scoring == MOE_ROUTE_HASH)) return MOE_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    StageScope sc(MOE_STAGE_STATS, s);
    const double *p_sum =
        (P || loss) ? (const double *)p_partial + (size_t)select_blocks(c) * c.n_routed : nullptr;
    hipError_t e = launch_balance_stats(c, expert_counts, p_sum, alpha1, f, P, loss, s);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int moe_seq_balance_stats(const moe_config *cfg, const float *logits, const float *logit_offset,
                          const int32_t *topk_idx, const int32_t *seg_offsets, int32_t n_seg,
                          float beta, float *f_seq, float *p_seq, float *loss_seq,
                          void *workspace, size_t ws_bytes, void *stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    const moe_config &c = *cfg;
    if (c.scoring == MOE_ROUTE_HASH || n_seg < 1) return MOE_ERR_INVALID_ARG;
    if (!logits || !topk_idx || !seg_offsets || !f_seq || !p_seq || !loss_seq || !workspace)
        return MOE_ERR_INVALID_ARG;
    if (ws_bytes < route_logits_bytes(c)) return MOE_ERR_WORKSPACE;
    hipError_t e = launch_seq_stats(c, logits, logit_offset, topk_idx, seg_offsets, n_seg, beta,
                                    (float *)workspace, f_seq, p_seq, loss_seq,
                                    (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int moe_device_balance_stats(const moe_config *cfg, const float *f, const float *P, int32_t n_dev,
                             float alpha2, float *f_dev, float *P_dev, float *loss,
                             void *stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    const moe_config &c = *cfg;
    if (!f || !P || !f_dev || !P_dev) return MOE_ERR_INVALID_ARG;
    if (n_dev < 1 || c.n_routed % n_dev) return MOE_ERR_INVALID_ARG;
    hipError_t e = launch_device_stats(c, f, P, n_dev, alpha2, f_dev, P_dev, loss,
                                       (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int moe_bias_update(const moe_config *cfg, const int32_t *expert_counts, int64_t n_tokens,
                    float alpha, float *bias, void *stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!expert_counts || !bias || n_tokens < 1) return MOE_ERR_INVALID_ARG;
    hipError_t e = launch_bias_update(*cfg, expert_counts, n_tokens, alpha, bias,
                                      (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
}

const char *moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED:
            return "unsupported configuration (sizes must be multiples of 64, matrices 16-byte aligned)";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return hipGetErrorString(g_last_hip);
        default: return "unknown status";
    }
}

int moe_profile_enable(int max_records) {
    if (max_records < 1) return MOE_ERR_INVALID_ARG;
    if ((int)g_prof.ev.size() < 2 * max_records) {
        const size_t old = g_prof.ev.size();
        g_prof.ev.resize(2 * (size_t)max_records);
        for (size_t i = old; i < g_prof.ev.size(); ++i) {
            hipError_t e = hipEventCreate(&g_prof.ev[i]);
            if (e != hipSuccess) {
                g_prof.ev.resize(i);
                return hip_fail(e);
            }
        }
    }
    g_prof.stage.assign(max_records, 0);
    g_prof.cap = max_records;
    g_prof.used = 0;
    g_prof.on = true;
    return MOE_OK;
}

int moe_profile_collect(moe_stage_times *out) {
    if (!out) return MOE_ERR_INVALID_ARG;
    memset(out, 0, sizeof *out);
    g_prof.on = false;
    for (int i = 0; i < g_prof.used; ++i) {
        hipError_t e = hipEventSynchronize(g_prof.ev[2 * i + 1]);
        if (e != hipSuccess) return hip_fail(e);
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
        if (e != hipSuccess) return hip_fail(e);
        out->launches[g_prof.stage[i]] += 1;
        out->ms[g_prof.stage[i]] += ms;
    }
    g_prof.used = 0;
    return MOE_OK;
}

}  // extern "C"
