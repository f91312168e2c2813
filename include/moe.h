/*
 * moe.h -- C ABI of libmoe.so, an MI355X (gfx950) DeepSeekMoE layer forward.
 *
 * The layer ("core design 2" equation of the DeepSeekMoE reading notes,
 * heloowird.com):
 *
 *   h_t = u_t + sum_{j < K_s} FFN^shared_j(u_t) + sum_{i < N'} g_{i,t} FFN_i(u_t)
 *
 * where g_{i,t} is non-zero only for the K' routed experts whose selection
 * score is among the K' largest ("core design 1", top-k gate equation).
 * Every FFN is SwiGLU without biases, W2 (SiLU(W1 u) * (W3 u)), the 3-matrix
 * form the MoE tutorial at ai.clawlihai.cn names as the one real models use.
 *
 * Conventions shared by every entry point
 *  - Every array pointer is a DEVICE pointer owned by the caller unless the
 *    comment says otherwise.  The library never allocates or frees device
 *    memory: scratch lives in a caller-provided workspace of at least
 *    moe_workspace_bytes(cfg, which) bytes, 256-byte aligned.
 *  - Row-major layouts; "bf16" means IEEE bfloat16 bit patterns.  The
 *    activation, weight and output matrices (x, w_gate, w13, w2, the shared
 *    weights, h) must be 16-byte aligned (MOE_ERR_UNSUPPORTED otherwise);
 *    allocator-returned buffers are.
 *  - All work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *    void*; NULL is the default stream).  Results are valid once the caller
 *    has synchronised that stream.
 *  - Arguments are validated on the host, synchronously, before anything is
 *    enqueued; on a non-zero return nothing has been enqueued (MOE_ERR_HIP
 *    aside, which reports a failed launch).
 *  - The entry points keep no state between calls and may be called from
 *    several host threads on distinct workspaces.  Calls sharing a
 *    workspace must be ordered on one stream.
 *  - Inputs must be finite; behaviour on NaN or Inf is unspecified.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1)   /* NULL pointer, bad size or mode        */
#define MOE_ERR_UNSUPPORTED (-2)   /* valid but not implemented (sizes, alignment) */
#define MOE_ERR_WORKSPACE (-3)     /* workspace smaller than required       */
#define MOE_ERR_HIP (-4)           /* a HIP launch or runtime call failed   */

/* ---- scoring modes ------------------------------------------------------
 * SOFTMAX       s = softmax over the N' routed logits (freedeepseekapi.com
 *               blog, sec. 2; the P_i definition of the DeepSeekMoE notes)
 * SIGMOID       s = 1 / (1 + e^-l)     (DeepSeek-V4 book ch. 02, sec. 1, V3)
 * SQRT_SOFTPLUS s = sqrt(log(1 + e^l)) (DeepSeek-V4 book ch. 02, sec. 2, V4)
 * HASH          expert = fmix32(token_id) mod N', K' = 1, g = 1 (V4 book
 *               ch. 02, sec. 5; fmix32 is MurmurHash3's 32-bit finaliser)   */
#define MOE_SCORE_SOFTMAX 0
#define MOE_SCORE_SIGMOID 1
#define MOE_SCORE_SQRT_SOFTPLUS 2
#define MOE_ROUTE_HASH 3

/* ---- element types ------------------------------------------------------ */
#define MOE_F32 0   /* fp32 activations and weights, fp32 arithmetic         */
#define MOE_BF16 1  /* bf16 activations and weights, fp32 accumulation       */

/* ---- flags ---------------------------------------------------------------- */
#define MOE_LOGITS_IN 1u   /* moe_route reads the router logits from `logits`
                              instead of computing x W_g^T                    */
#define MOE_LOGITS_OUT 2u  /* moe_route also writes the logits it computes    */

/* Layer shape.  Field names follow the pages' notation; the config fields
 * num_experts / num_experts_per_tok / n_routed_experts /
 * moe_intermediate_size that the MoE tutorial lists map to n_routed, top_k,
 * n_routed and d_ff. */
typedef struct {
    int32_t T;           /* tokens in the batch, >= 1                         */
    int32_t d_model;     /* hidden size d, a multiple of 64                   */
    int32_t n_routed;    /* N' (= m N) routed experts, 1..1024                */
    int32_t top_k;       /* K' (= m K - K_s), 1..min(N', 16); 1 under HASH    */
    int32_t n_shared;    /* K_s shared experts, >= 0                          */
    int32_t d_ff;        /* routed expert width (coarse width / m), mult. 64  */
    int32_t d_ff_shared; /* shared expert width, multiple of 64 if K_s > 0    */
    int32_t scoring;     /* MOE_SCORE_* or MOE_ROUTE_HASH                     */
    int32_t renorm;      /* 1: g = s / sum over the selected s (V4 book ch. 02
                            sec. 1); 0: g = s (top-k gate equation)           */
    int32_t dtype;       /* MOE_F32 or MOE_BF16                               */
    uint32_t flags;      /* MOE_LOGITS_IN | MOE_LOGITS_OUT                    */
    int32_t n_groups;    /* node-limited routing (V4 book ch. 02 sec. 4, V3's
                            limit of M nodes per token): the N' experts form
                            n_groups contiguous groups of N'/n_groups; 0 = no
                            limit.  1..64, a divisor of N'; not under HASH    */
    int32_t topk_groups; /* M: groups a token may draw its K' experts from;
                            1..n_groups with M * N'/n_groups >= K'.  The pages
                            give no ranking rule: a group ranks by its best
                            selection key (ties: lower group index)         */
} moe_config;

/* Which workspace a size query is for. */
#define MOE_WS_ROUTE 0    /* scratch of moe_route                               */
#define MOE_WS_FORWARD 1  /* scratch of moe_forward                             */
#define MOE_WS_PSTAT 2    /* the p_partial buffer moe_route fills for
                             moe_balance_stats (its content is internal: score
                             sums per block of the selection, then the batch's
                             sums, all double)                                 */
#define MOE_WS_SEQSTAT 3  /* scratch of moe_seq_balance_stats                   */

/* Bytes of the requested buffer for this config; 0 if the config is invalid
 * or unsupported.  MOE_WS_ROUTE also depends on the current device: the
 * router GEMM splits d into as many ranges as it takes to cover the
 * device's compute units, and the workspace holds one partial per range.
 * Query it with the device current that the calls will run on. */
size_t moe_workspace_bytes(const moe_config *cfg, int which);

/*
 * moe_route -- router of the layer: logits, scores, selection, gates, counts.
 *
 * Computes, per token t (freedeepseekapi.com blog sec. 2; DeepSeekMoE notes
 * top-k gate equation; V4 book ch. 02 secs. 1-3 and 5):
 *   l_t   = x_t W_g^T (+ logit_offset, added in fp32 before scoring)
 *   s_t   = score(l_t), evaluated in double from the fp32 logit and rounded
 *           once to fp32
 *   key   = s + bias (fp32 add) when bias != NULL -- the bias decides who is
 *           selected and nothing else (V4 book ch. 02 sec. 3; MoE tutorial,
 *           load-balancing section) -- else key = l (every score function is
 *           increasing, so this is the score order)
 *   topk_idx[t] = the K' experts with the largest key, larger key first,
 *           the smaller expert index first among equal keys; with
 *           cfg->n_groups > 0, only experts of the cfg->topk_groups groups
 *           whose best key ranks highest (ties: lower group index) compete
 *   topk_w[t][k] = s[idx]  or  s[idx] / sum_k' s[idx_k'] (renorm; double sum
 *           in k order, rounded once)
 *   expert_counts[i] = #{(t, k) : topk_idx[t][k] == i}  (overwritten)
 *   p_partial: partial sums of s (one row per block of the selection)
 *           and the batch's sums, read by moe_balance_stats for P_i (may be
 *           NULL; must be NULL under HASH)
 * Arguments
 *   x          [T][d] bf16 or fp32 (cfg->dtype); unused with MOE_LOGITS_IN
 *              or HASH
 *   w_gate     [N'][d] same dtype; unused with MOE_LOGITS_IN or HASH
 *   logit_offset [N'] fp32 or NULL
 *   bias       [N'] fp32 or NULL
 *   token_ids  [T] uint32, required under HASH, else ignored
 *   logits     [T][N'] fp32: input with MOE_LOGITS_IN, output with
 *              MOE_LOGITS_OUT, else NULL.  Always the raw x W_g^T (no offset).
 *   topk_idx   [T][K'] int32 out;  topk_w [T][K'] fp32 out
 *   expert_counts [N'] int32 out
 *   workspace  >= moe_workspace_bytes(cfg, MOE_WS_ROUTE) bytes; required
 *              for learned routing (not under HASH): it holds the expert
 *              histograms of the selection's blocks (added in block order,
 *              so no device-wide atomics), and, when the router GEMM runs,
 *              its output -- the logits (unless MOE_LOGITS_OUT and an
 *              unsplit GEMM), or, where d is split to cover the compute
 *              units, one partial sum per split, which the selection adds in
 *              split order as it reads them
 * Errors: INVALID_ARG for a NULL required pointer, an out-of-range field,
 * HASH with K' != 1, missing token_ids, or p_partial under HASH;
 * UNSUPPORTED for d or widths not multiples of 64, or N' d >= 2^31 when the
 * router GEMM runs (it addresses W_g with 32-bit offsets); WORKSPACE when
 * ws_bytes is too small; HIP when a launch fails.
 */
int moe_route(const moe_config *cfg, const void *x, const void *w_gate,
              const float *logit_offset, const float *bias,
              const uint32_t *token_ids, float *logits, int32_t *topk_idx,
              float *topk_w, int32_t *expert_counts, void *p_partial,
              void *workspace, size_t ws_bytes, void *stream);

/*
 * moe_forward -- experts and combine for a given routing.
 *
 *   h_t = x_t + sum_{j < K_s} FFN^shared_j(x_t)
 *             + sum_{k < K'} topk_w[t][k] FFN_{topk_idx[t][k]}(x_t)
 *
 * ("core design 2" equation; K_s = 0 gives the "core design 1" layer).  Any
 * routing is accepted, not only one produced by moe_route.  An index outside
 * [0, N') contributes nothing.  Each selected (token, expert) pair is
 * computed once (dropless).  The result is bitwise reproducible run to run.
 * Arithmetic: bf16 products with fp32 accumulation; the SwiGLU hidden
 * activation is rounded to the input dtype before the down projection (for
 * gate-1 groups with bf16, to a pair of bf16 values; for the shared experts
 * of a batch of more than 128 tokens, to fp16, their down projection then
 * running on fp16 products against W2 converted to fp16 -- or on the bf16
 * pair when fp16 cannot hold a value of z or of that W2); with bf16, each
 * gate-scaled expert output is held as fp16 until the sum (as fp32 where it
 * exceeds fp16's range); the sum is formed in fp32 and rounded once
 * (nearest-even) into h.
 * Arguments
 *   x          [T][d] (cfg->dtype)
 *   topk_idx   [T][K'] int32, topk_w [T][K'] fp32
 *   w13        [N'][2 d_ff][d]: rows 0..d_ff-1 are W1 (the SiLU branch),
 *              rows d_ff..2 d_ff-1 are W3
 *   w2         [N'][d][d_ff]
 *   w13_shared [K_s][2 d_ff_shared][d], w2_shared [K_s][d][d_ff_shared]
 *              (NULL when K_s == 0)
 *   h          [T][d] out, cfg->dtype; must not alias x
 *   workspace  >= moe_workspace_bytes(cfg, MOE_WS_FORWARD) bytes
 * Errors as for moe_route.
 */
int moe_forward(const moe_config *cfg, const void *x, const int32_t *topk_idx,
                const float *topk_w, const void *w13, const void *w2,
                const void *w13_shared, const void *w2_shared, void *h,
                void *workspace, size_t ws_bytes, void *stream);

/*
 * moe_forward_static -- moe_forward with no workspace argument and no
 * allocation, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * Computes exactly what moe_forward computes (the same kernels), using a
 * library-owned device array of MOE_STATIC_SCRATCH_BYTES as its workspace.
 * Each GPU the library runs on holds its own copy of that array until the
 * process ends (it is part of the library's device code, placed when the
 * library is loaded on that GPU); its address is looked up once per device
 * on the first call with that device current.  The call itself allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).
 *  - Configs whose moe_workspace_bytes(cfg, MOE_WS_FORWARD) exceeds
 *    MOE_STATIC_SCRATCH_BYTES return MOE_ERR_UNSUPPORTED (at the V3 layer
 *    shape, batches of up to 128 tokens fit: decode-sized work).
 *  - Every call on one GPU shares that GPU's array and leaves its contents
 *    behind; nothing in it needs to start at zero (the call clears what its
 *    kernels count from).  Calls that overlap on one GPU -- on different
 *    streams, or from host threads without ordering -- RACE on the array and
 *    give undefined results: order them on one stream.
 * Arguments and the other errors as for moe_forward.
 */
#define MOE_STATIC_SCRATCH_BYTES (64ull << 20)
int moe_forward_static(const moe_config *cfg, const void *x, const int32_t *topk_idx,
                       const float *topk_w, const void *w13, const void *w2,
                       const void *w13_shared, const void *w2_shared, void *h, void *stream);

/*
 * moe_balance_stats -- expert-level balance statistics of the DeepSeekMoE
 * notes ("Expert-level balance loss" equations), routed experts only:
 *   f_i = N' c_i / (K' T)          (c = expert_counts)
 *   P_i = (1/T) sum_t s_{i,t}      (from moe_route's p_partial)
 *   loss[0] = alpha1 / N' * sum_i f_i P_i,  loss[1] = sum_i f_i P_i
 * Arguments: expert_counts [N'] int32; p_partial as filled by moe_route for
 * the same cfg (NULL allowed only when P and loss are NULL); f [N'] fp32 out;
 * P [N'] fp32 out or NULL; loss [2] fp32 out or NULL.
 * Errors: INVALID_ARG for NULL f, or P/loss requested without p_partial or
 * under HASH routing.
 */
int moe_balance_stats(const moe_config *cfg, const int32_t *expert_counts,
                      const void *p_partial, float alpha1, float *f, float *P,
                      float *loss, void *stream);

/*
 * moe_seq_balance_stats -- in-sequence balance statistics (DeepSeek-V4 book
 * ch. 02 sec. 3, change 2: L_seq = beta * sum_i f_i^seq p_i^seq).
 *
 * The batch's tokens are cut into n_seg segments (sequences): segment s
 * holds tokens seg_offsets[s] .. seg_offsets[s+1]-1.  Per segment:
 *   f_seq[s][i] = N' / (K' T_s) * #{(t, k) : t in s, topk_idx[t][k] == i}
 *                 (the DeepSeekMoE notes' f_i normalisation; computed in
 *                 double, rounded once)
 *   p_seq[s][i] = (1/T_s) sum_{t in s} s_{i,t}, s the raw score (no bias)
 *                 recomputed from `logits` exactly as moe_route computes it
 *                 (double sum, rounded once)
 *   loss_seq[s] = beta * sum_i f_seq[s][i] p_seq[s][i] (double, rounded once)
 * An empty segment gives zeros.
 * Arguments
 *   logits      [T][N'] fp32, the raw x W_g^T (as moe_route's MOE_LOGITS_OUT)
 *   logit_offset [N'] fp32 or NULL, as passed to moe_route
 *   topk_idx    [T][K'] int32 from moe_route (ids outside [0, N') ignored)
 *   seg_offsets [n_seg + 1] int32 device array, non-decreasing, from 0 to
 *               at most T (values are clamped to [0, T]; a decreasing pair
 *               is an empty segment)
 *   f_seq, p_seq [n_seg][N'] fp32 out;  loss_seq [n_seg] fp32 out
 *   workspace   >= moe_workspace_bytes(cfg, MOE_WS_SEQSTAT) bytes
 * Errors: INVALID_ARG for a NULL pointer, n_seg < 1, or HASH routing (no
 * scores); WORKSPACE; HIP.
 */
int moe_seq_balance_stats(const moe_config *cfg, const float *logits,
                          const float *logit_offset, const int32_t *topk_idx,
                          const int32_t *seg_offsets, int32_t n_seg, float beta,
                          float *f_seq, float *p_seq, float *loss_seq,
                          void *workspace, size_t ws_bytes, void *stream);

/*
 * moe_device_balance_stats -- device-level balance loss of the DeepSeekMoE
 * notes: the routed experts split into n_dev groups E_d (contiguous runs of
 * N'/n_dev experts, the experts one device holds),
 *   f_dev[d] = (1/|E_d|) sum_{j in E_d} f[j],   P_dev[d] = sum_{j in E_d} P[j],
 *   loss[0]  = alpha2 * sum_d f_dev[d] P_dev[d]
 * each a double sum in index order, rounded once.  f, P: [N'] fp32 as
 * written by moe_balance_stats.  f_dev, P_dev: [n_dev] fp32 out; loss: [1]
 * fp32 out or NULL.
 * Errors: INVALID_ARG for a NULL pointer, n_dev < 1 or N' % n_dev != 0; HIP.
 */
int moe_device_balance_stats(const moe_config *cfg, const float *f, const float *P,
                             int32_t n_dev, float alpha2, float *f_dev, float *P_dev,
                             float *loss, void *stream);

/*
 * moe_bias_update -- the aux-loss-free bias update of V3 (DeepSeek-V4 book
 * ch. 02 sec. 3):  b_i <- b_i + alpha * (K'/N' - c_i / n_tokens), where c_i
 * are the expert counts accumulated over a window of n_tokens tokens (one
 * batch: moe_route's expert_counts and T).  K'/N' is the uniform share; the
 * update is evaluated in double and rounded once to fp32, in place.
 * Arguments: expert_counts [N'] int32; bias [N'] fp32 in/out.
 * Errors: INVALID_ARG for a NULL pointer or n_tokens < 1; HIP.
 */
int moe_bias_update(const moe_config *cfg, const int32_t *expert_counts, int64_t n_tokens,
                    float alpha, float *bias, void *stream);

/* Human-readable text of a status code (static storage; for MOE_ERR_HIP the
 * text of the last HIP error seen by this thread). */
const char *moe_status_string(int status);

/* ---- stage timing (benchmarking aid) ------------------------------------
 * While enabled, the entry points record a HIP event before and after each
 * kernel stage on the stream they launch on; moe_profile_collect waits for
 * those events and returns the summed milliseconds and launch counts per
 * stage.  Process-wide state: enable only from one host thread.  Creating
 * events is the only allocation involved (host-side driver objects). */
#define MOE_STAGE_ROUTER_GEMM 0  /* x W_g^T                                 */
#define MOE_STAGE_SELECT 1       /* scores, top-k, gates, counts, P partials */
#define MOE_STAGE_PERMUTE 2      /* histogram, scan, expert-contiguous order */
#define MOE_STAGE_GATE_UP 3      /* grouped [W1;W3] GEMM + SwiGLU            */
#define MOE_STAGE_DOWN 4         /* grouped W2 GEMM (+ gate scale)           */
#define MOE_STAGE_COMBINE 5      /* residual + shared + gated routed sum     */
#define MOE_STAGE_STATS 6        /* f_i, P_i, loss                           */
#define MOE_N_STAGES 7

typedef struct {
    int32_t launches[MOE_N_STAGES];
    double ms[MOE_N_STAGES];
} moe_stage_times;

/* max_records: how many stage executions to record (each uses 2 events). */
int moe_profile_enable(int max_records);
/* Waits for the recorded events, fills *out, disables recording. */
int moe_profile_collect(moe_stage_times *out);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
