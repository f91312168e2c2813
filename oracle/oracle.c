/*
 * oracle.c -- plain, slow, obviously correct CPU oracle for the DeepSeekMoE
 * layer forward, its router and its balance statistics.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant
 * with the HIP library.
 *
 * Every floating-point accumulation is done in double precision.  Inputs are
 * either fp32 or bf16 (raw 16-bit patterns); a bf16 value is widened exactly
 * by placing its 16 bits in the high half of an fp32 word.
 *
 * Sources (web pages; sections/equations named, no line numbers):
 *  [P1] "DeepSeekMoE: Towards Ultimate Expert Specialization ..." reading
 *       notes (heloowird.com): background eq. for h_t; "core design 1"
 *       (fine-grained segmentation) eqs. for h_t and the top-k gate g_{i,t};
 *       "core design 2" (shared expert isolation) eq. for h_t; expert-level
 *       balance loss eqs. for L_ExpBal, f_i, P_i and the worked example.
 *  [P2] "MoE architecture ..." (freedeepseekapi.com) sec. 2, gating network
 *       G(x) = Softmax(W_g x).
 *  [P3] DeepSeek-V4 book ch. 02 (igloomatics.github.io): sec. 1 (V3
 *       sigmoid + renormalisation), sec. 2 eq. s = sqrt(Softplus(l)),
 *       sec. 3 (biased selection score s~ = s + b), sec. 5 (hash routing).
 *  [P4] MoE tutorial (ai.clawlihai.cn), "load balancing" section: the bias
 *       changes only who is selected and carries no gradient; "hands-on"
 *       section: real experts are mostly 3-matrix (SwiGLU) FFNs.
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes of the repository):
 *  - FFN_i is SwiGLU without biases: W2 (SiLU(W1 u) * (W3 u)), with W1 and W3
 *    stored stacked as W13 = [W1; W3] (rows 0..f-1 are W1, rows f..2f-1 W3).
 *  - The softmax runs over the routed experts only.
 *  - Scores are evaluated in double from the fp32 logit and rounded once to
 *    fp32 ("s32").  With a bias the selection key is the fp32 sum s32 + b;
 *    without one the key is the logit itself (every score function is
 *    strictly increasing, so ordering by the logit is ordering by the exact
 *    score).
 *  - Ties: larger key first, then the smaller expert index.
 *  - Renormalised gates divide s32 by the double sum of the selected s32
 *    (the bias is never part of a gate).
 *  - Hash routing uses the 32-bit MurmurHash3 finaliser ("fmix32") of the
 *    token id, modulo the number of routed experts, one expert per token,
 *    gate 1.
 *  - P_i is the mean of the raw score s32 (no bias) over tokens.
 *  - An optional per-expert logit offset is added, in fp32, to the router
 *    logit before scoring (the form in which [P2] writes a bias, used here
 *    only to build skewed workloads).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_SOFTMAX 0
#define OR_SIGMOID 1
#define OR_SQRT_SOFTPLUS 2
#define OR_HASH 3

#define OR_F32 0
#define OR_BF16 1

static double widen(const void *p, int dtype, size_t i)
{
    if (dtype == OR_F32)
        return (double)((const float *)p)[i];
    uint32_t bits = ((uint32_t)((const uint16_t *)p)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* [P2] sec. 2: router logits l = W_g x, one row of W_g per routed expert.
 * Accumulated in double and rounded once to fp32.  tokens == NULL means
 * tokens 0..n_tok-1; otherwise the listed token rows of x. */
void oracle_router_logits(int64_t n_tok, const int64_t *tokens, int64_t d,
                          int64_t n_routed, int dtype, const void *x,
                          const void *w_gate, float *logits)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_tok; ++r) {
        int64_t t = tokens ? tokens[r] : r;
        for (int64_t i = 0; i < n_routed; ++i) {
            double acc = 0.0;
            for (int64_t k = 0; k < d; ++k)
                acc += widen(x, dtype, (size_t)(t * d + k)) *
                       widen(w_gate, dtype, (size_t)(i * d + k));
            logits[r * n_routed + i] = (float)acc;
        }
    }
}

/* Threads the OpenMP loops of this oracle use. */
int oracle_threads(void) { return omp_get_max_threads(); }

/* MurmurHash3's 32-bit finaliser (public domain, Austin Appleby). */
uint32_t oracle_fmix32(uint32_t h)
{
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

/* Scores of one token, [P1] eq. for P_i (softmax probability), [P3] sec. 1
 * (sigmoid), [P3] sec. 2 (sqrt of softplus).  l: fp32 logits (offset
 * already added).  s64 receives the double value, s32 its fp32 rounding. */
static void token_scores(int scoring, int64_t n, const float *l, double *s64,
                         float *s32)
{
    if (scoring == OR_SOFTMAX) {
        double m = (double)l[0];
        for (int64_t i = 1; i < n; ++i)
            if ((double)l[i] > m)
                m = (double)l[i];
        double sum = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            s64[i] = exp((double)l[i] - m);
            sum += s64[i];
        }
        for (int64_t i = 0; i < n; ++i)
            s64[i] = s64[i] / sum;
    } else if (scoring == OR_SIGMOID) {
        for (int64_t i = 0; i < n; ++i)
            s64[i] = 1.0 / (1.0 + exp(-(double)l[i]));
    } else { /* OR_SQRT_SOFTPLUS: log(1 + e^l), written so it never overflows */
        for (int64_t i = 0; i < n; ++i) {
            double v = (double)l[i];
            double sp = v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));
            s64[i] = sqrt(sp);
        }
    }
    for (int64_t i = 0; i < n; ++i)
        s32[i] = (float)s64[i];
}

/* Routing for n_tok tokens.
 *  logits  [n_tok][n_routed] fp32 router output (before the offset), unused
 *          under hash routing
 *  offset  [n_routed] fp32 or NULL: added to the logit before scoring
 *  bias    [n_routed] fp32 or NULL: selection-only bias ([P3] sec. 3, [P4])
 *  token_ids [n_tok] u32: hash routing only ([P3] sec. 5)
 * Outputs:
 *  idx     [n_tok][top_k] int32, key-descending order ([P1] top-k gate eq.)
 *  gate    [n_tok][top_k] fp32 gate values g
 *  s32_out [n_tok][n_routed] fp32 scores, or NULL (undefined under hash)
 *  gap_out [n_tok] double, or NULL: (K'-th) - (K'+1-th) selection score in
 *          score units (s, or s + b with a bias), evaluated in double;
 *          +INFINITY when top_k == n_routed or under hash routing.
 * Returns 0, or -1 on an invalid argument. */
int oracle_route(int64_t n_tok, int64_t n_routed, int64_t top_k, int scoring,
                 int renorm, const float *logits, const float *offset,
                 const float *bias, const uint32_t *token_ids,
                 int64_t n_groups, int64_t topk_groups, int32_t *idx,
                 float *gate, float *s32_out, double *gap_out)
{
    if (n_tok < 0 || n_routed < 1 || top_k < 1 || top_k > n_routed)
        return -1;
    if (n_groups < 0 || (n_groups > 0 && (n_routed % n_groups != 0 ||
                                          topk_groups < 1 ||
                                          topk_groups > n_groups ||
                                          topk_groups * (n_routed / n_groups) < top_k)))
        return -1;
    if (scoring == OR_HASH) {
        if (n_groups > 0)
            return -1;
        if (!token_ids || top_k != 1)
            return -1;
        for (int64_t t = 0; t < n_tok; ++t) {
            idx[t] = (int32_t)(oracle_fmix32(token_ids[t]) % (uint32_t)n_routed);
            gate[t] = 1.0f;
            if (gap_out)
                gap_out[t] = INFINITY;
        }
        return 0;
    }
    if (scoring < OR_SOFTMAX || scoring > OR_SQRT_SOFTPLUS || !logits)
        return -1;

    int bad = 0;
#pragma omp parallel
    {
        float *l = malloc(sizeof(float) * n_routed);
        double *s64 = malloc(sizeof(double) * n_routed);
        float *s32 = malloc(sizeof(float) * n_routed);
        float *key = malloc(sizeof(float) * n_routed);
        char *taken = malloc((size_t)n_routed);
        char *allowed = malloc((size_t)n_routed);
        int64_t ng = n_groups > 0 ? n_groups : 1;
        float *gkey = malloc(sizeof(float) * ng);
        double *gscore = malloc(sizeof(double) * ng);
        char *gtaken = malloc((size_t)ng);
        if (!l || !s64 || !s32 || !key || !taken || !allowed || !gkey || !gscore || !gtaken) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < n_tok; ++t) {
                for (int64_t i = 0; i < n_routed; ++i) {
                    float v = logits[t * n_routed + i];
                    l[i] = offset ? v + offset[i] : v; /* fp32 add */
                }
                token_scores(scoring, n_routed, l, s64, s32);
                for (int64_t i = 0; i < n_routed; ++i) {
                    key[i] = bias ? s32[i] + bias[i] : l[i]; /* fp32 add */
                    taken[i] = 0;
                    allowed[i] = 1;
                }
                /* node-limited routing ([P3] sec. 4): only experts of the
                 * topk_groups groups with the largest best key may be taken */
                double group_gap = INFINITY;
                if (n_groups > 0) {
                    const int64_t gsz = n_routed / n_groups;
                    for (int64_t g = 0; g < n_groups; ++g) {
                        gkey[g] = key[g * gsz];
                        gscore[g] = s64[g * gsz] + (bias ? (double)bias[g * gsz] : 0.0);
                        for (int64_t i = g * gsz + 1; i < (g + 1) * gsz; ++i) {
                            if (key[i] > gkey[g])
                                gkey[g] = key[i];
                            double v = s64[i] + (bias ? (double)bias[i] : 0.0);
                            if (v > gscore[g])
                                gscore[g] = v;
                        }
                        gtaken[g] = 0;
                    }
                    double last = 0.0;
                    for (int64_t m = 0; m < topk_groups; ++m) {
                        int64_t best = -1;
                        for (int64_t g = 0; g < n_groups; ++g)
                            if (!gtaken[g] && (best < 0 || gkey[g] > gkey[best]))
                                best = g;
                        gtaken[best] = 1;
                        last = gscore[best];
                    }
                    for (int64_t g = 0; g < n_groups; ++g)
                        if (!gtaken[g] && last - gscore[g] < group_gap)
                            group_gap = last - gscore[g];
                    for (int64_t i = 0; i < n_routed; ++i)
                        allowed[i] = gtaken[i / gsz];
                }
                /* top-k by (key desc, index asc): k passes of a plain argmax */
                for (int64_t k = 0; k < top_k; ++k) {
                    int64_t best = -1;
                    for (int64_t i = 0; i < n_routed; ++i) {
                        if (taken[i] || !allowed[i])
                            continue;
                        if (best < 0 || key[i] > key[best])
                            best = i;
                    }
                    taken[best] = 1;
                    idx[t * top_k + k] = (int32_t)best;
                }
                /* gates: g = s ([P1]) or s / sum_selected s ([P3] sec. 1) */
                double den = 0.0;
                for (int64_t k = 0; k < top_k; ++k)
                    den += (double)s32[idx[t * top_k + k]];
                for (int64_t k = 0; k < top_k; ++k) {
                    double s = (double)s32[idx[t * top_k + k]];
                    gate[t * top_k + k] = renorm ? (float)(s / den) : (float)s;
                }
                if (gap_out) {
                    /* next candidate: the best allowed expert not taken */
                    int64_t nxt = -1;
                    for (int64_t i = 0; i < n_routed; ++i)
                        if (!taken[i] && allowed[i] && (nxt < 0 || key[i] > key[nxt]))
                            nxt = i;
                    double g = INFINITY;
                    if (nxt >= 0) {
                        int64_t kth = idx[t * top_k + top_k - 1];
                        double a = s64[kth] + (bias ? (double)bias[kth] : 0.0);
                        double b = s64[nxt] + (bias ? (double)bias[nxt] : 0.0);
                        g = a - b;
                    }
                    gap_out[t] = g < group_gap ? g : group_gap;
                }
                if (s32_out)
                    memcpy(s32_out + t * n_routed, s32, sizeof(float) * n_routed);
            }
        }
        free(l);
        free(s64);
        free(s32);
        free(key);
        free(taken);
        free(allowed);
        free(gkey);
        free(gscore);
        free(gtaken);
    }
    return bad ? -1 : 0;
}

/* c_i = number of (token, slot) pairs that select routed expert i. */
void oracle_counts(int64_t n_tok, int64_t n_routed, int64_t top_k,
                   const int32_t *idx, int32_t *counts)
{
    for (int64_t i = 0; i < n_routed; ++i)
        counts[i] = 0;
    for (int64_t p = 0; p < n_tok * top_k; ++p)
        if (idx[p] >= 0 && idx[p] < n_routed)
            counts[idx[p]] += 1;
}

/* [P1] expert-level balance: f_i = N'/(K'T) * c_i, P_i = (1/T) sum_t s_{i,t},
 * L_ExpBal = alpha1 * (1/N') * sum_i f_i P_i, routed experts only.
 * scores may be NULL (then P and the loss are not written).
 * loss2[0] = L_ExpBal, loss2[1] = sum_i f_i P_i. */
void oracle_balance_stats(int64_t n_tok, int64_t n_routed, int64_t top_k,
                          const int32_t *counts, const float *scores,
                          double alpha1, double *f, double *P, double *loss2)
{
    for (int64_t i = 0; i < n_routed; ++i)
        f[i] = (double)(n_routed * (int64_t)counts[i]) /
               (double)(top_k * n_tok);
    if (!scores)
        return;
    double raw = 0.0;
    for (int64_t i = 0; i < n_routed; ++i) {
        double acc = 0.0;
        for (int64_t t = 0; t < n_tok; ++t)
            acc += (double)scores[t * n_routed + i];
        P[i] = acc / (double)n_tok;
        raw += f[i] * P[i];
    }
    if (loss2) {
        loss2[0] = alpha1 / (double)n_routed * raw;
        loss2[1] = raw;
    }
}

/* [P3] sec. 3, change 2: the in-sequence balance loss
 * L_seq = beta * sum_i f_i^seq p_i^seq, per segment (sequence) s of the
 * batch: tokens seg_off[s] .. seg_off[s+1]-1.  Readings: f_i^seq is
 * normalised like f_i of [P1] (N'/(K' T_s) times the selections of i in the
 * segment), p_i^seq is the mean raw score s32 of i over the segment's tokens
 * (as P_i), and an empty segment gives f = p = 0 and L = 0.
 * Outputs f_seq, p_seq [n_seg][n_routed], loss [n_seg], all double. */
void oracle_seq_balance_stats(int64_t n_tok, int64_t n_routed, int64_t top_k,
                              int64_t n_seg, const int64_t *seg_off,
                              const int32_t *idx, const float *scores, double beta,
                              double *f_seq, double *p_seq, double *loss)
{
    for (int64_t s = 0; s < n_seg; ++s) {
        const int64_t t0 = seg_off[s], t1 = seg_off[s + 1], ts = t1 - t0;
        double raw = 0.0;
        for (int64_t i = 0; i < n_routed; ++i) {
            int64_t c = 0;
            double acc = 0.0;
            for (int64_t t = t0; t < t1; ++t) {
                for (int64_t k = 0; k < top_k; ++k)
                    if (idx[t * top_k + k] == i)
                        c += 1;
                acc += (double)scores[t * n_routed + i];
            }
            double f = ts > 0 ? (double)(n_routed * c) / (double)(top_k * ts) : 0.0;
            double p = ts > 0 ? acc / (double)ts : 0.0;
            f_seq[s * n_routed + i] = f;
            p_seq[s * n_routed + i] = p;
            raw += f * p;
        }
        loss[s] = beta * raw;
    }
    (void)n_tok;
}

/* [P1] device-level balance loss: the routed experts split into n_dev
 * groups E_d; f'_d = mean of f_j over E_d, P'_d = sum of P_j over E_d,
 * L_DevBal = alpha2 * sum_d f'_d P'_d.  Reading: the groups are n_dev
 * contiguous runs of N'/n_dev experts.  f and P are the fp32 outputs of the
 * expert-level statistics. */
void oracle_device_balance_stats(int64_t n_routed, int64_t n_dev, const float *f,
                                 const float *P, double alpha2, double *f_dev,
                                 double *P_dev, double *loss)
{
    const int64_t gsz = n_routed / n_dev;
    double raw = 0.0;
    for (int64_t d = 0; d < n_dev; ++d) {
        double fs = 0.0, ps = 0.0;
        for (int64_t j = d * gsz; j < (d + 1) * gsz; ++j) {
            fs += (double)f[j];
            ps += (double)P[j];
        }
        f_dev[d] = fs / (double)gsz;
        P_dev[d] = ps;
        raw += f_dev[d] * P_dev[d];
    }
    *loss = alpha2 * raw;
}

/* [P3] sec. 3, the aux-loss-free bias update of V3:
 * b_i <- b_i + alpha (f* - f_i), f* = K'/N' the uniform share and f_i the
 * share of tokens routed to expert i over the window (counts c_i over
 * n_tok tokens: f_i = c_i / n_tok, so sum_i f_i = K' = sum_i f*).
 * Evaluated in double, rounded once to fp32. */
void oracle_bias_update(int64_t n_routed, int64_t top_k, int64_t n_tok,
                        const int32_t *counts, double alpha, const float *bias_in,
                        float *bias_out)
{
    const double target = (double)top_k / (double)n_routed;
    for (int64_t i = 0; i < n_routed; ++i) {
        double share = (double)counts[i] / (double)n_tok;
        bias_out[i] = (float)((double)bias_in[i] + alpha * (target - share));
    }
}

/* One SwiGLU expert on one token: y = W2 (SiLU(W1 u) * (W3 u)).
 * w13 [2f][d] (rows 0..f-1 = W1, f..2f-1 = W3), w2 [d][f]. */
static void swiglu_expert(int64_t d, int64_t f, int dtype, const void *x,
                          int64_t t, const void *w13, size_t w13_base,
                          const void *w2, size_t w2_base, double *z, double *y)
{
    for (int64_t r = 0; r < f; ++r) {
        double a = 0.0, b = 0.0;
        for (int64_t k = 0; k < d; ++k) {
            double xv = widen(x, dtype, (size_t)(t * d + k));
            a += widen(w13, dtype, w13_base + (size_t)(r * d + k)) * xv;
            b += widen(w13, dtype, w13_base + (size_t)((f + r) * d + k)) * xv;
        }
        z[r] = a / (1.0 + exp(-a)) * b;
    }
    for (int64_t n = 0; n < d; ++n) {
        double acc = 0.0;
        for (int64_t r = 0; r < f; ++r)
            acc += widen(w2, dtype, w2_base + (size_t)(n * f + r)) * z[r];
        y[n] = acc;
    }
}

/* Layer output, [P1] core design 2:
 *   h_t = u_t + sum_{shared j} FFN_j(u_t) + sum_k g_{t,k} FFN_{idx[t][k]}(u_t)
 * for the listed tokens (tokens == NULL: 0..n_out-1), in double.
 *  x    [T][d]; idx/gate [T][top_k] (rows indexed by the token id)
 *  w13  [n_routed][2f][d], w2 [n_routed][d][f]
 *  w13s [n_shared][2fs][d], w2s [n_shared][d][fs]
 *  h    [n_out][d] double.
 * Routed indices outside [0, n_routed) contribute nothing. */
void oracle_forward(int64_t n_out, const int64_t *tokens, int64_t d,
                    int64_t n_routed, int64_t top_k, int64_t n_shared,
                    int64_t f, int64_t fs, int dtype, const void *x,
                    const int32_t *idx, const float *gate, const void *w13,
                    const void *w2, const void *w13s, const void *w2s,
                    double *h)
{
    int64_t fmax = f > fs ? f : fs;
#pragma omp parallel
    {
        double *z = malloc(sizeof(double) * (size_t)(fmax > 0 ? fmax : 1));
        double *y = malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_out; ++r) {
            int64_t t = tokens ? tokens[r] : r;
            double *out = h + r * d;
            for (int64_t c = 0; c < d; ++c)
                out[c] = widen(x, dtype, (size_t)(t * d + c));
            for (int64_t j = 0; j < n_shared; ++j) {
                swiglu_expert(d, fs, dtype, x, t, w13s, (size_t)(j * 2 * fs * d),
                              w2s, (size_t)(j * d * fs), z, y);
                for (int64_t c = 0; c < d; ++c)
                    out[c] += y[c];
            }
            for (int64_t k = 0; k < top_k; ++k) {
                int32_t e = idx[t * top_k + k];
                if (e < 0 || e >= n_routed)
                    continue;
                double g = (double)gate[t * top_k + k];
                swiglu_expert(d, f, dtype, x, t, w13, (size_t)e * (size_t)(2 * f * d),
                              w2, (size_t)e * (size_t)(d * f), z, y);
                for (int64_t c = 0; c < d; ++c)
                    out[c] += g * y[c];
            }
        }
        free(z);
        free(y);
    }
}
