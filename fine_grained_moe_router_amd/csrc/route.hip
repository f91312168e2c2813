// route.hip -- the router of the DeepSeekMoE layer on gfx950:
//   * router GEMM l = x W_g^T (gating network of the freedeepseekapi.com MoE
//     blog, sec. 2): bf16 MFMA with fp32 accumulation, or fp32 SIMT;
//   * per-token scoring, selection bias, top-K', gates, expert counts and
//     per-block partial sums of the scores, one wavefront per token
//     (top-k gate equation of the DeepSeekMoE reading notes; V4 book ch. 02
//     sec. 1 sigmoid + renormalisation, sec. 2 sqrt(softplus), sec. 3 the
//     selection-only bias);
//   * hash routing (V4 book ch. 02 sec. 5);
//   * the expert-level balance statistics f_i, P_i, L_ExpBal (DeepSeekMoE
//     notes, "Expert-level balance loss").
#include <math.h>

#include "common.h"
#include "mfma_pipe.h"
#include "simt_tile.h"

namespace moe {

// ============================================================ router GEMM

// bf16: the 256 x 256 tile engine of the expert GEMMs (mfma_pipe.h).  Block
// (m, n, z) computes tokens m*256.., logits n*256.. over k-tiles
// [z*kps, (z+1)*kps) of d; a tile spans all 256 experts of a V3-sized
// router, so x is read once.  With one split the block writes the logits;
// with more it writes its partial sum to out + z * stride, and the select
// kernel adds the partials of each logit in split order as it reads them
// (no separate reduction pass, no logits round trip).
template <int NF>
__device__ __forceinline__ void router_tile(char *lds, const OperandRows<PipeTile> &rows, int K, int T,
                                            int N, int m0, int n0, float *__restrict__ out) {
    using P = PipeTile;
    f32x16 acc[NF > 0 ? NF : 1][P::FN];
    // transposed accumulators: a lane holds one token row and, per register
    // quad, four consecutive experts, stored as one 16-byte write where the
    // rows are 16-byte aligned (N' a multiple of 4, an aligned buffer)
    pipe_gemm_nf<P, false, NF, true, false, (1 << NF) - 1, false, true>(lds, rows, K, 0, 1, 0, 0,
                                                                       acc);
    const bool wide = (N & 3) == 0 && ((uintptr_t)out & 15) == 0;
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        const int tid = opaque_tid();
        const int row = m0 + pipe_out_row_tr<P>(tid, i);
        if (row >= T) continue;
        float *orow = out + (size_t)row * N;
#pragma unroll
        for (int j = 0; j < P::FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = n0 + pipe_out_col_tr<P>(tid, j, 4 * q);
                if (wide) {
                    if (col < N)
                        *(f32x4 *)(orow + col) = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                                       acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                } else {
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        if (col + s < N) orow[col + s] = acc[i][j][4 * q + s];
                }
            }
    }
}

__global__ __launch_bounds__(PipeTile::NT) void k_router_bf16(int T, int d, int N, int kps, int rb,
                                                              size_t stride,
                                                              const uint16_t *__restrict__ x,
                                                              const uint16_t *__restrict__ wg,
                                                              float *__restrict__ out) {
    __shared__ __attribute__((aligned(16))) char lds[PipeTile::LDS_BYTES];
    using P = PipeTile;
    // rb (256 or 128) token rows per block: a half tile computes half the
    // fragments (wave_frags), so twice the row blocks need half the K splits
    const int m0 = blockIdx.x * rb, n0 = blockIdx.y * P::BN;
    const int k0 = blockIdx.z * kps * P::BK;
    const int K = min(d - k0, kps * P::BK);
    out += (size_t)blockIdx.z * stride;
    const int nrows = min(rb, T - m0);
    // Both operands are affine: token rows m0.. and expert rows n0.. (token
    // rows past T are not fetched; expert rows past N' fetch row N' - 1).
    OperandRows<P> rows;
    rows.abase = x + k0;
    rows.bbase = wg + k0;
    const int r0 = P::load_row(threadIdx.x, 0);
    rows.aoff[0] = (uint32_t)(m0 + r0) * (uint32_t)d;
    rows.boff[0] = (uint32_t)(n0 + r0) * (uint32_t)d;
    rows.astep = rows.bstep = (uint32_t)(P::NT / P::CHUNKS) * (uint32_t)d;
    rows.amask = valid_row_mask<P>(nrows);
    rows.azero = pad_row_mask<P>(nrows);
    rows.bmask = valid_row_mask<P>(N - n0);
    rows.blast = (uint32_t)(N - 1) * (uint32_t)d;
    // a wave whose experts (its FN fragments of 32 columns) all lie past N'
    // -- the rest of a ragged last column tile, or all but the first wave
    // column for N' <= 64 -- issues no MFMAs (its loads and barriers stay)
    const bool cols = n0 + P::wave_n(threadIdx.x) * P::FN * 32 < N;
    switch (cols ? wave_frags<P>(nrows) : 0) {
        case 4: return router_tile<4>(lds, rows, K, T, N, m0, n0, out);
        case 3: return router_tile<3>(lds, rows, K, T, N, m0, n0, out);
        case 2: return router_tile<2>(lds, rows, K, T, N, m0, n0, out);
        case 1: return router_tile<1>(lds, rows, K, T, N, m0, n0, out);
        default: return router_tile<0>(lds, rows, K, T, N, m0, n0, out);
    }
}

__global__ __launch_bounds__(256) void k_router_f32(int T, int d, int N, const float *__restrict__ x,
                                                    const float *__restrict__ wg,
                                                    float *__restrict__ logits) {
    __shared__ float As[kSBK * kSPad], Bs[kSBK * kSPad];
    const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
    const int lr = threadIdx.x >> 2;
    const float *arow = (m0 + lr < T) ? x + (size_t)(m0 + lr) * d : nullptr;
    const float *brow = (n0 + lr < N) ? wg + (size_t)(n0 + lr) * d : nullptr;
    float acc[4][4];
    SimtTile<false>::run(arow, brow, d, 0, 1, 0, As, Bs, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = m0 + SimtTile<false>::out_row(i), col = n0 + SimtTile<false>::out_col(j);
            if (row < T && col < N) logits[(size_t)row * N + col] = acc[i][j];
        }
}

// Token rows per block of the bf16 router GEMM: 128 where 256-row tiles
// would need more than four K splits to cover the CUs (half the splits,
// half the partial sums written and read back by the selection), else 256.
int router_rows_per_block(const moe_config &c) {
    const int tiles = ((c.T + PipeTile::BM - 1) / PipeTile::BM) *
                      ((c.n_routed + PipeTile::BN - 1) / PipeTile::BN);
    return (c.T > PipeTile::BM / 2 && (device_cu_count() + tiles - 1) / tiles > 4) ? PipeTile::BM / 2
                                                                                   : PipeTile::BM;
}

// K splits of the bf16 router GEMM: enough blocks to cover the CUs (one
// tile per CU), each split at least 8 k-tiles long.
int router_splits(const moe_config &c) {
    if (c.dtype != MOE_BF16) return 1;
    const int rb = router_rows_per_block(c);
    const int tiles = ((c.T + rb - 1) / rb) * ((c.n_routed + PipeTile::BN - 1) / PipeTile::BN);
    const int nk = c.d_model / PipeTile::BK;
    int z = min(min(16, nk / 8), (device_cu_count() + tiles - 1) / tiles);
    if (z <= 1) return 1;
    const int kps = (nk + z - 1) / z;
    return (nk + kps - 1) / kps;
}

hipError_t launch_router_logits(const moe_config &c, const void *x, const void *wg, float *out,
                                size_t stride, hipStream_t s) {
    const int z = router_splits(c);
    if (c.dtype == MOE_BF16) {
        const int nk = c.d_model / PipeTile::BK;
        const int kps = (nk + z - 1) / z;
        const int rb = router_rows_per_block(c);
        dim3 grid((c.T + rb - 1) / rb, (c.n_routed + PipeTile::BN - 1) / PipeTile::BN, z);
        hipLaunchKernelGGL(k_router_bf16, grid, dim3(PipeTile::NT), 0, s, c.T, c.d_model,
                           c.n_routed, kps, rb, stride, (const uint16_t *)x, (const uint16_t *)wg,
                           out);
    } else {
        dim3 grid((c.T + 63) / 64, (c.n_routed + 63) / 64);
        hipLaunchKernelGGL(k_router_f32, grid, dim3(256), 0, s, c.T, c.d_model, c.n_routed,
                           (const float *)x, (const float *)wg, out);
    }
    return hipGetLastError();
}

// ============================================================ selection

constexpr int kSelWaves = 8;
constexpr int kMaxTopK = 16;

// One token per wavefront for small batches, two at prefill sizes (512
// blocks of 8 waves at T = 8192: two blocks fit a CU by registers, so the
// whole batch is in flight at once).  Each block writes its expert
// histogram and its partial sums of the scores to a row of its own, and
// k_route_tail adds the rows in block order: no device-wide atomics on the
// N' counters (from hundreds of blocks on eight XCDs they serialise on a
// few cache lines).
int select_tokens_per_block(const moe_config &c) { return c.T >= 4096 ? 2 * kSelWaves : kSelWaves; }

int select_blocks(const moe_config &c) {
    const int tpb = select_tokens_per_block(c);
    return (c.T + tpb - 1) / tpb;
}

// Score of one expert, in double from the fp32 logit (V4 book ch. 02: sec. 1
// sigmoid, sec. 2 sqrt(log(1 + e^l)) written so that it cannot overflow).
__device__ __forceinline__ double score_pointwise(int scoring, float l) {
    const double v = (double)l;
    if (scoring == MOE_SCORE_SIGMOID) return 1.0 / (1.0 + exp(-v));
    const double sp = v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));
    return sqrt(sp);
}

// A wavefront holds one token's N' experts: lane `lane` owns the J
// consecutive experts J lane .. J lane + J - 1 (those below N'), so a row of
// logits (or a split partial) arrives in one, two or four wide loads per
// lane rather than J narrow ones.
template <int J>
__device__ __forceinline__ int lane_expert(int lane, int j) { return J * lane + j; }

// J consecutive floats from p, in 16- or 8-byte loads where J allows (p
// must then be aligned to them; see wave_token_logits).
template <int J>
__device__ __forceinline__ void load_row_part(const float *p, float (&v)[J]) {
    if constexpr (J % 4 == 0) {
#pragma unroll
        for (int j = 0; j < J; j += 4) {
            const float4 q = *(const float4 *)(p + j);
            v[j] = q.x;
            v[j + 1] = q.y;
            v[j + 2] = q.z;
            v[j + 3] = q.w;
        }
    } else if constexpr (J % 2 == 0) {
#pragma unroll
        for (int j = 0; j < J; j += 2) {
            const float2 q = *(const float2 *)(p + j);
            v[j] = q.x;
            v[j + 1] = q.y;
        }
    } else {
#pragma unroll
        for (int j = 0; j < J; ++j) v[j] = p[j];
    }
}

// Raw logits of one token held by one wavefront (lane_expert).  The logit is
// row[e], or with a split router GEMM the sum of its `splits` partials
// row[e] + row[stride + e] + ..., added in split order in fp32 (so it is one
// fixed value whoever reads it).  A lane whose experts all exist loads them
// whole; the lane holding the end of a ragged N' loads one by one.
template <int J>
__device__ __forceinline__ void wave_token_logits(int N, const float *row, int splits,
                                                  size_t stride, int lane, float (&raw)[J]) {
    const int e0 = lane_expert<J>(lane, 0);
    // whole-lane loads need every expert present and an aligned start: every
    // row is 16-byte aligned when the buffer is and N' is a multiple of 4
    const bool aligned = ((uintptr_t)row & 15) == 0 && ((stride & 3) == 0 || splits == 1);
    const bool whole = e0 + J <= N && ((N % 4 == 0 && aligned) || J == 1);
    if (whole) {
        load_row_part<J>(row + e0, raw);
        for (int z = 1; z < splits; ++z) {
            float pz[J];
            load_row_part<J>(row + (size_t)z * stride + e0, pz);
#pragma unroll
            for (int j = 0; j < J; ++j) raw[j] += pz[j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int e = e0 + j;
            raw[j] = (e < N) ? row[e] : -INFINITY;
        }
        for (int z = 1; z < splits; ++z) {
            const float *pz = row + (size_t)z * stride;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int e = e0 + j;
                if (e < N) raw[j] += pz[e];
            }
        }
    }
}

// Logits plus the optional offset (an fp32 add) and scores s32 of one token
// held by one wavefront.  Scores are evaluated in double from the fp32 logit
// and rounded once.
template <int J>
__device__ __forceinline__ void wave_token_scores(int N, int scoring, const float (&raw)[J],
                                                  const float *offset, int lane, float (&l)[J],
                                                  float (&s32)[J]) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int e = lane_expert<J>(lane, j);
        float v = raw[j];
        if (offset && e < N) v = v + offset[e];  // fp32 add
        l[j] = v;
    }
    if (scoring == MOE_SCORE_SOFTMAX) {
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < J; ++j) m = fmaxf(m, l[j]);
        m = wave_max_f32(m);
        double ex[J], part = 0.0;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int e = lane_expert<J>(lane, j);
            ex[j] = (e < N) ? exp((double)l[j] - (double)m) : 0.0;
            part += ex[j];
        }
        const double sum = wave_sum_f64(part);
#pragma unroll
        for (int j = 0; j < J; ++j) s32[j] = (float)(ex[j] / sum);
    } else {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int e = lane_expert<J>(lane, j);
            s32[j] = (e < N) ? (float)score_pointwise(scoring, l[j]) : 0.0f;
        }
    }
}

// Wave-wide argmax of (v desc, index asc) over the lanes whose idx is not
// 0x7fffffff; every lane receives the winner.  (v, index) pairs are totally
// ordered, so the winner does not depend on the order of the reduction.  It
// runs on DPP lane moves, without the LDS crossbar: swaps within quads, then
// within half rows and rows (mirrors), then row broadcasts that leave the
// wave's winner in lane 63, which is read back into a scalar.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void argmax_dpp_step(float &v, int &idx) {
    const float ov = __int_as_float(__builtin_amdgcn_update_dpp(
        __float_as_int(-INFINITY), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
    const int oi = __builtin_amdgcn_update_dpp(0x7fffffff, idx, CTRL, ROW_MASK, 0xF, false);
    if (oi != 0x7fffffff && (idx == 0x7fffffff || ov > v || (ov == v && oi < idx))) {
        v = ov;
        idx = oi;
    }
}
__device__ __forceinline__ void wave_argmax_pairs(float &v, int &idx) {
    argmax_dpp_step<0xB1, 0xF>(v, idx);    // quad_perm [1,0,3,2]: lane ^ 1
    argmax_dpp_step<0x4E, 0xF>(v, idx);    // quad_perm [2,3,0,1]: lane ^ 2
    argmax_dpp_step<0x141, 0xF>(v, idx);   // row_half_mirror: the two quads of 8 lanes
    argmax_dpp_step<0x140, 0xF>(v, idx);   // row_mirror: the two halves of a 16-lane row
    argmax_dpp_step<0x142, 0xA>(v, idx);   // row_bcast:15 into rows 1, 3
    argmax_dpp_step<0x143, 0xC>(v, idx);   // row_bcast:31 into rows 2, 3
    v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
    idx = __builtin_amdgcn_readlane(idx, 63);
}

// The same winner from a wave-wide maximum of the key alone and a ballot
// of the lanes holding it: lanes own increasing expert ranges, so among
// equal keys the lowest such lane holds the lowest index.  The maximum runs
// on 32-bit integers that order like the floats (sign-magnitude folded to
// two's complement, -0 taken as +0 so that equal keys stay equal), one DPP
// max per step.  Lanes with no candidate (idx 0x7fffffff) and NaN keys take
// INT_MIN and never win; if no lane has a candidate left the pairwise
// reduction above decides.
__device__ __forceinline__ int ordered_key(float f) {
    f = f + 0.0f;   // -0 -> +0
    const int b = __float_as_int(f);
    return (f != f) ? INT_MIN : (b ^ ((b >> 31) & 0x7FFFFFFF));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int max_dpp_step(int v) {
    return max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ void wave_argmax(float &v, int &idx) {
    const int o = idx != 0x7fffffff ? ordered_key(v) : INT_MIN;
    int m = o;
    m = max_dpp_step<0xB1, 0xF>(m);
    m = max_dpp_step<0x4E, 0xF>(m);
    m = max_dpp_step<0x141, 0xF>(m);
    m = max_dpp_step<0x140, 0xF>(m);
    m = max_dpp_step<0x142, 0xA>(m);
    m = max_dpp_step<0x143, 0xC>(m);
    m = __builtin_amdgcn_readlane(m, 63);
    if (m != INT_MIN) {
        const int w = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(o == m));
        idx = __builtin_amdgcn_readlane(idx, w);
        v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), w));
    } else {
        wave_argmax_pairs(v, idx);
    }
}

// One wavefront per token.  Lane `lane` owns experts lane_expert(lane, j),
// j < J (J consecutive experts: a split partial's row arrives in one wide
// load per lane; V3 prefill select 47 -> 41 us, decode 30 -> 20 us).  Two
// tokens per wave side by side was measured and is slower: the extra
// registers cost more occupancy than the overlapped argmax chains gain.
// Node-limited routing (n_groups > 0): the experts of the topk_groups groups
// with the largest best key are the only candidates; the others are marked
// taken before the top-K' rounds.
// SC: the scoring function (MOE_SCORE_*), a template argument so that only
// its fp64 path is compiled into each instance.
template <int J, int SC>
__global__ __launch_bounds__(kSelWaves * kWave) void k_select(
    int T, int N, int K, int renorm, int tpb, int n_groups, int topk_groups,
    const float *__restrict__ logits, int splits, size_t stride, float *__restrict__ lg_out,
    const float *__restrict__ offset,
    const float *__restrict__ bias, int32_t *__restrict__ idx_out, float *__restrict__ w_out,
    int32_t *__restrict__ hist_part, double *__restrict__ p_partial) {
    __shared__ int32_t hist[J * kWave];
    __shared__ double psum[kSelWaves][J * kWave];
    __shared__ float kbuf[kSelWaves][J * kWave];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    for (int e = threadIdx.x; e < J * kWave; e += blockDim.x) hist[e] = 0;
    __syncthreads();

    double pacc[J];
#pragma unroll
    for (int j = 0; j < J; ++j) pacc[j] = 0.0;

    const int t0 = blockIdx.x * tpb;
    const int t1 = min(T, t0 + tpb);
    for (int t = t0 + wave; t < t1; t += kSelWaves) {
        float raw[J], l[J], key[J], s32[J];
        wave_token_logits<J>(N, logits + (size_t)t * N, splits, stride, lane, raw);
        if (lg_out) {
#pragma unroll
            for (int j = 0; j < J; ++j)
                if (lane_expert<J>(lane, j) < N) lg_out[(size_t)t * N + lane_expert<J>(lane, j)] = raw[j];
        }
        wave_token_scores<J>(N, SC, raw, offset, lane, l, s32);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int e = lane_expert<J>(lane, j);
            key[j] = bias ? ((e < N) ? s32[j] + bias[e] : -INFINITY) : l[j];  // fp32 add
            if (e < N) pacc[j] += (double)s32[j];
        }
        uint32_t taken = 0;
        if (n_groups > 0) {
            // best key of each group (lane g holds group g), via this wave's LDS row
#pragma unroll
            for (int j = 0; j < J; ++j)
                if (lane_expert<J>(lane, j) < N) kbuf[wave][lane_expert<J>(lane, j)] = key[j];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int gsz = N / n_groups;
            float gk = -INFINITY;
            if (lane < n_groups) {
                gk = kbuf[wave][lane * gsz];
                for (int i = 1; i < gsz; ++i) gk = fmaxf(gk, kbuf[wave][lane * gsz + i]);
            }
            __builtin_amdgcn_wave_barrier();   // reads done before the next token's writes
            uint64_t chosen = 0;
            bool gdone = false;
            for (int m = 0; m < topk_groups; ++m) {
                float v = gk;
                int gi = (lane < n_groups && !gdone) ? lane : 0x7fffffff;
                wave_argmax(v, gi);
                chosen |= 1ull << gi;
                if (lane == gi) gdone = true;
            }
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int e = lane_expert<J>(lane, j);
                if (e < N && !((chosen >> (e / gsz)) & 1ull)) taken |= 1u << j;
            }
        }
        // ---- top-K': K' rounds of a wave-wide argmax on (key desc, index asc).
        // Lane k keeps round k's winner and its score (two registers, not
        // K'-long arrays in every lane); the renormalisation's double sum
        // of the selected s runs in round order as the rounds go.
        int my_sel = 0;
        float my_sv = 0.0f;
        double den = 0.0;
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) {
            if (k < K) {
                float bk = -INFINITY;
                int bi = 0x7fffffff;
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    const int e = lane_expert<J>(lane, j);
                    if (e < N && !((taken >> j) & 1u) && (key[j] > bk || bi == 0x7fffffff)) {
                        bk = key[j];
                        bi = e;
                    }
                }
                wave_argmax(bk, bi);
                float mine = 0.0f;
#pragma unroll
                for (int j = 0; j < J; ++j)
                    if (lane_expert<J>(lane, j) == bi) {
                        taken |= 1u << j;
                        mine = s32[j];
                    }
                // from the lane that owns expert bi (bi is the same in every lane)
                const float svk =
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), (bi / J) & 63));
                den += (double)svk;
                if (lane == k) {
                    my_sel = bi;
                    my_sv = svk;
                }
            }
        }
        // ---- gates: s, or s / (double sum of the selected s in k order)
        if (lane < K) {
            const float g = renorm ? (float)((double)my_sv / den) : my_sv;
            idx_out[(size_t)t * K + lane] = my_sel;
            w_out[(size_t)t * K + lane] = g;
            atomicAdd(&hist[my_sel], 1);
        }
    }
    // ---- this block's expert histogram and partial sums of s (waves added
    // in a fixed order), one row each for k_route_tail
    if (p_partial) {
#pragma unroll
        for (int j = 0; j < J; ++j) psum[wave][lane_expert<J>(lane, j)] = pacc[j];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < N; e += blockDim.x) {
        hist_part[(size_t)blockIdx.x * N + e] = hist[e];
        if (p_partial) {
            double s = psum[0][e];
            for (int w = 1; w < kSelWaves; ++w) s += psum[w][e];
            p_partial[(size_t)blockIdx.x * N + e] = s;
        }
    }
}

// Expert counts and score sums of the batch from the select blocks' rows:
// block = 16 experts x 64 lanes of rows; lane r adds rows r, r + 64, ... in
// order, then the 64 lane sums are added by a fixed binary tree (a fixed
// order, so the score sums do not depend on timing).  Spreading the experts
// over N'/16 blocks keeps hundreds of rows' loads in flight.  The score sums
// go to row nblk of p_partial, where moe_balance_stats reads them.
constexpr int kTailExperts = 16, kTailRows = 64;
__global__ __launch_bounds__(kTailExperts * kTailRows) void k_route_tail(
    int N, int nblk, const int32_t *__restrict__ hist_part, double *__restrict__ p_partial,
    int32_t *__restrict__ counts) {
    __shared__ int32_t hs[kTailRows][kTailExperts];
    __shared__ double ps[kTailRows][kTailExperts];
    const int c = threadIdx.x % kTailExperts, r = threadIdx.x / kTailExperts;
    const int e = blockIdx.x * kTailExperts + c;
    int h = 0;
    double p = 0.0;
    if (e < N) {
#pragma unroll 4
        for (int b = r; b < nblk; b += kTailRows) {
            h += hist_part[(size_t)b * N + e];
            if (p_partial) p += p_partial[(size_t)b * N + e];
        }
    }
    hs[r][c] = h;
    ps[r][c] = p;
    __syncthreads();
    for (int o = kTailRows / 2; o > 0; o >>= 1) {
        if (r < o) {
            hs[r][c] += hs[r + o][c];
            ps[r][c] += ps[r + o][c];
        }
        __syncthreads();
    }
    if (r == 0 && e < N) {
        counts[e] = hs[0][c];
        if (p_partial) p_partial[(size_t)nblk * N + e] = ps[0][c];
    }
}

hipError_t launch_select(const moe_config &c, const float *logits, int splits, size_t stride,
                         float *lg_out, const float *offset, const float *bias, int32_t *idx,
                         float *w, int32_t *counts, double *p_partial, int32_t *hist_part,
                         hipStream_t s) {
    const int J = (c.n_routed + 63) / 64;
    const int tpb = select_tokens_per_block(c);
    dim3 grid(select_blocks(c)), block(kSelWaves * kWave);
#define MOE_SEL_SC(JJ, SC)                                                                     \
    hipLaunchKernelGGL((k_select<JJ, SC>), grid, block, 0, s, c.T, c.n_routed, c.top_k,       \
                       c.renorm, tpb, c.n_groups, c.topk_groups, logits, splits, stride,       \
                       lg_out, offset, bias, idx, w,                                           \
                       hist_part, p_partial)
#define MOE_SEL(JJ)                                                                            \
    do {                                                                                       \
        if (c.scoring == MOE_SCORE_SOFTMAX) MOE_SEL_SC(JJ, MOE_SCORE_SOFTMAX);                 \
        else if (c.scoring == MOE_SCORE_SIGMOID) MOE_SEL_SC(JJ, MOE_SCORE_SIGMOID);            \
        else MOE_SEL_SC(JJ, MOE_SCORE_SQRT_SOFTPLUS);                                          \
    } while (0)
    if (J <= 1) MOE_SEL(1);
    else if (J <= 2) MOE_SEL(2);
    else if (J <= 4) MOE_SEL(4);
    else if (J <= 6) MOE_SEL(6);
    else if (J <= 8) MOE_SEL(8);
    else MOE_SEL(16);
#undef MOE_SEL_SC
#undef MOE_SEL
    hipLaunchKernelGGL(k_route_tail, dim3((c.n_routed + kTailExperts - 1) / kTailExperts),
                       dim3(kTailExperts * kTailRows), 0, s, c.n_routed, select_blocks(c), hist_part,
                       p_partial, counts);
    return hipGetLastError();
}

// ============================================================ hash routing

// MurmurHash3's 32-bit finaliser (public domain, Austin Appleby).
__device__ __forceinline__ uint32_t fmix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

// ============================================================ segment and device statistics

// Score rows: one wavefront per token writes s32[t][0..N) exactly as k_select
// computes them (V4 book ch. 02 sec. 3, change 2 needs the raw scores).
template <int J>
__global__ __launch_bounds__(kSelWaves * kWave) void k_scores(int T, int N, int scoring,
                                                              const float *__restrict__ logits,
                                                              const float *__restrict__ offset,
                                                              float *__restrict__ s32_out) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kSelWaves + (threadIdx.x >> 6);
    if (t >= T) return;
    float raw[J], l[J], s32[J];
    wave_token_logits<J>(N, logits + (size_t)t * N, 1, 0, lane, raw);
    wave_token_scores<J>(N, scoring, raw, offset, lane, l, s32);
#pragma unroll
    for (int j = 0; j < J; ++j)
        if (lane_expert<J>(lane, j) < N) s32_out[(size_t)t * N + lane_expert<J>(lane, j)] = s32[j];
}

__device__ __forceinline__ void seg_range(const int32_t *off, int s, int T, int &t0, int &t1) {
    t0 = min(max(off[s], 0), T);
    t1 = min(max(off[s + 1], 0), T);
    if (t1 < t0) t1 = t0;
}

// Block (segment s, 64 experts): 16 token lanes x 64 experts.  Token lane r
// adds the scores of tokens t0 + r, t0 + r + 16, ...; the 16 partial sums
// are then added in r order (a fixed order).  Selections are counted in an
// LDS histogram of the block's 64 experts (integer adds: order-free): lane
// k < K' of token lane r reads slot k of the token's selection.
constexpr int kSeqRows = 16;
__global__ __launch_bounds__(kSeqRows * kWave) void k_seq_sums(int T, int N, int K,
                                                               const int32_t *__restrict__ off,
                                                               const float *__restrict__ s32,
                                                               const int32_t *__restrict__ idx,
                                                               float *__restrict__ f_seq,
                                                               float *__restrict__ p_seq) {
    __shared__ double ps[kSeqRows][kWave];
    __shared__ int hist[kWave];
    const int s = blockIdx.x;
    const int c = threadIdx.x & 63, r = threadIdx.x >> 6;
    const int e0 = blockIdx.y * kWave;
    const int e = e0 + c;
    if (threadIdx.x < kWave) hist[threadIdx.x] = 0;
    __syncthreads();
    int t0, t1;
    seg_range(off, s, T, t0, t1);
    double acc = 0.0;
    const float *col = s32 + (e < N ? e : 0);
#pragma unroll 8
    for (int t = t0 + r; t < t1; t += kSeqRows) {
        if (e < N) acc += (double)col[(size_t)t * N];
        if (c < K) {
            const int sel = idx[(size_t)t * K + c] - e0;
            if (sel >= 0 && sel < kWave) atomicAdd(&hist[sel], 1);
        }
    }
    ps[r][c] = acc;
    __syncthreads();
    if (r == 0 && e < N) {
        double p = 0.0;
        for (int q = 0; q < kSeqRows; ++q) p += ps[q][c];
        const long long n = hist[c];
        const int ts = t1 - t0;
        f_seq[(size_t)s * N + e] = ts > 0 ? (float)((double)((long long)N * n) / (double)((long long)K * ts)) : 0.0f;
        p_seq[(size_t)s * N + e] = ts > 0 ? (float)(p / (double)ts) : 0.0f;
    }
}

// loss[s] = beta * sum_i f_seq[s][i] p_seq[s][i], a double tree sum.
__global__ __launch_bounds__(256) void k_seq_loss(int N, float beta, const float *__restrict__ f_seq,
                                                  const float *__restrict__ p_seq,
                                                  float *__restrict__ loss) {
    __shared__ double red[256];
    const int s = blockIdx.x;
    double acc = 0.0;
    for (int i = threadIdx.x; i < N; i += 256)
        acc += (double)f_seq[(size_t)s * N + i] * (double)p_seq[(size_t)s * N + i];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) loss[s] = (float)((double)beta * red[0]);
}

hipError_t launch_seq_stats(const moe_config &c, const float *logits, const float *offset,
                            const int32_t *idx, const int32_t *seg_off, int n_seg, float beta,
                            float *scores, float *f_seq, float *p_seq, float *loss,
                            hipStream_t s) {
    const int J = (c.n_routed + 63) / 64;
    dim3 grid((c.T + kSelWaves - 1) / kSelWaves), block(kSelWaves * kWave);
#define MOE_SC(JJ)                                                                             \
    hipLaunchKernelGGL(k_scores<JJ>, grid, block, 0, s, c.T, c.n_routed, c.scoring, logits,    \
                       offset, scores)
    if (J <= 1) MOE_SC(1);
    else if (J <= 2) MOE_SC(2);
    else if (J <= 4) MOE_SC(4);
    else if (J <= 6) MOE_SC(6);
    else if (J <= 8) MOE_SC(8);
    else MOE_SC(16);
#undef MOE_SC
    hipLaunchKernelGGL(k_seq_sums, dim3(n_seg, J), dim3(kSeqRows * kWave), 0, s, c.T,
                       c.n_routed, c.top_k, seg_off, scores, idx, f_seq, p_seq);
    hipLaunchKernelGGL(k_seq_loss, dim3(n_seg), dim3(256), 0, s, c.n_routed, beta, f_seq, p_seq,
                       loss);
    return hipGetLastError();
}

// Device-level balance loss (DeepSeekMoE notes): thread d sums its group of
// N / n_dev experts in index order; the loss adds the groups in order.
__global__ __launch_bounds__(64) void k_device_stats(int N, int n_dev, float alpha2,
                                                     const float *__restrict__ f,
                                                     const float *__restrict__ P,
                                                     float *__restrict__ f_dev,
                                                     float *__restrict__ P_dev,
                                                     float *__restrict__ loss) {
    const int gsz = N / n_dev;
    double raw = 0.0;
    for (int d0 = 0; d0 < n_dev; d0 += 64) {
        const int d = d0 + (int)threadIdx.x;
        double fd = 0.0, pd = 0.0;
        if (d < n_dev) {
            for (int j = d * gsz; j < (d + 1) * gsz; ++j) {
                fd += (double)f[j];
                pd += (double)P[j];
            }
            fd /= (double)gsz;
            f_dev[d] = (float)fd;
            P_dev[d] = (float)pd;
        }
        // fixed-order sum of the 64 products of this chunk (lane 0 adds them)
        const double prod = (d < n_dev) ? fd * pd : 0.0;
        for (int q = 0; q < 64; ++q) {
            const double v = __shfl(prod, q, kWave);
            if (d0 + q < n_dev) raw += v;
        }
    }
    if (loss && threadIdx.x == 0) loss[0] = (float)((double)alpha2 * raw);
}

hipError_t launch_device_stats(const moe_config &c, const float *f, const float *P, int n_dev,
                               float alpha2, float *f_dev, float *P_dev, float *loss,
                               hipStream_t s) {
    hipLaunchKernelGGL(k_device_stats, dim3(1), dim3(64), 0, s, c.n_routed, n_dev, alpha2, f, P,
                       f_dev, P_dev, loss);
    return hipGetLastError();
}

// Aux-loss-free bias update (V4 book ch. 02 sec. 3, V3):
// b_i += alpha (K'/N' - c_i / n_tok), in double, rounded once.
__global__ __launch_bounds__(256) void k_bias_update(int N, int K, long long n_tok, float alpha,
                                                     const int32_t *__restrict__ c,
                                                     float *__restrict__ b) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= N) return;
    const double target = (double)K / (double)N;
    const double share = (double)c[i] / (double)n_tok;
    b[i] = (float)((double)b[i] + (double)alpha * (target - share));
}

hipError_t launch_bias_update(const moe_config &c, const int32_t *counts, long long n_tok,
                              float alpha, float *bias, hipStream_t s) {
    hipLaunchKernelGGL(k_bias_update, dim3((c.n_routed + 255) / 256), dim3(256), 0, s, c.n_routed,
                       c.top_k, n_tok, alpha, counts, bias);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_hash_route(int T, int N, const uint32_t *__restrict__ tid,
                                                    int32_t *__restrict__ idx,
                                                    float *__restrict__ w,
                                                    int32_t *__restrict__ counts) {
    extern __shared__ int32_t hhist[];
    for (int e = threadIdx.x; e < N; e += blockDim.x) hhist[e] = 0;
    __syncthreads();
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < T) {
        const int e = (int)(fmix32(tid[t]) % (uint32_t)N);
        idx[t] = e;
        w[t] = 1.0f;
        atomicAdd(&hhist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < N; e += blockDim.x)
        if (hhist[e]) atomicAdd(&counts[e], hhist[e]);
}

hipError_t launch_hash_route(const moe_config &c, const uint32_t *tid, int32_t *idx, float *w,
                             int32_t *counts, hipStream_t s) {
    hipLaunchKernelGGL(k_hash_route, dim3((c.T + 255) / 256), dim3(256),
                       (size_t)c.n_routed * sizeof(int32_t), s, c.T, c.n_routed, tid, idx, w,
                       counts);
    return hipGetLastError();
}

// ============================================================ utilities

__global__ void k_fill_i32(int32_t *p, int n, int32_t v) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t *p, int n, int32_t v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

// ============================================================ balance stats

// f_i = N' c_i / (K' T); P_i = (1/T) times the batch's score sum (row
// p_sum, written by k_route_tail); loss = alpha1 / N' sum_i f_i P_i (double,
// fixed tree order).  One block, one thread per expert.
__global__ __launch_bounds__(1024) void k_balance(int T, int N, int K, const int32_t *__restrict__ c,
                                                  const double *__restrict__ p_sum, float alpha1,
                                                  float *__restrict__ f, float *__restrict__ P,
                                                  float *__restrict__ loss) {
    __shared__ double red[1024];
    const int e = threadIdx.x;
    double acc = 0.0;
    if (e < N) {
        const double fe = (double)((int64_t)N * c[e]) / (double)((int64_t)K * T);
        f[e] = (float)fe;
        if (p_sum) {
            const double pe = p_sum[e] / (double)T;
            if (P) P[e] = (float)pe;
            acc = fe * pe;
        }
    }
    if (!loss) return;
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int o = blockDim.x / 2; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        loss[0] = (float)((double)alpha1 / (double)N * red[0]);
        loss[1] = (float)red[0];
    }
}
hipError_t launch_balance_stats(const moe_config &c, const int32_t *counts, const double *p_sum,
                                float alpha1, float *f, float *P, float *loss, hipStream_t s) {
    hipLaunchKernelGGL(k_balance, dim3(1), dim3(1024), 0, s, c.T, c.n_routed, c.top_k, counts,
                       p_sum, alpha1, f, P, loss);
    return hipGetLastError();
}

}  // namespace moe
