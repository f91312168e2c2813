// common.h -- device helpers and the launch interface shared by the HIP
// sources of libmoe.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---- element types --------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;     // CDNA wavefront width
constexpr int kXcds = 8;      // MI355X: 8 accelerator complex dies, 32 CUs each

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32, in the default
// rounding mode), two values per instruction: lo in bits 0-15.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ---- fp16 staging of the expert outputs (bf16 layers) ----------------------
// The gate-scaled expert outputs travel from the down projection to the
// combine as fp16: 11 significant bits against bf16's 8, at half the bytes of
// fp32.  A value with no finite fp16 form (|v| >= 65520 rounds to infinity;
// NaN stays NaN) keeps that non-finite half as a mark and is also written as
// fp32 at the same index of an fp32 array, where the reader takes it from.
// So the combine sees every value either as fp16(v) or as v itself.
__device__ __forceinline__ float f16_lo(uint32_t p) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(p & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t p) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(p >> 16));
}
__device__ __forceinline__ bool f16_marked(uint32_t h) { return (h & 0x7C00u) == 0x7C00u; }
__device__ __forceinline__ bool f16x4_marked(uint2 p) {
    return ((p.x & 0x7C00u) == 0x7C00u) | ((p.x & 0x7C000000u) == 0x7C000000u) |
           ((p.y & 0x7C00u) == 0x7C00u) | ((p.y & 0x7C000000u) == 0x7C000000u);
}
// Four staged values (p: their halves, f: the same four slots of the fp32
// array).
__device__ __forceinline__ float4 f16x4_value(uint2 p, const float *f) {
    float4 v = make_float4(f16_lo(p.x), f16_hi(p.x), f16_lo(p.y), f16_hi(p.y));
    if (f16x4_marked(p)) {
        if (f16_marked(p.x)) v.x = f[0];
        if (f16_marked(p.x >> 16)) v.y = f[1];
        if (f16_marked(p.y)) v.z = f[2];
        if (f16_marked(p.y >> 16)) v.w = f[3];
    }
    return v;
}

// ---- wave reductions (64 lanes) --------------------------------------------
__device__ __forceinline__ double wave_sum_f64(double v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// ---- forward workspace layout ----------------------------------------------
// Groups: g < N' are the routed experts (rows = the (token, slot) pairs that
// chose g, in pair order); g == N' (present when K_s > 0) is every shared
// expert at once (rows = all tokens, hidden width K_s * d_ff_shared).
struct FwdLayout {
    int n_chunks;       // permutation chunks
    int chunk;          // pairs per chunk
    int G;              // groups
    size_t off_chunk;   // int32 [n_chunks][N']: per-chunk counts, then bases
    size_t off_meta;    // int32 meta block (see MetaIdx)
    size_t off_perm;    // int32 [T*K']: pair id at each expert-ordered row
    size_t off_gsort;   // fp32 [T*K']: gate of each expert-ordered row
    size_t off_rtd;     // RowTileDesc [max_row_tiles]: the group record of each row tile
    int max_row_tiles;  // bound on the row tiles of all groups
    size_t off_zr;      // [T*K'][d_ff] dtype: routed hidden activations
    size_t off_zs;      // [T][K_s*d_ff_shared] dtype: shared hidden activations
    size_t off_yr;      // fp32 [T*K'][d]: gate-scaled routed outputs, pair order
    size_t off_ys;      // fp32 [T][d]: summed shared-expert outputs
    size_t off_yrh;     // bf16 layers: fp16 copies of the two above, read by
    size_t off_ysh;     //   the combine (fp32 only where fp16 overflows)
    size_t off_zs16;    // shared_f16: fp16 [T][K_s*d_ff_shared], z of the shared group
    size_t off_w2s16;   // shared_f16: fp16 [K_s][d][d_ff_shared], the shared W2
    size_t total;
};

// Offsets (in int32 elements) of the arrays inside the meta block.
//   group_off[G+1], group_cnt[G+1]   rows of each group
//   tile1[G+1], tile2[G+1]           tile prefix sums of the two GEMMs
//   mt[G+1]                          row-tile prefix sums (256-row tiles)
//   xs1[9], xs2[9]                   per-XCD row-tile ranges of the two GEMMs
//   q1[8], q2[8]                     per-XCD work counters of the two GEMMs
//   bad                              count of out-of-range expert ids
// q1, q2 and bad start at zero (set by the permutation).
struct MetaIdx {
    int group_off, group_cnt, tile1, tile2, mt, xs1, xs2, q1, q2, bad, f16bad, size;
};
__host__ __device__ inline MetaIdx meta_index(int G) {
    MetaIdx m;
    m.group_off = 0;
    m.group_cnt = G + 1;
    m.tile1 = 2 * G + 2;
    m.tile2 = 3 * G + 3;
    m.mt = 4 * G + 4;
    m.xs1 = 5 * G + 5;
    m.xs2 = 5 * G + 14;
    m.q1 = 5 * G + 23;
    m.q2 = 5 * G + 31;
    m.bad = 5 * G + 39;
    m.f16bad = 5 * G + 40;
    m.size = 5 * G + 41;
    return m;
}

// Tile shapes the permutation kernel prepares work lists for.
struct TileShape {
    int bm1, bz1;  // gate/up GEMM: rows per tile, hidden columns per tile
    int bm2, bn2;  // down GEMM: rows per tile, output columns per tile
};

// The group of a row tile of the bf16 GEMMs, in one 32-byte record (written
// by the permutation for every row tile of the group), so an item resolves
// to its tile with one dependent load.
struct alignas(32) RowTileDesc {
    int32_t g;      // group
    int32_t mt0;    // its first row tile
    int32_t R;      // its row tiles
    int32_t cnt;    // its rows
    int32_t goff;   // its first row in expert order (0 for the shared group)
    int32_t pad[3];
};

// Arguments of the grouped expert GEMMs.
struct GroupedArgs {
    int T, d, top_k, n_routed, n_shared, f, fs, G;
    int split_r, split_s;     // hidden activation carried as a bf16 (hi, lo) pair
    const int32_t *group_off, *group_cnt, *tile_base;
    // work queues of the bf16 kernels: row-tile prefix sums, per-XCD
    // row-tile ranges and item counters, column tiles per row tile
    const int32_t *mt_base, *xsplit;
    const RowTileDesc *rtd;   // group of each row tile
    int32_t *queue;
    int nt_routed, nt_shared;
    const int32_t *perm;      // pair id per expert-ordered row
    const float *gsort;       // gate per expert-ordered row
    const void *x, *w13, *w2, *w13s, *w2s;
    void *zr, *zs;
    float *yr, *ys;
    uint16_t *yrh, *ysh;      // fp16 outputs of the bf16 kernels (see f16x4_value)
    // The shared experts' fp16 down pass (shared_f16): z as one fp16 plane,
    // W2 of the shared experts converted to fp16, and the flag either
    // conversion sets when fp16 cannot hold a value (the down launch then
    // takes the (hi, lo) pass)
    int shared_f16;
    uint16_t *zs16;
    const uint16_t *w2s16;
    int32_t *f16bad;
};

// ---- launchers (each returns hipSuccess or the launch error) ---------------
int router_splits(const moe_config &c);   // K splits of the router GEMM
// Writes x W_g^T to out (one split), or split z's partial sum to
// out + z * stride (floats) for z < router_splits(c).
hipError_t launch_router_logits(const moe_config &c, const void *x, const void *wg, float *out,
                                size_t stride, hipStream_t s);
hipError_t launch_seq_stats(const moe_config &c, const float *logits, const float *offset,
                            const int32_t *idx, const int32_t *seg_off, int n_seg, float beta,
                            float *scores, float *f_seq, float *p_seq, float *loss,
                            hipStream_t s);
hipError_t launch_device_stats(const moe_config &c, const float *f, const float *P, int n_dev,
                               float alpha2, float *f_dev, float *P_dev, float *loss,
                               hipStream_t s);
hipError_t launch_bias_update(const moe_config &c, const int32_t *counts, long long n_tok,
                              float alpha, float *bias, hipStream_t s);
// logits: [T][N'] fp32, or `splits` partial sums stride floats apart
// (added in split order); lg_out: where to write the summed raw logits, or
// NULL.  hist_part: int32 [select_blocks][N'] scratch; p_partial:
// [select_blocks + 1][N'] doubles or NULL (the last row receives the
// batch's score sums); counts: [N'] out.
hipError_t launch_select(const moe_config &c, const float *logits, int splits, size_t stride,
                         float *lg_out, const float *offset, const float *bias, int32_t *idx,
                         float *w, int32_t *counts, double *p_partial, int32_t *hist_part,
                         hipStream_t s);
hipError_t launch_hash_route(const moe_config &c, const uint32_t *tid, int32_t *idx,
                             float *w, int32_t *counts, hipStream_t s);
hipError_t launch_fill_i32(int32_t *p, int n, int32_t v, hipStream_t s);
// p_sum: [N'] score sums of the batch (row select_blocks of p_partial) or NULL
hipError_t launch_balance_stats(const moe_config &c, const int32_t *counts, const double *p_sum,
                                float alpha1, float *f, float *P, float *loss, hipStream_t s);
int select_blocks(const moe_config &c);   // blocks of the select kernel

// Whether a group's hidden activation z is stored as two bf16 planes
// (hi = bf16(z), lo = bf16(z - hi)) so that the down projection sees z to
// about 16 significant bits: done where the gate is 1 (the shared experts,
// and routed experts when K' = 1), since there a bf16 rounding of z would
// reach h unscaled.
inline bool z_split_shared(const moe_config &c) { return c.dtype == MOE_BF16 && c.n_shared > 0; }
inline bool z_split_routed(const moe_config &c) { return c.dtype == MOE_BF16 && c.top_k == 1; }
// The shared group's down projection in fp16 instead of the (hi, lo) pass:
// z rounded once to fp16 (11 significant bits, 8 times bf16's precision)
// against W2 converted to fp16, which halves the shared group's down work.
// Used where the shared group has more than 128 rows (fewer: the folded
// (hi, lo) tile below), as long as fp16 holds every value of z and W2.
inline bool shared_f16(const moe_config &c) {
    return c.dtype == MOE_BF16 && c.n_shared > 0 && c.T > 128;
}

FwdLayout fwd_layout(const moe_config &c);
TileShape tile_shape(const moe_config &c);
hipError_t launch_permute(const moe_config &c, const FwdLayout &L, const int32_t *idx,
                          const float *topk_w, char *ws, hipStream_t s);
hipError_t launch_gate_up(const moe_config &c, const GroupedArgs &a, hipStream_t s);
hipError_t launch_down(const moe_config &c, const GroupedArgs &a, hipStream_t s);
hipError_t launch_combine(const moe_config &c, const void *x, const int32_t *idx,
                          const float *yr, const float *ys, const uint16_t *yrh,
                          const uint16_t *ysh, void *h, hipStream_t s);

int device_cu_count();

}  // namespace moe
