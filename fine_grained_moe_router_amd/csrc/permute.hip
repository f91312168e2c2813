// permute.hip -- expert histogram, prefix scan and stable permutation of the
// (token, slot) pairs into expert-contiguous order, plus the work lists of
// the two grouped expert GEMMs.  Everything stays on the device: no count
// ever travels to the host.
//
// The gate matrix g of the DeepSeekMoE notes is sparse (K' non-zeros per
// token, top-k gate equation); it arrives as topk_idx[T][K'].  Pair
// p = t K' + k.  Expert e's rows are the pairs with topk_idx == e in
// ascending p (a stable counting sort): chunk histograms, a scan over
// (expert, chunk), then a per-chunk placement pass.
#include "common.h"

namespace moe {

// Pairs per chunk: a multiple of 64, at most 256 chunks (small batches get
// 64-pair chunks, so the placement pass has several blocks and short scans).
static int perm_chunk(int pairs) {
    int per = (pairs + 255) / 256;
    per = ((per + 63) / 64) * 64;
    return per < 64 ? 64 : per;
}

TileShape tile_shape(const moe_config &c) {
    if (c.dtype == MOE_BF16) return TileShape{256, 128, 256, 256};
    return TileShape{64, 32, 64, 64};
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

FwdLayout fwd_layout(const moe_config &c) {
    FwdLayout L;
    const size_t P = (size_t)c.T * c.top_k;
    const size_t eb = c.dtype == MOE_BF16 ? 2 : 4;
    L.chunk = perm_chunk((int)P);
    L.n_chunks = (int)((P + L.chunk - 1) / L.chunk);
    L.G = c.n_routed + (c.n_shared > 0 ? 1 : 0);
    size_t o = 0;
    L.off_chunk = o;
    o = align256(o + (size_t)L.n_chunks * c.n_routed * 4);
    L.off_meta = o;
    o = align256(o + (size_t)meta_index(L.G).size * 4);
    L.off_perm = o;
    o = align256(o + P * 4);
    L.off_gsort = o;
    o = align256(o + P * 4);
    // row tiles: sum over groups of ceil(rows / bm1) <= P / bm1 + G, plus the
    // shared group's T / bm1 + 1
    const TileShape ts = tile_shape(c);
    L.max_row_tiles = (int)(P / ts.bm1) + L.G + (int)(c.T / ts.bm1) + 2;
    L.off_rtd = o;
    o = align256(o + (size_t)L.max_row_tiles * sizeof(RowTileDesc));
    L.off_zr = o;
    o = align256(o + P * c.d_ff * eb * (z_split_routed(c) ? 2 : 1));
    L.off_zs = o;
    o = align256(o + (size_t)c.T * c.n_shared * c.d_ff_shared * eb * (z_split_shared(c) ? 2 : 1));
    L.off_yr = o;
    o = align256(o + P * c.d_model * 4);
    L.off_ys = o;
    o = align256(o + (size_t)(c.n_shared > 0 ? c.T : 0) * c.d_model * 4);
    const size_t hb = c.dtype == MOE_BF16 ? 2 : 0;   // fp16 staging, bf16 layers only
    L.off_yrh = o;
    o = align256(o + P * c.d_model * hb);
    L.off_ysh = o;
    o = align256(o + (size_t)(c.n_shared > 0 ? c.T : 0) * c.d_model * hb);
    const bool f16 = shared_f16(c);
    L.off_zs16 = o;
    o = align256(o + (f16 ? (size_t)c.T * c.n_shared * c.d_ff_shared * 2 : 0));
    L.off_w2s16 = o;
    o = align256(o + (f16 ? (size_t)c.n_shared * c.d_model * c.d_ff_shared * 2 : 0));
    L.total = o;
    return L;
}

// Per-chunk histogram of routed expert ids.  Out-of-range ids are counted
// in meta[bad] and otherwise ignored.
__global__ __launch_bounds__(256) void k_perm_hist(int P, int N, int chunk,
                                                   const int32_t *__restrict__ idx,
                                                   int32_t *__restrict__ cc,
                                                   int32_t *__restrict__ bad) {
    extern __shared__ int32_t h[];
    for (int e = threadIdx.x; e < N; e += blockDim.x) h[e] = 0;
    __syncthreads();
    const int p0 = blockIdx.x * chunk, p1 = min(P, p0 + chunk);
    int nbad = 0;
    for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
        const int e = idx[p];
        if (e >= 0 && e < N) atomicAdd(&h[e], 1);
        else ++nbad;
    }
    if (nbad) atomicAdd(bad, nbad);
    __syncthreads();
    for (int e = threadIdx.x; e < N; e += blockDim.x) cc[(size_t)blockIdx.x * N + e] = h[e];
}

// Exclusive scan of data[0..n) (n <= 2 * blockDim.x, blockDim.x a multiple
// of 64) held in LDS; returns the total.  Each thread adds a pair, each
// wavefront scans its 64 pair sums with lane shuffles, and the first
// wavefront scans the wavefront totals: four barriers in all.  tmp:
// blockDim.x / 64 ints of LDS.
__device__ int block_excl_scan(int32_t *data, int n, int32_t *tmp) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, nw = blockDim.x >> 6;
    const int a = (2 * t < n) ? data[2 * t] : 0;
    const int b = (2 * t + 1 < n) ? data[2 * t + 1] : 0;
    int v = a + b;   // inclusive scan of the pair sums within the wavefront
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    if (lane == 63) tmp[w] = v;
    __syncthreads();
    if (w == 0) {    // inclusive scan of the wavefront totals
        int s = (lane < nw) ? tmp[lane] : 0;
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(s, o, 64);
            if (lane >= o) s += u;
        }
        if (lane < nw) tmp[lane] = s;
    }
    __syncthreads();
    const int excl = (w ? tmp[w - 1] : 0) + v - (a + b);
    const int total = tmp[nw - 1];
    __syncthreads();   // tmp is free again
    if (2 * t < n) data[2 * t] = excl;
    if (2 * t + 1 < n) data[2 * t + 1] = excl + a;
    __syncthreads();
    return total;
}

// Rows per row tile of a group of cnt rows in R tiles of at most bm rows:
// the rows are dealt out evenly in 32-row fragments (the expert GEMMs'
// row_tile); the last tile holds the rest.
__device__ __forceinline__ int tile_rows(int cnt, int R, int bm) {
    return min(bm, 32 * ((cnt + 32 * R - 1) / (32 * R)));
}

// Per-XCD row-tile ranges of one GEMM, balanced by estimated cost: a row
// tile with r valid rows costs nt (2 + ceil(r / 64)) (nt column tiles, each
// streaming its weight tile and issuing MFMAs for ceil(r / 64) 64-row
// slices), with nt scaled by the group's relative K where it differs.  Row
// tile i of group g starts at cost gcost_base[g] + i nt (2 + ceil(rpt / 64))
// (all but a group's last row tile hold rpt rows).  XCD x takes the row
// tiles whose start cost lies in [x C / 8, (x + 1) C / 8).
__device__ void xcd_splits(int G, int bm, const int32_t *cnt, const int32_t *mtb,
                           const int32_t *ntg, int32_t *gcost, int32_t *tmp, int32_t *out) {
    for (int g = threadIdx.x; g < G; g += blockDim.x) {
        const int mt = mtb[g + 1] - mtb[g];
        const int rpt = mt > 0 ? tile_rows(cnt[g], mt, bm) : 0;
        const int last = cnt[g] - (mt - 1) * rpt;
        gcost[g] = mt > 0 ? ntg[g] * (2 * mt + (mt - 1) * ((rpt + 63) / 64) + (last + 63) / 64) : 0;
    }
    __syncthreads();
    const int C = block_excl_scan(gcost, G, tmp);   // gcost now holds the group start costs
    const int M = mtb[G];
    if (threadIdx.x <= 8) out[threadIdx.x] = (threadIdx.x == 0) ? 0 : M;
    __syncthreads();
    for (int m = threadIdx.x; m < M; m += blockDim.x) {
        int lo = 0, hi = G;   // mtb[lo] <= m < mtb[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (mtb[mid] <= m) lo = mid;
            else hi = mid;
        }
        const int rpt = tile_rows(cnt[lo], mtb[lo + 1] - mtb[lo], bm);
        const long long start =
            gcost[lo] + (long long)(m - mtb[lo]) * ntg[lo] * (2 + (rpt + 63) / 64);
        long long prev = -1;
        if (m > 0) {
            const int pm = m - 1;
            int plo = (mtb[lo] <= pm) ? lo : lo - 1;
            while (plo > 0 && mtb[plo] > pm) --plo;
            const int prpt = tile_rows(cnt[plo], mtb[plo + 1] - mtb[plo], bm);
            prev = gcost[plo] + (long long)(pm - mtb[plo]) * ntg[plo] * (2 + (prpt + 63) / 64);
        }
        for (int x = 1; x < 8; ++x) {
            const long long target = (long long)x * C / 8;
            if (start >= target && prev < target) out[x] = m;
        }
    }
    __syncthreads();
}

// Chunk bases: block e turns expert e's chunk counts into exclusive prefix
// sums over the chunks (the row of each chunk's first pair of e, relative
// to the expert) and leaves the expert's row count in group_cnt[e].  At most
// 256 chunks (perm_chunk), one per thread.
__global__ __launch_bounds__(256) void k_chunk_scan(int N, int n_chunks, int32_t *__restrict__ cc,
                                                    int32_t *__restrict__ group_cnt) {
    __shared__ int32_t v[256];
    const int e = blockIdx.x, c = threadIdx.x;
    const int x = (c < n_chunks) ? cc[(size_t)c * N + e] : 0;
    v[c] = x;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {   // inclusive scan
        const int y = (c >= o) ? v[c - o] : 0;
        __syncthreads();
        v[c] += y;
        __syncthreads();
    }
    if (c < n_chunks) cc[(size_t)c * N + e] = v[c] - x;
    if (c == 255) group_cnt[e] = v[255];
}

// One block.  Computes group row counts/offsets, the tile prefix sums of
// both GEMMs, the row-tile prefix sums and the per-XCD row-tile ranges.
__global__ __launch_bounds__(1024) void k_perm_scan(int N, int T, int n_shared, int f, int fsum,
                                                    int d, int split_r, int split_s, TileShape ts,
                                                    int32_t *__restrict__ meta,
                                                    RowTileDesc *__restrict__ rtd) {
    __shared__ int32_t cnt[2048], t1[2048], t2[2048], tmp[1024];
    __shared__ int32_t mtb[2048], nt1[2048], nt2[2048], gcost[2048];
    const int G = N + (n_shared > 0 ? 1 : 0);
    const MetaIdx mi = meta_index(G);
    for (int e = threadIdx.x; e < 2048; e += blockDim.x) {
        cnt[e] = 0;
        t1[e] = 0;
        t2[e] = 0;
    }
    __syncthreads();
    // group row counts (the chunk scan left each routed expert's total)
    for (int e = threadIdx.x; e < N; e += blockDim.x) cnt[e] = meta[mi.group_cnt + e];
    if (threadIdx.x == 0 && n_shared > 0) cnt[N] = T;
    __syncthreads();
    const int ntn2 = (d + ts.bn2 - 1) / ts.bn2;
    // The down GEMM's K differs between groups (d_ff for a routed expert,
    // K_s d_ff_s for the shared group, doubled for a (hi, lo) split): its
    // row-tile cost scales with K relative to the routed K (capped at 64).
    const int k_routed = f * (split_r ? 2 : 1);
    const int k_shared = fsum * (split_s ? 2 : 1);
    const int kfac_shared = min(64, (k_shared + k_routed - 1) / k_routed);
    for (int g = threadIdx.x; g < G; g += blockDim.x) {
        const int c = cnt[g];
        const int width = (g < N) ? f : fsum;
        nt1[g] = (width + ts.bz1 - 1) / ts.bz1;
        nt2[g] = ntn2 * ((g < N) ? 1 : kfac_shared);
        t1[g] = ((c + ts.bm1 - 1) / ts.bm1) * nt1[g];
        t2[g] = ((c + ts.bm2 - 1) / ts.bm2) * ntn2;
        mtb[g] = (c + ts.bm1 - 1) / ts.bm1;
        meta[mi.group_cnt + g] = c;
    }
    __syncthreads();
    const int tot1 = block_excl_scan(t1, G, tmp);
    const int tot2 = block_excl_scan(t2, G, tmp);
    const int totm = block_excl_scan(mtb, G, tmp);
    if (threadIdx.x == 0) mtb[G] = totm;
    __syncthreads();
    for (int g = threadIdx.x; g <= G; g += blockDim.x) meta[mi.mt + g] = mtb[g];
    xcd_splits(G, ts.bm1, cnt, mtb, nt1, gcost, tmp, meta + mi.xs1);
    xcd_splits(G, ts.bm1, cnt, mtb, nt2, gcost, tmp, meta + mi.xs2);
    // row offsets of the routed groups (the shared group reads rows 0..T-1)
    if (threadIdx.x == 0 && n_shared > 0) cnt[N] = 0;
    __syncthreads();
    block_excl_scan(cnt, N, tmp);
    for (int g = threadIdx.x; g < G; g += blockDim.x) {
        const int goff = (g < N) ? cnt[g] : 0;
        meta[mi.group_off + g] = goff;
        meta[mi.tile1 + g] = t1[g];
        meta[mi.tile2 + g] = t2[g];
        RowTileDesc dsc;
        dsc.g = g;
        dsc.mt0 = mtb[g];
        dsc.R = mtb[g + 1] - mtb[g];
        dsc.cnt = meta[mi.group_cnt + g];  // this thread's own earlier store
        dsc.goff = goff;
        dsc.pad[0] = dsc.pad[1] = dsc.pad[2] = 0;
        for (int m = mtb[g]; m < mtb[g + 1]; ++m) rtd[m] = dsc;
    }
    if (threadIdx.x == 0) {
        meta[mi.tile1 + G] = tot1;
        meta[mi.tile2 + G] = tot2;
    }
}

// Stable placement, one wavefront per chunk.  The chunk's pairs are taken
// 64 at a time in pair order, one per lane.  A lane whose pair chose expert
// e writes it (and its gate) to row
//     group_off[e] + (pairs of e in earlier chunks) + (pairs of e before it
//     in this chunk),
// the last term being a running count per expert in LDS plus the number of
// lower lanes in the same 64 that chose e.  The lanes that chose e are found
// by matching e bit by bit, one ballot per bit of N' - 1; the highest of them
// then advances e's count.  Out-of-range ids are skipped.
__global__ __launch_bounds__(64) void k_perm_scatter(int P, int N, int chunk,
                                                     const int32_t *__restrict__ idx,
                                                     const float *__restrict__ topk_w,
                                                     const int32_t *__restrict__ cc,
                                                     const int32_t *__restrict__ group_off,
                                                     int32_t *__restrict__ perm,
                                                     float *__restrict__ gsort) {
    extern __shared__ int32_t next_row[];   // [N']
    const int lane = threadIdx.x;
    for (int e = lane; e < N; e += 64)
        next_row[e] = group_off[e] + cc[(size_t)blockIdx.x * N + e];
    __syncthreads();
    const int bits = N > 1 ? 32 - __clz(N - 1) : 0;
    const uint64_t below = (1ull << lane) - 1;
    const int p0 = blockIdx.x * chunk, p1 = min(P, p0 + chunk);
    int p = p0 + lane;
    int e = p < p1 ? idx[p] : -1;
    float g = p < p1 ? topk_w[p] : 0.f;
    for (int base = p0; base < p1; base += 64, p += 64) {
        // the next 64 pairs' loads are in flight while these are placed
        const int pn = p + 64;
        const int en = pn < p1 ? idx[pn] : -1;
        const float gn = pn < p1 ? topk_w[pn] : 0.f;
        const bool ok = e >= 0 && e < N;
        uint64_t same = __ballot(ok);
        for (int b = 0; b < bits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t m = __ballot(ok && bit);
            same &= bit ? m : ~m;
        }
        if (ok) {
            const int row = next_row[e] + __popcll(same & below);
            perm[row] = p;
            gsort[row] = g;
            if ((same >> lane) == 1ull) next_row[e] = row + 1;   // highest lane of e's set
        }
        e = en;
        g = gn;
    }
}

hipError_t launch_permute(const moe_config &c, const FwdLayout &L, const int32_t *idx,
                          const float *topk_w, char *ws, hipStream_t s) {
    const int P = c.T * c.top_k;
    const int N = c.n_routed;
    int32_t *cc = (int32_t *)(ws + L.off_chunk);
    int32_t *meta = (int32_t *)(ws + L.off_meta);
    const MetaIdx mi = meta_index(L.G);
    hipError_t e = launch_fill_i32(meta + mi.q1, mi.f16bad + 1 - mi.q1, 0, s);   // q1, q2, bad, f16bad
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_perm_hist, dim3(L.n_chunks), dim3(256), (size_t)N * 4, s, P, N, L.chunk,
                       idx, cc, meta + mi.bad);
    hipLaunchKernelGGL(k_chunk_scan, dim3(N), dim3(256), 0, s, N, L.n_chunks, cc,
                       meta + mi.group_cnt);
    hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, s, N, c.T, c.n_shared, c.d_ff,
                       c.n_shared * c.d_ff_shared, c.d_model, z_split_routed(c) ? 1 : 0,
                       // the shared group's down K: one fp16 pass, or the (hi, lo) pair
                       (z_split_shared(c) && !shared_f16(c)) ? 1 : 0, tile_shape(c), meta,
                       (RowTileDesc *)(ws + L.off_rtd));
    hipLaunchKernelGGL(k_perm_scatter, dim3(L.n_chunks), dim3(64), (size_t)N * 4, s, P, N,
                       L.chunk, idx, topk_w, cc, meta + mi.group_off, (int32_t *)(ws + L.off_perm),
                       (float *)(ws + L.off_gsort));
    return hipGetLastError();
}

}  // namespace moe
