// expert_gemm.hip -- the grouped expert contractions of the DeepSeekMoE layer.
//
// Every routed expert and the shared experts are SwiGLU FFNs,
// W2 (SiLU(W1 u) * (W3 u)) (the 3-matrix form named in the MoE tutorial at
// ai.clawlihai.cn); the layer is the "core design 2" equation of the
// DeepSeekMoE notes.  Two launches:
//   gate/up:  z = SiLU(X_e W1_e^T) * (X_e W3_e^T)   for each group e
//   down:     y = z W2_e^T (routed rows scaled by their gate)
// Group e < N' owns the pairs routed to expert e (rows gathered from x on
// load, in the expert-contiguous order built by permute.hip).  Group N'
// holds all K_s shared experts at once: every token is a row, and the K_s
// hidden blocks of width d_ff_shared sit side by side (K_s shared experts
// of width f act as one of width K_s f), so the down projection sums them
// inside one K loop.
//
// Scheduling: persistent blocks, one per CU.  The bf16 kernels pull
// (row tile, column tile) items from per-XCD work queues (see "Work queue"
// below).  The fp32 kernels (64-row tiles, SIMT) order their tiles (group,
// row tile, column tile) with the column tile fastest, so the column tiles
// that share token rows are adjacent; the range is cut into 8 contiguous
// pieces, one per XCD (block b runs on XCD b % 8), and every block strides
// through its XCD's piece.
#include "common.h"
#include "mfma_pipe.h"
#include "simt_tile.h"

namespace moe {

__device__ __forceinline__ int find_group(const int32_t *__restrict__ base, int G, int tile) {
    int lo = 0, hi = G;  // base[lo] <= tile < base[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (base[mid] <= tile) lo = mid;
        else hi = mid;
    }
    return lo;
}

struct TileJob {
    int g, i, j, row0, nrows, goff;
    bool shared;
    bool single;    // the group's only row tile
};

// Whether a tile's weight loads are non-temporal: when its group has a
// single row tile, no other tile reads its weight tile, so its weight lines
// need not be kept for reuse.  The bytes fetched past L2 stay the same; what
// changes is beyond L2 (the Infinity Cache's allocation, which the L2
// counters do not separate from HBM): thin-tile launches run 7-10% faster.
__device__ __forceinline__ bool streams_weights(const TileJob &tj) { return tj.single; }

__device__ __forceinline__ TileJob decode_tile(const GroupedArgs &a, int tile, int bm) {
    TileJob t;
    t.g = find_group(a.tile_base, a.G, tile);
    const int rel = tile - a.tile_base[t.g];
    const int cnt = a.group_cnt[t.g];
    const int mt = (cnt + bm - 1) / bm;
    const int nt = (a.tile_base[t.g + 1] - a.tile_base[t.g]) / mt;
    t.i = rel / nt;               // column tile fastest: column tiles sharing rows adjacent
    t.j = rel - t.i * nt;
    t.row0 = t.i * bm;
    t.nrows = min(bm, cnt - t.row0);
    t.shared = (t.g == a.n_routed);
    t.single = (mt == 1);
    t.goff = t.shared ? 0 : a.group_off[t.g];
    return t;
}

// Block b's share of the logical tiles: XCD b % 8 takes one contiguous
// eighth; its blocks stride through it.
struct TileRange {
    int first, end, step;
};
__device__ __forceinline__ TileRange tile_range(int total) {
    const int xcd = blockIdx.x % kXcds;
    const int slot = blockIdx.x / kXcds;
    const int nslots = gridDim.x / kXcds;
    const int per = (total + kXcds - 1) / kXcds;
    const int start = xcd * per;
    TileRange r;
    r.first = start + slot;
    r.end = min(total, start + per);
    r.step = nslots;
    return r;
}

// ---------------------------------------------------------------- bf16 MFMA



// Work queue of the bf16 kernels.  XCD x owns the row tiles
// [xsplit[x], xsplit[x+1]) (balanced by cost); its work items are the
// (row tile, column tile) pairs of that range.  The blocks of the XCD pull
// items in order from the XCD's counter, so the blocks busy at any moment
// hold consecutive items and share their operands through the XCD's L2;
// pulling also balances tiles of unequal cost (a block whose XCD has no
// items left takes them from the other XCDs' queues).  Item order within a
// group: a routed expert with at most kColMajorRows row tiles in the range
// lists them row tile fastest -- its row tiles that stream the same weight
// tile start together, and its 16 (gate/up) or 28 (down) column tiles take
// at most one XCD's worth of blocks.  A longer group (the shared experts, a
// Zipf-hot expert with up to 25 row tiles at the V4 shape) is listed in
// panels of kPanelRows row tiles x kPanelCols column tiles, 64 items, two
// rounds of one XCD's blocks: the blocks that run together share a few
// token-row tiles and weight tiles through the XCD's L2, and a weight tile
// is streamed once per 8 row tiles instead of once per row tile.
// Interleaved A/B: 4 x 8 panels against column-fastest order, V4 skew
// gate/up -4.3%, down -3%, V3 prefill gate/up -0.8%; then 8 x 8 against
// 4 x 8, gate/up -1% (V4 skew, V3 prefill) and -3% (the 16B shape's shared
// experts), down within noise.
constexpr int kColMajorRows = 4;
constexpr int kPanelRows = 8, kPanelCols = 8;

struct XcdQueue {
    int m0, ms, m1, ntr, nts, nr_items, total;
};
__device__ __forceinline__ XcdQueue xcd_queue(const GroupedArgs &a, int x) {
    XcdQueue q;
    q.m0 = a.xsplit[x];
    q.m1 = a.xsplit[x + 1];
    // the shared group (if any) is the last group: its row tiles come last
    const int first_shared = a.mt_base[a.n_routed];
    q.ms = min(max(first_shared, q.m0), q.m1);
    q.ntr = a.nt_routed;
    q.nts = a.nt_shared;
    q.nr_items = (q.ms - q.m0) * q.ntr;
    q.total = q.nr_items + (q.m1 - q.ms) * q.nts;
    return q;
}
// Item -> (row tile m, column tile j, the group's descriptor).  The routed
// items of a group with rows lo .. lo + r - 1 of the range are items
// (lo - m0) nt ... + r nt - 1.
__device__ __forceinline__ void queue_item(const GroupedArgs &a, const XcdQueue &q, int item,
                                           int &m, int &j, RowTileDesc &d) {
    int lo, r, local, nt;
    if (item < q.nr_items) {
        nt = q.ntr;
        d = a.rtd[q.m0 + item / nt];
        lo = max(d.mt0, q.m0);
        r = min(d.mt0 + d.R, q.ms) - lo;
        local = item - (lo - q.m0) * nt;
    } else {
        nt = q.nts;
        lo = q.ms;
        r = q.m1 - q.ms;
        local = item - q.nr_items;
        d = a.rtd[q.ms];
    }
    if (item < q.nr_items && r <= kColMajorRows) {
        j = local / r;
        m = lo + (local - j * r);
    } else {
        // panel rb of (up to) kPanelRows row tiles spans all nt column tiles
        // in blocks of kPanelCols; inside a block the row tile runs fastest
        const int rb = local / (kPanelRows * nt);
        const int pr = min(kPanelRows, r - rb * kPanelRows);
        const int idx = local - rb * kPanelRows * nt;
        const int cb = idx / (pr * kPanelCols);
        const int k = idx - cb * pr * kPanelCols;
        m = lo + rb * kPanelRows + k % pr;
        j = cb * kPanelCols + k / pr;
    }
}

// Tickets.  Right after the K loop of a tile (and once before the first),
// thread 0 takes a ticket from the counter of queue (x + k) % 8 (x: the
// block's XCD; k: how many queues the block has moved past its own, 0 while
// the XCD's own range lasts).  A ticket past that queue's end moves it on to
// the next queue -- work stealing once the XCD's own range is drained --
// until it holds an item or every queue is drained.  Taking the ticket only
// when the block is free (rather than one tile ahead) makes the order in
// which items start follow the queue order, which keeps consecutive items
// close in time (EA read traffic of the V3 gate/up launch 33.4 -> 31.1 GB).
// The ticket's atomic is issued right after the K loop and its result first
// used after the epilogue's stores, so its latency hides behind them.  The
// item (queue << 24 | index, or -1) reaches the other threads through one
// LDS word in the last B stage, after the down projection's row info
// (tile_info_offset): after the K loop no wave reads that stage (the
// epilogues stage their tiles in the others), and the next tile first writes
// it after the top barrier of its first k-tile, which every wave reaches
// only after it has read the word.
//
// The stealing state k is never kept per thread: every thread derives it
// from the item just published (queue_step), so all waves hold the same
// value and take the same branches.  A version that kept k in a per-thread
// variable advanced by thread 0 alone, and read it in every thread, faulted
// once stealing began: the waves took different paths around a barrier and
// read an LDS word that thread 0 had not written.
constexpr int kItemBits = 24;

// Row info of a down tile (pair id and gate of each of its rows) and then
// the queue word, in the last B stage.
template <class P>
constexpr int tile_info_offset() {
    static_assert(P::NT >= P::BM, "one tile row per thread");
    static_assert(P::BM * 8 + 4 <= P::B_STAGE, "row info and queue word fit one B stage");
    static_assert(P::A_STAGES * P::A_STAGE + (P::B_STAGES - 1) * P::B_STAGE >= P::BM * P::BN * 2,
                  "an fp16 output tile fits the stages before the last");
    return P::A_STAGES * P::A_STAGE + (P::B_STAGES - 1) * P::B_STAGE;
}
template <class P>
constexpr int queue_slot_offset() { return tile_info_offset<P>() + 8 * P::BM; }

// Queues moved past the block's own (0..7) to reach a published item; 8
// once every queue is drained (item -1).  The same in every thread.
__device__ __forceinline__ int queue_step(int item) {
    if (item < 0) return kXcds;
    return ((item >> kItemBits) - (int)(blockIdx.x % kXcds) + kXcds) % kXcds;
}
// Thread 0: the first ticket of a pull from queue step k (a counter value;
// unused once every queue is drained, k == kXcds).
__device__ __forceinline__ int take_ticket(const GroupedArgs &a, int k) {
    return (k < kXcds) ? atomicAdd(a.queue + (blockIdx.x % kXcds + k) % kXcds, 1) : 0;
}
// Thread 0: the item a pull ends with, from its first ticket; a ticket past
// its queue's end moves on to the next queue with a new ticket.
__device__ __forceinline__ int resolve_ticket(const GroupedArgs &a, int k, int ticket) {
    const int x = blockIdx.x % kXcds;
    while (k < kXcds) {
        const int y = (x + k) % kXcds;
        if (ticket < xcd_queue(a, y).total) return (y << kItemBits) | ticket;
        if (++k < kXcds) ticket = atomicAdd(a.queue + (x + k) % kXcds, 1);
    }
    return -1;
}
// Called by every thread with thread 0's first ticket of the pull from
// queue step k; returns the item to every thread.
template <class P>
__device__ __forceinline__ int publish_item(char *lds, const GroupedArgs &a, int k, int ticket) {
    int32_t *slot = (int32_t *)(lds + queue_slot_offset<P>());
    if (threadIdx.x == 0) *slot = resolve_ticket(a, k, ticket);
    lds_barrier();
    return __builtin_amdgcn_readfirstlane(*slot);
}
template <class P>
__device__ __forceinline__ int first_item(char *lds, const GroupedArgs &a) {
    const int ticket = threadIdx.x == 0 ? take_ticket(a, 0) : 0;
    return publish_item<P>(lds, a, 0, ticket);
}
__device__ __forceinline__ void item_tile(const GroupedArgs &a, int item, int &m, int &j,
                                          RowTileDesc &d) {
    const XcdQueue q = xcd_queue(a, item >> kItemBits);
    queue_item(a, q, item & ((1 << kItemBits) - 1), m, j, d);
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Transposed accumulators (TR) hold, in lanes l and l + 32, the two 4-column
// halves of each 8-column chunk q of one row (pk[q][0..1]: two packed
// 16-bit values each).  Exchange them so that lane l holds chunks 0 and 2
// whole and lane l + 32 chunks 1 and 3: chunk qp + (l >> 5) is then
// {pk[qp][0], pk[qp][1], pk[qp + 1][0], pk[qp + 1][1]} for qp = 0, 2.
// permlane32_swap trades the upper 32 lanes of its first operand with the
// lower 32 lanes of its second.  Every lane of the wave must take part.
__device__ __forceinline__ void swap_tr_halves(uint32_t (&pk)[4][2]) {
#pragma unroll
    for (int qp = 0; qp < 4; qp += 2)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const auto sw = __builtin_amdgcn_permlane32_swap(pk[qp][w], pk[qp + 1][w], false, false);
            pk[qp][w] = sw[0];
            pk[qp + 1][w] = sw[1];
        }
}
__device__ __forceinline__ u32x4 tr_chunk(const uint32_t (&pk)[4][2], int qp) {
    return u32x4{pk[qp][0], pk[qp][1], pk[qp + 1][0], pk[qp + 1][1]};
}

// 4x4 transpose across the four lanes of a quad (lanes 4q .. 4q+3): on
// entry lane p holds column p of the block (v[r] = M[r][p]), on exit row p
// (v[c] = M[p][c]).  Two exchange stages, lane ^ 1 then lane ^ 2, with DPP
// quad permutations.
__device__ __forceinline__ float quad_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ void quad_transpose(float (&v)[4], int p) {
#pragma unroll
    for (int k = 0; k < 4; k += 2) {
        const float got = quad_xor1((p & 1) ? v[k] : v[k + 1]);
        if (p & 1) v[k] = got;
        else v[k + 1] = got;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float got = quad_xor2((p & 2) ? v[k] : v[k + 2]);
        if (p & 2) v[k] = got;
        else v[k + 2] = got;
    }
}

// Output row of a lane after quad_transpose of accumulator registers
// 4 rq .. 4 rq + 3 of fragment i (its four consecutive columns start at
// pipe_out_col(tid, j) & ~3).
template <class P>
__device__ __forceinline__ int quad_row(int tid, int i, int rq) {
    const int lane = tid & 63;
    return P::a_row(P::wave_m(tid), i) + rq * 8 + (lane >> 5) * 4 + (lane & 3);
}

__device__ __forceinline__ uint2 pack_bf16x4(const float (&v)[4]) {
    uint2 o;
    o.x = pack_bf16x2(v[0], v[1]);
    o.y = pack_bf16x2(v[2], v[3]);
    return o;
}

// One gate/up tile whose wave computes NF row fragments (STREAM_B: its
// weight tile is read by no other tile).
template <class P, int NF, bool STREAM_B>
__device__ __forceinline__ int gate_up_tile(const GroupedArgs &a, const TileJob &tj, char *lds,
                                            const OperandRows<P> &rows, int zc0, int zw,
                                            size_t rbase, int k) {
    f32x16 acc[NF > 0 ? NF : 1][P::FN];
    pipe_gemm_nf<P, true, NF, false, STREAM_B>(lds, rows, a.d, 0, 1, 0, 0, acc);
    const int ticket = threadIdx.x == 0 ? take_ticket(a, k) : 0;
    // SwiGLU epilogue: z = SiLU(W1 u) * (W3 u) in fp32 (the sigmoid from the
    // hardware exponential and reciprocal, each within about an ulp), rounded
    // to bf16 (hi); for a split group the residual z - hi goes, rounded, zw
    // columns further.
    // Four rows' z of one column are transposed across a lane quad so each
    // lane stores four consecutive columns of one row (8 bytes).
    uint16_t *zout = (uint16_t *)(tj.shared ? a.zs : a.zr);
    const int split = tj.shared ? a.split_s : a.split_r;
    const size_t zstride = (size_t)zw * (split ? 2 : 1);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
#pragma unroll
        for (int jp = 0; jp < P::FN / 2; ++jp) {
            const int tid = opaque_tid();
            const int col = zc0 + (pipe_out_col<P, true>(tid, jp) & ~3);
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                float z[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float ga = acc[i][jp][4 * rq + q];              // W1 (gate) fragment
                    const float up = acc[i][jp + P::FN / 2][4 * rq + q];  // W3 (up) fragment
                    z[q] = ga * __builtin_amdgcn_rcpf(1.0f + __expf(-ga)) * up;
                }
                quad_transpose(z, tid & 3);
                const int row = quad_row<P>(tid, i, rq);
                if (row < tj.nrows && col < zw) {
                    uint16_t *dst = zout + (rbase + row) * zstride + col;
                    const uint2 hi = pack_bf16x4(z);
                    *(uint2 *)dst = hi;
                    if (split) {
                        float lo[4];
                        lo[0] = z[0] - bf16_to_f32((uint16_t)(hi.x & 0xFFFF));
                        lo[1] = z[1] - bf16_to_f32((uint16_t)(hi.x >> 16));
                        lo[2] = z[2] - bf16_to_f32((uint16_t)(hi.y & 0xFFFF));
                        lo[3] = z[3] - bf16_to_f32((uint16_t)(hi.y >> 16));
                        *(uint2 *)(dst + zw) = pack_bf16x4(lo);
                    }
                    if (tj.shared && a.shared_f16) {
                        // z once more as fp16, for the shared group's fp16
                        // down pass; a value fp16 cannot hold flags it off
                        uint16_t h[4];
                        bool over = false;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            over |= !(fabsf(z[q]) < 65520.0f);
                            h[q] = __builtin_bit_cast(uint16_t, (_Float16)z[q]);
                        }
                        *(uint2 *)(a.zs16 + (rbase + row) * zw + col) =
                            make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
                        if (over) atomicOr(a.f16bad, 1);
                    }
                }
            }
            // keep one fragment pair live at a time
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    return publish_item<P>(lds, a, k, ticket);
}

// Row tile m.  A group of cnt rows has R = ceil(cnt / bm) row tiles; its
// rows are dealt out evenly in whole 32-row fragments: every tile but the
// last holds rpt = 32 ceil(cnt / (32 R)) rows (rpt <= bm, and the last tile
// is never empty).  The row tiles of one group then carry the same MFMA
// work and run at the same speed, so the tiles that stream one weight tile
// -- adjacent in the queue -- stay close enough for the later ones to find
// it in L2 (EA read traffic of the V3 gate/up launch 32.0 -> 25.7 GB).
__device__ __forceinline__ TileJob row_tile(const GroupedArgs &a, const RowTileDesc &d, int m,
                                           int bm) {
    TileJob t;
    t.g = d.g;
    t.i = m - d.mt0;
    t.j = 0;
    const int cnt = d.cnt;
    const int R = d.R;
    const int rpt = min(bm, 32 * ((cnt + 32 * R - 1) / (32 * R)));
    t.row0 = t.i * rpt;
    t.nrows = min(rpt, cnt - t.row0);
    t.goff = d.goff;
    t.shared = (t.g == a.n_routed);
    t.single = (R == 1);
    return t;
}

template <class P>
__device__ __forceinline__ int gate_up_body(const GroupedArgs &a, const TileJob &tj, char *lds,
                                            int k) {
    const int fsum = a.n_shared * a.fs;
    const int zw = tj.shared ? fsum : a.f;         // hidden width of the group
    const int zc0 = tj.j * (P::BN / 2);            // first hidden column of the tile
    const int goff = tj.goff;
    OperandRows<P> rows;
    rows.abase = (const uint16_t *)a.x;
#pragma unroll
    for (int l = 0; l < P::A_LD; ++l) {
        int r = P::load_row(threadIdx.x, l);
        r = (r < tj.nrows) ? r : 0;   // rows past the end are not fetched
        const int tok = tj.shared ? tj.row0 + r : a.perm[goff + tj.row0 + r] / a.top_k;
        rows.aoff[l] = (uint32_t)tok * (uint32_t)a.d;
    }
    rows.amask = valid_row_mask<P>(tj.nrows);
    rows.azero = pad_row_mask<P>(tj.nrows);
    // B rows: hidden columns zc0 .. zc0+127 of W1 (tile rows 0..127) and of
    // W3 (tile rows 128..255); the shared group's hidden columns run across
    // its K_s experts.
    rows.bbase = tj.shared ? (const uint16_t *)a.w13s
                           : (const uint16_t *)a.w13 + (size_t)tj.g * 2 * a.f * a.d;
    const int wwidth = tj.shared ? a.fs : a.f;
#pragma unroll
    for (int l = 0; l < P::B_LD; ++l) {
        const int r = P::load_row(threadIdx.x, l);
        const bool up = r >= P::BN / 2;
        int zc = zc0 + (up ? r - P::BN / 2 : r);
        zc = (zc < zw) ? zc : zw - 1;   // columns past the end: discarded
        const int js = zc / wwidth, c = zc - js * wwidth;
        rows.boff[l] = ((uint32_t)js * 2 * wwidth + (up ? wwidth : 0) + c) * (uint32_t)a.d;
    }
    const size_t rbase = tj.shared ? (size_t)tj.row0 : (size_t)goff + tj.row0;
    const bool stream_b = streams_weights(tj);
    switch (wave_frags<P>(tj.nrows) + (stream_b ? 5 : 0)) {
        case 4: return gate_up_tile<P, 4, false>(a, tj, lds, rows, zc0, zw, rbase, k);
        case 3: return gate_up_tile<P, 3, false>(a, tj, lds, rows, zc0, zw, rbase, k);
        case 2: return gate_up_tile<P, 2, false>(a, tj, lds, rows, zc0, zw, rbase, k);
        case 1: return gate_up_tile<P, 1, false>(a, tj, lds, rows, zc0, zw, rbase, k);
        case 0: return gate_up_tile<P, 0, false>(a, tj, lds, rows, zc0, zw, rbase, k);
        case 9: return gate_up_tile<P, 4, true>(a, tj, lds, rows, zc0, zw, rbase, k);
        case 8: return gate_up_tile<P, 3, true>(a, tj, lds, rows, zc0, zw, rbase, k);
        case 7: return gate_up_tile<P, 2, true>(a, tj, lds, rows, zc0, zw, rbase, k);
        case 6: return gate_up_tile<P, 1, true>(a, tj, lds, rows, zc0, zw, rbase, k);
        default: return gate_up_tile<P, 0, true>(a, tj, lds, rows, zc0, zw, rbase, k);
    }
}

template <class P>
__global__ __launch_bounds__(P::NT) void k_gate_up_bf16(const GroupedArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[P::LDS_BYTES];
    int item = first_item<P>(lds, a);
    while (item >= 0) {
        int m, j;
        RowTileDesc d;
        item_tile(a, item, m, j, d);
        TileJob tj = row_tile(a, d, m, P::BM);
        tj.j = j;
        item = gate_up_body<P>(a, tj, lds, queue_step(item));
    }
}

// Byte offset of the 16-byte chunk c (eight halves) of row `row` in an fp16
// output tile staged in LDS: rows of BN halves (BN / 8 chunks); chunk c sits
// in slot c ^ (row & 15).  The 16 lanes of one LDS pass that write one chunk
// column of 16 consecutive rows, and the 16 that read 16 consecutive chunks
// of one row, then hit 16 distinct 16-byte bank groups of the 64-bank LDS.
template <class P>
__device__ __forceinline__ int stage_chunk(int row, int c) {
    static_assert(P::BN / 8 >= 16 && (P::BN / 8) % 16 == 0, "chunk swizzle spans whole groups");
    return row * (2 * P::BN) + ((c ^ (row & 15)) << 4);
}

// fp16 of g * v for the 16 accumulator registers of one transposed fragment
// (TR layout: this lane's row, four columns per register quad), packed two
// halves per word, and then exchanged between lanes l and l + 32 (which hold
// the two 4-column halves of each 8-column chunk of the same row): lane l
// leaves with chunks 0 and 2 of the fragment's 32 columns, lane l + 32 with
// chunks 1 and 3, each whole (pk[qp][0..1], pk[qp + 1][0..1] for the chunk
// qp + (l >> 5), qp = 0, 2).  hm: running packed maximum of |half| bits of
// this lane's values (0x7C00 and up: not finite).  Every lane of the wave
// must take part (the exchange is a cross-lane move).
__device__ __forceinline__ void pack_tr_fragment(const f32x16 &v, float g, bool valid,
                                                 uint32_t (&pk)[4][2], u16x2 &hm) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const f16x2 h2 = {(_Float16)(g * v[4 * q + 2 * w]), (_Float16)(g * v[4 * q + 2 * w + 1])};
            pk[q][w] = __builtin_bit_cast(uint32_t, h2);
            const u16x2 m = __builtin_bit_cast(u16x2, valid ? (pk[q][w] & 0x7FFF7FFFu) : 0u);
            hm = __builtin_elementwise_max(hm, m);
        }
    swap_tr_halves(pk);
}

// fp32 copies of the values of one transposed fragment that fp16 cannot hold
// (rare; the combine reads them in place of the fp16 ones).
template <class P>
__device__ __forceinline__ void store_f32_marked(const f32x16 &v, float g, int tid, int j,
                                                 int ncols, float *dst_row) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int col = pipe_out_col_tr<P>(tid, j, r);
        const float w = g * v[r];
        if (col < ncols && f16_marked(__builtin_bit_cast(uint16_t, (_Float16)w))) dst_row[col] = w;
    }
}

// One down-projection tile whose wave computes NF row fragments.  Thread t
// brings the destination row and gate of tile row t (fetched before the K
// loop).  The MFMAs run transposed (TR), so a lane holds four consecutive
// output columns of one row per register quad and one gate per fragment.
// Epilogue: every wave packs fp16(gate * y) of its fragments, exchanges
// halves across the wave (pack_tr_fragment) and writes whole 16-byte chunks
// into the tile staged in LDS (the A stages and the first two B stages);
// then each wave stores two whole rows of 512 bytes at a time with 16-byte
// lane stores.  A value beyond fp16's range (rare) is also stored as fp32.
// The next item is resolved before the stores are issued, so thread 0 waits
// for the ticket's atomic alone, not for the stores' completion.
//
// FOLD: a split tile of at most 128 rows whose lo plane sits in the tile's
// rows 128-255 (row 128 + r holds lo of row r; see down_body): each W2
// k-range is read once for both planes, the wave computes its hi fragments
// i < NF and their lo partners i + 2, and y = hi part + lo part is added in
// fp32 before the epilogue.
//
// F16: the shared group's fp16 pass (z's fp16 plane against the fp16 copy
// of the shared W2, K = K_s d_ff_s).
template <class P, int NF, bool STREAM_B, bool FOLD, bool F16 = false>
__device__ __forceinline__ int down_tile(const GroupedArgs &a, const TileJob &tj, char *lds,
                                         const OperandRows<P> &rows, int K, int split, int n0,
                                         int my_pair, float my_gate, int k) {
    constexpr int NP = (FOLD && NF > 0) ? NF + 2 : NF;   // fragments the K loop spans
    constexpr int FMASK = FOLD ? ((1 << NF) - 1) * 5 : (1 << NP) - 1;
    f32x16 acc[NP > 0 ? NP : 1][P::FN];
    if constexpr (F16) {
        pipe_gemm_nf<P, false, NF, true, false, (1 << NF) - 1, true, true>(
            lds, rows, K, a.fs, a.n_shared, (size_t)a.d * a.fs, 0, acc);
    } else if constexpr (FOLD) {
        if (tj.shared)
            pipe_gemm_nf<P, false, NP, false, STREAM_B, FMASK, false, true>(
                lds, rows, K, a.fs, a.n_shared, (size_t)a.d * a.fs, 0, acc);
        else
            pipe_gemm_nf<P, false, NP, false, STREAM_B, FMASK, false, true>(lds, rows, K, 0, 1, 0, 0,
                                                                           acc);
#pragma unroll
        for (int i = 0; i < NF; ++i)
#pragma unroll
            for (int j = 0; j < P::FN; ++j) acc[i][j] += acc[i + 2][j];
    } else if (tj.shared) {
        pipe_gemm_nf<P, false, NF, true, STREAM_B, (1 << NF) - 1, false, true>(
            lds, rows, K, a.fs, a.n_shared, (size_t)a.d * a.fs, split ? K / 2 : 0, acc);
    } else {
        pipe_gemm_nf<P, false, NF, true, STREAM_B, (1 << NF) - 1, false, true>(
            lds, rows, K, 0, 1, 0, split ? K / 2 : 0, acc);
    }
    int32_t *rdst = (int32_t *)(lds + tile_info_offset<P>());   // destination row
    float *rgate = (float *)(lds + tile_info_offset<P>() + 4 * P::BM);
    int32_t *slot = (int32_t *)(lds + queue_slot_offset<P>());
    if (threadIdx.x < P::BM) {
        rdst[threadIdx.x] = tj.shared ? tj.row0 + (int)threadIdx.x : my_pair;
        rgate[threadIdx.x] = tj.shared ? 1.0f : my_gate;
    }
    lds_barrier();   // publishes the row info
    const int ticket = threadIdx.x == 0 ? take_ticket(a, k) : 0;
    const int tid = opaque_tid();
    const int lane = tid & 63;
    const int ncols = min(P::BN, a.d - n0);
    uint16_t *yh = tj.shared ? a.ysh : a.yrh;
    float *yf = tj.shared ? a.ys : a.yr;
    if (tj.nrows <= 8) {
        // A tile of at most 8 rows (decode-sized groups): they all sit in
        // fragment 0 of wave row 0 (rows 0-7 in lanes 0-7 and 32-39) and are
        // stored straight from registers, 16 bytes a lane, with no staging.
        if (threadIdx.x == 0) *slot = resolve_ticket(a, k, ticket);
        lds_barrier();
        const int item = __builtin_amdgcn_readfirstlane(*slot);
        if (NF > 0 && P::wave_m(tid) == 0) {
            const int row = pipe_out_row_tr<P>(tid, 0);   // lane & 31
            const bool valid = row < tj.nrows;
            const float g = rgate[row];
            const size_t o = (size_t)rdst[valid ? row : 0] * a.d + n0;
            u16x2 hm = {0, 0};
#pragma unroll
            for (int j = 0; j < P::FN; ++j) {
                uint32_t pk[4][2];
                pack_tr_fragment(acc[0][j], g, valid, pk, hm);
#pragma unroll
                for (int qp = 0; qp < 4; qp += 2) {
                    const int col = (P::wave_n(tid) * P::FN + j) * 32 + (qp + (lane >> 5)) * 8;
                    if (valid && col < ncols)
                        *(u32x4 *)(yh + o + col) = tr_chunk(pk, qp);
                }
            }
            if (valid && (hm[0] >= 0x7C00u || hm[1] >= 0x7C00u))
#pragma unroll
                for (int j = 0; j < P::FN; ++j) store_f32_marked<P>(acc[0][j], g, tid, j, ncols, yf + o);
        }
        return item;
    }
    char *const st = lds;
    u16x2 hm = {0, 0};   // largest |half| of a valid row: 0x7C00 and up = not finite
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        const int row = pipe_out_row_tr<P>(tid, i);
        const float g = rgate[row];
        const bool valid = row < tj.nrows;
#pragma unroll
        for (int j = 0; j < P::FN; ++j) {
            uint32_t pk[4][2];
            pack_tr_fragment(acc[i][j], g, valid, pk, hm);
#pragma unroll
            for (int qp = 0; qp < 4; qp += 2) {
                const int c = (P::wave_n(tid) * P::FN + j) * 4 + qp + (lane >> 5);
                *(u32x4 *)(st + stage_chunk<P>(row, c)) = tr_chunk(pk, qp);
            }
        }
    }
    if (hm[0] >= 0x7C00u || hm[1] >= 0x7C00u) {
        // some value of this lane has no finite fp16 form: store it as fp32
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            const int row = pipe_out_row_tr<P>(tid, i);
            if (row < tj.nrows) {
                const float g = rgate[row];
#pragma unroll
                for (int j = 0; j < P::FN; ++j)
                    store_f32_marked<P>(acc[i][j], g, tid, j, ncols, yf + (size_t)rdst[row] * a.d + n0);
            }
        }
    }
    if (threadIdx.x == 0) *slot = resolve_ticket(a, k, ticket);
    lds_barrier();   // the staged tile is complete and the next item published
    const int item = __builtin_amdgcn_readfirstlane(*slot);
    constexpr int CHUNKS = P::BN / 8;   // 16-byte chunks per row
    constexpr int ITERS = P::BM * CHUNKS / P::NT, BATCH = 4;
    static_assert(ITERS % BATCH == 0, "whole batches");
    // BATCH rows' chunks and destinations are read from LDS before any is
    // stored (rows past the tile's end read stale values and are not
    // stored), so the LDS latency is paid once per batch, not once per row
#pragma unroll
    for (int it0 = 0; it0 < ITERS; it0 += BATCH) {
        u32x4 v[BATCH];
        int dr[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int q = (it0 + u) * P::NT + tid;
            const int row = q / CHUNKS, c = q % CHUNKS;
            v[u] = *(const u32x4 *)(st + stage_chunk<P>(row, c));
            dr[u] = rdst[row];
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int q = (it0 + u) * P::NT + tid;
            const int row = q / CHUNKS, c = q % CHUNKS;
            // read by the combine only, after this launch: not kept in cache
            if (row < tj.nrows && c * 8 < ncols)
                __builtin_nontemporal_store(v[u], (u32x4 *)(yh + (size_t)dr[u] * a.d + n0 + c * 8));
        }
    }
    lds_barrier();   // every wave is done with the staged tile before the next prologue
    return item;
}

template <class P>
__device__ __forceinline__ int down_body(const GroupedArgs &a, const TileJob &tj, char *lds,
                                         int k, bool f16) {
    const int fsum = a.n_shared * a.fs;
    const int n0 = tj.j * P::BN;
    const int goff = tj.goff;
    // K runs over z, or over (hi, lo) of a split group: the two halves of
    // each 64-wide k-range back to back, so W2 streams once
    const int split = tj.shared ? a.split_s : a.split_r;
    const int Kh = tj.shared ? fsum : a.f;   // z's width (one plane)
    const int K = Kh * (split ? 2 : 1);
    const size_t rbase = tj.shared ? (size_t)tj.row0 : (size_t)goff + tj.row0;
    const int wk = tj.shared ? a.fs : a.f;   // row length of the W2 matrix
    const uint16_t *zbase = (const uint16_t *)(tj.shared ? a.zs : a.zr) + rbase * K;
    const uint16_t *w2base = tj.shared ? (const uint16_t *)a.w2s
                                       : (const uint16_t *)a.w2 + (size_t)tj.g * a.d * a.f;
    const int r0 = P::load_row(threadIdx.x, 0);
    int my_pair = 0;
    float my_gate = 0.0f;
    if (!tj.shared && (int)threadIdx.x < tj.nrows) {
        my_pair = a.perm[rbase + threadIdx.x];
        my_gate = a.gsort[rbase + threadIdx.x];
    }
    OperandRows<P> rows;
    rows.abase = zbase;
    rows.bbase = w2base;
    if (tj.shared && f16) {
        // fp16 pass: z rows rbase.. of the fp16 plane (K = K_s d_ff_s) and
        // the fp16 shared W2, both affine as below
        rows.abase = a.zs16 + rbase * fsum;
        rows.bbase = a.w2s16;
        rows.aoff[0] = (uint32_t)r0 * (uint32_t)fsum;
        rows.astep = (uint32_t)(P::NT / P::CHUNKS) * (uint32_t)fsum;
        rows.amask = valid_row_mask<P>(tj.nrows);
        rows.azero = pad_row_mask<P>(tj.nrows);
        rows.boff[0] = (uint32_t)(n0 + r0) * (uint32_t)wk;
        rows.bstep = (uint32_t)(P::NT / P::CHUNKS) * (uint32_t)wk;
        rows.bmask = valid_row_mask<P>(a.d - n0);
        rows.blast = (uint32_t)(a.d - 1) * (uint32_t)wk;
        switch (wave_frags<P>(tj.nrows)) {
            case 4: return down_tile<P, 4, false, false, true>(a, tj, lds, rows, fsum, 0, n0, my_pair, my_gate, k);
            case 3: return down_tile<P, 3, false, false, true>(a, tj, lds, rows, fsum, 0, n0, my_pair, my_gate, k);
            case 2: return down_tile<P, 2, false, false, true>(a, tj, lds, rows, fsum, 0, n0, my_pair, my_gate, k);
            case 1: return down_tile<P, 1, false, false, true>(a, tj, lds, rows, fsum, 0, n0, my_pair, my_gate, k);
            default: return down_tile<P, 0, false, false, true>(a, tj, lds, rows, fsum, 0, n0, my_pair, my_gate, k);
        }
    }
    if (split && tj.nrows <= P::BM / 2) {
        // Folded split tile (few rows: a hash-routed expert, a decode-sized
        // shared group): tile row r < 128 fetches the hi plane of z row r,
        // tile row 128 + r its lo plane, so one pass over the W2 k-ranges
        // serves both (K = one plane) instead of reading every W2 tile twice
        // over twice the k-tiles.  Per-load offsets: not affine across the
        // two halves.
        const int pad = min(P::BM / 2, (tj.nrows + 31) & ~31);
        uint32_t amask = 0, azero = 0;
#pragma unroll
        for (int n = 0; n < P::A_LD; ++n) {
            const int row = P::load_row(threadIdx.x, n);
            const int zr = row & (P::BM / 2 - 1);
            rows.aoff[n] = (uint32_t)zr * (uint32_t)K + (row >= P::BM / 2 ? (uint32_t)Kh : 0u);
            amask |= (zr < tj.nrows ? 1u : 0u) << n;
            azero |= (zr >= tj.nrows && zr < pad ? 1u : 0u) << n;
        }
#pragma unroll
        for (int n = 0; n < P::B_LD; ++n)
            rows.boff[n] = (uint32_t)min(n0 + P::load_row(threadIdx.x, n), a.d - 1) * (uint32_t)wk;
        rows.amask = amask;
        rows.azero = azero;
        const bool stream_b = streams_weights(tj);
        switch (wave_frags<P>(tj.nrows) + (stream_b ? 3 : 0)) {
            case 2: return down_tile<P, 2, false, true>(a, tj, lds, rows, Kh, split, n0, my_pair, my_gate, k);
            case 1: return down_tile<P, 1, false, true>(a, tj, lds, rows, Kh, split, n0, my_pair, my_gate, k);
            case 0: return down_tile<P, 0, false, true>(a, tj, lds, rows, Kh, split, n0, my_pair, my_gate, k);
            case 5: return down_tile<P, 2, true, true>(a, tj, lds, rows, Kh, split, n0, my_pair, my_gate, k);
            case 4: return down_tile<P, 1, true, true>(a, tj, lds, rows, Kh, split, n0, my_pair, my_gate, k);
            default: return down_tile<P, 0, true, true>(a, tj, lds, rows, Kh, split, n0, my_pair, my_gate, k);
        }
    }
    // Both operands are affine: z rows rbase.. and W2 rows n0.. (z rows past
    // the group are not fetched; W2 rows past d fetch row d - 1).
    rows.aoff[0] = (uint32_t)r0 * (uint32_t)K;
    rows.astep = (uint32_t)(P::NT / P::CHUNKS) * (uint32_t)K;
    rows.amask = valid_row_mask<P>(tj.nrows);
    rows.azero = pad_row_mask<P>(tj.nrows);
    rows.boff[0] = (uint32_t)(n0 + r0) * (uint32_t)wk;
    rows.bstep = (uint32_t)(P::NT / P::CHUNKS) * (uint32_t)wk;
    rows.bmask = valid_row_mask<P>(a.d - n0);
    rows.blast = (uint32_t)(a.d - 1) * (uint32_t)wk;
    // a split tile reads each W2 tile twice in a row (once per half), the
    // second time from L2: it keeps the default policy
    const bool stream_b = streams_weights(tj) && !split;
    switch (wave_frags<P>(tj.nrows) + (stream_b ? 5 : 0)) {
        case 4: return down_tile<P, 4, false, false>(a, tj, lds, rows, K, split, n0, my_pair, my_gate, k);
        case 3: return down_tile<P, 3, false, false>(a, tj, lds, rows, K, split, n0, my_pair, my_gate, k);
        case 2: return down_tile<P, 2, false, false>(a, tj, lds, rows, K, split, n0, my_pair, my_gate, k);
        case 1: return down_tile<P, 1, false, false>(a, tj, lds, rows, K, split, n0, my_pair, my_gate, k);
        case 0: return down_tile<P, 0, false, false>(a, tj, lds, rows, K, split, n0, my_pair, my_gate, k);
        case 9: return down_tile<P, 4, true, false>(a, tj, lds, rows, K, split, n0, my_pair, my_gate, k);
        case 8: return down_tile<P, 3, true, false>(a, tj, lds, rows, K, split, n0, my_pair, my_gate, k);
        case 7: return down_tile<P, 2, true, false>(a, tj, lds, rows, K, split, n0, my_pair, my_gate, k);
        case 6: return down_tile<P, 1, true, false>(a, tj, lds, rows, K, split, n0, my_pair, my_gate, k);
        default: return down_tile<P, 0, true, false>(a, tj, lds, rows, K, split, n0, my_pair, my_gate, k);
    }
}

template <class P>
__global__ __launch_bounds__(P::NT) void k_down_bf16(const GroupedArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[P::LDS_BYTES];
    // the shared group's fp16 pass, unless fp16 could not hold a value of z
    // or of the shared W2 (flag set by the gate/up launch or the conversion)
    const bool f16 = a.shared_f16 && __builtin_amdgcn_readfirstlane(a.f16bad[0]) == 0;
    int item = first_item<P>(lds, a);
    while (item >= 0) {
        int m, j;
        RowTileDesc d;
        item_tile(a, item, m, j, d);
        TileJob tj = row_tile(a, d, m, P::BM);
        tj.j = j;
        item = down_body<P>(a, tj, lds, queue_step(item), f16);
    }
}

// The shared experts' W2 as fp16, for the shared group's fp16 down pass.  A
// bf16 value in fp16's normal range converts exactly (its 8 significant bits
// fit fp16's 11); below it, bits under 2^-24 are lost; a value fp16 cannot
// hold (|w| >= 65520, or not finite) sets the flag, and the down launch
// takes the (hi, lo) pass instead.
__global__ __launch_bounds__(256) void k_shared_w2_f16(size_t n4, const uint2 *__restrict__ src,
                                                       uint2 *__restrict__ dst,
                                                       int32_t *__restrict__ bad) {
    bool over = false;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
         i += (size_t)gridDim.x * blockDim.x) {
        const uint2 v = src[i];
        const float f[4] = {bf16_to_f32((uint16_t)(v.x & 0xFFFF)), bf16_to_f32((uint16_t)(v.x >> 16)),
                            bf16_to_f32((uint16_t)(v.y & 0xFFFF)), bf16_to_f32((uint16_t)(v.y >> 16))};
        uint16_t h[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            over |= !(fabsf(f[q]) < 65520.0f);
            h[q] = __builtin_bit_cast(uint16_t, (_Float16)f[q]);
        }
        dst[i] = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
    }
    if (over) atomicOr(bad, 1);
}

// ---------------------------------------------------------------- fp32 SIMT

__global__ __launch_bounds__(256) void k_gate_up_f32(const GroupedArgs a) {
    __shared__ float As[kSBK * kSPad], Bs[kSBK * kSPad];
    const TileRange tr = tile_range(a.tile_base[a.G]);
    const float *x = (const float *)a.x;
    const int fsum = a.n_shared * a.fs;
    const int lr = threadIdx.x >> 2;
    for (int tile = tr.first; tile < tr.end; tile += tr.step) {
        const TileJob tj = decode_tile(a, tile, 64);
        const int zc0 = tj.j * 32;
        const int goff = tj.goff;
        const float *arow = nullptr;
        if (lr < tj.nrows) {
            const int tok = tj.shared ? tj.row0 + lr : a.perm[goff + tj.row0 + lr] / a.top_k;
            arow = x + (size_t)tok * a.d;
        }
        const float *wbase;
        int wrow0, wup;
        if (tj.shared) {
            const int js = zc0 / a.fs;
            wbase = (const float *)a.w13s + (size_t)js * 2 * a.fs * a.d;
            wrow0 = zc0 - js * a.fs;
            wup = a.fs;
        } else {
            wbase = (const float *)a.w13 + (size_t)tj.g * 2 * a.f * a.d;
            wrow0 = zc0;
            wup = a.f;
        }
        const int wr = (lr < 32) ? wrow0 + lr : wup + wrow0 + (lr - 32);
        const float *brow = wbase + (size_t)wr * a.d;
        float acc[4][4];
        SimtTile<true>::run(arow, brow, a.d, 0, 1, 0, As, Bs, acc);
        float *zout = (float *)(tj.shared ? a.zs : a.zr);
        const int zw = tj.shared ? fsum : a.f;
        const size_t rbase = tj.shared ? (size_t)tj.row0 : (size_t)goff + tj.row0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = SimtTile<true>::out_row(i);
            if (row >= tj.nrows) continue;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float ga = acc[i][j], up = acc[i][j + 2];
                zout[(rbase + row) * zw + zc0 + SimtTile<true>::out_col(j)] =
                    ga / (1.0f + expf(-ga)) * up;
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_down_f32(const GroupedArgs a) {
    __shared__ float As[kSBK * kSPad], Bs[kSBK * kSPad];
    const TileRange tr = tile_range(a.tile_base[a.G]);
    const int fsum = a.n_shared * a.fs;
    const int lr = threadIdx.x >> 2;
    for (int tile = tr.first; tile < tr.end; tile += tr.step) {
        const TileJob tj = decode_tile(a, tile, 64);
        const int n0 = tj.j * 64;
        const int goff = tj.goff;
        const int K = tj.shared ? fsum : a.f;
        const float *zin = (const float *)(tj.shared ? a.zs : a.zr);
        const size_t rbase = tj.shared ? (size_t)tj.row0 : (size_t)goff + tj.row0;
        const float *arow = (lr < tj.nrows) ? zin + (rbase + lr) * K : nullptr;
        const int n = n0 + lr;
        const float *brow = nullptr;
        if (n < a.d)
            brow = tj.shared ? (const float *)a.w2s + (size_t)n * a.fs
                             : (const float *)a.w2 + (size_t)tj.g * a.d * a.f + (size_t)n * a.f;
        float acc[4][4];
        SimtTile<false>::run(arow, brow, K, tj.shared ? a.fs : 0, a.n_shared, (size_t)a.d * a.fs,
                             As, Bs, acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = SimtTile<false>::out_row(i);
            if (row >= tj.nrows) continue;
            float *dst;
            float gate = 1.0f;
            if (tj.shared) {
                dst = a.ys + (size_t)(tj.row0 + row) * a.d;
            } else {
                const int pair = a.perm[rbase + row];
                gate = a.gsort[rbase + row];
                dst = a.yr + (size_t)pair * a.d;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + SimtTile<false>::out_col(j);
                if (col < a.d) dst[col] = gate * acc[i][j];
            }
        }
    }
}

// ---------------------------------------------------------------- launch

int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Persistent grid: as many blocks as fit at once (per_cu per CU), no more than
// the largest possible tile count, a multiple of the XCD count.
static int persistent_grid(long long max_tiles, int per_cu) {
    long long g = (long long)device_cu_count() * per_cu;
    if (g > max_tiles) g = max_tiles;
    g = (g + kXcds - 1) / kXcds * kXcds;
    return (int)(g < kXcds ? kXcds : g);
}

static long long max_tiles(const moe_config &c, int bm, int ncols_tile, int width_r, int width_s) {
    const long long P = (long long)c.T * c.top_k;
    long long rt = (P + bm - 1) / bm + c.n_routed;  // sum over experts of ceil(cnt / bm)
    long long n = rt * ((width_r + ncols_tile - 1) / ncols_tile);
    if (c.n_shared > 0) n += ((c.T + bm - 1) / bm) * ((width_s + ncols_tile - 1) / ncols_tile);
    return n;
}

hipError_t launch_gate_up(const moe_config &c, const GroupedArgs &a0, hipStream_t s) {
    const TileShape ts = tile_shape(c);
    const long long mt = max_tiles(c, ts.bm1, ts.bz1, c.d_ff, c.n_shared * c.d_ff_shared);
    if (c.dtype == MOE_BF16) {
        const int grid = persistent_grid(1ll << 30, 1);
        GroupedArgs a = a0;
        a.nt_routed = (c.d_ff + ts.bz1 - 1) / ts.bz1;
        a.nt_shared = (c.n_shared * c.d_ff_shared + ts.bz1 - 1) / ts.bz1;
        hipLaunchKernelGGL(k_gate_up_bf16<PipeTile>, dim3(grid), dim3(PipeTile::NT), 0, s, a);
    }
    else
        hipLaunchKernelGGL(k_gate_up_f32, dim3(persistent_grid(mt, 4)), dim3(256), 0, s, a0);
    return hipGetLastError();
}

hipError_t launch_down(const moe_config &c, const GroupedArgs &a0, hipStream_t s) {
    const TileShape ts = tile_shape(c);
    const long long mt = max_tiles(c, ts.bm2, ts.bn2, c.d_model, c.d_model);
    if (c.dtype == MOE_BF16) {
        const int grid = persistent_grid(1ll << 30, 1);
        GroupedArgs a = a0;
        if (a.shared_f16) {
            const size_t n = (size_t)c.n_shared * c.d_model * c.d_ff_shared;
            hipLaunchKernelGGL(k_shared_w2_f16, dim3(1024), dim3(256), 0, s, n / 4,
                               (const uint2 *)a.w2s, (uint2 *)a.w2s16, a.f16bad);
        }
        a.nt_routed = a.nt_shared = (c.d_model + ts.bn2 - 1) / ts.bn2;
        hipLaunchKernelGGL(k_down_bf16<PipeTile>, dim3(grid), dim3(PipeTile::NT), 0, s, a);
    } else {
        hipLaunchKernelGGL(k_down_f32, dim3(persistent_grid(mt, 4)), dim3(256), 0, s, a0);
    }
    return hipGetLastError();
}

}  // namespace moe
