// mfma_pipe.h -- the bf16 MFMA tile engine of the grouped expert GEMMs and
// the router GEMM (gfx950).
//
// C[256][256] = A[256][K] B[256][K]^T, both operands K-contiguous, fp32
// accumulation with v_mfma_f32_32x32x16_bf16.  Eight waves, two per SIMD,
// in a 2 x 4 grid, each owning a 128 x 64 accumulator block (128 registers
// per lane).  With one 128 x 128 wave per SIMD (the fewest LDS bytes per
// MFMA) nothing hides a wave's waits on its loads, LDS reads and barriers:
// a skeleton of this pipeline with every operand in L2 ran at 1.72 us per
// k-tile with one wave per SIMD and 1.37 us with two (the MFMAs alone take
// 0.85 us).  A 384 x 256 tile (eight 96 x 128 waves, 17% fewer L2->LDS
// bytes per multiply-add) was faster in a probe with its token rows in L2,
// but its LDS holds only two weight stages, and with gathered token rows
// its gate/up launch ran 4-8% slower than this tile's.
//
// Memory pipeline.  k-tiles of 64 values: each row contributes one whole
// 128-byte cache line per k-tile (half-line requests halve the per-CU rate
// of L2 hits).  Global data goes straight into LDS with 16-byte
// global_load_lds (no register staging); a lane's LDS slot is fixed by its
// lane id, so the swizzle is applied by choosing which global chunk each
// lane fetches.  LDS row = 128 bytes = 8 chunks of 16 bytes; chunk c of row
// r sits in slot c ^ ((r >> 1) & 7), so the 16 lanes that read one chunk
// column of 16 consecutive rows hit 16 distinct 16-byte groups of the
// 64-bank LDS.
//
// The two operands get different depths: B (expert weights, streamed from
// HBM once, long latency) has three 32 KB stages -- its loads run two
// k-tiles ahead -- while A (token rows, shared by the column tiles that run
// together on one XCD and mostly served by L2) has two.  2 x 32 + 3 x 32 KB
// is the whole 160 KB LDS.  The next k-tile's loads are spread evenly
// through the MFMA stream, so a busy load queue never holds a run of MFMAs
// back.
//
// Partial row tiles: wave row wm owns the 32-row fragments 2 i + wm
// (i < 4), so a tile with n valid rows issues MFMAs only for fragments that
// hold a valid row -- the work of a partial tile scales with ceil(n / 64).
#pragma once

#include <type_traits>

#include "common.h"

namespace moe {

struct PipeTile {
    static constexpr int WM = 2, WN = 4;                   // wave grid
    static constexpr int FM = 4, FN = 2;                   // 32x32 fragments per wave
    static constexpr int BM = 32 * FM * WM, BN = 32 * FN * WN, BK = 64, NT = 64 * WM * WN;
    static constexpr int A_STAGES = 2, B_STAGES = 3;
    static constexpr int CHUNKS = BK / 8;                  // 16-byte chunks per row
    static constexpr int A_LD = BM * CHUNKS / NT;          // global_load_lds per thread, A
    static constexpr int B_LD = BN * CHUNKS / NT;          // and B
    static constexpr int A_STAGE = BM * CHUNKS * 16;       // bytes
    static constexpr int B_STAGE = BN * CHUNKS * 16;
    static constexpr int LDS_BYTES = A_STAGES * A_STAGE + B_STAGES * B_STAGE;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    static_assert(NT == 512 && (BM * CHUNKS) % NT == 0 && (BN * CHUNKS) % NT == 0, "loads");
    static_assert(FN % 2 == 0, "gate/up fragment pairs");

    __device__ static __forceinline__ int slot(int row, int chunk) {
        return chunk ^ ((row >> 1) & 7);
    }
    // Row of the tile that load n of thread tid fills; the global chunk it
    // fetches is the same for every n.
    __device__ static __forceinline__ int load_row(int tid, int n) {
        return tid / CHUNKS + n * (NT / CHUNKS);
    }
    __device__ static __forceinline__ int load_chunk(int tid) {
        return slot(load_row(tid, 0), tid % CHUNKS);   // slot() is its own inverse
    }
    // Wave coordinates (the same in every lane of a wave; read from lane 0
    // so the compiler keeps them, and what derives from them, scalar).
    __device__ static __forceinline__ int wave_m(int tid) {
        return __builtin_amdgcn_readfirstlane((tid >> 6) % WM);
    }
    __device__ static __forceinline__ int wave_n(int tid) {
        return __builtin_amdgcn_readfirstlane((tid >> 6) / WM);
    }
    // B tile row feeding fragment j of wave column wn.  SPLIT (gate/up): the
    // tile's first BN/2 rows are W1 rows and the last BN/2 the W3 rows of the
    // same hidden units; fragments j < FN/2 come from the first half and
    // fragment j + FN/2 from the second half at the same offset, so
    // fragments j and j + FN/2 hold the two halves of one SwiGLU.
    template <bool SPLIT>
    __device__ static __forceinline__ int b_row(int wn, int j) {
        if (SPLIT) {
            const int h = (j >= FN / 2) ? 1 : 0;
            return h * (BN / 2) + (wn * (FN / 2) + j - h * (FN / 2)) * 32;
        }
        return (wn * FN + j) * 32;
    }
    // Tile row of fragment i of wave row wm.
    __device__ static __forceinline__ int a_row(int wm, int i) { return (WM * i + wm) * 32; }
};

// Row addresses of the rows one thread fetches: a uniform base plus 32-bit
// element offsets (keeps the per-thread state small).  Affine operands (the
// rows of consecutive loads a fixed step apart) give only load 0's offset
// and the step, which saves the vector registers of the others.
template <class P>
struct OperandRows {
    const uint16_t *abase, *bbase;
    uint32_t aoff[P::A_LD];
    uint32_t boff[P::B_LD];
    uint32_t astep, bstep;      // affine operands: element step from load n to n + 1
    uint32_t amask;             // bit n: A load n fetches a valid row (the rest are skipped)
    // bit n: A load n's row is past the valid rows but inside a fragment the
    // tile computes; its LDS slot is zeroed in both A stages instead, so the
    // MFMAs over it multiply zeros (less power than stale values)
    uint32_t azero = 0;
    // Affine operands: bit n of bmask set when B load n fetches a valid row;
    // the others fetch row blast (an element offset, the tile's last valid
    // row) instead, so every B load is issued (the three-stage wait counts
    // them).
    uint32_t bmask, blast;
};

// Workgroup barrier without a memory fence.  __syncthreads() would also wait
// for every outstanding global_load_lds (vmcnt(0)), which drains the load
// pipeline; here each thread first waits for exactly the loads it needs
// (wait_vmcnt), and the barrier then makes them visible to all waves.  The
// signal fences stop the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): own LDS reads/writes done
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Cache policy of an operand load: the default, or non-temporal (the `nt`
// bit) for data no other load will read again, so that its lines are the
// first to leave L2.
constexpr int kCpolDefault = 0, kCpolStream = 2;

template <int CPOL = kCpolDefault>
__device__ __forceinline__ void load_lds16(const uint16_t *src, char *lds_dst) {
    __builtin_amdgcn_global_load_lds((const void *)src,
                                     (__attribute__((address_space(3))) void *)lds_dst, 16, 0, CPOL);
}
// The same from a wave-uniform base plus a 32-bit byte offset: the form the
// instruction takes natively (64-bit base in scalar registers, one vector
// register of offset), so no 64-bit per-row address stays live in vector
// registers across the K loop.  `base` must be the same in every lane.
__device__ __forceinline__ const uint16_t *uniform_ptr(const uint16_t *p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint16_t *)(((uint64_t)hi << 32) | lo);
}
template <int CPOL = kCpolDefault>
__device__ __forceinline__ void load_lds16_at(const uint16_t *base, uint32_t byte_off,
                                              char *lds_dst) {
    load_lds16<CPOL>((const uint16_t *)((const char *)base + byte_off), lds_dst);
}

// Run the K loop of one tile.  A rows past the valid count are not fetched
// (rows.amask): their LDS rows keep stale values, which only reach output
// rows that are discarded.  Every B row must be dereferenceable.  NF: how
// many of this wave's row fragments hold a valid row (0..FM) -- all waves
// run the same loads and barriers, a wave with fewer valid fragments issues
// fewer MFMAs.  B's k offset of k-tile k0 is k0, or
// ((k0 / bsplit) % bmod) * bstride + k0 % bsplit (B made of several matrices
// side by side along K, possibly repeated).  AFF: both operands are affine
// (rows.aoff[0], rows.astep; rows.boff[0], rows.bstep).  STREAM_B: B is
// read by this tile alone and once, so its loads are non-temporal.  FMASK:
// which of the NF leading fragments the wave computes (all by default; a
// folded split tile skips the fragments between its hi and lo rows).  F16:
// both operands are fp16 (v_mfma_f32_32x32x16_f16) instead of bf16.  TR:
// the MFMAs take the B fragment as their first operand, so each accumulator
// holds its block transposed: lane l owns tile row a_row(wm, i) + (l & 31)
// and register r column b_row(wn, j) + 8 (r >> 2) + 4 (l >> 5) + (r & 3)
// (four consecutive columns per register quad; see pipe_out_row_tr).
template <class P, bool SPLIT, int NF, bool AFF = false, bool STREAM_B = false,
          int FMASK = (1 << NF) - 1, bool F16 = false, bool TR = false>
__device__ __forceinline__ void pipe_gemm_nf(char *lds, const OperandRows<P> &rows, int K,
                                             int bsplit, int bmod, size_t bstride, int a_half,
                                             f32x16 (&acc)[NF > 0 ? NF : 1][P::FN]) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = P::wave_m(tid);
    const int wn = P::wave_n(tid);
    const int ca = P::load_chunk(tid) * 8;
    char *const a_lds = lds;
    char *const b_lds = lds + P::A_STAGES * P::A_STAGE;
    constexpr int NA = NF > 0 ? NF : 1;
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < P::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto koff_of = [&](int k0) -> size_t {
        return (bsplit > 0) ? (size_t)((k0 / bsplit) % bmod) * bstride + (size_t)(k0 % bsplit)
                            : (size_t)k0;
    };
    // a_half > 0: A rows are two halves of a_half values (a bf16 (hi, lo)
    // pair) and k-tile kt is half kt % 2 of k-range kt / 2; B's k-tile is
    // k-range kt / 2 for both, so each B tile is loaded twice in a row (the
    // second time from L2) instead of once per half pass.
    auto a_col = [&](int kt) -> int {
        return a_half ? (kt & 1) * a_half + (kt >> 1) * P::BK : kt * P::BK;
    };
    auto b_koff = [&](int kt) -> size_t { return koff_of((a_half ? kt >> 1 : kt) * P::BK); };
    // Byte offsets (below 2^32: the API bounds every operand matrix to 2^31
    // elements): row offset and chunk per thread, k offset per k-tile.  The
    // bases are per tile, so the same in every lane; reading them from lane 0
    // puts them in scalar registers even where the compiler cannot prove it.
    const uint16_t *const abase = uniform_ptr(rows.abase);
    const uint16_t *const bbase = uniform_ptr(rows.bbase);
    constexpr int NAB = AFF ? 1 : P::A_LD, NBB = AFF ? 1 : P::B_LD;
    uint32_t abyte[NAB], bbyte[NBB];
#pragma unroll
    for (int n = 0; n < NAB; ++n) abyte[n] = 2u * (rows.aoff[n] + (uint32_t)ca);
#pragma unroll
    for (int n = 0; n < NBB; ++n) bbyte[n] = 2u * (rows.boff[n] + (uint32_t)ca);
    auto a_byte = [&](int n) -> uint32_t {
        if constexpr (AFF) return abyte[0] + 2u * (uint32_t)n * rows.astep;
        else return abyte[n];
    };
    uint32_t bclamp = 0;
    if constexpr (AFF) bclamp = 2u * (rows.blast + (uint32_t)ca);
    auto b_byte = [&](int n) -> uint32_t {
        if constexpr (AFF)
            return ((rows.bmask >> n) & 1) ? bbyte[0] + 2u * (uint32_t)n * rows.bstep : bclamp;
        else return bbyte[n];
    };
    // kbyte: the k-tile's byte offset along the rows, taken once per k-tile
    // through readfirstlane so that it stays one scalar (otherwise the
    // compiler may turn it into one vector induction variable per load);
    // stage_off: byte offset of the destination stage within the A (B) area.
    auto a_kbyte = [&](int kt) -> uint32_t {
        return __builtin_amdgcn_readfirstlane(2u * (uint32_t)a_col(kt));
    };
    auto b_kbyte = [&](size_t koff) -> uint32_t {
        return __builtin_amdgcn_readfirstlane(2u * (uint32_t)koff);
    };
    auto a_load = [&](int n, uint32_t kbyte, uint32_t stage_off) {
        if ((rows.amask >> n) & 1)
            load_lds16_at(abase, a_byte(n) + kbyte,
                          a_lds + stage_off + (n * P::NT + wave * 64) * 16);
    };
    auto b_load = [&](int n, uint32_t kbyte, uint32_t stage_off) {
        load_lds16_at<STREAM_B ? kCpolStream : kCpolDefault>(
            bbase, b_byte(n) + kbyte, b_lds + stage_off + (n * P::NT + wave * 64) * 16);
    };
    const int nk = K / P::BK;
#pragma unroll
    for (int n = 0; n < P::A_LD; ++n)
        if ((rows.azero >> n) & 1)
#pragma unroll
            for (int st = 0; st < P::A_STAGES; ++st)
                *(u32x4 *)(a_lds + st * P::A_STAGE + (n * P::NT + tid) * 16) = u32x4{0, 0, 0, 0};
    // Prologue: A(0), B(0), B(1).  Every iteration kt then issues A(kt+1)
    // followed by B(kt+2), as far as they exist.  So at the top of iteration
    // kt < nk-1 the only loads issued after A(kt) and B(kt) are the B_LD
    // loads of B(kt+1) (every B load is issued, see OperandRows): vmcnt <=
    // B_LD means both operands of k-tile kt have landed (vector memory loads
    // complete in order); the last iteration has nothing in flight after
    // them and waits for everything.
    static_assert(P::A_STAGES == 2 && P::B_STAGES == 3, "the waits below assume 2 + 3 stages");
    constexpr int LB = P::B_STAGES - 1;
#pragma unroll
    for (int n = 0; n < P::A_LD; ++n) a_load(n, 0u, 0u);
#pragma unroll
    for (int s = 0; s < LB; ++s) {
        if (s >= nk) break;
        const uint32_t ko = b_kbyte(b_koff(s));
#pragma unroll
        for (int n = 0; n < P::B_LD; ++n) b_load(n, ko, (uint32_t)s * P::B_STAGE);
    }
    constexpr int SUB = P::BK / 16;          // MFMA k-substeps per k-tile
    constexpr int GROUPS = P::FM;            // MFMA groups (one fragment row each) per substep
    // Fragment rows start at multiples of 32, so the swizzled slot of this
    // lane's row (lane & 31 of the fragment) and chunk 2s + lane / 32 is the
    // same in every fragment: one byte offset per substep, loop-invariant.
    uint32_t lofs[SUB];
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
        const int r = lane & 31;
        lofs[s] = (uint32_t)(r * P::CHUNKS + P::slot(r, 2 * s + (lane >> 5))) * 16u;
    }
    constexpr int SLOTS = SUB * GROUPS;
    constexpr int LOADS = P::A_LD + P::B_LD;
    // One k-tile.  more_a: A(kt+1) exists (kt + 1 < nk); more_b: B(kt+2)
    // exists.  Both come in as std::true_type / std::false_type, so the main
    // loop below (where both hold) carries no per-load branches and no
    // choice of wait; the last two k-tiles are peeled off.
    static_assert((P::A_STAGE & (P::A_STAGE - 1)) == 0, "A stage toggle");
    uint32_t a_cur = 0, b_cur = 0;   // byte offsets of k-tile kt's A and B stages
    auto k_tile = [&](int kt, auto more_a_c, auto more_b_c) {
        constexpr bool more_a = decltype(more_a_c)::value;
        constexpr bool more_b = decltype(more_b_c)::value;
        // A(kt) and B(kt) have landed (this thread's share) ...
        if constexpr (more_a) wait_vmcnt<P::B_LD>();
        else wait_vmcnt<0>();
        lds_barrier();           // ... everyone's; the stages of k-tile kt-1 are free
        const uint32_t ka = a_kbyte(min(kt + 1, nk - 1));
        const uint32_t kbo = b_kbyte(b_koff(min(kt + LB, nk - 1)));
        // stage of k-tile kt + 1 (A, two stages) and kt + 2 = kt - 1 mod 3 (B)
        const uint32_t sa_next = a_cur ^ (uint32_t)P::A_STAGE;
        const uint32_t sb_next = b_cur == 0 ? 2u * P::B_STAGE : b_cur - P::B_STAGE;
        const char *Ab = a_lds + a_cur;
        const char *Bb = b_lds + b_cur;
        using V8 = std::conditional_t<F16, f16x8, bf16x8>;
        V8 a[2][NA], b[2][P::FN];
        auto frag_load = [&](int s, V8 (&av)[NA], V8 (&bv)[P::FN]) {
            const char *As = Ab + lofs[s];
            const char *Bs = Bb + lofs[s];
#pragma unroll
            for (int j = 0; j < P::FN; ++j) {
                const int row0 = P::template b_row<SPLIT>(wn, j);   // a multiple of 32
                bv[j] = __builtin_bit_cast(V8, *(const u32x4 *)(Bs + row0 * P::CHUNKS * 16));
            }
#pragma unroll
            for (int i = 0; i < NF; ++i) {
                if (!((FMASK >> i) & 1)) continue;
                const int row0 = P::a_row(wm, i);
                av[i] = __builtin_bit_cast(V8, *(const u32x4 *)(As + row0 * P::CHUNKS * 16));
            }
        };
        frag_load(0, a[0], b[0]);
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
            const int cur = s & 1;
            if (s + 1 < SUB) frag_load(s + 1, a[(s + 1) & 1], b[(s + 1) & 1]);
#pragma unroll
            for (int q = 0; q < GROUPS; ++q) {
#pragma unroll
                for (int i = 0; i < NF; ++i)
                    if (i == q && ((FMASK >> i) & 1))
#pragma unroll
                        for (int j = 0; j < P::FN; ++j)
                            if constexpr (F16 && TR)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                    b[cur][j], a[cur][i], acc[i][j], 0, 0, 0);
                            else if constexpr (F16)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                    a[cur][i], b[cur][j], acc[i][j], 0, 0, 0);
                            else if constexpr (TR)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                    b[cur][j], a[cur][i], acc[i][j], 0, 0, 0);
                            else
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                    a[cur][i], b[cur][j], acc[i][j], 0, 0, 0);
                // this group's share of the next loads, A loads first, then B,
                // at raised wave priority: where both waves of a SIMD can
                // issue, this wave's loads leave before the other wave's
                // MFMAs and LDS reads (interleaved A/B: V4 skew gate/up -0.7%,
                // down -1.2%; V3 prefill -0.2% / -0.5%; decode -0.5 to -1.8%.
                // The MFMAs at raised priority instead: gate/up +2%)
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int n = 0; n < LOADS; ++n) {
                    if (n * SLOTS / LOADS != s * GROUPS + q) continue;
                    if (n < P::A_LD) {
                        if constexpr (more_a) a_load(n, ka, sa_next);
                    } else if constexpr (more_b) {
                        b_load(n - P::A_LD, kbo, sb_next);
                    }
                }
                __builtin_amdgcn_s_setprio(0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        a_cur = sa_next;
        b_cur = b_cur == 2u * P::B_STAGE ? 0u : b_cur + P::B_STAGE;
    };
    using yes = std::true_type;
    using no = std::false_type;
    int kt = 0;
    for (; kt + LB < nk; ++kt) k_tile(kt, yes{}, yes{});
    if (kt + 1 < nk) k_tile(kt++, yes{}, no{});   // kt = nk - 2: B(nk) does not exist
    if (kt < nk) k_tile(kt, no{}, no{});          // the last k-tile
    wait_vmcnt<0>();
    lds_barrier();     // every wave done with the stages before the LDS is reused
}

// Bit n set when load n of this thread fetches one of the nrows valid rows
// (A and B loads cover the rows alike).
template <class P>
__device__ __forceinline__ uint32_t valid_row_mask(int nrows) {
    uint32_t m = 0;
#pragma unroll
    for (int n = 0; n < P::A_LD; ++n)
        m |= (P::load_row(threadIdx.x, n) < nrows ? 1u : 0u) << n;
    return m;
}

// Bits of the A loads whose rows lie past nrows but inside the last 32-row
// fragment a tile with nrows valid rows computes.
template <class P>
__device__ __forceinline__ uint32_t pad_row_mask(int nrows) {
    const int computed = min(P::BM, (nrows + 31) & ~31);
    return valid_row_mask<P>(computed) & ~valid_row_mask<P>(nrows);
}

// Fragments (of FM) this thread's wave row must compute for a tile with
// nrows valid rows: those i with WM i + wm < ceil(nrows / 32).
template <class P>
__device__ __forceinline__ int wave_frags(int nrows) {
    const int wm = P::wave_m(threadIdx.x);
    const int nblk = (nrows + 31) >> 5;
    return min(P::FM, max(0, (nblk - wm + P::WM - 1) / P::WM));
}

// Thread id the compiler cannot treat as loop-invariant: epilogue address
// arithmetic stays next to its use instead of being hoisted out of the
// persistent tile loop (where 64 precomputed offsets would spill).
__device__ __forceinline__ int opaque_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// Output coordinates of accumulator register r of fragment (i, j), given
// tid = opaque_tid().
template <class P>
__device__ __forceinline__ int pipe_out_row(int tid, int i, int r) {
    const int lane = tid & 63;
    return P::a_row(P::wave_m(tid), i) + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}
// Transposed accumulators (TR): tile row of fragment i (one per lane) and
// tile column of register r of fragment j.
template <class P>
__device__ __forceinline__ int pipe_out_row_tr(int tid, int i) {
    return P::a_row(P::wave_m(tid), i) + (tid & 31);
}
template <class P>
__device__ __forceinline__ int pipe_out_col_tr(int tid, int j, int r) {
    return (P::wave_n(tid) * P::FN + j) * 32 + (r >> 2) * 8 + ((tid & 63) >> 5) * 4 + (r & 3);
}
// SPLIT: hidden column (within a half) of gate/up pair j (< FN/2); else
// column of the tile.
template <class P, bool SPLIT>
__device__ __forceinline__ int pipe_out_col(int tid, int j) {
    const int lane = tid & 63;
    const int wn = P::wave_n(tid);
    return SPLIT ? (wn * (P::FN / 2) + j) * 32 + (lane & 31) : (wn * P::FN + j) * 32 + (lane & 31);
}

}  // namespace moe
