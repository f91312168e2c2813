// mfma_tile.h -- the bf16 MFMA main loop shared by the router GEMM and the
// grouped expert GEMMs (gfx950).
//
// Both operands are "K-contiguous": row r of A (M x K) and row n of B (N x K)
// are contiguous runs of K bf16 values, which is how x, W_g, W13, W2 and the
// hidden activations are stored.  C = A B^T is accumulated in fp32 with
// v_mfma_f32_32x32x16_bf16.
//
// Per k-tile of 64 values each row holds 8 chunks of 16 bytes.  Tiles sit in
// LDS as [row][chunk] with the chunk index XOR-ed by (row & 7): the 8 lanes
// that read one 16-byte chunk column of 8 consecutive rows hit 8 distinct
// bank groups, and the 8 lanes that store one row write it contiguously.
//
// The global -> LDS pipeline is double-buffered: while the MFMAs consume
// k-tile kt from LDS buffer kt&1, each thread holds k-tile kt+1 in registers
// and writes it to the other buffer afterwards; one barrier per k-tile.
#pragma once

#include "common.h"

namespace moe {

constexpr int kBK = 64;  // k values per tile

__device__ __forceinline__ int lds_idx(int row, int chunk) {
    return row * 8 + (chunk ^ (row & 7));
}

// BM x BN block tile, WM x WN waves, each wave (BM/WM) x (BN/WN) of output
// made of 32x32 MFMA blocks.  SPLIT: the B tile is two halves (rows
// [0, BN/2) and [BN/2, BN)); wave wn takes the same column range from each
// half, so fragment fn and fn + FN/2 of a lane cover the same output column
// of the two halves (used to pair the W1 and W3 products of SwiGLU).
template <int BM, int BN, int WM, int WN, bool SPLIT>
struct MfmaTile {
    static constexpr int NT = kWave * WM * WN;
    static constexpr int A_LD = BM * 8 / NT;
    static constexpr int B_LD = BN * 8 / NT;
    static constexpr int FM = BM / WM / 32;
    static constexpr int FN = BN / WN / 32;
    static constexpr int LDS_A = BM * 8;  // u32x4 per buffer
    static constexpr int LDS_B = BN * 8;
    static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "tile/threads");
    static_assert(A_LD >= 1 && B_LD >= 1 && FM >= 1 && FN >= 1, "tile too small");
    static_assert(!SPLIT || FN % 2 == 0, "split needs an even fragment count");

    // Row of the B tile feeding fragment fn of wave column wn, lane row 0.
    __device__ static __forceinline__ int b_frag_row(int wn, int fn) {
        if (!SPLIT) return wn * (BN / WN) + fn * 32;
        constexpr int H = FN / 2;
        constexpr int HW = BN / 2 / WN;
        return (fn < H) ? wn * HW + fn * 32 : BN / 2 + wn * HW + (fn - H) * 32;
    }

    // Row (within the thread's load set) handled by load slot i.
    __device__ static __forceinline__ int load_row(int tid, int i) {
        return (tid >> 3) + i * (NT / 8);
    }

    __device__ static __forceinline__ void gload(u32x4 (&ra)[A_LD], u32x4 (&rb)[B_LD],
                                                 const uint16_t *const (&arow)[A_LD],
                                                 const uint16_t *const (&brow)[B_LD], int k0,
                                                 int bsplit, int bmod, size_t bstride, int c) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const size_t koff = (bsplit > 0) ? (size_t)((k0 / bsplit) % bmod) * bstride +
                                               (size_t)(k0 % bsplit)
                                         : (size_t)k0;
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            ra[i] = arow[i] ? *(const u32x4 *)(arow[i] + k0 + c * 8) : zero;
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            rb[i] = brow[i] ? *(const u32x4 *)(brow[i] + koff + c * 8) : zero;
    }

    __device__ static __forceinline__ void lstore(u32x4 *As, u32x4 *Bs, const u32x4 (&ra)[A_LD],
                                                  const u32x4 (&rb)[B_LD], int buf, int tid,
                                                  int c) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) As[buf * LDS_A + lds_idx(load_row(tid, i), c)] = ra[i];
#pragma unroll
        for (int i = 0; i < B_LD; ++i) Bs[buf * LDS_B + lds_idx(load_row(tid, i), c)] = rb[i];
    }

    // Main loop.  arow[i]/brow[i]: base pointers of the rows this thread
    // loads (nullptr -> zeros).  B's k offset of k-tile k0 is k0, or, when
    // bsplit > 0, ((k0 / bsplit) % bmod) * bstride + k0 % bsplit (B made of
    // several matrices side by side along K, possibly repeated).
    __device__ static __forceinline__ void run(const uint16_t *const (&arow)[A_LD],
                                               const uint16_t *const (&brow)[B_LD],
                                               int K, int bsplit, int bmod, size_t bstride,
                                               u32x4 *As, u32x4 *Bs,
                                               f32x16 (&acc)[FM][FN]) {
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = tid >> 6;
        const int wm = wave % WM;
        const int wn = wave / WM;
        const int c = tid & 7;

#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        u32x4 ra[A_LD], rb[B_LD];
        const int nk = K / kBK;
        gload(ra, rb, arow, brow, 0, bsplit, bmod, bstride, c);
        lstore(As, Bs, ra, rb, 0, tid, c);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) gload(ra, rb, arow, brow, (kt + 1) * kBK, bsplit, bmod, bstride, c);
            const u32x4 *Ab = As + cur * LDS_A;
            const u32x4 *Bb = Bs + cur * LDS_B;
#pragma unroll
            for (int s = 0; s < kBK / 16; ++s) {
                const int ch = 2 * s + (lane >> 5);
                bf16x8 a[FM], b[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int row = wm * (BM / WM) + i * 32 + (lane & 31);
                    u32x4 v = Ab[lds_idx(row, ch)];
                    a[i] = __builtin_bit_cast(bf16x8, v);
                }
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int row = b_frag_row(wn, j) + (lane & 31);
                    u32x4 v = Bb[lds_idx(row, ch)];
                    b[j] = __builtin_bit_cast(bf16x8, v);
                }
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j],
                                                                            0, 0, 0);
            }
            if (kt + 1 < nk) lstore(As, Bs, ra, rb, cur ^ 1, tid, c);
            __syncthreads();
        }
    }

    // Output coordinates of accumulator register r of fragment (i, j):
    // tile row, and tile column (for SPLIT: the column within a half).
    __device__ static __forceinline__ int out_row(int i, int r) {
        const int lane = threadIdx.x & 63;
        const int wm = (threadIdx.x >> 6) % WM;
        return wm * (BM / WM) + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
    }
    __device__ static __forceinline__ int out_col(int j) {
        const int lane = threadIdx.x & 63;
        const int wn = (threadIdx.x >> 6) / WM;
        if (!SPLIT) return wn * (BN / WN) + j * 32 + (lane & 31);
        return wn * (BN / 2 / WN) + j * 32 + (lane & 31);
    }
};

}  // namespace moe
