// simt_tile.h -- fp32 tile loop (no matrix cores) for the MOE_F32 element
// type: C[64][64] = A[64][K] B[64][K]^T with 256 threads, 4x4 outputs each.
#pragma once

#include "common.h"

namespace moe {

constexpr int kSBK = 16;   // k values per fp32 tile
constexpr int kSPad = 68;  // padded LDS row (floats)

// SPLIT: thread tx owns columns 2tx, 2tx+1 of the first B half and the same
// two columns of the second half (rows 32 + 2tx, 33 + 2tx), so SwiGLU's W1 and
// W3 products of one hidden unit land in the same thread.
template <bool SPLIT>
struct SimtTile {
    __device__ static __forceinline__ int out_row(int i) { return (threadIdx.x >> 4) * 4 + i; }
    __device__ static __forceinline__ int out_col(int j) {
        const int tx = threadIdx.x & 15;
        return SPLIT ? 2 * tx + j : tx * 4 + j;   // SPLIT: j < 2, column within a half
    }

    // arow/brow: base of the single A row / B row this thread loads (row
    // tid / 4, k sub-range (tid % 4) * 4); nullptr -> zeros.
    __device__ static __forceinline__ void run(const float *arow, const float *brow, int K,
                                               int bsplit, int bmod, size_t bstride, float *As,
                                               float *Bs,
                                               float (&acc)[4][4]) {
        const int tid = threadIdx.x;
        const int lr = tid >> 2, lk = (tid & 3) * 4;
        const int tx = tid & 15, ty = tid >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
        for (int k0 = 0; k0 < K; k0 += kSBK) {
            size_t koff = (bsplit > 0) ? (size_t)((k0 / bsplit) % bmod) * bstride +
                                             (size_t)(k0 % bsplit)
                                       : (size_t)k0;
            float4 va = arow ? *(const float4 *)(arow + k0 + lk) : make_float4(0, 0, 0, 0);
            float4 vb = brow ? *(const float4 *)(brow + koff + lk) : make_float4(0, 0, 0, 0);
            As[(lk + 0) * kSPad + lr] = va.x;
            As[(lk + 1) * kSPad + lr] = va.y;
            As[(lk + 2) * kSPad + lr] = va.z;
            As[(lk + 3) * kSPad + lr] = va.w;
            Bs[(lk + 0) * kSPad + lr] = vb.x;
            Bs[(lk + 1) * kSPad + lr] = vb.y;
            Bs[(lk + 2) * kSPad + lr] = vb.z;
            Bs[(lk + 3) * kSPad + lr] = vb.w;
            __syncthreads();
#pragma unroll
            for (int k = 0; k < kSBK; ++k) {
                float a[4], b[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = As[k * kSPad + ty * 4 + i];
                if (SPLIT) {
                    b[0] = Bs[k * kSPad + 2 * tx];
                    b[1] = Bs[k * kSPad + 2 * tx + 1];
                    b[2] = Bs[k * kSPad + 32 + 2 * tx];
                    b[3] = Bs[k * kSPad + 33 + 2 * tx];
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) b[j] = Bs[k * kSPad + tx * 4 + j];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
            }
            __syncthreads();
        }
    }
};

}  // namespace moe
