// combine.hip -- the sum of the DeepSeekMoE layer ("core design 2" equation
// of the DeepSeekMoE notes):
//   h_t = u_t + sum_shared FFN(u_t) + sum_k g_{t,k} FFN_{idx[t][k]}(u_t)
// The gate-scaled routed outputs arrive in pair order (t K' + k), the summed
// shared output per token: fp32 for fp32 layers, fp16 for bf16 layers (with
// fp32 kept where fp16 overflows; f16x4_value).  Each thread adds four columns
// in a fixed order (residual, shared, then k = 0..K'-1) in fp32 and rounds
// once, so the result is the same bit pattern on every run (no atomics).
#include "common.h"

namespace moe {

constexpr int kMaxTopK = 16;   // the API's bound on K'

template <bool BF16>
__global__ __launch_bounds__(256) void k_combine(int T, int d, int K, int N, int has_shared,
                                                 const void *__restrict__ x,
                                                 const int32_t *__restrict__ idx,
                                                 const float *__restrict__ yr,
                                                 const float *__restrict__ ys,
                                                 const uint16_t *__restrict__ yrh,
                                                 const uint16_t *__restrict__ ysh,
                                                 void *__restrict__ h) {
    const int ncb = (d / 4 + blockDim.x - 1) / blockDim.x;
    const int t = blockIdx.x / ncb;
    const int c = ((blockIdx.x % ncb) * blockDim.x + threadIdx.x) * 4;
    if (t >= T || c >= d) return;
    const size_t o = (size_t)t * d + c;
    // Every load is issued before the first add (K' <= kMaxTopK), so the
    // K' + 2 reads of a thread overlap instead of waiting one by one.
    uint2 xv = make_uint2(0, 0), sv = make_uint2(0, 0), yv[kMaxTopK];
    float4 xf = make_float4(0, 0, 0, 0), sf = xf, yf[kMaxTopK];
    bool live[kMaxTopK];
    if constexpr (BF16) xv = *(const uint2 *)((const uint16_t *)x + o);
    else xf = *(const float4 *)((const float *)x + o);
    if (has_shared) {
        if constexpr (BF16) sv = *(const uint2 *)(ysh + o);
        else sf = *(const float4 *)(ys + o);
    }
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        live[k] = false;
        if (k < K) {
            const int e = idx[(size_t)t * K + k];
            live[k] = e >= 0 && e < N;
            const size_t oy = ((size_t)t * K + k) * d + c;
            if (live[k]) {
                if constexpr (BF16) yv[k] = *(const uint2 *)(yrh + oy);
                else yf[k] = *(const float4 *)(yr + oy);
            }
        }
    }
    float4 acc;
    if constexpr (BF16) {
        acc.x = bf16_to_f32((uint16_t)(xv.x & 0xffffu));
        acc.y = bf16_to_f32((uint16_t)(xv.x >> 16));
        acc.z = bf16_to_f32((uint16_t)(xv.y & 0xffffu));
        acc.w = bf16_to_f32((uint16_t)(xv.y >> 16));
    } else {
        acc = xf;
    }
    if (has_shared) {
        const float4 v = BF16 ? f16x4_value(sv, ys + o) : sf;
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        if (!live[k]) continue;
        const float4 v = BF16 ? f16x4_value(yv[k], yr + ((size_t)t * K + k) * d + c) : yf[k];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    if (BF16) {
        uint2 v;
        v.x = pack_bf16x2(acc.x, acc.y);
        v.y = pack_bf16x2(acc.z, acc.w);
        *(uint2 *)((uint16_t *)h + o) = v;
    } else {
        *(float4 *)((float *)h + o) = acc;
    }
}

hipError_t launch_combine(const moe_config &c, const void *x, const int32_t *idx, const float *yr,
                          const float *ys, const uint16_t *yrh, const uint16_t *ysh, void *h,
                          hipStream_t s) {
    dim3 grid(((c.d_model / 4 + 255) / 256) * c.T);
    if (c.dtype == MOE_BF16)
        hipLaunchKernelGGL(k_combine<true>, grid, dim3(256), 0, s, c.T, c.d_model, c.top_k,
                           c.n_routed, c.n_shared > 0, x, idx, yr, ys, yrh, ysh, h);
    else
        hipLaunchKernelGGL(k_combine<false>, grid, dim3(256), 0, s, c.T, c.d_model, c.top_k,
                           c.n_routed, c.n_shared > 0, x, idx, yr, ys, yrh, ysh, h);
    return hipGetLastError();
}

}  // namespace moe
