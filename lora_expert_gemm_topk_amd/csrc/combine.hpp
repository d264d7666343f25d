// Top-k weighted combine: out[t, n] = rsf * sum_{j < K+S} w[t, j] * y2[t*(K+S)+j, n],
// summed in fp32 in slot order and rounded once to the output dtype.
// The scale rsf multiplies the whole combine, so with the shared slot
// weighted 1/rsf the fused layer equals rsf * routed output + the shared
// expert's MLP (secrett2633 analysis of vLLM PR 46545, "lessons" item 2).
// The bf16 layer keeps y2 in bf16, the activation type (the expert outputs
// are rounded once before the weighted sum), the fp32 layer in fp32.  Each
// thread owns 4 consecutive features of one token.
#pragma once

#include "common.hpp"

namespace moelora {

// BF16: y2 and out in bf16 (the bf16 layer), else both fp32.  A thread owns
// kCombineVec<BF16> consecutive features of one token: 16-byte loads of y2.
template <bool BF16>
constexpr int kCombineVec = BF16 ? 8 : 4;

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void *__restrict__ y2, const float *__restrict__ wts,
                                                      void *__restrict__ out, int T, int H, int Kp, float rsf) {
    constexpr int V = kCombineVec<BF16>;
    const int t = blockIdx.y;
    const int n = (blockIdx.x * 256 + (int)threadIdx.x) * V;
    if (t >= T || n >= H) return;
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    const float *wt = wts + (int64_t)t * Kp;
    for (int j = 0; j < Kp; ++j) {
        const float wj = wt[j];
        const int64_t off = ((int64_t)t * Kp + j) * H + n;
        float y[V];
        if constexpr (BF16) {
            const u32x4 u = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(y2) + off);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                y[2 * i] = __uint_as_float(u[i] << 16);
                y[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
            }
        } else {
            const float4 v = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(y2) + off);
            y[0] = v.x;
            y[1] = v.y;
            y[2] = v.z;
            y[3] = v.w;
        }
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] += wj * y[i];
    }
    if constexpr (BF16) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(acc[2 * i] * rsf, acc[2 * i + 1] * rsf);
        *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(out) + (int64_t)t * H + n) = v;
    } else {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + (int64_t)t * H + n) =
            make_float4(acc[0] * rsf, acc[1] * rsf, acc[2] * rsf, acc[3] * rsf);
    }
}

}  // namespace moelora
