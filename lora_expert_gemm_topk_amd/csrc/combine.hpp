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

// BF16: y2 and out in bf16 (the bf16 layer), else both fp32.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void *__restrict__ y2, const float *__restrict__ wts,
                                                      void *__restrict__ out, int T, int H, int Kp, float rsf) {
    const int t = blockIdx.y;
    const int n = (blockIdx.x * 256 + (int)threadIdx.x) * 4;
    if (t >= T || n >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const float *wt = wts + (int64_t)t * Kp;
    for (int j = 0; j < Kp; ++j) {
        const float wj = wt[j];
        float4 y;
        if (BF16) {
            const uint2 u = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(y2) +
                                                             ((int64_t)t * Kp + j) * H + n);
            y = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                            __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
        } else {
            y = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(y2) + ((int64_t)t * Kp + j) * H + n);
        }
        acc.x += wj * y.x;
        acc.y += wj * y.y;
        acc.z += wj * y.z;
        acc.w += wj * y.w;
    }
    acc.x *= rsf;
    acc.y *= rsf;
    acc.z *= rsf;
    acc.w *= rsf;
    if (BF16) {
        uint2 v = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(out) + (int64_t)t * H + n) = v;
    } else {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + (int64_t)t * H + n) = acc;
    }
}

}  // namespace moelora
