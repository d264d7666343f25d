// fp32 variant of the expert GEMMs and the LoRA shrink.
//
// Same layer, same alignment and same work decomposition as the bf16 path,
// but every product and sum is a true fp32 FMA on the vector ALUs (no bf16
// rounding of any operand).  It exists for full-precision checking of the
// layer (fp32 tolerance 1e-5), not for speed: one thread per output element,
// reduction in index order.
#pragma once

#include "common.hpp"

namespace moelora {

struct F32Params {
    const float *in;             // gate_up: x [T, Kdim]; down: h [cap, Kdim]
    const int32_t *sorted_ids;
    const int32_t *block_expert;
    const int32_t *counters;
    const int32_t *adapter_ids;
    const float *W;              // w13 [Ep, 2N, Kdim] or w2 [Ep, N, Kdim]
    const float *B;              // b13 [L, Ep, 2N, r] or b2 [L, Ep, N, r]
    const float *s;              // [cap][r]
    float *out;                  // gate_up: h [cap, N]; down: y2 [P, N]
    int Kdim, Nout, Kp, P, cap, Ep, L, r, lora, bt;
};

// sum_c x[c] * w[c] over K (a multiple of 8): 16-byte loads, four fp32
// accumulators (lanes of the float4) combined in a fixed order.
__device__ __forceinline__ float dot_f32(const float *x, const float *w, int K) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = 0; c < K; c += 4) {
        const float4 xv = *reinterpret_cast<const float4 *>(x + c);
        const float4 wv = *reinterpret_cast<const float4 *>(w + c);
        a.x = fmaf(xv.x, wv.x, a.x);
        a.y = fmaf(xv.y, wv.y, a.y);
        a.z = fmaf(xv.z, wv.z, a.z);
        a.w = fmaf(xv.w, wv.w, a.w);
    }
    return (a.x + a.y) + (a.z + a.w);
}

__global__ __launch_bounds__(256) void shrink_f32_kernel(const float *__restrict__ in, const int32_t *sorted_ids,
                                                         const float *__restrict__ A, const int32_t *items,
                                                         const int32_t *counters, float *s, int Kdim, int r,
                                                         int Ep, int Kp, int gather) {
    const int item = blockIdx.x;
    if (item >= counters[1]) return;
    const int4 it = reinterpret_cast<const int4 *>(items)[item];
    for (int q = (int)threadIdx.x; q < it.y * r; q += 256) {
        const int j = q / r, k = q % r;
        const int prow = it.x + j;
        const int64_t row = gather ? (int64_t)(sorted_ids[prow] / Kp) : (int64_t)prow;
        const float *x = in + row * Kdim;
        const float *a = A + (((int64_t)it.z * Ep + it.w) * r + k) * Kdim;
        s[(int64_t)prow * r + k] = dot_f32(x, a, Kdim);
    }
}

template <bool GU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(F32Params p) {
    const int b = blockIdx.y;
    if (b * p.bt >= p.counters[0]) return;
    const int e = p.block_expert[b];
    const int N = p.Nout;
    const int rows_per_expert = GU ? 2 * N : N;
    for (int q = (int)threadIdx.x; q < p.bt * 64; q += 256) {
        const int j = q / 64, n = blockIdx.x * 64 + q % 64;
        if (n >= N) continue;
        const int prow = b * p.bt + j;
        const int f = p.sorted_ids[prow];
        if (f >= p.P) {
            if (GU) p.out[(int64_t)prow * N + n] = 0.f;
            continue;
        }
        const float *x = p.in + (GU ? (int64_t)(f / p.Kp) : (int64_t)prow) * p.Kdim;
        const float *w0 = p.W + ((int64_t)e * rows_per_expert + n) * p.Kdim;
        const float *w1 = p.W + ((int64_t)e * rows_per_expert + N + n) * p.Kdim;
        float v0 = dot_f32(x, w0, p.Kdim), v1 = 0.f;
        if (GU) v1 = dot_f32(x, w1, p.Kdim);
        if (p.lora) {
            const int a = p.adapter_ids[f / p.Kp];
            if (a >= 0 && a < p.L) {
                const float *sv = p.s + (int64_t)prow * p.r;
                const float *B0 = p.B + (((int64_t)a * p.Ep + e) * rows_per_expert + n) * p.r;
                float d0 = 0.f, d1 = 0.f;
                for (int k = 0; k < p.r; ++k) d0 = fmaf(sv[k], B0[k], d0);
                v0 += d0;
                if (GU) {
                    const float *B1 = B0 + (int64_t)N * p.r;
                    for (int k = 0; k < p.r; ++k) d1 = fmaf(sv[k], B1[k], d1);
                    v1 += d1;
                }
            }
        }
        if (GU) p.out[(int64_t)prow * N + n] = (v0 / (1.0f + expf(-v0))) * v1;
        else p.out[(int64_t)f * N + n] = v0;
    }
}

}  // namespace moelora
