// Top-k router with the shared-slot append.
//
// One wavefront per token.  Each lane holds the logits of experts
// lane, lane+64, ...; K rounds of a wave-wide arg-max on the key
// (value descending, expert index ascending) pick the routed experts in slot
// order.  Softmax weights are taken in fp64 (exp of logit minus the top
// logit, summed left to right in slot order) and rounded once to fp32.  The
// S shared slots follow with ids E..E+S-1 and the constant weight 1/rsf
// (secrett2633 analysis of vLLM PR 46545, "code analysis" part 1 and
// "lessons" item 2).
#pragma once

#include "common.hpp"

namespace moelora {

struct RouteParams {
    const float *logits;  // [T, E]
    int T, E, K, S;
    float shared_w;       // fl32(1/rsf)
    int renorm;
    int32_t *ids;         // [T, K+S]
    float *wts;           // [T, K+S]
};

struct Cand {
    float v;
    int i;  // expert index; INT_MAX = none
};

__device__ __forceinline__ bool better(const Cand &a, const Cand &b) {
    if (b.i == 0x7fffffff) return a.i != 0x7fffffff;
    if (a.i == 0x7fffffff) return false;
    return a.v > b.v || (a.v == b.v && a.i < b.i);
}

// Route token t with the whole wavefront; writes ids and weights of its K+S
// slots (unless `write` is false) and returns to lane j the expert id of
// slot j (-1 for j >= K+S; slots beyond lane 63 are written but not returned).
template <int VPL>
__device__ int route_one_token(const RouteParams &rp, int t, bool write = true) {
    const int lane = lane_id();
    const int E = rp.E, K = rp.K, S = rp.S;
    const float *l = rp.logits + (int64_t)t * E;
    float v[VPL];
    bool live[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int e = lane + 64 * j;
        live[j] = e < E;
        v[j] = live[j] ? l[e] : 0.0f;
    }
    float myv = 0.0f;
    int myi = -1;
    for (int s = 0; s < K; ++s) {
        Cand c{0.0f, 0x7fffffff};
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            Cand d{v[j], lane + 64 * j};
            if (live[j] && better(d, c)) c = d;
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            Cand o{__shfl_xor(c.v, off, 64), __shfl_xor(c.i, off, 64)};
            if (better(o, c)) c = o;
        }
        // every lane now holds the same winner
        if ((c.i & 63) == lane) {
#pragma unroll
            for (int j = 0; j < VPL; ++j)
                if (j == (c.i >> 6)) live[j] = false;
        }
        if (lane == s) {
            myv = c.v;
            myi = c.i;
        }
    }
    const double m = (double)__shfl(myv, 0, 64);
    const double ex = (lane < K) ? exp((double)myv - m) : 0.0;
    double sum = 0.0;
    if (rp.renorm) {
        for (int j = 0; j < K; ++j) sum += __shfl(ex, j, 64);
    } else {
        for (int e = 0; e < E; ++e) sum += exp((double)l[e] - m);
    }
    const int Kp = K + S;
    if (write && lane < K) {
        rp.ids[(int64_t)t * Kp + lane] = myi;
        rp.wts[(int64_t)t * Kp + lane] = (float)(ex / sum);
    }
    if (write && lane < S) {
        rp.ids[(int64_t)t * Kp + K + lane] = E + lane;
        rp.wts[(int64_t)t * Kp + K + lane] = rp.shared_w;
    }
    if (lane >= K) myi = (lane < Kp) ? E + (lane - K) : -1;
    return myi;
}

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(RouteParams rp) {
    const int t = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (t >= rp.T) return;
    route_one_token<VPL>(rp, t);
}

}  // namespace moelora
