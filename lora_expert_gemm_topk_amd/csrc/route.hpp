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
//
// Biased variant (the router module that analysis names in "code analysis"
// part 1 is a top-k router with a bias; the page gives no formula, and the
// reading implemented is): fp64 score s_e per expert, the sigmoid of the
// logit or the softmax over all E logits (exp of logit minus the largest,
// divided by the sum over experts in index order); the choice takes the K
// largest keys s_e + b_e (b the per-expert fp32 bias, 0 when absent), lower
// index on an exact tie; the weights are the unbiased scores of the chosen
// experts, divided by their slot-order sum when renormalizing, rounded once
// to fp32.  The bias steers the choice only.
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
    int scoring = -1;     // -1: plain top-k of the logits; 0: biased, softmax scores; 1: biased, sigmoid scores
    const float *bias = nullptr;  // [E] (biased router only; nullptr = zero bias)
};

// The value of `v` in lane j, j the same in every lane: v_readlane (a
// scalar read) rather than a permute through the LDS crossbar.
__device__ __forceinline__ float lane_value(float v, int j) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), j));
}
__device__ __forceinline__ double lane_value(double v, int j) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, j);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), j);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// The plain router's candidates as one 64-bit integer: the high half an
// order-preserving key of the value (larger value, larger key; -0 taken as
// +0 so that equal values tie), the low half the complement of the expert
// index, so a larger integer is the better candidate under (value desc,
// index asc) and 0 is "none" (every finite value's key is at least 2^23).
__device__ __forceinline__ uint32_t order_key(float x) {
    const uint32_t b = x == 0.0f ? 0u : __float_as_uint(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float order_key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}
__device__ __forceinline__ uint64_t pack_cand(float v, int e) {
    return ((uint64_t)order_key(v) << 32) | (uint32_t)~e;
}

// One step of a wavefront-wide arg-max over packed candidates: each lane of
// the rows in ROW_MASK compares with the candidate DPP pattern CTRL brings
// it (lanes without a source see 0, "none").  The order is total, so the
// winner does not depend on the pattern.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void cand_dpp_step(uint64_t &c) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)c, CTRL, ROW_MASK, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(c >> 32), CTRL, ROW_MASK, 0xf, false);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    if (o > c) c = o;
}

// The best candidate of the wavefront, in every lane: exchanges within quads
// (lane xor 1, xor 2), half-rows and rows (mirrors), then across rows (row
// broadcasts) leave it in lane 63, which is read out.  Register-to-register
// steps (DPP) instead of LDS-routed shuffles: the router's K rounds each run
// one of these.
__device__ __forceinline__ uint64_t wave_best(uint64_t c) {
    cand_dpp_step<0xb1, 0xf>(c);   // quad_perm [1,0,3,2]
    cand_dpp_step<0x4e, 0xf>(c);   // quad_perm [2,3,0,1]
    cand_dpp_step<0x141, 0xf>(c);  // row_half_mirror
    cand_dpp_step<0x140, 0xf>(c);  // row_mirror
    cand_dpp_step<0x142, 0xa>(c);  // row_bcast15 into rows 1, 3
    cand_dpp_step<0x143, 0xc>(c);  // row_bcast31 into rows 2, 3
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)c, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(c >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// DPP move of one 32-bit word (lanes without a source, or outside ROW_MASK,
// get `none`).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_int(int x, int none) {
    return __builtin_amdgcn_update_dpp(none, x, CTRL, ROW_MASK, 0xf, false);
}
// The biased router's candidates: an order-preserving 64-bit key of its fp64
// key (-0 taken as +0; 0 is "none", below every finite value) and the
// complemented expert index, compared as one 96-bit unsigned integer; the
// winner's unbiased score is read from its lane afterwards.
struct Cand64 {
    uint64_t k;
    uint32_t i;
};
__device__ __forceinline__ uint64_t order_key(double x) {
    const uint64_t b = x == 0.0 ? 0ull : __builtin_bit_cast(uint64_t, x);
    return (b >> 63) ? ~b : (b | (1ull << 63));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void cand_dpp_step(Cand64 &c) {
    const uint32_t klo = (uint32_t)dpp_int<CTRL, ROW_MASK>((int)(uint32_t)c.k, 0);
    const uint32_t khi = (uint32_t)dpp_int<CTRL, ROW_MASK>((int)(uint32_t)(c.k >> 32), 0);
    const uint32_t oi = (uint32_t)dpp_int<CTRL, ROW_MASK>((int)c.i, 0);
    const uint64_t ok = ((uint64_t)khi << 32) | klo;
    const bool take = ok > c.k || (ok == c.k && oi > c.i);
    c.k = take ? ok : c.k;
    c.i = take ? oi : c.i;
}
__device__ __forceinline__ Cand64 wave_best(Cand64 c) {
    cand_dpp_step<0xb1, 0xf>(c);
    cand_dpp_step<0x4e, 0xf>(c);
    cand_dpp_step<0x141, 0xf>(c);
    cand_dpp_step<0x140, 0xf>(c);
    cand_dpp_step<0x142, 0xa>(c);
    cand_dpp_step<0x143, 0xc>(c);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)c.k, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(c.k >> 32), 63);
    return Cand64{((uint64_t)hi << 32) | lo, (uint32_t)__builtin_amdgcn_readlane((int)c.i, 63)};
}

// The largest of the wavefront's values, in every lane (a maximum is exact
// in any order).  Lanes without a value pass -inf.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, __builtin_bit_cast(float, dpp_int<0xb1, 0xf>(__builtin_bit_cast(int, x), (int)0xff800000u)));
    x = fmaxf(x, __builtin_bit_cast(float, dpp_int<0x4e, 0xf>(__builtin_bit_cast(int, x), (int)0xff800000u)));
    x = fmaxf(x, __builtin_bit_cast(float, dpp_int<0x141, 0xf>(__builtin_bit_cast(int, x), (int)0xff800000u)));
    x = fmaxf(x, __builtin_bit_cast(float, dpp_int<0x140, 0xf>(__builtin_bit_cast(int, x), (int)0xff800000u)));
    x = fmaxf(x, __builtin_bit_cast(float, dpp_int<0x142, 0xa>(__builtin_bit_cast(int, x), (int)0xff800000u)));
    x = fmaxf(x, __builtin_bit_cast(float, dpp_int<0x143, 0xc>(__builtin_bit_cast(int, x), (int)0xff800000u)));
    return lane_value(x, 63);
}

// Biased router for token t (see the file comment): returns to lane j the
// expert id of slot j like route_one_token.
template <int VPL>
__device__ int route_one_token_bias(const RouteParams &rp, int t, bool write) {
    const int lane = lane_id();
    const int E = rp.E, K = rp.K, S = rp.S;
    const float *l = rp.logits + (int64_t)t * E;
    double sc[VPL], key[VPL];
    bool live[VPL];
    float lf[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int e = lane + 64 * j;
        live[j] = e < E;
        lf[j] = live[j] ? l[e] : -__builtin_huge_valf();
    }
    if (rp.scoring == 0) {
        // largest logit (exact), then the exps of each lane's own logits,
        // summed in expert order
        float mx = lf[0];
#pragma unroll
        for (int j = 1; j < VPL; ++j) mx = fmaxf(mx, lf[j]);
        const double m = (double)wave_max(mx);
        double den = 0.0;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            sc[j] = live[j] ? exp((double)lf[j] - m) : 0.0;
            for (int q = 0; q < 64 && 64 * j + q < E; ++q) den += lane_value(sc[j], q);
        }
#pragma unroll
        for (int j = 0; j < VPL; ++j) sc[j] = sc[j] / den;
    } else {
#pragma unroll
        for (int j = 0; j < VPL; ++j) sc[j] = 1.0 / (1.0 + exp(-(live[j] ? (double)lf[j] : 0.0)));
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int e = lane + 64 * j;
        key[j] = sc[j] + ((live[j] && rp.bias) ? (double)rp.bias[e] : 0.0);
    }
    uint64_t kk[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) kk[j] = order_key(key[j]);
    double mys = 0.0;
    int myi = -1;
    for (int s = 0; s < K; ++s) {
        Cand64 c{0ull, 0u};
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const uint32_t di = ~(uint32_t)(lane + 64 * j);
            if (live[j] && (kk[j] > c.k || (kk[j] == c.k && di > c.i))) c = Cand64{kk[j], di};
        }
        c = wave_best(c);  // every lane now holds the same winner
        const int ci = (int)~c.i;
        // the winner's unbiased score, from its lane
        double cs = 0.0;
#pragma unroll
        for (int j = 0; j < VPL; ++j)
            if (j == (ci >> 6)) cs = lane_value(sc[j], ci & 63);
        if ((ci & 63) == lane) {
#pragma unroll
            for (int j = 0; j < VPL; ++j)
                if (j == (ci >> 6)) live[j] = false;
        }
        if (lane == s) {
            mys = cs;
            myi = ci;
        }
    }
    double sum = 0.0;
    for (int j = 0; j < K; ++j) sum += lane_value(mys, j);
    const int Kp = K + S;
    if (write && lane < K) {
        rp.ids[(int64_t)t * Kp + lane] = myi;
        rp.wts[(int64_t)t * Kp + lane] = (float)(rp.renorm ? mys / sum : mys);
    }
    if (write && lane < S) {
        rp.ids[(int64_t)t * Kp + K + lane] = E + lane;
        rp.wts[(int64_t)t * Kp + K + lane] = rp.shared_w;
    }
    if (lane >= K) myi = (lane < Kp) ? E + (lane - K) : -1;
    return myi;
}

// Route token t with the whole wavefront; writes ids and weights of its K+S
// slots (unless `write` is false) and returns to lane j the expert id of
// slot j (-1 for j >= K+S; slots beyond lane 63 are written but not returned).
template <int VPL>
__device__ int route_one_token(const RouteParams &rp, int t, bool write = true) {
    if (rp.scoring >= 0) return route_one_token_bias<VPL>(rp, t, write);
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
    uint64_t cand[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) cand[j] = pack_cand(v[j], lane + 64 * j);
    float myv = 0.0f;
    int myi = -1;
    for (int s = 0; s < K; ++s) {
        uint64_t c = 0;
#pragma unroll
        for (int j = 0; j < VPL; ++j)
            if (live[j] && cand[j] > c) c = cand[j];
        c = wave_best(c);  // every lane now holds the same winner
        const int ci = (int)~(uint32_t)c;
        if ((ci & 63) == lane) {
#pragma unroll
            for (int j = 0; j < VPL; ++j)
                if (j == (ci >> 6)) live[j] = false;
        }
        if (lane == s) {
            myv = order_key_value((uint32_t)(c >> 32));  // a zero comes back as +0: same exp below
            myi = ci;
        }
    }
    const double m = (double)lane_value(myv, 0);
    const double ex = (lane < K) ? exp((double)myv - m) : 0.0;
    double sum = 0.0;
    if (rp.renorm) {
        for (int j = 0; j < K; ++j) sum += lane_value(ex, j);
    } else {
        // softmax over all E: each lane's exps of its own logits, summed in
        // expert order
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const double xj = lane + 64 * j < E ? exp((double)v[j] - m) : 0.0;
            for (int q = 0; q < 64 && 64 * j + q < E; ++q) sum += lane_value(xj, q);
        }
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
