// Check of the input preconditions that the layer itself does not check on
// the device (moe_lora_check_inputs): router logits (and the biased
// router's expert bias) finite, adapter ids in
// [-1, L), and for MXFP8 weights scale bytes in [1, 254] (E8M0: 0xFF is NaN,
// 0x00 the smallest power of two, outside the range the encoder writes) and
// no NaN code (E4M3: S.1111.111).  Two launches, no atomics: every workgroup
// of the first ORs the flags of its grid-stride share into one word of the
// workspace, the one workgroup of the second ORs those words into the
// caller's status word.
#pragma once

#include "common.hpp"
#include "moe_lora.h"

namespace moelora {

constexpr int kCheckBlocks = 512;

struct CheckParams {
    const float *logits;         // [n_logits] f32
    int64_t n_logits;
    const float *bias = nullptr; // [n_bias] f32 (biased router) or null
    int64_t n_bias = 0;
    const int32_t *adapter_ids;  // [n_adapters] or null
    int64_t n_adapters;
    int L;
    const uint8_t *mx[4];  // w13 codes, w13 scales, w2 codes, w2 scales (null: none); 16-B aligned
    int64_t n_mx[4];
    int32_t *partial;      // [kCheckBlocks] (null: nothing to check)
    int32_t *status;
};

__device__ __forceinline__ bool mx_bad_byte(uint32_t b, bool scale) {
    return scale ? (b == 0u || b == 255u) : ((b & 0x7fu) == 0x7fu);
}

// OR of `flag` over the workgroup (256 threads), valid on thread 0.
__device__ __forceinline__ int block_or_flags(int flag) {
    __shared__ int wflag[4];
    int wf = 0;
    for (int bit = 0; bit < 3; ++bit)
        if (__ballot((flag >> bit) & 1) != 0) wf |= 1 << bit;
    if (lane_id() == 0) wflag[threadIdx.x >> 6] = wf;
    __syncthreads();
    return wflag[0] | wflag[1] | wflag[2] | wflag[3];
}

__global__ __launch_bounds__(256) void check_inputs_kernel(CheckParams p) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int flag = 0;
    for (int64_t i = i0; i < p.n_logits; i += stride)
        if (!isfinite(p.logits[i])) flag |= MOE_LORA_BAD_LOGIT;
    for (int64_t i = i0; i < p.n_bias; i += stride)
        if (!isfinite(p.bias[i])) flag |= MOE_LORA_BAD_LOGIT;
    for (int64_t i = i0; i < p.n_adapters; i += stride) {
        const int a = p.adapter_ids[i];
        if (a < -1 || a >= p.L) flag |= MOE_LORA_BAD_ADAPTER;
    }
    for (int q = 0; q < 4; ++q) {
        if (p.mx[q] == nullptr) continue;
        const bool scale = q & 1;
        const int64_t nv = p.n_mx[q] >> 4;
        const u32x4 *v = reinterpret_cast<const u32x4 *>(p.mx[q]);
        bool bad = false;
        for (int64_t i = i0; i < nv; i += stride) {
            const u32x4 w = v[i];
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int b = 0; b < 4; ++b) bad |= mx_bad_byte((w[c] >> (8 * b)) & 0xffu, scale);
        }
        for (int64_t i = (nv << 4) + i0; i < p.n_mx[q]; i += stride) bad |= mx_bad_byte(p.mx[q][i], scale);
        if (bad) flag |= MOE_LORA_BAD_MXFP8;
    }
    const int f = block_or_flags(flag);
    if (threadIdx.x == 0) p.partial[blockIdx.x] = f;
}

__global__ __launch_bounds__(256) void check_inputs_reduce_kernel(CheckParams p) {
    int flag = 0;
    if (p.partial)
        for (int i = threadIdx.x; i < kCheckBlocks; i += 256) flag |= p.partial[i];
    const int f = block_or_flags(flag);
    if (threadIdx.x == 0) *p.status = f;
}

}  // namespace moelora
