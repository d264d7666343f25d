// Device helpers shared by the gfx950 kernels of the MoE-LoRA layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moelora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32, which
// converts two values per instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Lanes of the wave whose `key` equals this lane's (restricted to lanes with
// `valid`).  Bit-sliced: one ballot per key bit.  Result only meaningful on
// valid lanes.
__device__ __forceinline__ uint64_t match_key(uint32_t key, bool valid, int nbits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1u;
        const uint64_t bal = __ballot(valid && bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// silu(z) = z * sigmoid(z); the reciprocal is the hardware approximation
// (v_rcp_f32, about 1 ulp), far below the bf16 rounding of every result.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// 16-byte global load that returns zeros when `ok` is false.
__device__ __forceinline__ u32x4 ld16(const void *p, bool ok) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ok) v = *reinterpret_cast<const u32x4 *>(p);
    return v;
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Packed operand layout ("row groups x K slabs").  Rows are taken in groups of
// 16 and K in slabs of 32; each (group, slab) pair is one 1 KiB block, blocks
// group-major (a group's slabs are consecutive).  Inside a block, element
// (r, k) sits at element index (k/8)*128 + r*8 + k%8: 16-byte chunk
// (k/8)*16 + r.  That is the per-lane order of a v_mfma_f32_16x16x32_bf16
// operand fragment (lane = (k/8)*16 + r holds 8 consecutive k of row r), so a
// wave fetches a whole fragment with one 16-byte load per lane reading 1 KiB
// contiguously, and an LDS copy of a block serves 32x32x16 fragment reads
// without bank conflicts (16 consecutive lanes read 256 contiguous bytes).
// K past the last element of a slab is zero.
constexpr int kGroupRows = 16;
constexpr int kSlabK = 32;
constexpr int kBlockElems = kGroupRows * kSlabK;  // 512 bf16 = 1 KiB

// Element offset of (row, k) in a packed matrix with `nslab` slabs per group.
__host__ __device__ __forceinline__ int64_t packed_off(int64_t row, int64_t k, int64_t nslab) {
    return ((row >> 4) * nslab + (k >> 5)) * kBlockElems + ((k >> 3) & 3) * 128 + (row & 15) * 8 + (k & 7);
}

// Map workgroup i (dispatched to XCD i % 8) to a logical index such that each
// XCD owns one contiguous range of logical indices.  Bijective on [0, total).
__device__ __forceinline__ int xcd_logical(int i, int total) {
    const int q = total / 8, rem = total % 8;
    const int x = i % 8, k = i / 8;
    return (x < rem) ? x * (q + 1) + k : rem * (q + 1) + (x - rem) * q + k;
}

}  // namespace moelora
