// Re-layout kernels into the packed layout of common.hpp.
//
// Gather-and-pack of the gate_up activations for the LDS-tiled GEMM:
// The grouped GEMM reads each expert's tokens in sorted order; with x
// row-major every 32-wide K slab of a 16-row group is 16 scattered 64-byte
// pieces.  This kernel writes x once per sorted row into the packed layout of
// common.hpp (xp[group][slab] 1 KiB blocks), so the GEMM's token copies read
// 1 KiB contiguously, the access shape L2 serves best.  Padding rows and K
// past H are zeros.
#pragma once

#include "common.hpp"

namespace moelora {

struct PackXParams {
    const uint16_t *x;          // [T, H]
    const int32_t *sorted_ids;  // [cap]
    const int32_t *counters;    // [0] = padded row count
    uint16_t *xp;               // packed, cap/16 groups x nslab blocks
    int H, P, Kp;
};

// One workgroup per 16-row group g; wave w packs slabs w, w+4, ...  Lane l
// reads row l/4, chunk l%4 of the slab (4 lanes cover one row's 64 contiguous
// bytes) and writes it to its place in the block.
__device__ __forceinline__ void pack_x_group(const PackXParams &p, int g) {
    if (g * 16 >= p.counters[0]) return;
    const int lane = lane_id(), w = (int)(threadIdx.x >> 6);
    const int r = lane >> 2, c = lane & 3;
    const int f = p.sorted_ids[g * 16 + r];
    const bool ok = f < p.P;
    const uint16_t *row = p.x + (ok ? (int64_t)(f / p.Kp) * p.H : 0) + c * 8;
    const int nslab = (p.H + kSlabK - 1) / kSlabK;
    uint16_t *dst = p.xp + (int64_t)g * nslab * kBlockElems + (c * 16 + r) * 8;
    for (int s = w; s < nslab; s += 4) {
        const int k = s * kSlabK + c * 8;
        const u32x4 v = ld16(row + s * kSlabK, ok && k < p.H);  // H is a multiple of 8
        *reinterpret_cast<u32x4 *>(dst + (int64_t)s * kBlockElems) = v;
    }
}

__global__ __launch_bounds__(256) void pack_x_kernel(PackXParams p) { pack_x_group(p, (int)blockIdx.x); }

// Packed expert weights (see moe_lora_pack_weights): w13 with the gate and up
// rows of 8 features per 16-row group, w2 with 16 consecutive rows per
// group; groups per expert rounded up to whole 256-row GEMM tiles.
__host__ __device__ inline int64_t packed_w13_groups(int64_t I) { return 16 * ((I + 127) / 128); }
__host__ __device__ inline int64_t packed_w2_groups(int64_t H) { return 16 * ((H + 255) / 256); }

// Packed MXFP8 codes (see moe_lora_pack_mxfp8_weights): for every 16
// consecutive rows of an expert's code matrix and every 128-wide chunk c of
// K, one 2 KiB block [q][lane][16 bytes] with lane = 16 g + r holding codes
// 128 c + 32 g + 16 q .. + 15 of row r (zeros past K).  That is the per-lane
// order of the streaming GEMM's MXFP8 fragment loads, so each of its load
// instructions reads 1 KiB contiguously.
__host__ __device__ inline int64_t packed_mx_chunks(int64_t K) { return (K + 127) / 128; }

struct PackMxParams {
    const uint8_t *src;  // [rows_total, K] row-major codes (rows_total a multiple of 16)
    uint8_t *dst;        // [rows_total / 16][chunks][2 KiB]
    int64_t pieces;      // 16-byte pieces of dst
    int K, nch;
};

__global__ __launch_bounds__(256) void pack_mx_kernel(PackMxParams p) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < p.pieces; i += (int64_t)gridDim.x * 256) {
        const int64_t grp = i / ((int64_t)p.nch * 128);
        const int rem = (int)(i - grp * p.nch * 128);
        const int c = rem >> 7, q = (rem >> 6) & 1, lane = rem & 63;
        const int64_t row = grp * 16 + (lane & 15);
        const int k = 128 * c + 32 * (lane >> 4) + 16 * q;  // K is a multiple of 32: a piece is all in or all out
        u32x4 v = {0u, 0u, 0u, 0u};
        if (k < p.K) v = *reinterpret_cast<const u32x4 *>(p.src + row * p.K + k);
        *reinterpret_cast<u32x4 *>(p.dst + i * 16) = v;
    }
}

struct PackWParams {
    const uint16_t *src;  // [E', rows_src, K] row-major
    uint16_t *dst;        // [E'][G][nslab] blocks
    int64_t rows_src;     // rows per expert in src: 2I (w13) or H (w2)
    int K, nslab, G;
    int N;                // features (w13: I) or rows (w2: H) that exist
    int gate_up;          // 1: w13 group order
};

// grid (G, E'): one workgroup per (group, expert); wave w packs slabs w,
// w+4, ...  Lane l reads row l/4, chunk l%4 (coalesced 64 bytes per row).
__global__ __launch_bounds__(256) void pack_w_kernel(PackWParams p) {
    const int q = blockIdx.x, e = blockIdx.y;
    const int lane = lane_id(), w = (int)(threadIdx.x >> 6);
    const int r = lane >> 2, c = lane & 3;
    int srow;
    bool ok;
    if (p.gate_up) {
        const int f = 8 * q + 2 * (r >> 2) + (r & 1);
        ok = f < p.N;
        srow = ((r & 3) < 2) ? f : p.N + f;
    } else {
        srow = 16 * q + r;
        ok = srow < p.N;
    }
    const uint16_t *row = p.src + ((int64_t)e * p.rows_src + (ok ? srow : 0)) * p.K + c * 8;
    uint16_t *dst = p.dst + ((int64_t)e * p.G + q) * p.nslab * kBlockElems + (c * 16 + r) * 8;
    for (int s = w; s < p.nslab; s += 4) {
        const int k = s * kSlabK + c * 8;
        *reinterpret_cast<u32x4 *>(dst + (int64_t)s * kBlockElems) = ld16(row + s * kSlabK, ok && k < p.K);
    }
}

}  // namespace moelora
