// LoRA shrink: s[p, k] = sum_c in[p, c] * A[a, e, k, c] for the rows p of one
// (adapter, expert) work item.
//
// The shrink is the skinny side of LoRA: r (16..64) output columns against a
// reduction over H or I.  Following the split-K idea for skinny LoRA
// products (aitrends.kr summary of the AWS multi-LoRA MoE post, "section
// details" and "practical takeaways"), the reduction is split twice: across
// `split` workgroups (grid.y) and, inside a workgroup, across its 4
// wavefronts.  Partials go to s_part[split][row][r] in fp32 and are summed
// in fixed order by the consumer (the expand in the next GEMM's epilogue), so
// the result does not depend on scheduling.  For the LDS-tiled GEMM the
// shrink runs unsplit and writes its sums rounded once to bf16, the operand
// type the tiled kernel streams.  Items past the item count exit at once: a
// layer call whose tokens carry no adapter does no shrink work.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16): the MFMA M side is the
// rank index k (A rows), the N side is the item's rows (tokens), K is the
// reduction.  Rows k >= r and tokens past the item length load zeros.
#pragma once

#include "common.hpp"
#include "pack.hpp"
#include "route.hpp"

namespace moelora {

struct ShrinkParams {
    const uint16_t *in;        // gate_up: x [T, H]; down: h (row = sorted position), row-major or packed
    const int32_t *sorted_ids; // gate_up only: pair index per sorted position
    const uint16_t *A;         // [L, Ep, r, Kdim]
    const int32_t *items;      // [max_items][4]
    const int32_t *counters;   // [1] = item count
    float *s_part;             // [split][cap][r] fp32, or [cap][r] bf16 when out_bf16
    int Kdim, r, Ep, Kp, P, cap;
    int out_bf16;              // 1: split == 1, write the sum rounded once to bf16
    int in_packed;             // down only: h in the packed layout of common.hpp
    int chunks_per_split;      // in units of 32 along Kdim
};

// NT: 16-row token subtiles per item (lora_block_m = 16*NT); MT: 16-row
// rank subtiles (r <= 16*MT); GATHER: rows come from x through sorted_ids.
// One workgroup's work: item `item`, K split `ks`.
template <int NT, int MT, bool GATHER>
__device__ __forceinline__ void shrink_item(const ShrinkParams &p, int item, int ks) {
    __shared__ float red[4][16 * NT][16 * MT + 4];
    if (item >= p.counters[1]) return;
    const int4 it = reinterpret_cast<const int4 *>(p.items)[item];
    const int p0 = it.x, len = it.y, a = it.z, e = it.w;
    const int lane = lane_id(), w = (int)(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    const int64_t Kd = p.Kdim;

    // Per-lane pointers for the N side (tokens) at this lane's k-group of
    // chunk 0, advanced by xstep per 32-wide chunk: gathered x rows, rows of
    // h, or rows of the packed h (one 1 KiB block per 16 rows x 32 k).
    const uint16_t *xrow[NT];
    bool xok[NT];
    const int64_t nslab = (Kd + kSlabK - 1) / kSlabK;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int j = nt * 16 + l16;
        xok[nt] = j < len;
        if (GATHER) {
            const int64_t row = xok[nt] ? p.sorted_ids[p0 + j] / p.Kp : 0;
            xrow[nt] = p.in + row * Kd + g * 8;
        } else if (p.in_packed) {
            const int64_t row = p0 + (xok[nt] ? j : 0);
            xrow[nt] = p.in + packed_off(row, (int64_t)g * 8, nslab);
        } else {
            const int64_t row = p0 + (xok[nt] ? j : 0);
            xrow[nt] = p.in + row * Kd + g * 8;
        }
    }
    const int64_t xstep = (GATHER || !p.in_packed) ? kSlabK : kBlockElems;
    const uint16_t *arow[MT];
    bool aok[MT];
    const uint16_t *Abase = p.A + ((int64_t)a * p.Ep + e) * p.r * Kd;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int k = mt * 16 + l16;
        aok[mt] = k < p.r;
        arow[mt] = Abase + (int64_t)(aok[mt] ? k : 0) * Kd;
    }

    f32x4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nch = (int)((Kd + 31) / 32);
    const int c_beg = ks * p.chunks_per_split;
    const int c_end = min(nch, c_beg + p.chunks_per_split);
    // Chunks c_beg + w, +4, +8, ... go to wave w; a wave issues the loads of
    // kBatch chunks before their MFMAs so its memory requests overlap (chunks
    // past the end load zeros, whose products add exact zeros).
    constexpr int kBatch = 4;
    for (int c = c_beg + w; c < c_end; c += 4 * kBatch) {
        u32x4 av[kBatch][MT], xv[kBatch][NT];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int cc = c + 4 * u;
            const int64_t k0 = (int64_t)cc * 32 + g * 8;
            const bool kin = cc < c_end && k0 < Kd;  // Kdim is a multiple of 8
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) av[u][mt] = ld16(arow[mt] + k0, aok[mt] && kin);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) xv[u][nt] = ld16(xrow[nt] + (int64_t)cc * xstep, xok[nt] && kin);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[u][mt]), as_bf16x8(xv[u][nt]),
                                                                          acc[mt][nt], 0, 0, 0);
    }
    // D layout: lane holds rank rows 4*g .. 4*g+3 of column (token) l16.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[w][nt * 16 + l16][mt * 16 + g * 4 + i] = acc[mt][nt][i];
    __syncthreads();
    const int R4 = (p.r + 3) / 4;
    float *dst = p.s_part + ((int64_t)ks * p.cap + p0) * p.r;
    uint16_t *dst16 = reinterpret_cast<uint16_t *>(p.s_part) + (int64_t)p0 * p.r;
    for (int q = (int)threadIdx.x; q < len * R4; q += 256) {
        const int j = q / R4, k = (q % R4) * 4;
        for (int i = 0; i < 4 && k + i < p.r; ++i) {
            const float v = ((red[0][j][k + i] + red[1][j][k + i]) + red[2][j][k + i]) + red[3][j][k + i];
            if (p.out_bf16) dst16[(int64_t)j * p.r + k + i] = f32_to_bf16(v);
            else dst[(int64_t)j * p.r + k + i] = v;
        }
    }
}

// The items of one (adapter, expert) bin are consecutive in the item list;
// with an unsplit shrink each XCD takes one contiguous range of items, so a
// bin's A slice is fetched into one XCD's L2 and its other items hit there.
__device__ __forceinline__ int shrink_item_of(int b, int n_items) { return xcd_logical(b, n_items); }

template <int NT, int MT, bool GATHER>
__global__ __launch_bounds__(256) void shrink_kernel(ShrinkParams p) {
    int item = (int)blockIdx.x;
    if (gridDim.y == 1) {
        const int n = p.counters[1];
        if (item >= n) return;
        item = shrink_item_of(item, n);
    }
    shrink_item<NT, MT, GATHER>(p, item, (int)blockIdx.y);
}

// The gate_up shrink (unsplit, x gathered) and the gather-and-pack of x for
// the LDS-tiled GEMM in one launch: both need only the alignment, one mostly
// reads and the other mostly writes, so their memory traffic overlaps and
// one kernel boundary goes.  Workgroups [0, n_items) take shrink items (they
// are dispatched first), the rest one 16-row pack group each.
template <int NT, int MT>
__global__ __launch_bounds__(256) void pack_x_shrink_kernel(PackXParams xp, ShrinkParams sp, int n_items) {
    const int b = (int)blockIdx.x;
    if (b < n_items) {
        const int n = sp.counters[1];
        if (b < n) shrink_item<NT, MT, true>(sp, shrink_item_of(b, n), 0);
    } else {
        pack_x_group(xp, b - n_items);
    }
}

// ---------------------------------------------------------------------------
// Per-row gate_up shrink for the streaming GEMM (few rows per expert, decode).
//
// With a handful of rows per (adapter, expert) bin the item shrink above is
// latency bound, and it has to wait for the alignment.  The gate_up shrink
// needs only the routing (the expert of each pair) and the token's adapter,
// so it runs in the router's launch: workgroup (t, j) routes token t again
// in its first wavefront (workgroup j = 0 writes the routing) and then
// computes pair f = t*(K+S) + j's r sums, s13[f][k] = x[t] . A13[a,e][k],
// stored by pair index.  The loads for the whole reduction are issued at
// once: thread i takes the 16-byte chunks i and i + 256 (then i + 512, ...)
// of every A row, so each load instruction of a wavefront reads 1 KiB
// contiguously.  Each thread sums its chunks in order, each wavefront folds
// its 64 lanes with a fixed butterfly and the 4 wavefront sums are added in
// wave order: the result depends on nothing but the inputs.  A bin's slice
// of A is read once per pair (the pairs of a bin share it in L2).
struct RowShrinkParams {
    const uint16_t *in;           // x [T, Kdim]
    const uint16_t *A;            // A13 [L, Ep, r, Kdim]
    const int32_t *adapter_ids;   // [T]
    float *s;                     // s13 [P][r] fp32 by pair
    int Kdim, r, Ep, Kp, P, L;
};

// s_out[k] = sum_c in[c] * A[k][c] for k < r (r <= RMAX), by the whole
// workgroup of 256 threads; Kdim is a multiple of 8.
template <int RMAX>
__device__ __forceinline__ void shrink_row_wg(const uint16_t *__restrict__ in, const uint16_t *__restrict__ A,
                                              int Kdim, int r, float *__restrict__ s_out) {
    __shared__ float red[4][RMAX];
    const int tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nch = Kdim >> 3;
    float acc[RMAX];
#pragma unroll
    for (int k = 0; k < RMAX; ++k) acc[k] = 0.f;
    // rows k >= r repeat row r-1 (their sums are never stored), so every
    // load is in bounds and none is predicated
    for (int c0 = tid; c0 < nch; c0 += 512) {
        const int c1 = c0 + 256;
        const bool has1 = c1 < nch;
        const u32x4 x0 = *reinterpret_cast<const u32x4 *>(in + (int64_t)c0 * 8);
        const u32x4 x1 = ld16(in + (int64_t)c1 * 8, has1);
#pragma unroll
        for (int kb = 0; kb < RMAX; kb += 16) {
            u32x4 a0[16], a1[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int64_t row = (int64_t)min(kb + q, r - 1) * Kdim;
                a0[q] = *reinterpret_cast<const u32x4 *>(A + row + (int64_t)c0 * 8);
                a1[q] = ld16(A + row + (int64_t)c1 * 8, has1);
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                float v = acc[kb + q];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v = fmaf(bf16_to_f32((uint16_t)(a0[q][i] & 0xffffu)), bf16_to_f32((uint16_t)(x0[i] & 0xffffu)), v);
                    v = fmaf(bf16_to_f32((uint16_t)(a0[q][i] >> 16)), bf16_to_f32((uint16_t)(x0[i] >> 16)), v);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v = fmaf(bf16_to_f32((uint16_t)(a1[q][i] & 0xffffu)), bf16_to_f32((uint16_t)(x1[i] & 0xffffu)), v);
                    v = fmaf(bf16_to_f32((uint16_t)(a1[q][i] >> 16)), bf16_to_f32((uint16_t)(x1[i] >> 16)), v);
                }
                acc[kb + q] = v;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < RMAX; ++k) {
        float v = acc[k];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        acc[k] = v;
    }
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < RMAX; ++k) red[w][k] = acc[k];
    }
    __syncthreads();
    if (tid < r) s_out[tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

// Router + gate_up shrink: grid (T, K+S), K+S <= 64.
template <int VPL, int RMAX>
__global__ __launch_bounds__(256) void route_shrink_kernel(RouteParams rp, RowShrinkParams sp) {
    const int t = (int)blockIdx.x, j = (int)blockIdx.y;
    __shared__ int e_slot;
    if (threadIdx.x < 64) {
        const int myi = route_one_token<VPL>(rp, t, j == 0);
        const int e = __builtin_amdgcn_readlane(myi, j);
        if (threadIdx.x == 0) e_slot = e;
    }
    const int a = sp.adapter_ids[t];
    if (!(a >= 0 && a < sp.L)) return;  // the same for the whole workgroup; no barrier passed yet
    __syncthreads();
    const int e = e_slot;
    const int64_t Kd = sp.Kdim;
    shrink_row_wg<RMAX>(sp.in + (int64_t)t * Kd, sp.A + ((int64_t)a * sp.Ep + e) * sp.r * Kd, sp.Kdim, sp.r,
                        sp.s + ((int64_t)t * sp.Kp + j) * sp.r);
}

}  // namespace moelora
