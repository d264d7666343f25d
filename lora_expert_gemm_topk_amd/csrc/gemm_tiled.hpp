// Grouped expert GEMM for many rows per expert (prefill): LDS-tiled, matrix
// cores (v_mfma_f32_32x32x16_bf16), LoRA expand and SwiGLU in the epilogue.
//
// Same contract as the streaming kernel (gemm_stream.hpp): weights are the
// MFMA M side, the expert block's tokens the N side, y13 -> SwiGLU -> h (bf16,
// sorted row) for gate_up and y2 (fp32, pair row) for down.
//
// Workgroup tile: BW weight rows x BT tokens, 4 wavefronts in a 2 x 2 grid,
// each owning (BW/2) x (BT/2) as (BW/64) x (BT/64) MFMA tiles of 32 x 32.
// K advances 64 at a time through two LDS buffers: while the MFMAs read one
// buffer, the next 64-wide slab of weights and (gathered) tokens is in flight
// from global memory in registers and lands in the other buffer; one barrier
// per slab.  LDS rows are padded to 144 bytes so the 16-byte fragment reads of
// 8 consecutive lanes hit 8 different bank groups.
//
// gate_up row order inside a tile: rows 4a, 4a+1 hold gate features
// i0+2a, i0+2a+1 and rows 4a+2, 4a+3 the matching up features.  The 32 x 32
// accumulator gives each lane 4 consecutive rows, so every lane holds whole
// (gate, up) pairs and SwiGLU needs no data exchange.
//
// LoRA expand (aitrends.kr summary of the AWS multi-LoRA MoE post, "section
// details": LoRA sum folded into the expand step) runs as extra MFMA k-steps
// on the same accumulators after the main loop: for each adapter present in a
// 32-token tile, A = B13/B2 rows of (adapter, expert), B = the shrink result
// of the tile's tokens that carry that adapter (others zero).  Tokens of an
// expert block are grouped by adapter by the alignment, so a tile usually
// sees one or two adapters.
//
// Workgroups are numbered so that each XCD (8 per MI355X, dispatched round
// robin) receives one contiguous range of (weight tile, expert block) pairs,
// expert blocks fastest: the blocks of one expert that share a weight tile run
// on the same XCD and reuse that tile from its L2.
#pragma once

#include "common.hpp"
#include "gemm_stream.hpp"

namespace moelora {

constexpr int kTileBK = 64;
constexpr int kLdsRowBytes = kTileBK * 2 + 16;  // 144: padded row of one 64-wide K slab

// Map workgroup i (dispatched to XCD i % 8) to a logical index such that each
// XCD owns one contiguous range of logical indices.  Bijective on [0, total).
__device__ __forceinline__ int xcd_logical(int i, int total) {
    const int q = total / 8, rem = total % 8;
    const int x = i % 8, k = i / 8;
    return (x < rem) ? x * (q + 1) + k : rem * (q + 1) + (x - rem) * q + k;
}

// global row of tile row rr for gate_up (interleaved gate/up pairs) or down
template <bool GU>
__device__ __forceinline__ int tile_weight_row(int rr, int i0, int N, bool &ok) {
    if (GU) {
        const int a = rr >> 2, q = rr & 3;
        const int feat = i0 + 2 * a + (q & 1);
        ok = feat < N;
        return (q < 2) ? feat : N + feat;
    }
    const int feat = i0 + rr;
    ok = feat < N;
    return feat;
}

template <int BW, int BT, bool GU>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(GemmParams p, int n_wtiles, int max_blocks) {
    constexpr int MT = BW / 64, NT = BT / 64;          // 32x32 tiles per wave
    constexpr int ROWS = BW + BT;                       // LDS rows per stage
    constexpr int CHUNKS = ROWS * (kTileBK / 8);        // 16-byte chunks per stage
    constexpr int CPT = CHUNKS / 256;                   // chunks per thread
    static_assert(CHUNKS % 256 == 0, "tile rows must fill the workgroup");
    constexpr int STAGE_BYTES = ROWS * kLdsRowBytes;
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * STAGE_BYTES];

    const int logical = xcd_logical((int)blockIdx.x, (int)gridDim.x);
    const int wt = logical / max_blocks, b = logical % max_blocks;
    const int npp = p.counters[0];
    if (wt >= n_wtiles || b * BT >= npp) return;
    const int e = p.block_expert[b];
    const int tid = (int)threadIdx.x, lane = lane_id(), w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int l32 = lane & 31, lh = lane >> 5;
    const int N = p.Nout;
    const int64_t Kd = p.Kdim;
    const int i0 = wt * (GU ? BW / 2 : BW);
    const int rows_per_expert = GU ? 2 * N : N;

    // ---- per-thread global source rows for the stage loads -------------
    const uint16_t *src[CPT];
    bool sok[CPT];
    int soff[CPT];  // byte offset inside a stage
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + 256 * j;
        const int rr = c >> 3, piece = c & 7;
        soff[j] = rr * kLdsRowBytes + piece * 16;
        if (rr < BW) {
            bool ok;
            const int grow = tile_weight_row<GU>(rr, i0, N, ok);
            sok[j] = ok;
            src[j] = p.W + ((int64_t)e * rows_per_expert + (ok ? grow : 0)) * Kd + piece * 8;
        } else {
            const int prow = b * BT + (rr - BW);
            const int f = p.sorted_ids[prow];
            sok[j] = f < p.P;
            int64_t row = 0;
            if (sok[j]) row = GU ? (f / p.Kp) : prow;
            src[j] = p.in + row * Kd + piece * 8;
        }
    }

    u32x4 stg[CPT];
    auto gload = [&](int kt) {
        const int64_t k0 = (int64_t)kt * kTileBK;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int piece = (tid + 256 * j) & 7;
            stg[j] = ld16(src[j] + k0, sok[j] && (k0 + piece * 8 < Kd));
        }
    };
    auto swrite = [&](int buf) {
        unsigned char *base = lds + buf * STAGE_BYTES;
#pragma unroll
        for (int j = 0; j < CPT; ++j) *reinterpret_cast<u32x4 *>(base + soff[j]) = stg[j];
    };

    f32x16 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[mt][nt][q] = 0.f;

    const int a_row0 = wm * (BW / 2) + l32;        // + mt*32
    const int b_row0 = BW + wn * (BT / 2) + l32;   // + nt*32
    auto compute = [&](int buf) {
        const unsigned char *base = lds + buf * STAGE_BYTES;
#pragma unroll
        for (int ks = 0; ks < kTileBK / 16; ++ks) {
            const int koff = ks * 32 + lh * 16;
            u32x4 af[MT], bfr[NT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                af[mt] = *reinterpret_cast<const u32x4 *>(base + (a_row0 + mt * 32) * kLdsRowBytes + koff);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                bfr[nt] = *reinterpret_cast<const u32x4 *>(base + (b_row0 + nt * 32) * kLdsRowBytes + koff);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[mt]), as_bf16x8(bfr[nt]),
                                                                          acc[mt][nt], 0, 0, 0);
        }
    };

    const int nk = (int)((Kd + kTileBK - 1) / kTileBK);
    gload(0);
    swrite(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more) gload(kt + 1);
        compute(kt & 1);
        if (more) swrite((kt + 1) & 1);
        __syncthreads();
    }

    // ---- LoRA expand: extra MFMA k-steps per adapter present --------------
    int prow_t[NT], f_t[NT], a_t[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        prow_t[nt] = b * BT + wn * (BT / 2) + nt * 32 + l32;
        f_t[nt] = p.sorted_ids[prow_t[nt]];
        int a = -1;
        if (p.lora && f_t[nt] < p.P) {
            a = p.adapter_ids[f_t[nt] / p.Kp];
            if (a >= p.L) a = -1;
        }
        a_t[nt] = a;
    }
    if (p.lora) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            uint64_t remaining = __ballot(a_t[nt] >= 0);
            while (remaining) {
                const int src_lane = __ffsll((unsigned long long)remaining) - 1;
                const int a = __shfl(a_t[nt], src_lane, 64);
                const bool mine = a_t[nt] == a;
                remaining &= ~__ballot(mine);
                const uint16_t *Bae = p.B + ((int64_t)a * p.Ep + e) * (int64_t)rows_per_expert * p.r;
                for (int k0 = 0; k0 < p.r; k0 += 16) {
                    const int kk = k0 + lh * 8;
                    const bool kin = kk < p.r;
                    float s[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) s[i] = 0.f;
                    if (mine && kin) {
                        for (int sp = 0; sp < p.split; ++sp) {
                            const float4 *sv = reinterpret_cast<const float4 *>(
                                p.s_part + ((int64_t)sp * p.cap + prow_t[nt]) * p.r + kk);
                            const float4 lo = sv[0], hi = sv[1];
                            s[0] += lo.x; s[1] += lo.y; s[2] += lo.z; s[3] += lo.w;
                            s[4] += hi.x; s[5] += hi.y; s[6] += hi.z; s[7] += hi.w;
                        }
                    }
                    u32x4 sb;
                    sb[0] = pack_bf16x2(s[0], s[1]);
                    sb[1] = pack_bf16x2(s[2], s[3]);
                    sb[2] = pack_bf16x2(s[4], s[5]);
                    sb[3] = pack_bf16x2(s[6], s[7]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        bool ok;
                        const int grow = tile_weight_row<GU>(wm * (BW / 2) + mt * 32 + l32, i0, N, ok);
                        const u32x4 bw = ld16(Bae + (int64_t)(ok ? grow : 0) * p.r + kk, ok && kin);
                        acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(bw), as_bf16x8(sb),
                                                                              acc[mt][nt], 0, 0, 0);
                    }
                }
            }
        }
    }

    // ---- epilogue --------------------------------------------------------
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int prow = prow_t[nt], f = f_t[nt];
            const bool valid = f < p.P;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int rr = wm * (BW / 2) + mt * 32 + g4 * 8 + lh * 4;  // first of 4 consecutive rows
                if (GU) {
                    const int feat = i0 + 2 * (rr >> 2);
                    if (feat >= N) continue;
                    uint32_t v = 0u;
                    if (valid) {
                        const float g0 = acc[mt][nt][4 * g4 + 0], g1 = acc[mt][nt][4 * g4 + 1];
                        const float u0 = acc[mt][nt][4 * g4 + 2], u1 = acc[mt][nt][4 * g4 + 3];
                        v = pack_bf16x2(silu(g0) * u0, silu(g1) * u1);
                    }
                    *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(p.out) + (int64_t)prow * N + feat) = v;
                } else {
                    const int feat = i0 + rr;
                    if (feat >= N || !valid) continue;
                    const float4 v = make_float4(acc[mt][nt][4 * g4 + 0], acc[mt][nt][4 * g4 + 1],
                                                 acc[mt][nt][4 * g4 + 2], acc[mt][nt][4 * g4 + 3]);
                    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.out) + (int64_t)f * N + feat) = v;
                }
            }
        }
    }
}

}  // namespace moelora
