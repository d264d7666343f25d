// Grouped expert GEMM for many rows per expert (prefill): LDS-tiled, matrix
// cores (v_mfma_f32_32x32x16_bf16), LoRA expand and SwiGLU in the epilogue.
//
// Same contract as the streaming kernel (gemm_stream.hpp): weights are the
// MFMA M side, the expert's tokens the N side, y13 -> SwiGLU -> h (bf16,
// sorted row) for gate_up and y2 (fp32, pair row) for down.
//
// Work unit: one (weight tile of BW rows, token tile) pair.  Token tiles come
// from a list built by the alignment: up to BT consecutive sorted rows of ONE
// expert, a multiple of 32 rows (experts are padded to 32 only), so a large
// expert is cut into full BT-row tiles plus one shorter tail tile.  MFMA
// column tiles (32 tokens) past the tile's rows are skipped outright, which
// keeps the padding cost at 32-row granularity while the tile stays large.
//
// Workgroup: 4 wavefronts in a 2 x 2 grid, each owning (BW/2) x (BT/2) as
// (BW/64) x (BT/64) MFMA tiles of 32 x 32; with BW = BT = 256 every wave does
// 16 MFMAs per 16-wide k-step on 8 fragment reads, which keeps LDS traffic
// (reads + stage fills) under the ~128 B/clk/CU that gfx950 sustains.
//
// K advances 32 at a time through a ring of kStages LDS stages of (BW+BT)
// rows x 64 bytes, filled by gfx950's direct global->LDS loads
// (global_load_lds_dwordx4: lane l's 16 bytes land at M0 + 16*l), so no
// registers stage the data and kStages-1 slabs are in flight while the MFMAs
// work on the oldest one.  Each wave waits only for its own loads of the slab
// it needs next (s_waitcnt vmcnt with the number of younger slabs still
// allowed in flight) and then meets the others at one barrier per slab; the
// wait and the barrier are one asm statement with a memory clobber, which
// keeps the compiler from moving LDS accesses across the barrier without the
// vmcnt(0) a fenced barrier would force.  The four 16-byte chunks of a row
// are XOR-swizzled (swz_slot) so that the fragment reads of 8 or 16
// consecutive lanes (consecutive rows, same chunk) hit distinct 16-byte slots.
// K beyond the reduction length reads a 16-byte zero chunk.
//
// gate_up row order inside a tile: rows 4a, 4a+1 hold gate features
// i0+2a, i0+2a+1 and rows 4a+2, 4a+3 the matching up features.  The 32 x 32
// accumulator gives each lane 4 consecutive rows, so every lane holds whole
// (gate, up) pairs and SwiGLU needs no data exchange.
//
// LoRA expand (aitrends.kr summary of the AWS multi-LoRA MoE post, "section
// details": LoRA sum folded into the expand step) runs as extra MFMA k-steps
// on the same accumulators after the main loop: for each adapter present in a
// 32-token column tile, A = B13/B2 rows of (adapter, expert), B = the shrink
// result of that tile's tokens carrying the adapter (others zero).  The
// alignment groups an expert's tokens by adapter, so a column tile usually
// sees one or two adapters.
//
// Workgroups are numbered so that each XCD (8 per MI355X, dispatched round
// robin) receives one contiguous range of work in expert-major order (expert,
// then weight tile, then the expert's token tiles): an XCD works through whole
// experts, so an expert's gathered token rows stay in that XCD's L2 while all
// of its weight tiles stream past, and the token tiles sharing a weight tile
// run side by side.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "gemm_stream.hpp"

namespace moelora {

constexpr int kTileBK = 32;   // K per LDS stage
#ifndef MOELORA_TILED_STAGES
#define MOELORA_TILED_STAGES 4
#endif
constexpr int kStages = MOELORA_TILED_STAGES;  // LDS ring depth

// 16 bytes of zeros: the source of every load past the end of K
__device__ __attribute__((aligned(16))) const uint16_t g_zero_chunk[8] = {0, 0, 0, 0, 0, 0, 0, 0};

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

// byte offset of 16-byte chunk `c` (0..3) of LDS row `row` inside a stage.
// The XOR term makes 8 consecutive rows (same c) fall in 8 different 16-byte
// slots of a 128-byte window AND 16 consecutive rows in 16 different slots of
// a 256-byte window, so fragment reads are conflict-free whether the LDS
// serves 8 or 16 lanes of a 16-byte read per cycle.
__device__ __forceinline__ int swz_slot(int row, int c) { return c ^ (((row >> 1) ^ (row >> 3)) & 3); }
__device__ __forceinline__ int swz(int row, int c) { return row * 64 + (swz_slot(row, c) << 4); }

// Wait until at most N direct-to-LDS loads of this wave are still in flight,
// then barrier; the memory clobber pins every LDS access to its side.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int BW, int BT, bool GU>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(GemmParams p, const int32_t *__restrict__ tiles,
                                                         const int32_t *__restrict__ n_tiles, int n_wtiles) {
    constexpr int MT = BW / 64, NT = BT / 64;          // 32x32 tiles per wave
    constexpr int ROWS = BW + BT;                       // LDS rows per stage
    constexpr int STAGE_BYTES = ROWS * 64;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kStages * STAGE_BYTES];

    // Logical order: expert-major, then weight tile, then the expert's token
    // tiles.  Expert e owns logical [n_wtiles*t0, n_wtiles*(t0+nt)) where t0 is
    // its first token tile and nt its tile count (both stored in every tile).
    // Only the first n_wtiles * n_tiles workgroups have work; the XCD remap
    // runs over exactly that many so every XCD gets an equal share.
    const int live = n_wtiles * n_tiles[0];
    if ((int)blockIdx.x >= live) return;
    const int logical = xcd_logical((int)blockIdx.x, live);
    const int tq = logical / n_wtiles;
    const int4 tq_tile = reinterpret_cast<const int4 *>(tiles)[tq];
    const int t0 = tq_tile.w, ntl = tq_tile.y >> 16;
    const int rel = logical - n_wtiles * t0;
    const int wt = rel / ntl, ti = t0 + rel % ntl;
    const int4 tile = reinterpret_cast<const int4 *>(tiles)[ti];
    const int row0 = tile.x, nrows = tile.y & 0xffff, e = tile.z;
    const int tid = (int)threadIdx.x, lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so tile branches stay scalar
    const int wm = w >> 1, wn = w & 1;
    const int l32 = lane & 31, lh = lane >> 5;
    const int N = p.Nout;
    const int64_t Kd = p.Kdim;
    const int i0 = wt * (GU ? BW / 2 : BW);
    const int rows_per_expert = GU ? 2 * N : N;
    // MFMA column tiles of this wave that hold at least one sorted row
    const int nt_live = max(0, min(NT, (nrows - wn * (BT / 2) + 31) / 32));

    // ---- direct-to-LDS stage loads ----------------------------------------
    // One wave instruction fills 16 rows x 64 bytes (1 KiB) of a stage; wave w
    // owns instructions w, w+4, ...  Lane l writes row R0 + l/4, slot l&3,
    // which holds logical chunk swz_slot(row, l&3).
    constexpr int GROUPS = ROWS / 16;               // 16-row groups per stage
    static_assert(GROUPS % 4 == 0, "row groups must split evenly over 4 waves");
    constexpr int LPW = GROUPS / 4;                 // load instructions per wave per stage
    const uint16_t *src[LPW];
    int chunk_of[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int rr = (w + 4 * j) * 16 + (lane >> 2);
        const int c = swz_slot(rr, lane & 3);  // slot -> chunk (the XOR is its own inverse)
        chunk_of[j] = c;
        const uint16_t *row;
        if (rr < BW) {
            bool ok;
            const int grow = tile_weight_row<GU>(rr, i0, N, ok);
            row = p.W + ((int64_t)e * rows_per_expert + (ok ? grow : 0)) * Kd;
        } else {
            const int j_tok = rr - BW;
            const int prow = row0 + min(j_tok, nrows - 1);
            const int f = p.sorted_ids[prow];
            int64_t xr = 0;
            if (j_tok < nrows && f < p.P) xr = GU ? (f / p.Kp) : prow;
            row = p.in + xr * Kd;
        }
        src[j] = row + c * 8;
    }
    typedef __attribute__((address_space(3))) unsigned char lds_t;
    lds_t *lds_base = (lds_t *)lds;
    auto issue = [&](int kt) {
        const int64_t k0 = (int64_t)kt * kTileBK;
        lds_t *stage = lds_base + (kt % kStages) * STAGE_BYTES;
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const bool kin = k0 + chunk_of[j] * 8 < Kd;
            const void *g = kin ? (const void *)(src[j] + k0) : (const void *)g_zero_chunk;
            __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)(stage + (w + 4 * j) * 1024),
                                             16, 0, 0);
        }
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
    // Fragment reads of one 16-wide k-step (NTL live column tiles) and its MFMAs.
    auto rd = [&](auto ntl, u32x4 *af, u32x4 *bfr, int stage, int ks) {
        constexpr int NTL = decltype(ntl)::value;
        const unsigned char *base = lds + stage * STAGE_BYTES;
        const int c = ks * 2 + lh;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            af[mt] = *reinterpret_cast<const u32x4 *>(base + swz(a_row0 + mt * 32, c));
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt)
            bfr[nt] = *reinterpret_cast<const u32x4 *>(base + swz(b_row0 + nt * 32, c));
    };
    auto mm = [&](auto ntl, const u32x4 *af, const u32x4 *bfr) {
        constexpr int NTL = decltype(ntl)::value;
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[mt]), as_bf16x8(bfr[nt]),
                                                                      acc[mt][nt], 0, 0, 0);
    };
    const int nk = (int)((Kd + kTileBK - 1) / kTileBK);
    // The whole K loop, specialised on the live column tiles so it has no
    // branches.  Two fragment register sets alternate: while the MFMAs of one
    // k-step run, the reads of the next are in flight.  The barrier that makes
    // slab kt+1 visible sits between the two k-steps of slab kt, so the first
    // reads of slab kt+1 overlap the second half of slab kt's MFMAs.  The slab
    // refilled right after that barrier, (kt + kStages - 1) mod kStages ==
    // (kt - 1) mod kStages, was last read before the previous barrier, so
    // every wave is done with it.
    // Wait for this wave's loads of the slab needed next, given `younger`
    // younger slabs that may stay in flight, then barrier.
    auto wait_slab = [&](int younger) {
        static_assert(kStages <= 6, "extend the wait ladder");
        if (younger >= 4) wait_vm_barrier<4 * LPW>();
        else if (younger == 3) wait_vm_barrier<3 * LPW>();
        else if (younger == 2) wait_vm_barrier<2 * LPW>();
        else if (younger == 1) wait_vm_barrier<LPW>();
        else wait_vm_barrier<0>();
    };
    auto mainloop = [&](auto ntl) {
        u32x4 a0[MT], b0[NT], a1[MT], b1[NT];
#pragma unroll
        for (int s = 0; s < kStages - 1; ++s)
            if (s < nk) issue(s);
        wait_slab(min(kStages - 2, nk - 1));
        rd(ntl, a0, b0, 0, 0);
        for (int kt = 0; kt < nk; ++kt) {
            rd(ntl, a1, b1, kt % kStages, 1);
            mm(ntl, a0, b0);
            if (kt + 1 < nk) {
                // issued so far: slabs 0 .. min(kt + kStages - 2, nk - 1)
                wait_slab(min(kStages - 3, nk - 2 - kt));
                if (kt + kStages - 1 < nk) issue(kt + kStages - 1);
                rd(ntl, a0, b0, (kt + 1) % kStages, 0);
            }
            mm(ntl, a1, b1);
        }
    };
    switch (nt_live) {
        case 0: mainloop(std::integral_constant<int, 0>{}); break;
        case 1: mainloop(std::integral_constant<int, (NT >= 1 ? 1 : NT)>{}); break;
        case 2: mainloop(std::integral_constant<int, (NT >= 2 ? 2 : NT)>{}); break;
        case 3: mainloop(std::integral_constant<int, (NT >= 3 ? 3 : NT)>{}); break;
        default: mainloop(std::integral_constant<int, NT>{}); break;
    }

    // ---- LoRA expand: extra MFMA k-steps per adapter present --------------
    int prow_t[NT], f_t[NT], a_t[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int j_tok = wn * (BT / 2) + nt * 32 + l32;
        prow_t[nt] = row0 + min(j_tok, nrows - 1);
        const int f = p.sorted_ids[prow_t[nt]];
        f_t[nt] = (j_tok < nrows) ? f : p.P;
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
            if (nt >= nt_live) break;
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
    for (int nt = 0; nt < NT; ++nt) {
        if (nt >= nt_live) break;
        const int j_tok = wn * (BT / 2) + nt * 32 + l32;
        if (j_tok >= nrows) continue;
        const int prow = prow_t[nt], f = f_t[nt];
        const bool valid = f < p.P;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
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
