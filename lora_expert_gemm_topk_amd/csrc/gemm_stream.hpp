// Grouped expert GEMM for few rows per expert (decode), streaming the expert
// weights once from HBM.
//
//   gate_up:  y13[p, n] = sum_h x[t(p), h] * W13[e, n, h]      n in the tile's
//             gate columns [i0, i0+BW/2) and the matching up columns
//             I + [i0, i0+BW/2); epilogue: + LoRA expand (s13 . B13[a,e]),
//             h = silu(gate) * up, stored bf16 at the sorted row p.
//   down:     y2[f, n]  = sum_i h[p, i] * W2[e, n, i]; epilogue: + LoRA
//             expand (s2 . B2[a,e]), stored bf16 at the pair row f.
// (aitrends.kr summary of the AWS multi-LoRA MoE post: LoRA shrink/expand
// fused into each expert projection, "section details"; an adapter path on
// gate_up and on down, "image analysis" diagram; the LoRA sum folded into
// the expand step.)
//
// One workgroup = one expert block of BT sorted rows x one tile of BW weight
// rows.  The weight tile is the MFMA M side (v_mfma_f32_16x16x32_bf16), the
// BT tokens the N side, so a lane's accumulator holds 4 consecutive output
// features of one token and gate/up pairs sit at the same register position.
// The 4 wavefronts split the reduction into 64-wide chunks (chunk c goes to
// wave c mod 4) and load their MFMA fragments straight from global memory,
// double-buffered in registers, so each weight byte is read exactly once per
// expert block and many loads are in flight per CU.  Partial tiles are summed
// across waves in LDS in a fixed order, which keeps the result deterministic.
// Blocks past the padded row count exit at once.
#pragma once

#include "align.hpp"
#include "common.hpp"
#include "pack.hpp"

namespace moelora {

// MXFP8 weights: most 32-element blocks per weight row (K <= 8192)
constexpr int kMxMaxBlocks = 256;

struct GemmParams {
    const uint16_t *in;          // gate_up: x [T, Kdim]; down: h [cap, Kdim] (LDS-tiled kernel: h packed)
    const int32_t *sorted_ids;   // [cap]
    const int32_t *sorted_adapter; // [cap] adapter per sorted row (LDS-tiled kernel only)
    const int32_t *block_expert; // [max_blocks]
    const int32_t *counters;     // [0] = padded row count
    const int32_t *adapter_ids;  // [T]
    const uint16_t *W;           // gate_up: w13 [Ep, 2*Nout, Kdim]; down: w2 [Ep, Nout, Kdim]
    const uint16_t *B;           // gate_up: b13 [L, Ep, 2*Nout, r]; down: b2 [L, Ep, Nout, r]
    const float *s_part;         // [split][cap][r] fp32; LDS-tiled kernel: bf16 [cap][r]
    void *out;                   // gate_up: h bf16 [cap, Nout] (LDS-tiled kernel: packed); down: y2 bf16 [P, Nout]
    int Kdim, Nout, Kp, P, cap, Ep, L, r, split, lora;
    int s_by_pair = 0;           // streaming kernel: s_part is [P][r] by pair index (split 1)
    const uint8_t *Wscale = nullptr;  // MXFP8 weights: E8M0 scale of each 32-element block, [rows][Kdim/32]
};

// LoRA expand in the epilogue: ranks per staged chunk and bf16 elements of
// B rows staged at once (16 KiB)
constexpr int kLoraRC = 32;
constexpr int kLoraStage = 8192;

// WP: weights in the packed layout of moe_lora_pack_weights.  A weight
// fragment is then one 16-row group (for gate_up the gate and up rows of 8
// features, in quads gate f, gate f+1, up f, up f+1), read 1 KiB-contiguous.
//
// MX: MXFP8 weights (row-major like the bf16 ones): one byte per element, an
// FP8 E4M3 code, and one E8M0 scale byte per 32-element block along K; the
// element is code * 2^(scale - 127).  The reduction then runs in 128-wide
// chunks: lane (row, g) loads the 32 codes of block 4c + g (whole 128-byte
// row segments per 4 lanes), takes the block's scale from a copy of the
// tile's scale rows staged in LDS once per workgroup, converts the codes with
// the hardware's scaled FP8 -> bf16 conversion (exact: E4M3 has 3 mantissa
// bits) and feeds the same bf16 MFMAs; the matching 32 activations are that
// lane's 64 bytes of x.  Weight bytes per layer call halve.
//
// ROUTE (gate_up of tiny calls without LoRA): the workgroup routes the
// tokens and aligns the pairs itself (route_align_in_block) instead of
// reading a layout written by earlier launches; workgroup (0, 0) stores the
// routing and the layout for the down GEMM and the combine.
template <int BW, int BT, bool GU, bool WP, bool MX, bool ROUTE>
__device__ __forceinline__ void gemm_stream_body(const GemmParams &p, const FusedRoute *fr) {
    constexpr int MS = BW / 16, NS = BT / 16;
    constexpr int LDW = BW + 4;
    __shared__ float buf[2][BT][LDW];
    // MXFP8: the scale bytes of the tile's BW weight rows, staged once
    __shared__ __attribute__((aligned(16))) uint8_t mx_sc[MX ? BW * kMxMaxBlocks : 16];
    // ROUTE: the slots' experts, the block's pairs, padded row count and expert
    __shared__ int r_e[ROUTE ? 64 : 1], r_rows[ROUTE ? BT : 1], r_blk[2];
    // LoRA expand staging: B rows of a batch of adapters [q][tile column][kc],
    // the rows' s values, and per row its adapter, adapter slot and s row
    constexpr bool LORA = !ROUTE;
    __shared__ __attribute__((aligned(16))) uint16_t l_b[LORA ? kLoraStage : 8];
    __shared__ __attribute__((aligned(16))) float l_s[LORA ? BT : 1][kLoraRC];
    __shared__ int l_a[BT], l_q[BT], l_srow[BT], l_list[BT + 1];

    const int b = blockIdx.y;
    int npp, e;
    if constexpr (ROUTE) {
        // While the routing's loads are in flight, wave 3 (which routes only
        // at T = 4) reads one dword of every expert's gate_up weights at this
        // workgroup's share of them and one of its down weights: the address
        // translations (and those lines) of the weights this call will stream
        // are then warm when the expert is known, instead of missing after
        // the routing.  The values are folded into nothing but a register.
        constexpr int kTouch = 5;  // experts in chunks of 64 (Ep <= 256 + 64)
        uint32_t touch[kTouch][2];
        const int Ep = fr->ap.Ep;
        const bool toucher = (threadIdx.x >> 6) == 3;
        if (toucher) {
            const int64_t o13 = (fr->stride13 / gridDim.x * blockIdx.x) & ~(int64_t)63;
            const int64_t o2 = (fr->stride2 / ((int64_t)gridDim.x * gridDim.y) * (blockIdx.y * gridDim.x + blockIdx.x)) &
                               ~(int64_t)63;
#pragma unroll
            for (int j = 0; j < kTouch; ++j) {
                const int ee = 64 * j + lane_id();
                touch[j][0] = touch[j][1] = 0u;
                if (ee < Ep) {
                    touch[j][0] = *reinterpret_cast<const uint32_t *>(fr->touch13 + ee * fr->stride13 + o13);
                    touch[j][1] = *reinterpret_cast<const uint32_t *>(fr->touch2 + ee * fr->stride2 + o2);
                }
            }
        }
        route_align_in_block<BT, 4>(*fr, b, blockIdx.x == 0 && b == 0, r_e, r_rows, r_blk);
        npp = r_blk[0];
        e = r_blk[1];
        if (toucher) {
            uint32_t s = 0;
#pragma unroll
            for (int j = 0; j < kTouch; ++j) s ^= touch[j][0] ^ touch[j][1];
            asm volatile("" ::"v"(s));
        }
    } else {
        npp = p.counters[0];
        e = 0;
    }
    if (b * BT >= npp) return;
    if constexpr (!ROUTE) e = p.block_expert[b];
    // the pair at sorted row prow of this block (P: padding)
    auto sorted_at = [&](int prow) -> int {
        if constexpr (ROUTE) return r_rows[prow - b * BT];
        else return p.sorted_ids[prow];
    };
    const int lane = lane_id(), w = (int)(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    const int64_t Kd = p.Kdim;
    const int N = p.Nout;
    const int i0 = blockIdx.x * (GU ? BW / 2 : BW);
    const int rows_per_expert = GU ? 2 * N : N;

    const uint16_t *wrow[MS];
    bool wok[MS];
    const int64_t nslab_w = (Kd + kSlabK - 1) / kSlabK;
    if constexpr (WP && !MX) {
        // the packed group count covers every tile of the grid
        const int64_t G = GU ? packed_w13_groups(N) : packed_w2_groups(N);
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
            wok[ms] = true;
            wrow[ms] = p.W + ((int64_t)e * G + (int64_t)blockIdx.x * MS + ms) * nslab_w * kBlockElems + l16 * 8;
        }
    } else {
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
        int col, grow;
        if (GU) {
            const int half = ms / (MS / 2);
            col = i0 + (ms % (MS / 2)) * 16 + l16;
            grow = half ? N + col : col;
        } else {
            col = i0 + ms * 16 + l16;
            grow = col;
        }
        wok[ms] = col < N;
        wrow[ms] = p.W + ((int64_t)e * rows_per_expert + (wok[ms] ? grow : 0)) * Kd;
    }
    }
    // MXFP8: the same rows as byte rows; with packed codes (WP) the lane's
    // place in its fragment's 2 KiB chunk blocks
    const uint8_t *wrow8[MS];
    if constexpr (MX) {
        const int64_t nchp = packed_mx_chunks(Kd);
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
            const int64_t row = (wrow[ms] - p.W) / Kd;  // e * rows_per_expert + row within the expert
            if constexpr (WP)
                wrow8[ms] = reinterpret_cast<const uint8_t *>(p.W) + ((row >> 4) * nchp * 2048 + lane * 16);
            else
                wrow8[ms] = reinterpret_cast<const uint8_t *>(p.W) + row * Kd;
        }
    }
    const uint16_t *xrow[NS];
    bool xok[NS];
    // LoRA: pair and adapter of rows ns*16 + l16, fetched now for the
    // epilogue (the loads retire long before the main loop's)
    int row_f[NS], row_a[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
        const int prow = b * BT + ns * 16 + l16;
        const int f = sorted_at(prow);
        xok[ns] = f < p.P;
        int64_t row = 0;
        if (xok[ns]) row = GU ? (f / p.Kp) : prow;
        xrow[ns] = p.in + row * Kd;
        row_f[ns] = f;
        row_a[ns] = (p.lora && xok[ns]) ? p.adapter_ids[f / p.Kp] : -1;
    }

    f32x4 acc[MS][NS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) acc[ms][ns] = f32x4{0.f, 0.f, 0.f, 0.f};

    constexpr int XQ = MX ? 4 : 2;        // 16-byte x loads per lane and chunk
    constexpr int KC = MX ? 128 : 64;     // reduction per chunk
    const int nch = (int)((Kd + KC - 1) / KC);
    u32x4 wa[2][MS][2], xa[2][NS][XQ];
    auto load_mx = [&](int buf_i, int c) {
        const int64_t k0 = (int64_t)c * 128 + g * 32;  // block 4c + g (K is a multiple of 32)
        const bool kin = k0 < Kd;
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
            const bool ok = wok[ms] && kin;
            if constexpr (WP) {
                wa[buf_i][ms][0] = ld16(wrow8[ms] + (int64_t)c * 2048, ok);
                wa[buf_i][ms][1] = ld16(wrow8[ms] + (int64_t)c * 2048 + 1024, ok);
            } else {
                wa[buf_i][ms][0] = ld16(wrow8[ms] + k0, ok);
                wa[buf_i][ms][1] = ld16(wrow8[ms] + k0 + 16, ok);
            }
        }
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
#pragma unroll
            for (int q = 0; q < XQ; ++q) xa[buf_i][ns][q] = ld16(xrow[ns] + k0 + 8 * q, xok[ns] && kin);
    };
    auto compute_mx = [&](int buf_i, int c) {
        const int64_t k0 = (int64_t)c * 128 + g * 32;
        const bool kin = k0 < Kd;
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
            // the block's scale from the staged copy (past K: any scale, the codes there are zero)
            const uint32_t sb = kin ? (uint32_t)mx_sc[(ms * 16 + l16) * (int)(Kd / 32) + (int)(k0 >> 5)] : 127u;
            const float sc = __uint_as_float(sb << 23);  // 2^(scale - 127)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                // codes 8s .. 8s+7 of the lane's 32: dwords 2s and 2s+1
                const uint32_t d0 = wa[buf_i][ms][s >> 1][2 * (s & 1)], d1 = wa[buf_i][ms][s >> 1][2 * (s & 1) + 1];
                u32x4 wb;
                wb[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, sc, false));
                wb[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, sc, true));
                wb[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, sc, false));
                wb[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, sc, true));
#pragma unroll
                for (int ns = 0; ns < NS; ++ns)
                    acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wb), as_bf16x8(xa[buf_i][ns][s]),
                                                                          acc[ms][ns], 0, 0, 0);
            }
        }
    };
    auto load = [&](int buf_i, int c) {
        if constexpr (MX) {
            load_mx(buf_i, c);
            return;
        }
        const int64_t k0 = (int64_t)c * 64 + g * 16;
        const bool k_lo = k0 < Kd, k_hi = k0 + 8 < Kd;
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
            if constexpr (WP) {
                // k0 = 64c + 16g (+8) sits in slab 2c + g/2, chunk 2(g%2) (+1)
                const int64_t slab = (int64_t)c * 2 + (g >> 1);
                const uint16_t *blk = wrow[ms] + slab * kBlockElems + (g & 1) * 256;
                wa[buf_i][ms][0] = ld16(blk, slab < nslab_w);
                wa[buf_i][ms][1] = ld16(blk + 128, slab < nslab_w);
            } else {
                wa[buf_i][ms][0] = ld16(wrow[ms] + k0, wok[ms] && k_lo);
                wa[buf_i][ms][1] = ld16(wrow[ms] + k0 + 8, wok[ms] && k_hi);
            }
        }
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
            xa[buf_i][ns][0] = ld16(xrow[ns] + k0, xok[ns] && k_lo);
            xa[buf_i][ns][1] = ld16(xrow[ns] + k0 + 8, xok[ns] && k_hi);
        }
    };
    auto compute = [&](int buf_i, int c) {
        if constexpr (MX) {
            compute_mx(buf_i, c);
            return;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int ns = 0; ns < NS; ++ns)
                    acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        as_bf16x8(wa[buf_i][ms][s]), as_bf16x8(xa[buf_i][ns][s]), acc[ms][ns], 0, 0, 0);
    };
    int c = w;
    if (c < nch) load(0, c);
    if constexpr (MX) {
        // Stage the scale rows while the first chunk is in flight.  A
        // fragment's 16 weight rows are consecutive rows of w13/w2 (rows start
        // at multiples of 16 and K is a multiple of 32), so their scales are
        // 16 * nblk contiguous bytes starting on a 16-byte boundary: copied
        // in 16-byte pieces to mx_sc[ms][row][block].
        const int nblk = (int)(Kd / 32);
        for (int i = (int)threadIdx.x; i < MS * nblk; i += 256) {
            const int ms = i / nblk, q = i - ms * nblk;
            int col0, grow0;
            if (GU) {
                col0 = i0 + (ms % (MS / 2)) * 16;
                grow0 = ms / (MS / 2) ? N + col0 : col0;
            } else {
                col0 = i0 + ms * 16;
                grow0 = col0;
            }
            if (col0 < N) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(
                    p.Wscale + ((int64_t)e * rows_per_expert + grow0) * nblk + (int64_t)q * 16);
                *reinterpret_cast<u32x4 *>(mx_sc + ms * 16 * nblk + q * 16) = v;
            }
        }
        __syncthreads();
    }
    while (c < nch) {
        if (c + 4 < nch) load(1, c + 4);
        compute(0, c);
        c += 4;
        if (c >= nch) break;
        if (c + 4 < nch) load(0, c + 4);
        compute(1, c);
        c += 4;
    }

    // Cross-wave reduction in fixed order: (w0 + w2) + (w1 + w3).
    auto put = [&](int slot) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int ns = 0; ns < NS; ++ns)
                *reinterpret_cast<f32x4 *>(&buf[slot][ns * 16 + l16][ms * 16 + g * 4]) = acc[ms][ns];
    };
    auto add = [&](int slot) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int ns = 0; ns < NS; ++ns)
                acc[ms][ns] += *reinterpret_cast<const f32x4 *>(&buf[slot][ns * 16 + l16][ms * 16 + g * 4]);
    };
    if (w >= 2) put(w - 2);
    __syncthreads();
    if (w < 2) add(w);
    __syncthreads();
    if (w == 1) put(0);
    __syncthreads();
    if (w == 0) {
        add(0);
        put(1);
    }
    __syncthreads();

    // LoRA expand on the finished tile: buf[1][j][c] += sum_k s[j][k] *
    // B[a_j, e, row(c), k] for the block's rows j with an adapter.  The B
    // rows of the adapters present (in batches that fit kLoraStage) and the
    // rows' s values (split-K partials summed in order) are staged in LDS with
    // all their loads in flight at once, ranks kLoraRC at a time; each column
    // then adds its 8-rank partial dot products in rank order.
    if constexpr (LORA) {
        if (p.lora) {
            // weight row (within the expert) of tile column c, or -1 past N
            auto col_row = [&](int c) -> int {
                if constexpr (GU && WP && !MX) {
                    // packed quads: gate f, gate f+1, up f, up f+1, gate f+2, ...
                    const int m = c & 7, feat = i0 + 4 * (c >> 3) + (m >> 2) * 2 + (m & 1);
                    return feat < N ? (((m >> 1) & 1) ? N + feat : feat) : -1;
                } else if constexpr (GU) {
                    const bool up = c >= BW / 2;
                    const int feat = i0 + (up ? c - BW / 2 : c);
                    return feat < N ? (up ? N + feat : feat) : -1;
                } else {
                    const int feat = i0 + c;
                    return feat < N ? feat : -1;
                }
            };
            if (w == 0 && l16 == lane) {
#pragma unroll
                for (int ns = 0; ns < NS; ++ns) {
                    const int j = ns * 16 + l16, a = row_a[ns];
                    l_a[j] = (a >= 0 && a < p.L) ? a : -1;
                    l_srow[j] = p.s_by_pair ? row_f[ns] : b * BT + j;
                }
            }
            __syncthreads();
            // adapter slots in order of first appearance among the rows
            if (w == 0) {
                const int a = lane < BT ? l_a[lane] : -1;
                int first = lane;
                for (int i = 0; i < BT; ++i)
                    if (i < first && l_a[i] == a) first = i;
                const bool lead = a >= 0 && first == lane;
                const uint64_t m = __ballot(lead);
                if (lane < BT) l_q[lane] = a >= 0 ? __popcll(m & ((1ull << first) - 1)) : -1;
                if (lead) l_list[__popcll(m & ((1ull << lane) - 1))] = a;
                if (lane == 0) l_list[BT] = __popcll(m);
            }
            __syncthreads();
            const int nad = l_list[BT];
            const int tid = (int)threadIdx.x;
            for (int k0 = 0; k0 < p.r; k0 += kLoraRC) {
                const int kc = min(kLoraRC, p.r - k0), kp8 = kc / 8;
                const int nab = kLoraStage / (BW * kc);  // adapters per batch
                for (int q0 = 0; q0 < nad; q0 += nab) {
                    const int nb = min(nab, nad - q0);
                    // B pieces (16 bytes = 8 ranks): (slot, column, piece)
                    const int npc = nb * BW * kp8;
                    u32x4 bv[kLoraStage / (8 * 256)];
#pragma unroll
                    for (int i = 0; i < kLoraStage / (8 * 256); ++i) {
                        const int u = tid + 256 * i;
                        bv[i] = u32x4{0u, 0u, 0u, 0u};
                        if (u < npc) {
                            const int qq = u / (BW * kp8), rem = u - qq * (BW * kp8);
                            const int c = rem / kp8, kq = rem - c * kp8;
                            const int grow = col_row(c);
                            const int a = l_list[q0 + qq];
                            const uint16_t *Bae = p.B + ((int64_t)a * p.Ep + e) * (int64_t)rows_per_expert * p.r;
                            if (grow >= 0) bv[i] = *reinterpret_cast<const u32x4 *>(Bae + (int64_t)grow * p.r + k0 + 8 * kq);
                        }
                    }
                    // s values of the batch's rows, 4 ranks per thread
                    float4 sv = make_float4(0.f, 0.f, 0.f, 0.f);
                    const int k4n = kc / 4;
                    const int sj = tid / k4n, sk = tid - sj * k4n;
                    const bool s_in = sj < BT && l_q[sj] >= q0 && l_q[sj] < q0 + nb;
                    if (s_in) {
                        for (int sp = 0; sp < p.split; ++sp) {
                            const float4 x4 = *reinterpret_cast<const float4 *>(
                                p.s_part + ((int64_t)sp * p.cap + l_srow[sj]) * p.r + k0 + 4 * sk);
                            sv.x += x4.x; sv.y += x4.y; sv.z += x4.z; sv.w += x4.w;
                        }
                    }
#pragma unroll
                    for (int i = 0; i < kLoraStage / (8 * 256); ++i) {
                        const int u = tid + 256 * i;
                        if (u < npc) *reinterpret_cast<u32x4 *>(l_b + (int64_t)u * 8) = bv[i];
                    }
                    if (s_in) *reinterpret_cast<float4 *>(&l_s[sj][4 * sk]) = sv;
                    __syncthreads();
                    // each (row, 4-column group): the 8-rank partial sums in rank order
                    for (int u = tid; u < BT * (BW / 4); u += 256) {
                        const int j = u / (BW / 4), c4 = u - j * (BW / 4);
                        const int q = l_q[j] - q0;
                        if (l_a[j] < 0 || q < 0 || q >= nb) continue;
#pragma unroll
                        for (int cc = 0; cc < 4; ++cc) {
                            const int c = 4 * c4 + cc;
                            if (col_row(c) < 0) continue;
                            float v = buf[1][j][c];
                            for (int g8 = 0; g8 < kp8; ++g8) {
                                const u32x4 bb = *reinterpret_cast<const u32x4 *>(l_b + ((int64_t)(q * BW + c) * kp8 + g8) * 8);
                                const float *s8 = &l_s[j][8 * g8];
                                float acc = 0.f;
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    acc += s8[2 * i] * bf16_to_f32((uint16_t)(bb[i] & 0xffffu));
                                    acc += s8[2 * i + 1] * bf16_to_f32((uint16_t)(bb[i] >> 16));
                                }
                                v += acc;
                            }
                            buf[1][j][c] = v;
                        }
                    }
                    __syncthreads();
                }
            }
        }
    }

    // Epilogue on the finished tile buf[1][token][feature].
    if (GU && WP && !MX) {
        // tile rows 8qp .. 8qp+7 = gate f, gate f+1, up f, up f+1, gate f+2,
        // gate f+3, up f+2, up f+3 with f = i0 + 4qp
        constexpr int QP = BW / 8;
        uint16_t *hout = reinterpret_cast<uint16_t *>(p.out);
        for (int q = (int)threadIdx.x; q < BT * QP; q += 256) {
            const int j = q / QP, qp = q % QP;
            const int prow = b * BT + j;
            const int col0 = i0 + 4 * qp;
            if (col0 >= N) continue;
            const int f = sorted_at(prow);
            uint2 packed = make_uint2(0u, 0u);
            if (f < p.P) {
                float v[8];  // gate col0..col0+3, up col0..col0+3
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    v[2 * h2 + 0] = buf[1][j][8 * qp + 4 * h2 + 0];
                    v[2 * h2 + 1] = buf[1][j][8 * qp + 4 * h2 + 1];
                    v[4 + 2 * h2 + 0] = buf[1][j][8 * qp + 4 * h2 + 2];
                    v[4 + 2 * h2 + 1] = buf[1][j][8 * qp + 4 * h2 + 3];
                }
                float hv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) hv[i] = silu(v[i]) * v[4 + i];
                packed.x = pack_bf16x2(hv[0], hv[1]);
                packed.y = pack_bf16x2(hv[2], hv[3]);
            }
            *reinterpret_cast<uint2 *>(hout + (int64_t)prow * N + col0) = packed;
        }
    } else if (GU) {
        constexpr int CG = BW / 8;  // 4-column groups in the gate half
        uint16_t *hout = reinterpret_cast<uint16_t *>(p.out);
        for (int q = (int)threadIdx.x; q < BT * CG; q += 256) {
            const int j = q / CG, cg = q % CG;
            const int prow = b * BT + j;
            const int col0 = i0 + cg * 4;
            if (col0 >= N) continue;
            const int f = sorted_at(prow);
            uint2 packed = make_uint2(0u, 0u);
            if (f < p.P) {
                float v[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[i] = buf[1][j][cg * 4 + i];
                    v[4 + i] = buf[1][j][BW / 2 + cg * 4 + i];
                }
                float hv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) hv[i] = silu(v[i]) * v[4 + i];
                packed.x = pack_bf16x2(hv[0], hv[1]);
                packed.y = pack_bf16x2(hv[2], hv[3]);
            }
            *reinterpret_cast<uint2 *>(hout + (int64_t)prow * N + col0) = packed;
        }
    } else {
        constexpr int CG = BW / 4;
        uint16_t *yout = reinterpret_cast<uint16_t *>(p.out);
        for (int q = (int)threadIdx.x; q < BT * CG; q += 256) {
            const int j = q / CG, cg = q % CG;
            const int prow = b * BT + j;
            const int col0 = i0 + cg * 4;
            if (col0 >= N) continue;
            const int f = sorted_at(prow);
            if (f >= p.P) continue;
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = buf[1][j][cg * 4 + i];
            *reinterpret_cast<uint2 *>(yout + (int64_t)f * N + col0) =
                make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
    }
}

// Three workgroups per CU at 16 rows per block (two at 32): the register
// budget that keeps that many resident.
template <int BT> constexpr int stream_waves_per_eu() { return BT == 16 ? 3 : 2; }

template <int BW, int BT, bool GU, bool WP, bool MX = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(stream_waves_per_eu<BT>())))
void gemm_stream_kernel(GemmParams p) {
    gemm_stream_body<BW, BT, GU, WP, MX, false>(p, nullptr);
}

template <int BW, int BT, bool WP, bool MX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(stream_waves_per_eu<BT>())))
void gemm_stream_route_kernel(GemmParams p, FusedRoute fr) {
    gemm_stream_body<BW, BT, true, WP, MX, true>(p, &fr);
}

}  // namespace moelora
