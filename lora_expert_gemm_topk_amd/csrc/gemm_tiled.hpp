// Grouped expert GEMM for many rows per expert (prefill): LDS-tiled, matrix
// cores (v_mfma_f32_32x32x16_bf16); LoRA expand as extra K slabs, SwiGLU in the epilogue.
//
// Same contract as the streaming kernel (gemm_stream.hpp): weights are the
// MFMA M side, the expert's tokens the N side, y13 -> SwiGLU -> h (bf16,
// sorted row) for gate_up and y2 (bf16, pair row) for down.  The token side
// comes in the packed layout of common.hpp: x gathered and packed per sorted
// row (pack.hpp) for gate_up, h as written by gate_up for down.
//
// Work unit: one (weight tile of BW rows, token tile) pair.  Token tiles come
// from a list built by the alignment: up to BT consecutive sorted rows of ONE
// expert, a multiple of 32 rows (experts are padded to 32 only); an expert's
// rows are cut into tiles of equal size (to 32 rows), so the token tiles that
// share a weight tile run at the same pace and meet its slabs in L2.  MFMA
// column tiles (32 tokens) past the tile's rows are skipped outright, which
// keeps the padding cost at 32-row granularity while the tile stays large.
//
// Workgroup: 4 wavefronts in a 2 x 2 grid, each owning BW/2 weight rows and
// every other 32-token column tile (so a short tile splits evenly), as
// (BW/64) x (BT/64) MFMA tiles of 32 x 32; with BW = BT = 256 every wave does
// 16 MFMAs per 16-wide k-step on 8 fragment reads, which keeps LDS traffic
// (reads + stage fills) under the ~128 B/clk/CU that gfx950 sustains.
//
// K advances 32 at a time through a ring of kStages LDS stages of (BW+BT)
// rows x 64 bytes, filled by gfx950's direct global->LDS loads
// (global_load_lds_dwordx4: lane l's 16 bytes land at M0 + 16*l), so no
// registers stage the data and kStages-1 slabs are in flight while the MFMAs
// work on the oldest one.  One load instruction fills one 16-row group of a
// stage: from a packed operand (the tokens, and the weights when packed) it
// copies one 1 KiB block, from a row-major one 16 rows x 64 bytes.  Each wave
// waits only for its own loads of the slab it needs next (s_waitcnt vmcnt
// with the number of younger slabs still allowed in flight) and then meets
// the others at one barrier per slab; the
// wait and the barrier are one asm statement with a memory clobber, which
// keeps the compiler from moving LDS accesses across the barrier without the
// vmcnt(0) a fenced barrier would force.  K beyond the reduction length reads
// a 16-byte zero chunk (row-major operands) or the zero tail of a packed slab.
//
// gate_up row order inside a tile: rows 4a, 4a+1 hold gate features
// i0+2a, i0+2a+1 and rows 4a+2, 4a+3 the matching up features.  The 32 x 32
// accumulator gives each lane 4 consecutive rows, so every lane holds whole
// (gate, up) pairs and SwiGLU needs no data exchange.
//
// LoRA expand runs as extra K slabs of the same ring and MFMAs, one per
// adapter present in the token tile and 32 rank columns (see `issue`), so it
// costs a few slabs of the main loop's kind and no separate epilogue pass;
// a wave runs a LoRA slab's MFMAs only on its column tiles that hold the
// adapter's rows.  This needs, per sorted row, the adapter (written by the
// alignment) and the shrink result in bf16 (written by an unsplit shrink).
//
// Workgroups are numbered so that each XCD (8 per MI355X, dispatched round
// robin) receives one contiguous range of work in expert-major order (expert,
// then weight tile, then the expert's token tiles): an XCD works through whole
// experts, so an expert's gathered token rows stay in that XCD's L2 while all
// of its weight tiles stream past, and the token tiles sharing a weight tile
// run side by side.  When the load is skewed the work goes token-tile-major
// in plain dispatch order instead (see the kernel).
#pragma once

#include <type_traits>
#include <utility>

#include "common.hpp"
#include "gemm_stream.hpp"
#include "pack.hpp"

namespace moelora {

constexpr int kTileBK = 32;   // K per LDS stage
#ifndef MOELORA_TILED_STAGES
#define MOELORA_TILED_STAGES 4
#endif
constexpr int kStages = MOELORA_TILED_STAGES;  // LDS ring depth
#ifndef MOELORA_SKEW_PANEL
#define MOELORA_SKEW_PANEL 1
#endif
constexpr int kSkewPanel = MOELORA_SKEW_PANEL;  // token tiles per XCD panel in the skewed work order
static_assert(kStages >= 3, "the K loop keeps at least two slabs in flight");
// MXFP8 weights in the tiled kernel: most 32-element scale blocks per row
// (K <= 3072), so the tile's scale rows fit in LDS beside the ring
constexpr int kMxTiledMaxBlocks = 96;

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>), in order
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Step plan of the MXFP8 steady-state k-step (MT row tiles, NTL live column
// tiles, row-tile-major MFMA order: step s runs row tile s / NTL, column
// tile s % NTL).  The codes of row tile mt for the next k-step are read at
// ra(mt), one step after this k-step's conversion of mt (at step
// (mt - 1) NTL) consumed them; row tile 0 of the next k-step is converted at
// CV0, after this k-step's last use of it; the B fragment reads and then the
// slab copies take the steps with no code read, in order (B reads beyond
// them go to the last step, copies beyond them after the k-step).
template <int MT, int NTL>
struct MxSched {
    static constexpr int NMM = MT * NTL;
    static constexpr int CV0 = NTL > NMM - 2 ? NTL : NMM - 2;
    static constexpr int ra(int mt) { return mt == 0 ? 0 : (mt - 1) * NTL + 1; }
    static constexpr bool taken(int st) {
        for (int m = 0; m < MT; ++m)
            if (ra(m) == st) return true;
        return false;
    }
    static constexpr int free_step(int k) {
        int c = 0;
        for (int st = 0; st < NMM; ++st)
            if (!taken(st)) {
                if (c == k) return st;
                ++c;
            }
        return -1;
    }
    static constexpr int rb(int nt) { return free_step(nt) >= 0 ? free_step(nt) : NMM - 1; }
    static constexpr int dstep(int d) { return free_step(NTL + d); }
};

// 16 bytes of zeros: the source of every load past the end of K
__device__ __attribute__((aligned(16))) const uint16_t g_zero_chunk[8] = {0, 0, 0, 0, 0, 0, 0, 0};

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

// Byte offset of 16-byte chunk `c` (0..3) of LDS row `row` inside a stage.
// A 16-row group of a stage is 1 KiB in one of two layouts:
//  * row-major (rows copied from a row-major operand): 4 consecutive lanes of
//    a copy fetch one row's 64 contiguous bytes (coalesced), and the chunks
//    of a row are XOR-swizzled (swz_slot) so that 8 or 16 consecutive rows at
//    one chunk fall in distinct 16-byte slots;
//  * packed (a block of a packed operand copied as is): the block order of
//    common.hpp, where 16 consecutive rows at one chunk are 256 contiguous
//    bytes.
// Either way the 32x32x16 fragment reads are free of bank conflicts.
__device__ __forceinline__ int swz_slot(int row, int c) { return c ^ (((row >> 1) ^ (row >> 3)) & 3); }
template <bool PACKED>
__device__ __forceinline__ int lds_off(int row, int c) {
    return PACKED ? (row >> 4) * 1024 + (c * 16 + (row & 15)) * 16 : row * 64 + (swz_slot(row, c) << 4);
}

// Direct global->LDS copy of 16 bytes per lane: lane l's bytes land at LDS
// address `dst` + 16*l (dst uniform).  Issued as inline asm so that the
// compiler does not track it: its own wait insertion would otherwise drain
// every outstanding slab load before each LDS fragment read it cannot prove
// disjoint from the slab being filled.  The K loop orders these copies
// itself (wait_vm_barrier); since loads retire in order for vmcnt, copies the
// compiler does not know of only make its own vmcnt waits stricter.
// M0 is a register the compiler reserves (it may hold a value of its own
// across this statement), so the statement saves it in a scratch SGPR, sets
// the LDS address, issues the copy (which reads M0 at issue) and restores
// it: to the compiler M0 is unchanged.
__device__ __forceinline__ void dma16(const void *g, __attribute__((address_space(3))) unsigned char *dst) {
    const uint32_t m0v = (uint32_t)(uintptr_t)dst;
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0v), "v"(g));
}

// dma16 from a wave-uniform base plus this lane's byte offset (the copy's
// scalar-base form: no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void dma16s(const void *base, uint32_t off,
                                       __attribute__((address_space(3))) unsigned char *dst) {
    const uint32_t m0v = (uint32_t)(uintptr_t)dst;
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0v), "v"(off), "s"((uint64_t)(uintptr_t)base));
}

// Barrier for LDS data only: waits for this wave's LDS accesses, not for its
// loads in flight.  (__syncthreads also waits for every outstanding global
// load, and placed before the K loop it leads the compiler to drain all slab
// loads before each fragment read of the loop.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// WP: weights in the packed layout of moe_lora_pack_weights (copied block by
// block like the tokens) instead of row-major.
//
// MX: MXFP8 expert weights (E4M3 codes, one E8M0 scale per 32 elements along
// K; row-major codes, or with WP the packed codes of
// moe_lora_pack_mxfp8_weights).  A K slab then carries 32 codes (bytes) per
// weight row: in each 1 KiB block of the stage's weight area, 32 tile rows,
// codes 0..15 of row r at 16 r and codes 16..31 at 512 + 16 r, so a lane's
// eight codes of a 16-wide k-step are one 8-byte LDS read.  The tile's
// scale rows (K/32 bytes per weight row) are copied to LDS once per tile;
// each fragment is converted with the hardware's scaled FP8 -> bf16
// conversion (exact: E4M3 has 3 mantissa bits) right before its first MFMA,
// and the same bf16 MFMAs run.  The weight area keeps its bf16 size, so the
// LoRA slabs (bf16 B rows) are unchanged, and every slab issues the same
// number of stage loads per wave (a K slab's spare weight-side loads copy
// the zero chunk), which keeps the slab waits exact.
template <int BW, int BT, bool GU, bool WP, bool MX = false>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(GemmParams p, const int32_t *__restrict__ tiles,
                                                         const int32_t *__restrict__ n_tiles, int n_wtiles,
                                                         const int32_t *__restrict__ xsplit) {
    constexpr int MT = BW / 64, NT = BT / 64;          // 32x32 tiles per wave
    constexpr int ROWS = BW + BT;                       // LDS rows per stage
    constexpr int STAGE_BYTES = ROWS * 64;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kStages * STAGE_BYTES];
    // MX: the tile's weight scales.  The tile's weight rows are NRUN runs of
    // consecutive rows (gate_up: its gate rows, then its up rows), so the
    // scales of a run are one contiguous byte range of K/32 bytes per row;
    // each run has RUN_BYTES of LDS (layout at the copy below).
    constexpr int NRUN = GU ? 2 : 1, RUN_ROWS = GU ? BW / 2 : BW;
    constexpr int RUN_CHUNKS = (RUN_ROWS * kMxTiledMaxBlocks + 15) / 16;  // most whole 16-byte pieces of a run
    constexpr int RUN_COPIES = (RUN_CHUNKS + 63) / 64;                    // 1 KiB copies per run, at most
    constexpr int RUN_BYTES = 16 + 1024 * RUN_COPIES + 32;  // + the 8-byte scale reads' overhang
    __shared__ __attribute__((aligned(16))) unsigned char mx_sc[MX ? NRUN * RUN_BYTES : 16];

    // Logical order: expert-major, then weight tile, then the expert's token
    // tiles.  Expert e owns logical [n_wtiles*t0, n_wtiles*(t0+nt)) where t0 is
    // its first token tile and nt its tile count (both stored in every tile).
    // XCD x (the workgroups with blockIdx mod 8 = x) takes the contiguous
    // range [xsplit[x], xsplit[x+1]), cut by the alignment at equal
    // estimated cost (tiles of fewer rows cost less), so the XCDs finish
    // together; workgroups past their XCD's range exit at once.
    //
    // When the load is skewed (one expert holds more than twice the mean tile
    // count of the experts with tiles) the per-XCD ranges would carry very
    // different amounts of work; the work is then enumerated token-tile-major
    // in dispatch order (token tile, then weight tile) and balances across the
    // whole chip instead (measured on a Zipf-skewed 128-expert prefill: 11-13%
    // faster; on uniform routing the XCD ranges are faster by ~12% on down).
    const int live = n_wtiles * n_tiles[0];
    const bool skewed = 2 * n_tiles[0] < n_tiles[1] * n_tiles[2];
    int wt, ti;
    if (skewed) {
        // token tiles in panels of kSkewPanel consecutive tiles, the panels
        // dealt to the XCDs in turn; an XCD runs a panel's items weight tile
        // by weight tile, so its L2 fetches the panel's token rows once and
        // each weight tile once per panel (on a Zipf-skewed 128-expert
        // prefill one tile per panel was fastest: larger panels read less
        // but leave the XCDs less evenly loaded)
        const int x = (int)blockIdx.x & 7, k = (int)(blockIdx.x >> 3);
        const int per = kSkewPanel * n_wtiles;
        const int j = k / per, kl = k - j * per;
        ti = (8 * j + x) * kSkewPanel + kl % kSkewPanel;
        wt = kl / kSkewPanel;
        if (ti >= n_tiles[0]) return;
    } else {
        const int x = (int)blockIdx.x & 7;
        const int logical = xsplit[x] + (int)(blockIdx.x >> 3);
        if (logical >= xsplit[x + 1]) return;
        const int tq = logical / n_wtiles;
        const int4 tq_tile = reinterpret_cast<const int4 *>(tiles)[tq];
        const int t0 = tq_tile.w, ntl = tq_tile.y >> 16;
        const int rel = logical - n_wtiles * t0;
        wt = rel / ntl;
        ti = t0 + rel % ntl;
    }
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
    // 32-row column tiles alternate between the two wave columns (tile c to
    // wn = c % 2), so a short tile splits its rows evenly between them
    const int nt_live = max(0, min(NT, (nrows / 32 - wn + 1) / 2));

    // ---- token metadata and the tile's adapter list ----------------------
    // tok_f / tok_a: pair index and adapter of each tile row (P / -1 past the
    // tile's rows); alist: the adapters present, ascending (the alignment
    // sorts an expert's rows by adapter, so each is one run of rows); arun:
    // the first and one-past-last row of each adapter's run.
    __shared__ int tok_f[BT], tok_a[BT], alist[BT], arun[2 * BT], wcnt[5];
    // ---- MX: the tile's scales, copied to LDS ahead of the ring ------------
    // Run u covers the weight rows of features i0 .. i0 + vrows - 1 (gate
    // rows, or up rows at u = 1): bytes [0, len) from rg.  Byte b of the
    // range lands at LDS run base + 16 + (rg mod 16) + b, which keeps the
    // 16-byte grid of the scale array (16-byte aligned) on that of LDS, so
    // the scale of (run row q, K block kb) sits at run base + 16 +
    // (rg mod 16) + q nb + kb.  The whole 16-byte pieces from rg rounded down
    // to the end rounded down (all inside the array) go by direct
    // global->LDS loads issued before the ring's (so every slab wait covers
    // them; lanes past the last piece copy the zero chunk into the run's
    // spare bytes); the last (end mod 16) bytes are fetched one per thread
    // and stored once the first slab wait has seen every copy land.
    const int nb = (int)(Kd / 32);
    int mx_off16[NRUN], mx_nch[NRUN], mx_tail[NRUN];
    uint32_t mx_byte = 0;
    if constexpr (MX) {
        const int vrows = max(0, min(RUN_ROWS, N - i0));
#pragma unroll
        for (int u = 0; u < NRUN; ++u) {
            const uint8_t *rg = p.Wscale + ((int64_t)e * rows_per_expert + (u ? N : 0) + i0) * nb;
            const uint8_t *g16 = rg - ((uintptr_t)rg & 15);
            const uint8_t *end = rg + vrows * nb;
            const uint8_t *end0 = end - ((uintptr_t)end & 15);
            mx_off16[u] = (int)((uintptr_t)rg & 15);
            mx_nch[u] = (int)((end0 - g16) >> 4);
            mx_tail[u] = (int)((uintptr_t)end & 15);
            typedef __attribute__((address_space(3))) unsigned char lds_b;
            lds_b *run = (lds_b *)mx_sc + u * RUN_BYTES + 16;
            for (int m = w; m * 64 < mx_nch[u]; m += 4) {
                const int c = m * 64 + lane;
                dma16(c < mx_nch[u] ? (const void *)(g16 + 16 * c) : (const void *)g_zero_chunk, run + 1024 * m);
            }
            // threads 16u .. 16u + 14: the tail bytes
            const int k = tid - 16 * u;
            if (k >= 0 && k < mx_tail[u]) mx_byte = end0[k];
        }
    }

    const int my_row = row0 + min(tid, nrows - 1);
    const int f_row = (tid < BT) ? p.sorted_ids[my_row] : p.P;
    const int a_row = (p.lora && tid < BT) ? p.sorted_adapter[my_row] : -1;

    // ---- direct-to-LDS stage loads ----------------------------------------
    // Wave w owns the stage's 16-row groups w, w+4, ...: instruction j fills
    // group w + 4j.  Groups below BW/16 hold weight rows, the rest token rows.
    // Weights (row-major): lane l fetches row l/4 of the group at the chunk
    // its slot l&3 holds (swizzled).  Tokens (packed x for gate_up, packed h
    // for down): lane l fetches bytes 16l .. 16l+15 of the block.
    constexpr int GROUPS = ROWS / 16;               // 16-row groups per stage
    static_assert(GROUPS % 4 == 0 && BW % 64 == 0, "row groups must split evenly over 4 waves");
    constexpr int LPW = GROUPS / 4;                 // load instructions per wave per stage
    constexpr int LPW_A = BW / 64;                  // of which weight groups
    constexpr bool B_PACKED = true;                 // tokens arrive packed (x packed per sorted row, h)
    // MX K slabs: 32 codes (bytes) per weight row fill half the weight area,
    // BW/128 loads per wave; the wave's other weight-side loads are not issued
    constexpr int MX_REAL = BW / 128;
    constexpr int LPW_K = MX ? LPW - LPW_A + MX_REAL : LPW;  // loads per wave of a K slab
    const int64_t nslab_in = (Kd + kSlabK - 1) / kSlabK;
    const uint16_t *src[LPW];
    int chunk_of[LPW];  // chunk (0..3) this lane moves, row-major groups
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int rr = (w + 4 * j) * 16 + (lane >> 2);
        const int c = swz_slot(rr, lane & 3);  // slot -> chunk (the XOR is its own inverse)
        chunk_of[j] = c;
        if (j < LPW_A && WP) {
            // packed weights: group (w + 4j) of this tile; a tile spans BW/16
            // whole groups (the packed group count is padded to full tiles)
            const int64_t G = GU ? packed_w13_groups(N) : packed_w2_groups(N);
            const int64_t gq = (int64_t)wt * (BW / 16) + (w + 4 * j);
            src[j] = p.W + ((int64_t)e * G + gq) * nslab_in * kBlockElems + lane * 8;
        } else if (j < LPW_A) {
            bool ok;
            const int grow = tile_weight_row<GU>(rr, i0, N, ok);
            src[j] = p.W + ((int64_t)e * rows_per_expert + (ok ? grow : 0)) * Kd + c * 8;
        } else {
            // the tile's rows start on a group boundary and fill whole groups;
            // groups past them repeat its last one (those columns are discarded)
            const int grp = row0 / 16 + min((w + 4 * j) - BW / 16, nrows / 16 - 1);
            src[j] = p.in + (int64_t)grp * nslab_in * kBlockElems + lane * 8;
        }
    }
    // per-slab advance of a source: 32 elements along a row, or one block
    auto src_step = [&](int j) -> int64_t {
        return (j < LPW_A ? WP : B_PACKED) ? (int64_t)kBlockElems : (int64_t)kTileBK;
    };
    // MX: weight-side load j < BW/128 of a K slab moves 32 tile rows: lane l
    // takes codes 16q .. 16q+15 (q = l/32) of tile row 32(w+4j) + l%32 to
    // byte 16l of the stage's 1 KiB block w+4j.  Packed codes: the slab is
    // 32-code group kt%4 of 128-wide chunk kt/4, whose 2 KiB block per 16 rows
    // holds half q of row r's group g at 1024q + 256g + 16r.  Rows past N
    // read the expert's row 0, as the bf16 weights do (their outputs are
    // dropped).
    const uint8_t *mx_src[MX_REAL];
    if constexpr (MX) {
        const uint8_t *W8 = reinterpret_cast<const uint8_t *>(p.W);
        const int64_t nch = packed_mx_chunks(Kd);
#pragma unroll
        for (int j = 0; j < MX_REAL; ++j) {
            const int trow = (w + 4 * j) * 32 + (lane & 31), q = lane >> 5;
            bool ok;
            const int R = tile_weight_row<GU>(trow, i0, N, ok);
            const int64_t grow = (int64_t)e * rows_per_expert + (ok ? R : 0);
            mx_src[j] = WP ? W8 + (grow >> 4) * nch * 2048 + 16 * (64 * q + (grow & 15)) : W8 + grow * Kd + 16 * q;
        }
    }
    // whether load j of a K slab is issued (MX: not the spare weight-side ones)
    auto k_issued = [](int j) { return !MX || j < MX_REAL || j >= LPW_A; };
    // source of issued load j of K slab kt (kt < nk)
    auto ksrc = [&](int j, int kt) -> const void * {
        if constexpr (MX) {
            if (j < MX_REAL) {
                const int64_t off = WP ? (int64_t)(kt >> 2) * 2048 + (kt & 3) * 256 : (int64_t)kt * kTileBK;
                return mx_src[j] + off;
            }
        }
        return src[j] + kt * src_step(j);
    };
    const int nk = (int)((Kd + kTileBK - 1) / kTileBK);
    typedef __attribute__((address_space(3))) unsigned char lds_t;
    lds_t *lds_base = (lds_t *)lds;
    auto dma = [&](const void *g, lds_t *stage, int j) { dma16(g, stage + (w + 4 * j) * 1024); };
    // Slab kt < nk: K columns [32 kt, 32 kt + 32) of the weights and tokens.
    auto issue = [&](int kt) {
        lds_t *stage = lds_base + (kt % kStages) * STAGE_BYTES;
        const int64_t k0 = (int64_t)kt * kTileBK;
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            if (!k_issued(j)) continue;
            // MX weights: K is a multiple of 32, every slab is whole
            const bool kin = (j < LPW_A ? (WP || MX) : B_PACKED) || k0 + chunk_of[j] * 8 < Kd;
            dma(kin ? ksrc(j, kt) : (const void *)g_zero_chunk, stage, j);
        }
    };
    const int rs = (p.r + kTileBK - 1) / kTileBK;  // 32-rank slabs per adapter

    f32x16 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[mt][nt][q] = 0.f;

    const int a_row0 = wm * (BW / 2) + l32;        // + mt*32
    const int b_row0 = BW + wn * 32 + l32;         // + nt*64
    // MX fragments: lane (l32, lh) of row tile mt reads the eight codes
    // 16 ks + 8 lh .. + 7 of tile row a_row0 + 32 mt and, at ks = 0, the
    // row's scale byte of the slab; mx_cvt turns them into the bf16 fragment,
    // exactly (E4M3 times a power of two fits bf16).  The scale stays a byte
    // until the conversion, so no instruction waits on its read before then.
    int mx_soff[MT];     // LDS offset of the row's scale of K block 0
    uint32_t mx_scl[MT]; // scale byte of the slab last read at ks = 0
    if constexpr (MX) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int tr = a_row0 + mt * 32;
            const int u = GU ? ((tr >> 1) & 1) : 0;                   // gate or up run
            const int q = GU ? 2 * (tr >> 2) + (tr & 1) : tr;        // row within the run
            mx_soff[mt] = u * RUN_BYTES + 16 + mx_off16[u] + q * nb;
            mx_scl[mt] = 0u;
        }
    }
    auto mx_rd_raw = [&](uint2 &r, const unsigned char *base, int mt, int ks, int slab) {
        r = *reinterpret_cast<const uint2 *>(base + ((a_row0 + mt * 32) >> 5) * 1024 + ks * 512 + l32 * 16 + lh * 8);
        if (ks == 0) mx_scl[mt] = mx_sc[mx_soff[mt] + slab];
    };
    // r's codes times 2^(scale - 127), `bits` = scale << 23 (that power of two in fp32)
    auto mx_cvt_bits = [&](u32x4 &a, uint2 r, uint32_t bits) {
        const float sc = __uint_as_float(bits);
        a[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.x, sc, false));
        a[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.x, sc, true));
        a[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.y, sc, false));
        a[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.y, sc, true));
    };
    auto mx_cvt_to = [&](u32x4 &a, uint2 r, int mt) { mx_cvt_bits(a, r, mx_scl[mt] << 23); };
    // the drain keeps a K slab's codes in dwords 0, 1 of the fragment itself
    auto mx_rd = [&](u32x4 &a, const unsigned char *base, int mt, int ks, int slab) {
        uint2 r;
        mx_rd_raw(r, base, mt, ks, slab);
        a[0] = r.x;
        a[1] = r.y;
    };
    auto mx_cvt = [&](u32x4 &a, int mt) { mx_cvt_to(a, make_uint2(a[0], a[1]), mt); };
    // Fragment reads of one 16-wide k-step (NTL live column tiles) of slab
    // `slab` held in ring stage `stage`, and its MFMAs.
    auto rd = [&](auto ntl, u32x4 *af, u32x4 *bfr, int stage, int ks, int slab) {
        constexpr int NTL = decltype(ntl)::value;
        const unsigned char *base = lds + stage * STAGE_BYTES;
        const int c = ks * 2 + lh;
        if (MX && slab < nk) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) mx_rd(af[mt], base, mt, ks, slab);
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                af[mt] = *reinterpret_cast<const u32x4 *>(base + lds_off<WP>(a_row0 + mt * 32, c));
        }
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt)
            bfr[nt] = *reinterpret_cast<const u32x4 *>(base + lds_off<B_PACKED>(b_row0 + nt * 64, c));
    };
    // mm restricted to the column tiles set in `live` (wave-uniform); `cvt`:
    // the A fragments still hold MX codes
    auto mm_live = [&](auto ntl, u32x4 *af, const u32x4 *bfr, int live, bool cvt) {
        constexpr int NTL = decltype(ntl)::value;
        if (MX && cvt) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) mx_cvt(af[mt], mt);
        }
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) {
            if (!((live >> nt) & 1)) continue;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[mt]), as_bf16x8(bfr[nt]),
                                                                      acc[mt][nt], 0, 0, 0);
        }
    };
    // Single steps of the above for K slabs: fragment read i (A fragments
    // first, then B) and MFMA i (column tile i / MT, row tile i % MT).
    auto rd_one = [&](auto i, u32x4 *af, u32x4 *bfr, const unsigned char *base, int ks) {
        constexpr int I = decltype(i)::value;
        const int c = ks * 2 + lh;
        if constexpr (I < MT) af[I] = *reinterpret_cast<const u32x4 *>(base + lds_off<WP>(a_row0 + I * 32, c));
        else bfr[I - MT] = *reinterpret_cast<const u32x4 *>(base + lds_off<B_PACKED>(b_row0 + (I - MT) * 64, c));
    };
    auto mm_one = [&](auto i, const u32x4 *af, const u32x4 *bfr) {
        constexpr int I = decltype(i)::value;
        acc[I % MT][I / MT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[I % MT]), as_bf16x8(bfr[I / MT]),
                                                                      acc[I % MT][I / MT], 0, 0, 0);
    };
    // Wait for this wave's loads of the slab needed next, given `younger`
    // younger slabs that may stay in flight, then barrier.  Loads issued before
    // the slabs (token metadata) are older than all of them, so they only make
    // a wait longer, never shorter.
    auto wait_slab = [&](int younger) {
        static_assert(kStages <= 6, "extend the wait ladder");
        // per younger slab the fewest loads a slab issues (LoRA slabs issue
        // LPW >= LPW_K): a wait that counts low only waits longer
        if (younger >= 4) wait_vm_barrier<4 * LPW_K>();
        else if (younger == 3) wait_vm_barrier<3 * LPW_K>();
        else if (younger == 2) wait_vm_barrier<2 * LPW_K>();
        else if (younger == 1) wait_vm_barrier<LPW_K>();
        else wait_vm_barrier<0>();
    };

    // Ring prologue: the K slabs; the adapter list is built while they are
    // in flight.
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < nk) issue(s);
    if (tid < BT) {
        tok_f[tid] = tid < nrows ? f_row : p.P;
        tok_a[tid] = (tid < nrows && a_row < p.L) ? a_row : -1;
    }
    // Every value loaded above is used here on all paths (the MX tail byte
    // is loaded first): a load whose only use is conditional would leave the
    // compiler a wait for it pending into the K loop, where it would put a
    // full vmcnt(0) wait in every iteration.
    asm volatile("" ::"v"(f_row), "v"(a_row), "v"(mx_byte));
    lds_barrier();
    {
        const int a = tid < BT ? tok_a[tid] : -1;
        const bool start = a >= 0 && (tid == 0 || tok_a[tid - 1] != a);
        const bool end = a >= 0 && (tid == BT - 1 || tok_a[tid + 1] != a);
        const uint64_t m = __ballot(start);
        if (lane == 0) wcnt[w] = __popcll(m);
        lds_barrier();
        int before = 0;
        for (int v = 0; v < w; ++v) before += wcnt[v];
        const int run = before + __popcll(m & lanemask_lt());  // runs starting before this row
        if (start) {
            alist[run] = a;
            arun[2 * run] = tid;
        }
        if (end) arun[2 * (run + (start ? 1 : 0)) - 1] = tid + 1;  // this row's run
        if (tid == 0) wcnt[4] = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
        lds_barrier();
    }
    const int n_adapters = __builtin_amdgcn_readfirstlane(wcnt[4]);

    // The whole K loop, specialised on the live column tiles so it has no
    // branches.  Two fragment register sets alternate: while the MFMAs of one
    // k-step run, the reads of the next are in flight.  The barrier that makes
    // slab kt+1 visible sits between the two k-steps of slab kt, so the first
    // reads of slab kt+1 overlap the second half of slab kt's MFMAs.  The slab
    // refilled right after that barrier, (kt + kStages - 1) mod kStages ==
    // (kt - 1) mod kStages, was last read before the previous barrier, so
    // every wave is done with it.  The steady state refills with slabs that
    // lie wholly inside K, so it needs no slab-kind or end-of-K branches and
    // is one basic block (measured ~15% faster than one loop with them).
    const int nk_full = (int)(Kd / kTileBK);

    // ---- LoRA expand (aitrends.kr summary of the AWS multi-LoRA MoE post,
    // "section details": the LoRA sum folded into the expand step) ---------
    // After the K loop, each adapter present in the token tile adds
    // B[a, e] (its rows of this weight tile) times the bf16 shrink rows of
    // its tokens, as MFMAs on the same accumulators.  The ring, now free,
    // streams only the weight side in units of BW x 32 ranks: an adapter's
    // 32-rank slab, or, where the rank range holds 64 ranks, one of its two
    // row halves (each copy instruction then reads whole 128-byte row
    // pieces); kStages*STAGE_BYTES / (BW*64) units fit, so many more are in
    // flight than whole slabs would allow.  Each unit's copies take a
    // wave-uniform base and per-lane offsets fixed for the tile, so issuing
    // them costs no vector instructions.  Each lane holds its
    // tokens' shrink rows in registers for 64 ranks at a time (read once per
    // tile) and zeroes those of other adapters before each MFMA; the MFMAs
    // of column tiles outside the adapter's run of rows (exact zeros) are
    // skipped.  Units go in adapter order, ranks ascending, so the sums are
    // those of the same products in the same order as full LoRA slabs.
    const uint16_t *s16 = reinterpret_cast<const uint16_t *>(p.s_part);
    auto lora_phase = [&](auto ntl) {
        constexpr int NTL = decltype(ntl)::value;
        constexpr int UBYTES = BW * 64;                          // one unit: BW x 32 bf16 values
        constexpr int NSLOT = kStages * STAGE_BYTES / UBYTES;    // units the ring holds
        static_assert(NSLOT >= 4 && NSLOT <= 12 && NSLOT % 2 == 0, "LoRA unit ring depth");
        // wait for unit u with `younger` later units still in flight, then barrier
        auto wait_unit = [&](int younger) {
            switch (younger) {
                case 0: wait_vm_barrier<0>(); break;
                case 1: wait_vm_barrier<LPW_A>(); break;
                case 2: wait_vm_barrier<2 * LPW_A>(); break;
                case 3: wait_vm_barrier<3 * LPW_A>(); break;
                case 4: wait_vm_barrier<4 * LPW_A>(); break;
                case 5: wait_vm_barrier<5 * LPW_A>(); break;
                case 6: wait_vm_barrier<6 * LPW_A>(); break;
                case 7: wait_vm_barrier<7 * LPW_A>(); break;
                case 8: wait_vm_barrier<8 * LPW_A>(); break;
                case 9: wait_vm_barrier<9 * LPW_A>(); break;
                default: wait_vm_barrier<10 * LPW_A>(); break;
            }
        };
        int myad[NTL > 0 ? NTL : 1];  // adapter of this lane's token in column tile nt
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) myad[nt] = tok_a[(2 * nt + wn) * 32 + l32];
        // Both unit forms place row tile mt of wave row wm at 4096 mt + (a
        // part fixed per lane), so a fragment read is (lane base ^ X) +
        // 4096 mt + slot with X and the slot the same for the whole wave.
        // 32-rank units: 1 KiB group g of the wave row's row tile mt (tile
        // rows (BW/2) wm + 32 mt + 16 g ..) sits at block 4 mt + 2 wm + g,
        // in the K slabs' group layout (packed or swizzled row-major).
        // Wide units (a whole 64-rank range): unit (adapter, row half h) holds
        // the 64 ranks of tile rows [h BW/2, (h+1) BW/2), the rows of wave row
        // h, in 1 KiB blocks of 8 rows x 64 ranks, so every copy instruction
        // reads 8 whole 128-byte row pieces (a 32-rank unit reads 16 half
        // lines when r >= 64).  Lane l of block b moves row l/8, rank chunk
        // (l%8) ^ (l/8) ^ (b%2) to 16-byte slot l%8 of its row: the fragment
        // reads of 16 consecutive rows then hit 16 different bank groups.
        // Rank chunk (of 8) lane l moves in copy j of a 32-rank / wide unit:
        auto nchunk = [&](int j) { return WP ? lane >> 4 : swz_slot((w + 4 * j) * 16 + (lane >> 2), lane & 3); };
        auto wchunk = [&](int j) { return (lane & 7) ^ (lane >> 3) ^ ((w + 4 * j) & 1); };
        // byte offsets of those 16 bytes from the unit's base (adapter,
        // expert, first rank of the range); rows past N read row 0 instead
        // (their accumulator rows are never stored)
        uint32_t noff[LPW_A], woff[2][LPW_A];
#pragma unroll
        for (int j = 0; j < LPW_A; ++j) {
            const int b = w + 4 * j;
            const int grp = ((b >> 1) & 1) * (BW / 32) + (b >> 2) * 2 + (b & 1);
            bool ok;
            int grow = tile_weight_row<GU>(grp * 16 + (WP ? (lane & 15) : (lane >> 2)), i0, N, ok);
            noff[j] = (uint32_t)(((ok ? grow : 0) * p.r + nchunk(j) * 8) * 2);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                grow = tile_weight_row<GU>(h * (BW / 2) + b * 8 + (lane >> 3), i0, N, ok);
                woff[h][j] = (uint32_t)(((ok ? grow : 0) * p.r + wchunk(j) * 8) * 2);
            }
        }
        // lane bases: row l32 of row tile 0 at rank chunk lh (chunk 2 ks + lh
        // of a 32-rank unit, 4 rcl + 2 ks + lh of a wide one: X flips the
        // bits of ks and rcl)
        const int nbase = (2 * wm + (l32 >> 4)) * 1024 +
                          (WP ? lh * 256 + (l32 & 15) * 16 : (l32 & 15) * 64 + ((lh ^ swz_slot(l32, 0)) << 4));
        const int wbase = (l32 >> 3) * 1024 + (l32 & 7) * 128 + ((lh ^ (l32 & 7) ^ ((l32 >> 3) & 1)) << 4);
        // every wave is past its last fragment read of the ring's K slabs
        lds_barrier();
        for (int c0 = 0; c0 < rs; c0 += 2) {      // ranks [32 c0, 32 c0 + 64)
            const int uc = min(2, rs - c0);        // 32-rank slabs per adapter in this range
            const int nu = n_adapters * uc;
            const bool wide = uc == 2;             // units of 64 ranks x half the rows
            const bool full = (c0 + uc) * kTileBK <= p.r;  // no rank of the range past r
            const int lbase = wide ? wbase : nbase;
            uint32_t off0[LPW_A];
#pragma unroll
            for (int j = 0; j < LPW_A; ++j) off0[j] = wide ? woff[0][j] : noff[j];
            // adapter q's units q uc .. q uc + uc - 1: the weight rows of a
            // slab (32 ranks) or of a row half (wide), ranks from 32 c0
            auto issue_adapter = [&](int q) {
                const int a = __builtin_amdgcn_readfirstlane(alist[q]);
                const uint16_t *base = p.B + ((int64_t)a * p.Ep + e) * (int64_t)rows_per_expert * p.r + c0 * kTileBK;
                lds_t *s0 = lds_base + ((q * uc) % NSLOT) * UBYTES;
                lds_t *s1 = lds_base + ((q * uc + 1) % NSLOT) * UBYTES;
                if (full) {
#pragma unroll
                    for (int j = 0; j < LPW_A; ++j) dma16s(base, off0[j], s0 + (w + 4 * j) * 1024);
                    if (wide) {
#pragma unroll
                        for (int j = 0; j < LPW_A; ++j) dma16s(base, woff[1][j], s1 + (w + 4 * j) * 1024);
                    }
                } else {
                    // rank chunks past r read zeros
                    const char *cb = reinterpret_cast<const char *>(base);
#pragma unroll
                    for (int j = 0; j < LPW_A; ++j) {
                        const bool in = c0 * kTileBK + (wide ? wchunk(j) : nchunk(j)) * 8 < p.r;
                        dma(in ? (const void *)(cb + off0[j]) : (const void *)g_zero_chunk, s0, j);
                    }
                    if (wide) {
#pragma unroll
                        for (int j = 0; j < LPW_A; ++j) {
                            const bool in = c0 * kTileBK + wchunk(j) * 8 < p.r;
                            dma(in ? (const void *)(cb + woff[1][j]) : (const void *)g_zero_chunk, s1, j);
                        }
                    }
                }
            };
            // units are consumed an adapter (uc units) at a time, one barrier
            // each; the ring holds NSLOT / uc adapters
            const int apr = wide ? NSLOT / 2 : NSLOT;
            for (int q = 0; q < min(n_adapters, apr - 1); ++q) issue_adapter(q);
            // shrink rows: lane (l32, lh) of column tile nt holds ranks
            // 32 c0 + 16 kq + 8 lh .. + 7 of tile row (2 nt + wn) 32 + l32
            u32x4 sfr[NTL > 0 ? NTL : 1][4];
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                const int jt = (2 * nt + wn) * 32 + l32;
#pragma unroll
                for (int kq = 0; kq < 4; ++kq) {
                    const int k = c0 * kTileBK + kq * 16 + lh * 8;
                    sfr[nt][kq] = ld16(s16 + (int64_t)(row0 + min(jt, nrows - 1)) * p.r + k, jt < nrows && k < p.r);
                }
            }
            // wait for the shrink rows here (with the units issued above),
            // not at a first use after later unit copies
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                for (int kq = 0; kq < 4; ++kq) asm volatile("" ::"v"(sfr[nt][kq]));
            for (int q = 0; q < n_adapters; ++q) {
                const int a = __builtin_amdgcn_readfirstlane(alist[q]);
                const int lo = __builtin_amdgcn_readfirstlane(arun[2 * q]);
                const int hi = __builtin_amdgcn_readfirstlane(arun[2 * q + 1]);
                const int u0 = q * uc;
                // issued so far: units 0 .. min(u0 + NSLOT - uc, nu) - 1; wait for this adapter's
                wait_unit(min(nu - u0 - uc, NSLOT - 2 * uc));
                // into the slots of adapter q - 1, which every wave is done with
                if (q + apr - 1 < n_adapters) issue_adapter(q + apr - 1);
#pragma unroll
                for (int rcl = 0; rcl < 2; ++rcl) {
                    if (rcl >= uc) break;
                    const int u = u0 + (wide ? wm : rcl);
                    const unsigned char *slot = lds + (u % NSLOT) * UBYTES;
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        if ((c0 + rcl) * kTileBK + ks * 16 >= p.r) break;  // ranks past r
                        const int x = wide ? (4 * rcl + 2 * ks) << 4 : ks * (WP ? 512 : 32);
                        const unsigned char *fr = slot + (lbase ^ x);
                        u32x4 af[MT];
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) af[mt] = *reinterpret_cast<const u32x4 *>(fr + mt * 4096);
#pragma unroll
                        for (int nt = 0; nt < NTL; ++nt) {
                            const int cr = (2 * nt + wn) * 32;
                            if (!(cr < hi && cr + 32 > lo)) continue;
                            const u32x4 sv = sfr[nt][rcl * 2 + ks];
                            const bool mine = myad[nt] == a;
                            u32x4 bv;
#pragma unroll
                            for (int i = 0; i < 4; ++i) bv[i] = mine ? sv[i] : 0u;
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt)
                                acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[mt]), as_bf16x8(bv),
                                                                                      acc[mt][nt], 0, 0, 0);
                        }
                    }
                }
            }
            // the next rank range (or the epilogue) reuses the ring
            lds_barrier();
        }
    };

    auto mainloop = [&](auto ntl) {
        u32x4 a0[MT], b0[NT], a1[MT], b1[NT];
        wait_slab(min(kStages - 2, nk - 1));
        if constexpr (MX) {
            // every scale copy has landed (older than slab 0): the tail bytes
#pragma unroll
            for (int u = 0; u < NRUN; ++u) {
                const int k = tid - 16 * u;
                if (k >= 0 && k < mx_tail[u]) mx_sc[u * RUN_BYTES + 16 + 16 * mx_nch[u] + k] = (unsigned char)mx_byte;
            }
            lds_barrier();
        }
        rd(ntl, a0, b0, 0, 0, 0);
        int kt = 0;
        constexpr int NTL = decltype(ntl)::value;
        constexpr int NMM = MT * NTL, NRD = MT + NTL;
        if constexpr (!MX) {
        // Steady state, one slab per iteration.  Instruction order is fixed by hand (a scheduling barrier after each
        // step): MFMA i of a k-step is followed by fragment read i of the next
        // k-step and, after the barrier, by one slab copy, so the wave keeps
        // its matrix core fed while the reads and copies issue between MFMAs
        // instead of in blocks (measured ~8% faster than blocked issue).
        for (; kt + kStages - 1 < nk_full; ++kt) {
            const unsigned char *cur = lds + (kt % kStages) * STAGE_BYTES;
            const unsigned char *nxt = lds + ((kt + 1) % kStages) * STAGE_BYTES;
            lds_t *fill = lds_base + ((kt + kStages - 1) % kStages) * STAGE_BYTES;
            const int kfill = kt + kStages - 1;
            static_for<NMM>([&](auto i) {
                mm_one(i, a0, b0);
                if constexpr (i < NRD) rd_one(i, a1, b1, cur, 1);
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (NMM < NRD) {
                static_for<NRD - NMM>([&](auto i) { rd_one(std::integral_constant<int, NMM + i>{}, a1, b1, cur, 1); });
            }
            wait_vm_barrier<(kStages - 3) * LPW>();
            __builtin_amdgcn_sched_barrier(0);
            static_for<NMM>([&](auto i) {
                mm_one(i, a1, b1);
                if constexpr (i < NRD) rd_one(i, a0, b0, nxt, 0);
                else if constexpr (i - NRD < LPW) dma(ksrc(i - NRD, kfill), fill, i - NRD);
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (NMM < NRD) {
                static_for<NRD - NMM>([&](auto i) { rd_one(std::integral_constant<int, NMM + i>{}, a0, b0, nxt, 0); });
            }
            constexpr int DONE = NMM > NRD ? NMM - NRD : 0;
            if constexpr (DONE < LPW) {
                static_for<LPW - DONE>([&](auto i) {
                    constexpr int j = DONE + decltype(i)::value;
                    dma(ksrc(j, kfill), fill, j);
                });
            }
        }
        } else {
        // MXFP8 steady state: the step plan of MxSched, one set of codes `r`
        // and one set of converted fragments (a0); each fragment is converted
        // NTL - 1 MFMAs before its first use, so no conversion stands
        // between two MFMAs of the matrix core's queue.  Four slabs per
        // iteration: sc4[mt] holds the scale bytes of the group's four slabs
        // for row tile mt (byte j: slab g + j), refreshed once per group with
        // one aligned 8-byte LDS read (one scale-byte read per row tile and
        // slab measured ~5% slower on the prefill GEMMs).
        using S = MxSched<MT, NTL>;
        uint2 r[MT];
        uint32_t sc4[MT];
        // scale bytes of slabs g .. g+3 of row tile mt (g a multiple of 4)
        auto rd_sc4 = [&](int mt, int g) {
            const int pos = mx_soff[mt] + g;
            const uint2 v = *reinterpret_cast<const uint2 *>(mx_sc + (pos & ~3));
            return __builtin_amdgcn_alignbyte(v.y, v.x, (uint32_t)(pos & 3));
        };
        auto sbits = [&](int mt, int j) { return ((sc4[mt] >> (8 * j)) & 0xffu) << 23; };
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            r[mt] = make_uint2(a0[mt][0], a0[mt][1]);
            sc4[mt] = rd_sc4(mt, 0);
        }
        if constexpr (NTL > 0) mx_cvt_bits(a0[0], r[0], sbits(0, 0));
        // issued load d of a K slab: weight-side d < MX_REAL, then the token side
        auto jd = [](int d) { return d < MX_REAL ? d : d - MX_REAL + LPW_A; };
        // One k-step of slab g + J on B fragments bc, reading the next k-step
        // (codes and B fragments bn, at ks / slab) from stage `src`.  Its
        // fragments convert with scale byte J, the next k-step's row tile 0
        // with byte JN; SECOND: also the slab copies of slab kfill into
        // `fill`, and with REFRESH the scale bytes of the next group (slab
        // `slab`), each read after this k-step's last use of the old ones.
        auto kstep = [&](auto second, auto refresh, int J, int JN, const u32x4 *bc, u32x4 *bn,
                         const unsigned char *src, int ks, int slab, lds_t *fill, int kfill) {
            constexpr bool SECOND = decltype(second)::value, REFRESH = decltype(refresh)::value;
            static_for<NMM>([&](auto i) {
                constexpr int I = decltype(i)::value, mt = I / NTL, nt = I % NTL;
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0[mt]), as_bf16x8(bc[nt]),
                                                                      acc[mt][nt], 0, 0, 0);
                if constexpr (nt == 0 && mt + 1 < MT) mx_cvt_bits(a0[mt + 1], r[mt + 1], sbits(mt + 1, J));
                if constexpr (I == S::CV0) mx_cvt_bits(a0[0], r[0], sbits(0, JN));
                static_for<MT>([&](auto m) {
                    constexpr int M = decltype(m)::value;
                    if constexpr (S::ra(M) == I) {
                        r[M] = *reinterpret_cast<const uint2 *>(src + ((a_row0 + M * 32) >> 5) * 1024 + ks * 512 +
                                                                l32 * 16 + lh * 8);
                        if constexpr (REFRESH) sc4[M] = rd_sc4(M, slab);
                    }
                });
                static_for<NTL>([&](auto n) {
                    constexpr int N_ = decltype(n)::value;
                    if constexpr (S::rb(N_) == I)
                        bn[N_] = *reinterpret_cast<const u32x4 *>(src + lds_off<B_PACKED>(b_row0 + N_ * 64, ks * 2 + lh));
                });
                if constexpr (SECOND) {
                    static_for<LPW_K>([&](auto d) {
                        if constexpr (S::dstep(decltype(d)::value) == I) dma(ksrc(jd(decltype(d)::value), kfill), fill, jd(decltype(d)::value));
                    });
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (SECOND) {
                static_for<LPW_K>([&](auto d) {
                    if constexpr (S::dstep(decltype(d)::value) < 0) dma(ksrc(jd(decltype(d)::value), kfill), fill, jd(decltype(d)::value));
                });
            }
        };
        for (; kt + 3 + kStages - 1 < nk_full; kt += 4) {
            static_for<4>([&](auto jj) {
                constexpr int J = decltype(jj)::value;
                const int sl = kt + J;
                const unsigned char *cur = lds + (sl % kStages) * STAGE_BYTES;
                const unsigned char *nxt = lds + ((sl + 1) % kStages) * STAGE_BYTES;
                lds_t *fill = lds_base + ((sl + kStages - 1) % kStages) * STAGE_BYTES;
                kstep(std::false_type{}, std::false_type{}, J, J, b0, b1, cur, 1, sl, fill, 0);
                wait_vm_barrier<(kStages - 3) * LPW_K>();
                __builtin_amdgcn_sched_barrier(0);
                kstep(std::true_type{}, std::integral_constant<bool, J == 3>{}, J, (J + 1) & 3, b1, b0, nxt, 0, sl + 1,
                      fill, sl + kStages - 1);
            });
        }
        // The last (at most 3) slabs of the steady state, one per iteration:
        // sc4 already holds their scale bytes (group g), picked at run time.
        const int g = kt;
        for (; kt + kStages - 1 < nk_full; ++kt) {
            const unsigned char *cur = lds + (kt % kStages) * STAGE_BYTES;
            const unsigned char *nxt = lds + ((kt + 1) % kStages) * STAGE_BYTES;
            lds_t *fill = lds_base + ((kt + kStages - 1) % kStages) * STAGE_BYTES;
            const int j = kt - g;
            kstep(std::false_type{}, std::false_type{}, j, j, b0, b1, cur, 1, kt, fill, 0);
            wait_vm_barrier<(kStages - 3) * LPW_K>();
            __builtin_amdgcn_sched_barrier(0);
            kstep(std::true_type{}, std::false_type{}, j, j + 1, b1, b0, nxt, 0, kt + 1, fill, kt + kStages - 1);
        }
        // the drain converts slab kt's codes with its scale byte kt - g
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) mx_scl[mt] = (sc4[mt] >> (8 * (kt - g))) & 0xffu;
        // the drain reads a K slab's codes from dwords 0, 1 of its fragments
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            a0[mt][0] = r[mt].x;
            a0[mt][1] = r[mt].y;
        }
        }
        // The rest: the drain of the ring.
        for (; kt < nk; ++kt) {
            const int live = (1 << NTL) - 1;
            // MX: both fragment sets of a K slab convert with its scale, a0's
            // and a1's before the reads of the next slab replace it
            rd(ntl, a1, b1, kt % kStages, 1, kt);
            mm_live(ntl, a0, b0, live, true);
            if constexpr (MX) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) mx_cvt(a1[mt], mt);
            }
            if (kt + 1 < nk) {
                // issued so far: slabs 0 .. min(kt + kStages - 2, nk - 1)
                wait_slab(min(kStages - 3, nk - 2 - kt));
                if (kt + kStages - 1 < nk) issue(kt + kStages - 1);
                rd(ntl, a0, b0, (kt + 1) % kStages, 0, kt + 1);
            }
            mm_live(ntl, a1, b1, live, false);
        }
        if (p.lora && n_adapters > 0) lora_phase(ntl);
    };
    switch (nt_live) {
        case 0: mainloop(std::integral_constant<int, 0>{}); break;
        case 1: mainloop(std::integral_constant<int, (NT >= 1 ? 1 : NT)>{}); break;
        case 2: mainloop(std::integral_constant<int, (NT >= 2 ? 2 : NT)>{}); break;
        case 3: mainloop(std::integral_constant<int, (NT >= 3 ? 3 : NT)>{}); break;
        default: mainloop(std::integral_constant<int, NT>{}); break;
    }

    // ---- epilogue --------------------------------------------------------
    if constexpr (GU) {
        // h = silu(gate) * up in bf16, into the packed layout.  Lane (l32, lh)
        // holds, for tile column (token) nt*32 + l32, the gate/up pairs of
        // features fb + mt*16 + g4*4 + {0, 1} with fb = i0 + wm*64 + lh*2, so
        // packed_off splits into a per-token part and a constant per (mt, g4).
        const int64_t nslab_out = (N + kSlabK - 1) / kSlabK;
        const int flim = (int)(nslab_out * kSlabK);  // features the packed h holds
        const int fb = i0 + wm * (BW / 4) + lh * 2;
        uint16_t *hbase = reinterpret_cast<uint16_t *>(p.out) + packed_off(0, fb, nslab_out);
        // Tiles wholly inside N (all but the last weight tile) store without
        // feature checks; the check is a template flag so that neither form
        // branches per element.
        auto emit = [&](auto checked) {
            constexpr bool CHK = decltype(checked)::value;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if (nt >= nt_live) break;
                const int j_tok = (2 * nt + wn) * 32 + l32;  // < nrows: nrows is a multiple of 32
                const int prow = row0 + j_tok;
                const bool valid = tok_f[j_tok] < p.P;
                uint16_t *hrow = hbase + (int64_t)(prow >> 4) * nslab_out * kBlockElems + (prow & 15) * 8;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int feat = fb + mt * 16 + g4 * 4;
                        const float g0 = acc[mt][nt][4 * g4 + 0], g1 = acc[mt][nt][4 * g4 + 1];
                        const float u0 = acc[mt][nt][4 * g4 + 2], u1 = acc[mt][nt][4 * g4 + 3];
                        const uint32_t hv = pack_bf16x2(silu(g0) * u0, silu(g1) * u1);
                        // padding rows and features past N stay zero
                        const uint32_t v = (valid && (!CHK || feat < N)) ? hv : 0u;
                        // feature offset fb + mt*16 + g4*4 relative to fb: slab mt/2,
                        // 8-column chunk 2*(mt%2) + g4/2, column 4*(g4%2)
                        const int koff = (mt >> 1) * kBlockElems + (2 * (mt & 1) + (g4 >> 1)) * 128 + (g4 & 1) * 4;
                        if (!CHK || feat < flim) *reinterpret_cast<uint32_t *>(hrow + koff) = v;
                    }
                }
            }
        };
        if (i0 + BW / 2 <= N) emit(std::false_type{});
        else emit(std::true_type{});
    } else {
        // y2 rows in bf16, staged through LDS so that every store writes
        // whole 256-byte row segments.  The ring is free once every wave is
        // past its last fragment read (no slab copy is in flight by then).
        // Wave w stages one 32-token column tile at a time, 32 rows x (BW/2)
        // values with rows padded by 16 bytes against bank conflicts.
        __syncthreads();
        constexpr int ROWF = BW / 2;                  // values of a staged row
        constexpr int RSTR = ROWF * 2 + 16;           // bytes between staged rows
        static_assert(4 * 32 * RSTR <= kStages * STAGE_BYTES, "epilogue staging must fit the ring");
        unsigned char *stg = lds + w * 32 * RSTR;
        const int fw = i0 + wm * ROWF;                // first feature of this wave
        uint16_t *y2 = reinterpret_cast<uint16_t *>(p.out);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (nt >= nt_live) break;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const uint2 v = make_uint2(pack_bf16x2(acc[mt][nt][4 * g4 + 0], acc[mt][nt][4 * g4 + 1]),
                                               pack_bf16x2(acc[mt][nt][4 * g4 + 2], acc[mt][nt][4 * g4 + 3]));
                    *reinterpret_cast<uint2 *>(stg + l32 * RSTR + (mt * 32 + g4 * 8 + lh * 4) * 2) = v;
                }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // lane (h, c): token 4*it + h of the column tile, values 8c .. 8c+7
            const int c = lane & 15, h = lane >> 4;
            const int feat = fw + c * 8;
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int t = 4 * it + h;
                const int j_tok = (2 * nt + wn) * 32 + t;
                if (c * 8 < ROWF) {
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + t * RSTR + c * 16);
                    const int f = j_tok < nrows ? tok_f[j_tok] : p.P;
                    if (f < p.P && feat < N) *reinterpret_cast<u32x4 *>(y2 + (int64_t)f * N + feat) = v;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
}

}  // namespace moelora
