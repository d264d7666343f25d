// Expert/adapter alignment of the (token, slot) pairs.
//
// The grouped GEMMs need the pairs of each expert contiguous and padded to
// the expert block size; the alignment expert count is the number of
// stacked w13 rows, shared experts included (secrett2633 analysis of vLLM
// PR 46545, "code analysis" part 2).  The LoRA shrink/expand needs, in
// addition, the pairs of one (adapter, expert) bin contiguous (aitrends.kr
// summary of the AWS multi-LoRA MoE post, "section details": expert routing
// and adapter choice are two sparsities at once).  Both come out of one
// layout: pairs sorted by (expert, adapter+1, pair index), padded per expert.
//
// Layout produced (the contract with the GEMM and shrink kernels):
//   sorted_ids[cap]         pair index f, or the sentinel P in the padding
//   sorted_adapter[cap]     optional: adapter of each sorted row, -1 for
//                           no LoRA and in the padding
//   block_expert[maxb]      expert of each block of bm rows, -1 after the end
//   *npp_out                padded row count (num_post_pad)
//   *nitems_out             LoRA work item count
//   items[max_items][4]     (start row, rows <= lbm, adapter, expert)
//   tiles[][4]              optional token tiles for the LDS-tiled GEMM: each
//                           expert's padded rows cut into ceil(rows/tile_rows)
//                           runs of equal length (to 32 rows): (start row, rows | tiles of the
//                           expert << 16, expert, first tile of the expert),
//                           with the tile count, the most tiles of one expert
//                           and the number of experts with tiles
//
// Implementation (below 8192 pairs; the multi-workgroup form for more pairs
// is described further down): one workgroup of NW wavefronts, no host
// synchronisation and no atomics on anything but LDS integer counters.  A
// stable sort by a
// composite key is done as two stable counting passes (least significant
// key first): by adapter+1, then by expert.  Each pass gives every wave a
// contiguous segment of the input; a wave walks its segment 64 pairs at a
// time in order, finds equal keys inside the wave with bit-sliced ballots,
// and keeps one running cursor per key in LDS.  Per-wave histograms plus a
// scan over (key, wave) make every position depend only on the input, so the
// result is deterministic and stable.  When the pairs fit, the per-pair
// expert and adapter keys and the intermediate order live in LDS as 16-bit
// values (one bulk load instead of four passes of dependent global loads).
#pragma once

#include "common.hpp"
#include "route.hpp"

namespace moelora {

// Fixed part of a tiled-GEMM work item's estimated cost, in units of one
// 32-row column tile's MFMA work (see align_finish).
constexpr int kTileCostFixed = 5;

struct AlignParams {
    const int32_t *topk_ids;
    const int32_t *adapter_ids;
    int32_t *sorted_ids;
    int32_t *sorted_adapter;  // optional [cap]
    int32_t *block_expert;
    int32_t *npp_out;
    int32_t *npp_copy = nullptr;  // optional second copy of the padded row count (a caller's buffer)
    int32_t *nitems_out;
    int32_t *items;
    int32_t *tmp;         // [P] global scratch (used when the keys do not fit in LDS)
    int32_t *tiles;       // optional GEMM token tiles [max_tiles][4]
    // with tiles: per tiled GEMM g (0 = gate_up, 1 = down) the XCD ranges of
    // its work items, xsplit[16 g + x] for x = 0..8 (see align_finish)
    int32_t *xsplit = nullptr;
    int nwt[2] = {0, 0};   // weight tiles of each GEMM
    int xcap[2] = {0, 0};  // most items one XCD may take (its share of the grid)
    int cus = 256;         // compute units of the device
    int32_t *ntiles_out;  // [3]: tile count, most tiles of one expert, experts with tiles
    int T, P, Kp, Ep, La, bm, lbm;
    int cap, max_blocks, max_items;
    int tile_rows;
    int nbits_a, nbits_e;
    int lds_keys;         // 1: stage keys and the intermediate order in LDS
    // multi-workgroup alignment (align_hist / align_scan / align_scatter)
    int32_t *hist;        // [nb][NK] per-(block, key) counts, then prefixes
    int32_t *ktot;        // [NK] pairs per key, then the key's first position
    int nb, chunk;        // blocks and pairs per block
    int nbits_k;          // bits of a composite key
};

// Ids outside their documented ranges (a precondition) are clamped so that
// they can never index memory out of bounds: an adapter outside [-1, La)
// counts as "no LoRA", an expert outside [0, Ep) as the nearest valid one.
__device__ __forceinline__ int adapter_key_of(int a, int La) { return (a >= 0 && a < La) ? a + 1 : 0; }
__device__ __forceinline__ int clamp_expert(int e, int Ep) { return min(max(e, 0), Ep - 1); }

// ints of LDS before the staged keys (histograms, offsets, scan scratch, LoRA counts)
__host__ __device__ inline int64_t align_lds_fixed_ints(int NW, int Ep, int La) {
    const int64_t nk = (int64_t)Ep * (La + 1);
    const int64_t tk = (Ep > La + 1 ? Ep : La + 1) + 1;
    int64_t n = (int64_t)NW * (La + 1) + (int64_t)NW * Ep + 2 * (int64_t)Ep + 1 + tk + 80 + (Ep + 1);
    if (La > 0) n += 2 * nk + 1;
    return n;
}

// LDS ints of the alignment; with lds_keys the 16-bit keys follow:
// expert of each pair [P], order after the adapter pass [P], adapter+1 of
// each token [T].
__host__ __device__ inline int64_t align_lds_ints(int NW, int Ep, int La, int64_t T, int64_t P, bool lds_keys) {
    int64_t n = align_lds_fixed_ints(NW, Ep, La);
    if (lds_keys) n += (2 * P + T + 1) / 2 + 1;
    return n;
}

// In-place exclusive scan of arr[0, n) in LDS by the whole workgroup.
// Returns the total to every thread.  scr holds >= 17 ints.
// Inclusive prefix sum over the 64 lanes (all active), by DPP: shifts by
// 1, 2, 4, 8 lanes inside each row of 16, then rows 1 and 3 add the last
// lane of the row before them and rows 2 and 3 add lane 31.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += dpp_int<0x111, 0xf>(x, 0);  // row_shr:1
    x += dpp_int<0x112, 0xf>(x, 0);  // row_shr:2
    x += dpp_int<0x114, 0xf>(x, 0);  // row_shr:4
    x += dpp_int<0x118, 0xf>(x, 0);  // row_shr:8
    x += dpp_int<0x142, 0xa>(x, 0);  // row_bcast15 into rows 1, 3
    x += dpp_int<0x143, 0xc>(x, 0);  // row_bcast31 into rows 2, 3
    return x;
}

__device__ inline int block_excl_scan(int *arr, int n, int *scr) {
    const int nt = (int)blockDim.x, tid = (int)threadIdx.x;
    const int nw = nt >> 6, lane = tid & 63, w = tid >> 6;
    const int per = (n + nt - 1) / nt;
    const int b = tid * per;
    const int e = min(n, b + per);
    int local = 0;
    for (int i = b; i < e; ++i) local += arr[i];
    const int x = wave_incl_scan(local);
    if (lane == 63) scr[w] = x;
    __syncthreads();
    if (w == 0) {
        // the wave totals (at most 16) scanned by wave 0
        const int t = lane < nw ? scr[lane] : 0;
        const int y = wave_incl_scan(t);
        if (lane < nw) scr[lane] = y - t;
        if (lane == nw - 1) scr[nw] = y;
    }
    __syncthreads();
    int run = scr[w] + x - local;
    const int total = scr[nw];
    for (int i = b; i < e; ++i) {
        const int t = arr[i];
        arr[i] = run;
        run += t;
    }
    __syncthreads();
    return total;
}

// Where the staged 16-bit keys start inside the alignment's LDS.
__device__ __forceinline__ uint16_t *align_keys(int *lds, int NW, int Ep, int La) {
    return reinterpret_cast<uint16_t *>(lds + align_lds_fixed_ints(NW, Ep, La));
}

// Everything after the scatter: padding rows, the tail, the block -> expert
// map, the GEMM token tiles, the LoRA items and the counts.  Needs offE[Ep+1]
// and totE[Ep] (expert offsets and pair counts) and, with LoRA, cnt2[NK]
// (pairs per (expert, adapter+1) key, overwritten here with each key's first
// row) in LDS; tk, scr and itemOff are LDS scratch.  Run by one whole
// workgroup.
__device__ void align_finish(const AlignParams &p, const int *offE, const int *totE, int *tk, int *scr,
                             int *cnt2, int *itemOff, int npp, int *cst) {
    const int NW = (int)(blockDim.x >> 6);
    const int tid = (int)threadIdx.x, nt = (int)blockDim.x;
    const int lane = tid & 63, w = tid >> 6;
    const int La = p.La, Ep = p.Ep, A1 = La + 1;
    const int NK = Ep * A1;
    const int P = p.P;
    // ---- padding, tail and block -> expert map ---------------------------
    for (int e = w; e < Ep; e += NW) {
        const int b = offE[e] + totE[e], end = offE[e + 1];
        for (int q = b + lane; q < end; q += 64) {
            p.sorted_ids[q] = P;
            if (p.sorted_adapter) p.sorted_adapter[q] = -1;
        }
    }
    for (int q = npp + tid; q < p.cap; q += nt) {
        p.sorted_ids[q] = P;
        if (p.sorted_adapter) p.sorted_adapter[q] = -1;
    }
    for (int b = tid; b < p.max_blocks; b += nt) {
        const int pos = b * p.bm;
        int ex = -1;
        if (pos < npp) {
            int lo = 0, hi = Ep - 1;  // last e with offE[e] <= pos
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (offE[mid] <= pos) lo = mid;
                else hi = mid - 1;
            }
            ex = lo;
        }
        p.block_expert[b] = ex;
    }

    // ---- token tiles of the LDS-tiled GEMM ---------------------------------
    // Besides the tiles: the largest tile count of one expert and the number
    // of experts with tiles, from which the GEMM decides whether the load is skewed.
    if (p.tiles != nullptr) {
        __syncthreads();
        if (tid == 0) {
            scr[20] = 0;
            scr[21] = 0;
        }
        // an expert's padded rows in ceil(rows / tile_rows) tiles of equal size
        // (rounded up to 32 rows; the last one takes what is left)
        auto tile_len = [&](int pad) {
            const int n = (pad + p.tile_rows - 1) / p.tile_rows;
            return n == 0 ? 0 : ((pad + n - 1) / n + 31) / 32 * 32;
        };
        for (int e = tid; e < Ep; e += nt) {
            const int pad = offE[e + 1] - offE[e], len = tile_len(pad);
            tk[e] = len == 0 ? 0 : (pad + len - 1) / len;
        }
        __syncthreads();
        for (int e = tid; e < Ep; e += nt) {
            atomicMax(&scr[20], tk[e]);
            if (tk[e] > 0) atomicAdd(&scr[21], 1);
        }
        const int ntiles = block_excl_scan(tk, Ep, scr);
        for (int e = tid; e < Ep; e += nt) {
            const int pad = offE[e + 1] - offE[e], len = tile_len(pad);
            int it = tk[e];
            const int t0 = it, nt_e = len == 0 ? 0 : (pad + len - 1) / len;
            for (int q = 0; q < pad; q += len) {
                int4 v;
                v.x = offE[e] + q;
                v.y = min(len, pad - q) | (nt_e << 16);
                v.z = e;
                v.w = t0;
                reinterpret_cast<int4 *>(p.tiles)[it++] = v;
            }
        }
        __syncthreads();
        if (tid == 0) {
            p.ntiles_out[0] = ntiles;
            p.ntiles_out[1] = scr[20];
            p.ntiles_out[2] = scr[21];
        }
        // XCD ranges of the tiled GEMMs' work.  The GEMM's logical order is
        // expert-major (expert, weight tile, token tile), and each XCD takes
        // one contiguous range of it.  The ranges are cut at equal estimated
        // cost rather than equal item count: an item's cost is taken as
        // kTileCostFixed + its 32-row column tiles (the weight slabs stream
        // through the CU whatever the token count; the MFMA work grows with
        // it), which follows the measured per-tile K-loop times of the
        // GPT-OSS prefill (tiles of 192 and 256 rows) closely.  With fewer
        // than 6 items per CU the rounding of each XCD's items to whole rounds
        // of its CUs outweighs their cost differences, and the ranges hold
        // equal item counts instead (measured on the GPT-OSS prefill: down,
        // 3.8 items per CU, 308 us with equal counts against 322 us by cost;
        // gate_up, 7.4 per CU, 587 against 541 us).  cst[Ep+1] is LDS
        // scratch for the per-expert cost prefix.
        if (p.xsplit != nullptr) {
            for (int e = tid; e < Ep; e += nt) {
                const int pad = offE[e + 1] - offE[e], len = tile_len(pad);
                const int nt_e = len == 0 ? 0 : (pad + len - 1) / len;
                cst[e] = nt_e == 0 ? 0
                                   : (nt_e - 1) * (kTileCostFixed + len / 32) +
                                         (kTileCostFixed + (pad - (nt_e - 1) * len) / 32);
            }
            __syncthreads();
            const int totc = block_excl_scan(cst, Ep, scr);
            if (tid < 16) {
                const int g = tid >> 3, x = tid & 7;
                const int64_t nwt = p.nwt[g];
                int item = 0;
                if (x > 0 && totc > 0) {
                    const int64_t target = (int64_t)x * nwt * totc / 8;
                    int lo = 0, hi = Ep - 1;  // last e with nwt * cst[e] <= target
                    while (lo < hi) {
                        const int mid = (lo + hi + 1) >> 1;
                        if (nwt * cst[mid] <= target) lo = mid;
                        else hi = mid - 1;
                    }
                    const int e = lo;
                    const int se = (e + 1 < Ep ? cst[e + 1] : totc) - cst[e];
                    const int pad = offE[e + 1] - offE[e], len = tile_len(pad);
                    const int nt_e = len == 0 ? 0 : (pad + len - 1) / len;
                    if (se > 0 && nt_e > 0) {
                        const int64_t r = target - nwt * cst[e];
                        const int64_t wt = min<int64_t>(r / se, nwt - 1);
                        const int64_t rr = r - wt * se;
                        const int tt = (int)min<int64_t>(rr / (kTileCostFixed + len / 32), nt_e - 1);
                        item = (int)(nwt * tk[e] + wt * nt_e + tt);
                    } else {
                        item = (int)(nwt * tk[e]);
                    }
                }
                const int live = p.nwt[g] * ntiles;
                if (live < 6 * p.cus) {
                    const int q = live / 8, rem = live % 8;
                    item = x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q;
                }
                scr[24 + tid] = item;
            }
            __syncthreads();
            if (tid < 2) {
                // monotone, every range within the XCD's share of the grid
                const int g = tid, cap = p.xcap[g];
                const int live = p.nwt[g] * ntiles;
                int prev = 0;
                p.xsplit[16 * g] = 0;
                for (int x = 1; x < 8; ++x) {
                    int v = scr[24 + 8 * g + x];
                    v = max(v, prev);
                    v = min(v, prev + cap);
                    v = max(v, live - (8 - x) * cap);
                    v = min(v, live);
                    p.xsplit[16 * g + x] = v;
                    prev = v;
                }
                p.xsplit[16 * g + 8] = live;
            }
        }
    }

    // ---- LoRA work items: (adapter >= 0, expert) runs cut to lbm rows ------
    int nitems = 0;
    if (La > 0 && p.items != nullptr) {
        for (int k = tid; k < NK; k += nt) {
            const int a1 = k % A1;
            itemOff[k] = (a1 == 0) ? 0 : (cnt2[k] + p.lbm - 1) / p.lbm;
        }
        __syncthreads();
        nitems = block_excl_scan(itemOff, NK, scr);
        // the key counts become each key's first row: its expert's offset
        // plus the counts of the expert's earlier keys
        for (int e = tid; e < Ep; e += nt) {
            int run = offE[e];
            for (int a1 = 0; a1 < A1; ++a1) {
                const int c = cnt2[e * A1 + a1];
                cnt2[e * A1 + a1] = run;
                run += c;
            }
        }
        __syncthreads();
        // item i belongs to the last key k with itemOff[k] <= i (keys
        // without items share the offset of the key after them)
        for (int i = tid; i < nitems; i += nt) {
            int lo = 0, hi = NK - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (itemOff[mid] <= i) lo = mid;
                else hi = mid - 1;
            }
            const int k = lo, e = k / A1, a1 = k - e * A1;
            const int first = cnt2[k];
            const int c = (a1 + 1 < A1 ? cnt2[k + 1] : offE[e] + totE[e]) - first;
            const int q = (i - itemOff[k]) * p.lbm;
            int4 v;
            v.x = first + q;
            v.y = min(p.lbm, c - q);
            v.z = a1 - 1;
            v.w = e;
            reinterpret_cast<int4 *>(p.items)[i] = v;
        }
        for (int q = nitems + tid; q < p.max_items; q += nt) {
            int4 v;
            v.x = 0;
            v.y = 0;
            v.z = -1;
            v.w = -1;
            reinterpret_cast<int4 *>(p.items)[q] = v;
        }
    }
    if (tid == 0) {
        *p.npp_out = npp;
        if (p.npp_copy) *p.npp_copy = npp;
        *p.nitems_out = nitems;
    }
}

// The alignment proper, run by one whole workgroup.  With p.lds_keys the
// keys are bulk-loaded into LDS first.
__device__ void align_body(const AlignParams &p, int *lds) {
    const int NW = (int)(blockDim.x >> 6);
    const int tid = (int)threadIdx.x, nt = (int)blockDim.x;
    const int lane = tid & 63, w = tid >> 6;
    const int La = p.La, Ep = p.Ep, A1 = La + 1;
    const int NK = Ep * A1;
    const int TK = (Ep > A1 ? Ep : A1) + 1;
    const int P = p.P;
    const bool lk = p.lds_keys != 0;

    int *histA = lds;                    // [NW][A1]
    int *histB = histA + NW * A1;        // [NW][Ep]
    int *offE = histB + NW * Ep;         // [Ep+1]
    int *totE = offE + Ep + 1;           // [Ep]
    int *tk = totE + Ep;                 // [TK]
    int *scr = tk + TK;                  // [80]
    int *cst = scr + 80;                 // [Ep+1]    tile cost prefix (align_finish)
    int *cnt2 = cst + Ep + 1;            // [NK]      (La > 0)
    int *itemOff = cnt2 + NK;            // [NK+1]    (La > 0)
    uint16_t *eL = align_keys(lds, NW, Ep, La);  // [P] expert of pair f
    uint16_t *oL = eL + P;                       // [P] order after the adapter pass
    uint16_t *aL = oL + P;                       // [T] adapter+1 of token t

    if (lk) {
        for (int f = tid; f < P; f += nt) eL[f] = (uint16_t)clamp_expert(p.topk_ids[f], Ep);
        for (int t = tid; t < p.T; t += nt) aL[t] = (uint16_t)(La > 0 ? adapter_key_of(p.adapter_ids[t], La) : 0);
    }
    auto get_e = [&](int f) -> int { return lk ? (int)eL[f] : clamp_expert(p.topk_ids[f], Ep); };
    auto get_a1 = [&](int f) -> int {
        return lk ? (int)aL[f / p.Kp] : adapter_key_of(p.adapter_ids[f / p.Kp], La);
    };
    auto get_order = [&](int i) -> int { return La > 0 ? (lk ? (int)oL[i] : p.tmp[i]) : i; };

    const int nzero = NW * A1 + NW * Ep + (La > 0 ? NK : 0);
    for (int i = tid; i < nzero; i += nt) {
        if (i < NW * A1 + NW * Ep) lds[i] = 0;
        else cnt2[i - NW * A1 - NW * Ep] = 0;
    }
    __syncthreads();

    const int seg = (P + NW - 1) / NW;
    const int s0 = min(P, w * seg), s1 = min(P, s0 + seg);

    // ---- pass A: stable counting sort by adapter+1 ------------------------
    if (La > 0) {
        for (int base = s0; base < s1; base += 64) {
            const int f = base + lane;
            const bool valid = f < s1;
            const int a1 = valid ? get_a1(f) : 0;
            const uint64_t m = match_key((uint32_t)a1, valid, p.nbits_a);
            if (valid) {
                if ((m & lanemask_lt()) == 0) histA[w * A1 + a1] += __popcll(m);
                atomicAdd(&cnt2[get_e(f) * A1 + a1], 1);
            }
        }
        __syncthreads();
        for (int a = tid; a < A1; a += nt) {
            int run = 0;
            for (int v = 0; v < NW; ++v) {
                const int c = histA[v * A1 + a];
                histA[v * A1 + a] = run;
                run += c;
            }
            tk[a] = run;
        }
        __syncthreads();
        block_excl_scan(tk, A1, scr);
        for (int i = tid; i < NW * A1; i += nt) histA[i] += tk[i % A1];
        __syncthreads();
        for (int base = s0; base < s1; base += 64) {
            const int f = base + lane;
            const bool valid = f < s1;
            const int a1 = valid ? get_a1(f) : 0;
            const uint64_t m = match_key((uint32_t)a1, valid, p.nbits_a);
            if (valid) {
                const int pos = histA[w * A1 + a1] + __popcll(m & lanemask_lt());
                if (lk) oL[pos] = (uint16_t)f;
                else p.tmp[pos] = f;
                if ((m & lanemask_lt()) == 0) histA[w * A1 + a1] += __popcll(m);
            }
        }
        __threadfence_block();
        __syncthreads();
    }

    // ---- pass B: stable counting sort by expert, padded per expert --------
    for (int base = s0; base < s1; base += 64) {
        const int i = base + lane;
        const bool valid = i < s1;
        const int f = valid ? get_order(i) : 0;
        const int e = valid ? get_e(f) : 0;
        const uint64_t m = match_key((uint32_t)e, valid, p.nbits_e);
        if (valid && (m & lanemask_lt()) == 0) histB[w * Ep + e] += __popcll(m);
    }
    __syncthreads();
    for (int e = tid; e < Ep; e += nt) {
        int run = 0;
        for (int v = 0; v < NW; ++v) {
            const int c = histB[v * Ep + e];
            histB[v * Ep + e] = run;
            run += c;
        }
        totE[e] = run;
        tk[e] = (run + p.bm - 1) / p.bm * p.bm;
    }
    __syncthreads();
    const int npp = block_excl_scan(tk, Ep, scr);
    for (int e = tid; e < Ep; e += nt) offE[e] = tk[e];
    if (tid == 0) offE[Ep] = npp;
    __syncthreads();
    for (int i = tid; i < NW * Ep; i += nt) histB[i] += offE[i % Ep];
    __syncthreads();
    for (int base = s0; base < s1; base += 64) {
        const int i = base + lane;
        const bool valid = i < s1;
        const int f = valid ? get_order(i) : 0;
        const int e = valid ? get_e(f) : 0;
        const uint64_t m = match_key((uint32_t)e, valid, p.nbits_e);
        if (valid) {
            const int pos = histB[w * Ep + e] + __popcll(m & lanemask_lt());
            p.sorted_ids[pos] = f;
            if (p.sorted_adapter) p.sorted_adapter[pos] = get_a1(f) - 1;
            if ((m & lanemask_lt()) == 0) histB[w * Ep + e] += __popcll(m);
        }
    }

    align_finish(p, offE, totE, tk, scr, cnt2, itemOff, npp, cst);
}

// ---- multi-workgroup alignment -------------------------------------------
// For many pairs one workgroup is latency bound, so the same stable sort by
// the composite key (expert, adapter+1) runs in four launches:
//   hist     nb blocks count the keys of their contiguous slices of pairs
//            (slice b = pairs [b*chunk, (b+1)*chunk)) into hist[b][key];
//   colscan  per key, an exclusive prefix over the blocks (in place) and the
//            key's total into ktot[key];
//   scan     one workgroup turns the totals into expert offsets, writes the
//            first position of each key back into ktot and builds the
//            padding, block map, tiles and items as the one-workgroup path;
//   scatter  nb blocks place their slices in pair order, one wave each.
// Every position depends only on the input, and the output is bitwise that
// of the one-workgroup path.
__device__ __forceinline__ int align_key_of(const AlignParams &p, int f) {
    const int e = clamp_expert(p.topk_ids[f], p.Ep);
    const int a1 = p.La > 0 ? adapter_key_of(p.adapter_ids[f / p.Kp], p.La) : 0;
    return e * (p.La + 1) + a1;
}

// grid nb, block 256, LDS NK ints
__global__ __launch_bounds__(256) void align_hist_kernel(AlignParams p) {
    extern __shared__ int cnt[];
    const int NK = p.Ep * (p.La + 1);
    const int tid = (int)threadIdx.x;
    for (int k = tid; k < NK; k += 256) cnt[k] = 0;
    __syncthreads();
    const int f0 = blockIdx.x * p.chunk, f1 = min(p.P, f0 + p.chunk);
    for (int f = f0 + tid; f < f1; f += 256) atomicAdd(&cnt[align_key_of(p, f)], 1);
    __syncthreads();
    int32_t *row = p.hist + (int64_t)blockIdx.x * NK;
    for (int k = tid; k < NK; k += 256) row[k] = cnt[k];
}

// grid ceil(NK/256), block 256: thread k scans column k of hist
__global__ __launch_bounds__(256) void align_colscan_kernel(AlignParams p) {
    const int NK = p.Ep * (p.La + 1);
    const int k = blockIdx.x * 256 + (int)threadIdx.x;
    if (k >= NK) return;
    int run = 0;
    int b = 0;
    for (; b + 8 <= p.nb; b += 8) {
        int c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = p.hist[(int64_t)(b + u) * NK + k];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            p.hist[(int64_t)(b + u) * NK + k] = run;
            run += c[u];
        }
    }
    for (; b < p.nb; ++b) {
        const int c = p.hist[(int64_t)b * NK + k];
        p.hist[(int64_t)b * NK + k] = run;
        run += c;
    }
    p.ktot[k] = run;
}

// ints of LDS the scan workgroup needs
__host__ __device__ inline int64_t align_scan_lds_ints(int Ep, int La) {
    const int64_t nk = (int64_t)Ep * (La + 1);
    const int64_t tk = (Ep > La + 1 ? Ep : La + 1) + 1;
    return 2 * nk + 1 + 2 * (int64_t)Ep + 1 + tk + 80 + (Ep + 1);
}

// one workgroup
__global__ __launch_bounds__(1024) void align_scan_kernel(AlignParams p) {
    extern __shared__ int lds[];
    const int tid = (int)threadIdx.x, nt = (int)blockDim.x;
    const int La = p.La, Ep = p.Ep, A1 = La + 1;
    const int NK = Ep * A1;
    const int TK = (Ep > A1 ? Ep : A1) + 1;
    int *cnt2 = lds;                 // [NK] pairs per key
    int *itemOff = cnt2 + NK;        // [NK+1] scratch of align_finish
    int *offE = itemOff + NK + 1;    // [Ep+1]
    int *totE = offE + Ep + 1;       // [Ep]
    int *tk = totE + Ep;             // [TK]
    int *scr = tk + TK;              // [80]
    int *cst = scr + 80;             // [Ep+1] tile cost prefix of align_finish
    for (int k0 = tid; k0 < NK; k0 += 8 * nt) {  // eight loads in flight per thread (clamped: no branches)
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = p.ktot[min(k0 + u * nt, NK - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (k0 + u * nt < NK) cnt2[k0 + u * nt] = v[u];
    }
    __syncthreads();
    for (int e = tid; e < Ep; e += nt) {
        int run = 0;
        for (int a1 = 0; a1 < A1; ++a1) run += cnt2[e * A1 + a1];
        totE[e] = run;
        tk[e] = (run + p.bm - 1) / p.bm * p.bm;
    }
    __syncthreads();
    const int npp = block_excl_scan(tk, Ep, scr);
    for (int e = tid; e < Ep; e += nt) offE[e] = tk[e];
    if (tid == 0) offE[Ep] = npp;
    __syncthreads();
    // first position of each key: its expert's offset plus the keys before it
    for (int e = tid; e < Ep; e += nt) {
        int run = offE[e];
        for (int a1 = 0; a1 < A1; ++a1) {
            p.ktot[e * A1 + a1] = run;
            run += cnt2[e * A1 + a1];
        }
    }
    align_finish(p, offE, totE, tk, scr, cnt2, itemOff, npp, cst);
}

// grid nb, block 256, LDS NK ints: the next position of each key.  All four
// waves load the cursors; wave 0 alone then walks the slice in pair order,
// in windows of kScatterWin pairs per lane whose keys are loaded up front so
// their loads overlap.  Past the one workgroup barrier only wave 0 runs, and
// its LDS accesses execute in program order, so no further barrier is needed.
// The loads are branch-free (clamped addresses, masked values), so each
// batch waits once instead of once per load, and the walk is a rolled loop
// (the window's keys shift through registers) rather than kScatterWin
// unrolled copies.
constexpr int kScatterWin = 16;
__global__ __launch_bounds__(256) void align_scatter_kernel(AlignParams p) {
    extern __shared__ int cur[];
    const int NK = p.Ep * (p.La + 1);
    const int tid = (int)threadIdx.x, lane = lane_id();
    const int32_t *row = p.hist + (int64_t)blockIdx.x * NK;
    for (int k0 = 0; k0 < NK; k0 += 4 * 256) {
        int v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int k = min(k0 + u * 256 + tid, NK - 1);
            v[u] = p.ktot[k] + row[k];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int k = k0 + u * 256 + tid;
            if (k < NK) cur[k] = v[u];
        }
    }
    __syncthreads();
    if (tid >= 64) return;
    const int f0 = blockIdx.x * p.chunk, f1 = min(p.P, f0 + p.chunk);
    for (int w0 = f0; w0 < f1; w0 += 64 * kScatterWin) {
        // the window's expert ids, then its adapter ids, each batch in flight at once
        int key[kScatterWin], av[kScatterWin];
#pragma unroll
        for (int u = 0; u < kScatterWin; ++u) key[u] = p.topk_ids[min(w0 + 64 * u + lane, f1 - 1)];
        if (p.La > 0) {
#pragma unroll
            for (int u = 0; u < kScatterWin; ++u) av[u] = p.adapter_ids[min(w0 + 64 * u + lane, f1 - 1) / p.Kp];
        }
#pragma unroll
        for (int u = 0; u < kScatterWin; ++u) {
            const int k = clamp_expert(key[u], p.Ep) * (p.La + 1) + (p.La > 0 ? adapter_key_of(av[u], p.La) : 0);
            key[u] = w0 + 64 * u + lane < f1 ? k : -1;
        }
#pragma unroll 1
        for (int u = 0; u < kScatterWin; ++u) {
            const int f = w0 + 64 * u + lane;
            if (w0 + 64 * u >= f1) break;  // uniform
            const int ku = key[0];
#pragma unroll
            for (int i = 0; i + 1 < kScatterWin; ++i) key[i] = key[i + 1];
            const bool valid = ku >= 0;
            const uint64_t m = match_key((uint32_t)(valid ? ku : 0), valid, p.nbits_k);
            const uint64_t lt = m & lanemask_lt();
            if (valid) {
                const int pos = cur[ku] + __popcll(lt);
                p.sorted_ids[pos] = f;
                if (p.sorted_adapter) p.sorted_adapter[pos] = ku % (p.La + 1) - 1;
            }
            __builtin_amdgcn_wave_barrier();
            if (valid && lt == 0) cur[ku] += __popcll(m);
            __builtin_amdgcn_wave_barrier();
        }
    }
}

__global__ __launch_bounds__(1024) void align_kernel(AlignParams p) {
    extern __shared__ int lds[];
    align_body(p, lds);
}

// ---- small calls: one pass over the composite key ------------------------
// For at most 1024 pairs and no GEMM token tiles (the streaming GEMM's
// decode-sized calls) one workgroup with one thread per pair sorts by the
// composite key (expert, adapter+1) in a single stable counting pass: the
// pairs of wave w are f = 64w .. 64w+63, equal keys inside a wave are found
// with bit-sliced ballots, and per-(wave, key) counts give each pair its
// place.  Key offsets come from two block scans (over the keys, unpadded,
// and over the experts, padded) instead of the two sorting passes and the
// per-expert loops of the general form, and the padding, block map and LoRA
// items are written by independent threads.  The layout is the same as the
// general form's, bit for bit.
//
// ROUTE: the same workgroup routes the tokens first (wave w routes tokens
// w, w + NW, ...; ids and weights are written out as by the router launch
// and kept in LDS for the sort), one launch instead of two for the small
// calls whose gate_up shrink does not run in the router's launch.
__host__ __device__ inline int64_t align_small_lds_ints(int NW, int Ep, int La, int64_t P) {
    const int64_t NK = (int64_t)Ep * (La + 1);
    return (int64_t)NW * NK + 3 * (NK + 1) + 2 * (int64_t)Ep + 1 + 80 + P;
}

template <bool ROUTE, int VPL>
__global__ __launch_bounds__(1024) void align_small_kernel(AlignParams p, RouteParams rp) {
    extern __shared__ int lds[];
    const int nt = (int)blockDim.x, NW = nt >> 6;
    const int tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int La = p.La, Ep = p.Ep, A1 = La + 1, NK = Ep * A1, P = p.P;
    int *histW = lds;                 // [NW][NK] pairs of wave v with key k, then their prefix over waves
    int *keyX = histW + NW * NK;      // [NK+1] pairs with a smaller key (exclusive scan of keyN)
    int *keyN = keyX + NK + 1;        // [NK+1] pairs per key
    int *itemOff = keyN + NK + 1;     // [NK+1] first LoRA item of each key
    int *offE = itemOff + NK + 1;     // [Ep+1] padded start of each expert
    int *totE = offE + Ep + 1;        // [Ep] pairs per expert
    int *scr = totE + Ep;             // [80] scan scratch
    int *idsL = scr + 80;             // [P] expert of each pair (ROUTE)

    if constexpr (ROUTE) {
        for (int t = w; t < rp.T; t += NW) {
            const int myi = route_one_token<VPL>(rp, t);  // K + S <= 64: every slot is returned
            if (lane < p.Kp) idsL[t * p.Kp + lane] = myi;
        }
    }
    for (int i = tid; i < NW * NK; i += nt) histW[i] = 0;
    const int f = tid;
    const bool valid = f < P;
    if constexpr (ROUTE) __syncthreads();
    int e = 0, a1 = 0;
    if (valid) {
        e = clamp_expert(ROUTE ? idsL[f] : p.topk_ids[f], Ep);
        if (La > 0) a1 = adapter_key_of(p.adapter_ids[f / p.Kp], La);
    }
    const int key = e * A1 + a1;
    __syncthreads();
    const uint64_t m = match_key((uint32_t)key, valid, p.nbits_k);
    const int rank = __popcll(m & lanemask_lt());
    if (valid && rank == 0) histW[w * NK + key] = __popcll(m);
    __syncthreads();
    for (int k = tid; k < NK; k += nt) {
        int run = 0;
        for (int v = 0; v < NW; ++v) {
            const int c = histW[v * NK + k];
            histW[v * NK + k] = run;
            run += c;
        }
        keyN[k] = run;
        keyX[k] = run;
    }
    __syncthreads();
    const int total = block_excl_scan(keyX, NK, scr);
    if (tid == 0) keyX[NK] = total;
    __syncthreads();
    for (int x = tid; x < Ep; x += nt) {
        const int c = keyX[(x + 1) * A1] - keyX[x * A1];
        totE[x] = c;
        offE[x] = (c + p.bm - 1) / p.bm * p.bm;
    }
    __syncthreads();
    const int npp = block_excl_scan(offE, Ep, scr);
    if (tid == 0) offE[Ep] = npp;
    __syncthreads();

    // scatter: expert start + keys of the expert before this one + earlier
    // waves + earlier lanes
    if (valid) {
        const int pos = offE[e] + (keyX[key] - keyX[e * A1]) + histW[w * NK + key] + rank;
        p.sorted_ids[pos] = f;
        if (p.sorted_adapter) p.sorted_adapter[pos] = a1 - 1;
    }
    // the last expert e' with offE[e'] <= pos (empty experts share offsets)
    auto expert_at = [&](int pos) {
        int lo = 0, hi = Ep - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (offE[mid] <= pos) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    };
    // padding rows: each expert's [offE + totE, next offE), then the tail
    for (int x = w; x < Ep; x += NW) {
        for (int q = offE[x] + totE[x] + lane; q < offE[x + 1]; q += 64) {
            p.sorted_ids[q] = P;
            if (p.sorted_adapter) p.sorted_adapter[q] = -1;
        }
    }
    for (int q = npp + tid; q < p.cap; q += nt) {
        p.sorted_ids[q] = P;
        if (p.sorted_adapter) p.sorted_adapter[q] = -1;
    }
    for (int b = tid; b < p.max_blocks; b += nt) {
        const int pos = b * p.bm;
        p.block_expert[b] = pos < npp ? expert_at(pos) : -1;
    }
    int nitems = 0;
    if (La > 0 && p.items != nullptr) {
        for (int k = tid; k < NK; k += nt) itemOff[k] = (k % A1 == 0) ? 0 : (keyN[k] + p.lbm - 1) / p.lbm;
        __syncthreads();
        nitems = block_excl_scan(itemOff, NK, scr);
        for (int k = tid; k < NK; k += nt) {
            const int ka = k % A1, c = keyN[k];
            if (ka == 0 || c == 0) continue;
            const int x = k / A1;
            const int start = offE[x] + (keyX[k] - keyX[x * A1]);
            int it = itemOff[k];
            for (int q = 0; q < c; q += p.lbm) {
                int4 v;
                v.x = start + q;
                v.y = min(p.lbm, c - q);
                v.z = ka - 1;
                v.w = x;
                reinterpret_cast<int4 *>(p.items)[it++] = v;
            }
        }
        for (int q = nitems + tid; q < p.max_items; q += nt) {
            int4 v;
            v.x = 0;
            v.y = 0;
            v.z = -1;
            v.w = -1;
            reinterpret_cast<int4 *>(p.items)[q] = v;
        }
    }
    if (tid == 0) {
        *p.npp_out = npp;
        if (p.npp_copy) *p.npp_copy = npp;
        *p.nitems_out = nitems;
    }
}

// ---- tiny calls: one wavefront ------------------------------------------
// At most 64 pairs and no GEMM token tiles: one wavefront, one lane per pair
// f, no LDS and no barrier.  Each lane reads every other lane's key (v_readlane
// in a 64-step loop) to count the pairs before it in (expert, adapter+1, f)
// order, within its expert and within its key, and the pairs of its expert;
// a second pass adds the padded sizes of the smaller experts (each counted
// once, by its first pair).  The lane then stores its pair; the first pair
// of each expert writes that expert's padding and block map, the first pair
// of each LoRA key its items.  The layout is the one the other forms write,
// bit for bit.

// Lane f's place in the layout (lanes >= P hold no pair).
struct TinyRank {
    int e, a1, key;
    int pos;            // sorted position of the pair
    int off_e, cnt_e, pad_e;  // its expert's first position, pairs and padded size
    int cnt_k, items_k, item0;  // its key's pairs, LoRA items and first item
    int npp, nitems;    // totals (every lane)
    bool valid, lead_e, lead_k;  // holds a pair; first pair of its expert / key
};

// `e`: lane f's expert (any value on lanes >= P).  Wave-uniform control flow.
__device__ __forceinline__ TinyRank tiny_align_rank(const AlignParams &p, int e) {
    TinyRank r;
    const int lane = lane_id();
    const int La = p.La, A1 = La + 1, P = p.P;
    r.valid = lane < P;
    r.e = e;
    r.a1 = (r.valid && La > 0) ? adapter_key_of(p.adapter_ids[lane / p.Kp], La) : 0;
    r.key = r.valid ? e * A1 + r.a1 : 0x7fffffff;
    // pass 1: ranks and counts
    int before_e = 0;   // pairs of this expert before this one
    int cnt_e = 0;      // pairs of this expert
    int before_k = 0;   // pairs of this key before this one
    int cnt_k = 0;      // pairs of this key
    for (int j = 0; j < P; ++j) {
        const int kj = __builtin_amdgcn_readlane(r.key, j);
        const int ej = __builtin_amdgcn_readlane(e, j);
        const bool earlier = kj < r.key || (kj == r.key && j < lane);
        cnt_e += ej == e;
        before_e += (ej == e && earlier) ? 1 : 0;
        cnt_k += kj == r.key;
        before_k += (kj == r.key && j < lane) ? 1 : 0;
    }
    r.cnt_e = cnt_e;
    r.cnt_k = cnt_k;
    r.pad_e = (cnt_e + p.bm - 1) / p.bm * p.bm;
    r.lead_e = r.valid && before_e == 0;
    r.lead_k = r.valid && before_k == 0;
    r.items_k = (La > 0 && r.a1 > 0) ? (cnt_k + p.lbm - 1) / p.lbm : 0;
    // pass 2: expert start (padded sizes of the smaller experts), first item
    // of this key, and the totals
    int off_e = 0, item0 = 0, npp = 0, nitems = 0;
    for (int j = 0; j < P; ++j) {
        const int ej = __builtin_amdgcn_readlane(e, j);
        const int kj = __builtin_amdgcn_readlane(r.key, j);
        const int pj = __builtin_amdgcn_readlane(r.pad_e, j);
        const int lj = __builtin_amdgcn_readlane(r.lead_e ? 1 : 0, j);
        const int ij = __builtin_amdgcn_readlane(r.lead_k ? r.items_k : 0, j);
        if (lj) {
            npp += pj;
            if (ej < e) off_e += pj;
        }
        nitems += ij;
        if (kj < r.key) item0 += ij;
    }
    r.off_e = off_e;
    r.item0 = item0;
    r.npp = npp;
    r.nitems = nitems;
    r.pos = off_e + before_e;
    return r;
}

// Store the layout ranked by tiny_align_rank (the whole wavefront calls it).
__device__ __forceinline__ void tiny_align_store(const AlignParams &p, const TinyRank &r) {
    const int lane = lane_id();
    const int P = p.P;
    if (r.valid) {
        p.sorted_ids[r.pos] = lane;
        if (p.sorted_adapter) p.sorted_adapter[r.pos] = r.a1 - 1;
    }
    if (r.lead_e) {
        for (int q = r.off_e + r.cnt_e; q < r.off_e + r.pad_e; ++q) {
            p.sorted_ids[q] = P;
            if (p.sorted_adapter) p.sorted_adapter[q] = -1;
        }
        for (int b = r.off_e / p.bm; b < (r.off_e + r.pad_e) / p.bm; ++b) p.block_expert[b] = r.e;
    }
    for (int q = r.npp + lane; q < p.cap; q += 64) {
        p.sorted_ids[q] = P;
        if (p.sorted_adapter) p.sorted_adapter[q] = -1;
    }
    for (int b = r.npp / p.bm + lane; b < p.max_blocks; b += 64) p.block_expert[b] = -1;
    const bool with_items = p.La > 0 && p.items != nullptr;
    if (with_items) {
        if (r.lead_k && r.items_k > 0) {
            // the key's run starts where its first pair sits
            int it = r.item0;
            for (int q = 0; q < r.cnt_k; q += p.lbm) {
                int4 v;
                v.x = r.pos + q;
                v.y = min(p.lbm, r.cnt_k - q);
                v.z = r.a1 - 1;
                v.w = r.e;
                reinterpret_cast<int4 *>(p.items)[it++] = v;
            }
        }
        for (int q = r.nitems + lane; q < p.max_items; q += 64) {
            int4 v;
            v.x = 0;
            v.y = 0;
            v.z = -1;
            v.w = -1;
            reinterpret_cast<int4 *>(p.items)[q] = v;
        }
    }
    if (lane == 0) {
        *p.npp_out = r.npp;
        if (p.npp_copy) *p.npp_copy = r.npp;
        *p.nitems_out = with_items ? r.nitems : 0;
    }
}

// Routing and alignment of a tiny call inside another kernel's workgroup of
// 256 threads, for a kernel whose workgroups each need one block of the
// layout: wave w < T routes token w, then wave 0 ranks the pairs.  Only the
// `writer` workgroup stores the routing and the layout (as the standalone
// kernels do, for the kernels launched after this one); every workgroup
// keeps in LDS the padded row count (s_blk[0]), the expert of its block b
// (s_blk[1]) and the pair of each of the block's BT rows (s_rows).
// Requires T <= 4, T*(K+S) <= 64, E <= 64*VPL and ap.bm == BT.
struct FusedRoute {
    AlignParams ap;
    RouteParams rp;
    // the host kernel's weights to touch while routing (see its use); per-expert byte strides
    const unsigned char *touch13 = nullptr, *touch2 = nullptr;
    int64_t stride13 = 0, stride2 = 0;
};

template <int BT, int VPL>
__device__ __forceinline__ void route_align_in_block(const FusedRoute &fr, int b, bool writer, int *s_e,
                                                     int *s_rows, int *s_blk) {
    const AlignParams &ap = fr.ap;
    const int w = (int)(threadIdx.x >> 6), lane = lane_id();
    if (w < fr.rp.T) {
        const int myi = route_one_token<VPL>(fr.rp, w, writer);  // slot j's expert in lane j
        if (lane < ap.Kp) s_e[w * ap.Kp + lane] = clamp_expert(myi, ap.Ep);
    }
    if ((int)threadIdx.x < BT) s_rows[threadIdx.x] = ap.P;
    if (threadIdx.x == 0) s_blk[1] = 0;
    __syncthreads();
    if (w == 0) {
        const TinyRank r = tiny_align_rank(ap, lane < ap.P ? s_e[lane] : 0);
        if (writer) tiny_align_store(ap, r);
        if (r.valid && r.pos >= b * BT && r.pos < (b + 1) * BT) s_rows[r.pos - b * BT] = lane;
        if (r.lead_e && r.off_e <= b * BT && b * BT < r.off_e + r.pad_e) s_blk[1] = r.e;
        if (lane == 0) s_blk[0] = r.npp;
    }
    __syncthreads();
}

// ROUTE: the wavefront routes the T <= 64 / (K+S) tokens first, one after
// another.
template <bool ROUTE, int VPL>
__global__ __launch_bounds__(64) void align_tiny_kernel(AlignParams p, RouteParams rp) {
    const int lane = (int)threadIdx.x;
    int e = 0;
    if constexpr (ROUTE) {
        for (int t = 0; t < rp.T; ++t) {
            const int myi = route_one_token<VPL>(rp, t);  // slot j's expert in lane j
            const int src = lane - t * p.Kp;
            const int got = __shfl(myi, max(0, min(src, 63)), 64);
            if (src >= 0 && src < p.Kp) e = clamp_expert(got, p.Ep);
        }
    } else {
        if (lane < p.P) e = clamp_expert(p.topk_ids[lane], p.Ep);
    }
    tiny_align_store(p, tiny_align_rank(p, e));
}

}  // namespace moelora
