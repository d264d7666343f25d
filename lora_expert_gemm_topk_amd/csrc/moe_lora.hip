// Host side of the MoE-LoRA layer: argument checking, plan (tile and split
// choice, workspace carving) and the launch sequence.  Every entry point is
// declared and documented in include/moe_lora.h.
//
// Launch sequence of moe_lora_forward on the caller's stream (no host sync,
// no allocation, grids sized for the worst case so nothing is read back):
//   route -> align -> [shrink13] -> gate_up GEMM (+expand13, SwiGLU)
//         -> [shrink2] -> down GEMM (+expand2) -> combine
// The alignment is one launch below MOELORA_ALIGN_MULTI_MIN pairs and four
// from there on.  With the LDS-tiled GEMMs (many rows per expert) x is also
// gathered and packed per sorted row: in the shrink13 launch when the layer
// has LoRA, else right after the alignment.
// The LoRA shrink launches are skipped on the host when the layer has no
// LoRA (L = 0 or r = 0), and on the device every shrink workgroup exits at
// once when no token of the call carries an adapter (aitrends.kr summary of
// the AWS multi-LoRA MoE post, "section details": layers without LoRA exit
// immediately).  No kernel is specialised on T: T is a runtime argument and
// the code object is loaded once (same post: per-length recompilation made
// the first version's time-to-first-token 10x the base model's).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "moe_lora.h"
#include "align.hpp"
#include "check.hpp"
#include "combine.hpp"
#include "fp32_path.hpp"
#include "gemm_stream.hpp"
#include "gemm_tiled.hpp"
#include "pack.hpp"
#include "route.hpp"
#include "shrink.hpp"

using namespace moelora;

// Scratch of moe_lora_forward_static: the layer's workspace for callers that
// cannot allocate.  One copy per GPU, allocated with the code object when the
// library is first used on that GPU and held until the process ends.  In
// host code this name is only a stand-in for the symbol: kernels get the
// device address that hipGetSymbolAddress returns (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[MOE_LORA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int64_t kLdsBytes = 160 * 1024;
#ifndef MOELORA_STREAM_BW
#define MOELORA_STREAM_BW 64
#endif
constexpr int kStreamBW = MOELORA_STREAM_BW;  // weight rows per streaming-GEMM workgroup

thread_local char g_errbuf[320];

struct Plan {
    int bm = 0, lbm = 0, split = 1, kind = 0, tile = 0;
    bool row_shrink = false;  // streaming path: gate_up shrink per pair in the router launch
    int64_t P = 0, Ep = 0, Kp = 0, La = 0;
    int64_t max_blocks = 0, cap = 0, max_items = 0, max_tiles = 0;
    int align_nw = 16;
    size_t align_lds = 0;
    bool lds_keys = false;   // alignment keys staged in LDS
    bool multi = false;      // multi-workgroup alignment
    bool small_align = false;  // one-pass alignment for small calls without GEMM token tiles
    bool route_in_align = false;  // small_align: the router runs in the alignment's launch
    bool route_in_gemm = false;   // the gate_up launch routes and aligns (tiny calls without LoRA)
    int align_small_nw = 4;
    size_t align_small_lds = 0;
    int anb = 0, achunk = 0; // its blocks and pairs per block
    int64_t tmp_ints = 0;    // ints of alignment scratch
    bool lora = false;
    // workspace offsets (bytes)
    size_t o_ids = 0, o_w = 0, o_sorted = 0, o_sadp = 0, o_bexp = 0, o_cnt = 0, o_items = 0, o_tmp = 0, o_tiles = 0;
    size_t o_queue = 0;
    size_t o_s13 = 0, o_s2 = 0, o_h = 0, o_y2 = 0, o_xp = 0, total = 0;
    size_t align_total = 0;  // tmp + nothing else, for moe_lora_align
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int bits_for(int64_t n) {  // bits to hold values 0..n-1
    int b = 0;
    while ((int64_t(1) << b) < n) ++b;
    return b;
}

int make_plan(const moe_lora_dims *d, Plan *pl) {
    if (!d || !pl) return MOE_LORA_EINVAL;
    if (d->T < 0 || d->H <= 0 || d->I <= 0 || d->E <= 0 || d->K <= 0 || d->K > d->E || d->S < 0 || d->L < 0 ||
        d->r < 0)
        return MOE_LORA_EINVAL;
    if (!(std::isfinite(d->routed_scaling_factor) && d->routed_scaling_factor > 0.0f)) return MOE_LORA_EINVAL;
    if (d->renormalize != 0 && d->renormalize != 1) return MOE_LORA_EINVAL;
    if (d->router < MOE_LORA_ROUTER_TOPK || d->router > MOE_LORA_ROUTER_BIAS_SIGMOID) return MOE_LORA_EINVAL;
    if (d->dtype != MOE_LORA_F32 && d->dtype != MOE_LORA_BF16) return MOE_LORA_EUNSUPPORTED;
    if (d->E > 1024 || d->K > 64 || d->S > 64) return MOE_LORA_EUNSUPPORTED;
    if (d->H % 8 != 0 || d->I % 8 != 0) return MOE_LORA_EUNSUPPORTED;
    if (d->H > (1 << 24) || d->I > (1 << 24)) return MOE_LORA_EUNSUPPORTED;
    const bool lora = d->L > 0 && d->r > 0;
    if (lora) {
        if (d->r > 128 || d->L > 1024) return MOE_LORA_EUNSUPPORTED;
        if (d->dtype == MOE_LORA_BF16 && d->r % 8 != 0) return MOE_LORA_EUNSUPPORTED;
    }
    Plan p;
    p.lora = lora;
    p.Kp = d->K + d->S;
    p.Ep = d->E + d->S;
    p.La = lora ? d->L : 0;
    if (d->T > (int64_t(1) << 31) / p.Kp) return MOE_LORA_EUNSUPPORTED;
    p.P = d->T * p.Kp;
    if (p.Ep * (p.La + 1) > 16384) return MOE_LORA_EUNSUPPORTED;

    // tile choice by the average rows per expert; never specialised on T itself
    const int64_t rho = p.P / p.Ep;
    if (d->block_m != 0 && d->block_m != 16 && d->block_m != 32 && d->block_m != 128 && d->block_m != 256)
        return MOE_LORA_EUNSUPPORTED;
    if (d->lora_block_m != 0 && d->lora_block_m != 16 && d->lora_block_m != 32) return MOE_LORA_EUNSUPPORTED;
    if (d->split_k < 0 || d->split_k > 16) return MOE_LORA_EINVAL;
    if (d->dtype == MOE_LORA_F32) {
        p.kind = 0;
        p.bm = d->block_m ? d->block_m : 16;
        if (p.bm > 32) return MOE_LORA_EUNSUPPORTED;
        p.tile = p.bm;
        p.lbm = d->lora_block_m ? d->lora_block_m : 16;
        p.split = 1;
    } else {
        const int tm = d->block_m ? d->block_m : (rho <= 12 ? 16 : (rho <= 40 ? 32 : (rho < 192 ? 128 : 256)));
        p.kind = tm <= 32 ? 1 : 2;
        p.bm = tm <= 32 ? tm : 32;  // the tiled GEMM pads experts to 32 rows and cuts tiles of tm rows
        p.tile = tm;
        p.lbm = d->lora_block_m ? d->lora_block_m : (rho <= 40 || d->r > 64 ? 16 : 32);
        if (p.lbm == 32 && d->r > 64) return MOE_LORA_EUNSUPPORTED;
        if (d->split_k) {
            p.split = d->split_k;
        } else {
            const int64_t ch = (std::max(d->H, d->I) + 31) / 32;
            p.split = (d->T <= 512) ? (int)std::min<int64_t>(2, std::max<int64_t>(1, ch / 16)) : 1;
        }
    }
    // The tiled kernel streams the shrink result through its LDS ring as bf16
    // rows, so the shrink runs unsplit and rounds its fp32 sums there.
    if (!lora || p.kind == 2) p.split = 1;
    // Unless a split is asked for, the streaming path runs the gate_up shrink
    // per pair inside the router launch (it needs only the routing and the
    // adapter ids; K+S <= 64).  The down shrink keeps the split-K items.
    p.row_shrink = lora && p.kind == 1 && d->split_k == 0 && p.Kp <= 64 && d->r <= 64;

    const int64_t nz = std::min(p.Ep, p.P);
    p.max_blocks = (p.P + p.bm - 1) / p.bm + nz;
    p.cap = p.max_blocks * p.bm;
    if (lora) {
        const int64_t bins = std::min(p.La * p.Ep, p.P);
        p.max_items = (p.P + p.lbm - 1) / p.lbm + bins;
    }
    if (p.kind == 2) p.max_tiles = (p.P + p.tile - 1) / p.tile + 2 * nz;
    if (p.cap >= (int64_t(1) << 31) - 1) return MOE_LORA_EUNSUPPORTED;

    // align workgroup: as many waves as the LDS allows, keys staged in LDS
    // when they fit (16-bit pair indices need P < 65536)
    // a small call needs few waves: one 64-pair step per wave and pass
#ifndef MOELORA_ALIGN_MAXNW
#define MOELORA_ALIGN_MAXNW 16
#endif
    int nw_max = MOELORA_ALIGN_MAXNW;
    while (nw_max > 4 && (int64_t)(nw_max / 2) * 64 >= p.P) nw_max /= 2;
    p.align_nw = 0;
    for (int pass = 0; pass < 2 && p.align_nw == 0; ++pass) {
        const bool lk = pass == 0;
        if (lk && p.P >= 65536) continue;
        for (int nw = nw_max; nw >= (lk ? 4 : 1); nw >>= 1) {
            const int64_t bytes = align_lds_ints(nw, (int)p.Ep, (int)p.La, d->T, p.P, lk) * 4;
            if (bytes <= kLdsBytes) {
                p.align_nw = nw;
                p.align_lds = (size_t)bytes;
                p.lds_keys = lk;
                break;
            }
        }
    }
    if (p.align_nw == 0) return MOE_LORA_EUNSUPPORTED;
    // many pairs: the multi-workgroup alignment (slices of 256..1024+ pairs,
    // at most 64 slices so the per-key column scans stay short)
#ifndef MOELORA_ALIGN_MULTI_MIN
#define MOELORA_ALIGN_MULTI_MIN 8192
#endif
    const int64_t NK = p.Ep * (p.La + 1);
    p.multi = p.P >= MOELORA_ALIGN_MULTI_MIN && NK * 4 <= kLdsBytes &&
              align_scan_lds_ints((int)p.Ep, (int)p.La) * 4 <= kLdsBytes;
    // small calls without GEMM token tiles: one thread per pair, one pass
    p.small_align = !p.multi && p.kind != 2 && p.P <= 1024;
    if (p.small_align) {
        p.align_small_nw = (int)std::max<int64_t>(4, (p.P + 63) / 64);
        const int64_t ints = align_small_lds_ints(p.align_small_nw, (int)p.Ep, (int)p.La, p.P);
        if (ints * 4 > 65536) p.small_align = false;
        else p.align_small_lds = (size_t)ints * 4;
    }
    // small calls whose gate_up shrink does not run in the router's launch
    // route inside the alignment's launch (every slot fits one wavefront)
    // when each of its waves routes one token at most: routing more tokens
    // one after another in a wave costs more than the launch it saves
    // (measured: T = 32 with 64 experts, 57 us against 19 us in two launches)
    p.route_in_align = p.small_align && !p.row_shrink && p.Kp <= 64 && d->T <= p.align_small_nw;
    // tiny calls without LoRA on the streaming GEMM: every gate_up workgroup
    // routes the tokens and aligns the pairs itself (a wave per token, then
    // one wave ranks them), so the call runs in three launches
    p.route_in_gemm = p.small_align && p.kind == 1 && !p.lora && p.P <= 64 && d->T >= 1 && d->T <= 4 &&
                      d->E <= 256;
    p.tmp_ints = p.P;
    if (p.multi) {
        p.achunk = (int)std::max<int64_t>(256, ((p.P + 63) / 64 + 63) / 64 * 64);
        p.anb = (int)((p.P + p.achunk - 1) / p.achunk);
        p.tmp_ints = std::max<int64_t>(p.P, (int64_t)p.anb * NK + NK);
    }

    const size_t A = 256;
    const size_t es = d->dtype == MOE_LORA_BF16 ? 2 : 4;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = round_up(o + std::max<size_t>(bytes, 1), A);
        return at;
    };
    p.o_ids = take(sizeof(int32_t) * p.P);
    p.o_w = take(sizeof(float) * p.P);
    p.o_sorted = take(sizeof(int32_t) * p.cap);
    p.o_sadp = take(p.kind == 2 ? sizeof(int32_t) * p.cap : 0);
    p.o_bexp = take(sizeof(int32_t) * p.max_blocks);
    p.o_cnt = take(sizeof(int32_t) * 16);
    p.o_items = take(sizeof(int32_t) * 4 * std::max<int64_t>(p.max_items, 1));
    p.o_tmp = take(sizeof(int32_t) * p.tmp_ints);
    p.o_tiles = take(sizeof(int32_t) * 4 * std::max<int64_t>(p.max_tiles, 1));
    p.o_queue = take(p.kind == 2 ? sizeof(int32_t) * 32 : 0);  // XCD ranges: gate_up's, then down's
    p.o_s13 = take(lora ? sizeof(float) * p.split * p.cap * d->r : 0);
    p.o_s2 = take(lora ? sizeof(float) * p.split * p.cap * d->r : 0);
    // room for h packed (the tiled GEMM's layout): whole 32-wide slabs
    p.o_h = take(es * p.cap * (d->dtype == MOE_LORA_BF16 ? (d->I + 31) / 32 * 32 : d->I));
    p.o_y2 = take(es * p.P * d->H);  // y2 in the layer's dtype
    // tiled GEMM: x gathered and packed per sorted row
    p.o_xp = take(p.kind == 2 ? es * p.cap * ((d->H + 31) / 32 * 32) : 0);
    p.total = o;
    p.align_total = round_up(sizeof(int32_t) * std::max<int64_t>(p.tmp_ints, 1), A) + round_up(sizeof(int32_t) * 16, A);
    *pl = p;
    return MOE_LORA_OK;
}

bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

int hip_fail(hipError_t e, const char *what) {
    snprintf(g_errbuf, sizeof g_errbuf, "HIP error in %s: %s (%d)", what, hipGetErrorString(e), (int)e);
    return MOE_LORA_EHIP;
}

std::once_flag g_attr_once;
hipError_t g_attr_err = hipSuccess;

void set_kernel_attributes() {
    const void *fns[] = {(const void *)align_kernel,
                         (const void *)align_hist_kernel,     (const void *)align_scan_kernel,
                         (const void *)align_scatter_kernel};
    for (const void *fn : fns) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
        if (e != hipSuccess) g_attr_err = e;
    }
}

RouteParams route_params(const moe_lora_dims *d, const float *logits, const float *bias, int32_t *ids,
                         float *w) {
    RouteParams rp;
    rp.scoring = d->router == MOE_LORA_ROUTER_TOPK ? -1 : (d->router == MOE_LORA_ROUTER_BIAS_SOFTMAX ? 0 : 1);
    rp.bias = bias;
    rp.logits = logits;
    rp.T = (int)d->T;
    rp.E = (int)d->E;
    rp.K = (int)d->K;
    rp.S = (int)d->S;
    rp.shared_w = 1.0f / d->routed_scaling_factor;
    rp.renorm = d->renormalize;
    rp.ids = ids;
    rp.wts = w;
    return rp;
}

template <int VPL>
void launch_route_shrink_vpl(const RouteParams &rp, const RowShrinkParams &sp, hipStream_t st) {
    const dim3 grid((unsigned)rp.T, (unsigned)(rp.K + rp.S)), block(256);
    if (sp.r <= 16) hipLaunchKernelGGL((route_shrink_kernel<VPL, 16>), grid, block, 0, st, rp, sp);
    else if (sp.r <= 32) hipLaunchKernelGGL((route_shrink_kernel<VPL, 32>), grid, block, 0, st, rp, sp);
    else hipLaunchKernelGGL((route_shrink_kernel<VPL, 64>), grid, block, 0, st, rp, sp);
}

// Router and gate_up shrink in one launch (plan.row_shrink): s13 by pair.
void launch_route_shrink(const Plan &pl, const moe_lora_dims *d, const moe_lora_args *a, int32_t *ids, float *w,
                         float *s13, hipStream_t st) {
    const RouteParams rp = route_params(d, a->router_logits, a->expert_bias, ids, w);
    RowShrinkParams sp{};
    sp.in = (const uint16_t *)a->hidden;
    sp.A = (const uint16_t *)a->a13;
    sp.adapter_ids = a->adapter_ids;
    sp.s = s13;
    sp.Kdim = (int)d->H;
    sp.r = (int)d->r;
    sp.Ep = (int)pl.Ep;
    sp.Kp = (int)pl.Kp;
    sp.P = (int)pl.P;
    sp.L = (int)pl.La;
    const int E = rp.E;
    if (E <= 64) launch_route_shrink_vpl<1>(rp, sp, st);
    else if (E <= 128) launch_route_shrink_vpl<2>(rp, sp, st);
    else if (E <= 256) launch_route_shrink_vpl<4>(rp, sp, st);
    else if (E <= 512) launch_route_shrink_vpl<8>(rp, sp, st);
    else launch_route_shrink_vpl<16>(rp, sp, st);
}

int launch_route(const moe_lora_dims *d, const float *logits, const float *bias, int32_t *ids, float *w,
                 hipStream_t st) {
    const RouteParams rp = route_params(d, logits, bias, ids, w);
    const dim3 grid((unsigned)((rp.T + 3) / 4)), block(256);
    const int E = rp.E;
    if (E <= 64) hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, st, rp);
    else if (E <= 128) hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, st, rp);
    else if (E <= 256) hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, st, rp);
    else if (E <= 512) hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, st, rp);
    else hipLaunchKernelGGL(route_kernel<16>, grid, block, 0, st, rp);
    return MOE_LORA_OK;
}

// Weight rows per tile of the LDS-tiled kernel.  256 (16 MFMAs per 8
// fragment reads per wave) measured fastest for both projections of the
// GPT-OSS-20B prefill layer even where N is not a multiple of the tile; 128
// only when N is too small to fill wider tiles.  (Both are whole multiples of
// the 128-row half tiles the packed weight layout is padded to.)
int tiled_bw(int N, bool gu) {
    const int feats = gu ? N * 2 : N;
    return feats <= 128 ? 128 : 256;
}

// Compute units of the current device, looked up once per device.
int device_cus() {
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// Weight tiles of the tiled gate_up (gu) or down GEMM.
int tiled_nwt(const moe_lora_dims *d, bool gu) {
    const int N = (int)(gu ? d->I : d->H);
    const int bw = tiled_bw(N, gu);
    const int per = gu ? bw / 2 : bw;
    return (N + per - 1) / per;
}

// Work items one XCD may take: twice its equal share of the most items the
// GEMM can have, so that ranges cut at equal cost always fit the grid.
int64_t tiled_xcap(const Plan &pl, int n_wt) { return 2 * (((int64_t)n_wt * pl.max_tiles + 7) / 8); }

// Alignment: one workgroup below the multi-workgroup threshold, else four launches.
AlignParams align_params(const Plan &pl, const moe_lora_dims *d, const int32_t *ids, const int32_t *adapter_ids,
                         int32_t *sorted, int32_t *sorted_adapter, int32_t *bexp, int32_t *npp, int32_t *items,
                         int32_t *nitems, int32_t *tmp, int32_t *tiles, int32_t *ntiles, int32_t *npp_copy,
                         int32_t *queue) {
    AlignParams ap;
    ap.T = (int)d->T;
    ap.lds_keys = pl.lds_keys ? 1 : 0;
    ap.topk_ids = ids;
    ap.adapter_ids = adapter_ids;
    ap.sorted_ids = sorted;
    ap.sorted_adapter = sorted_adapter;
    ap.block_expert = bexp;
    ap.npp_out = npp;
    ap.npp_copy = npp_copy;
    ap.nitems_out = nitems;
    ap.items = pl.lora ? items : nullptr;
    ap.tmp = tmp;
    ap.tiles = tiles;
    ap.ntiles_out = ntiles;
    ap.xsplit = tiles ? queue : nullptr;
    for (int g = 0; g < 2; ++g) {
        ap.nwt[g] = tiled_nwt(d, g == 0);
        ap.xcap[g] = (int)tiled_xcap(pl, ap.nwt[g]);
    }
    if (tiles) ap.cus = device_cus();
    ap.tile_rows = pl.tile;
    ap.P = (int)pl.P;
    ap.Kp = (int)pl.Kp;
    ap.Ep = (int)pl.Ep;
    ap.La = (int)pl.La;
    ap.bm = pl.bm;
    ap.lbm = pl.lbm;
    ap.cap = (int)pl.cap;
    ap.max_blocks = (int)pl.max_blocks;
    ap.max_items = (int)pl.max_items;
    ap.nbits_a = bits_for(pl.La + 1);
    ap.nbits_e = bits_for(pl.Ep);
    const int NK = (int)(pl.Ep * (pl.La + 1));
    ap.nbits_k = bits_for(NK);
    ap.nb = pl.anb;
    ap.chunk = pl.achunk;
    ap.hist = tmp;
    ap.ktot = tmp + (int64_t)pl.anb * NK;
    return ap;
}

int launch_align(const Plan &pl, const moe_lora_dims *d, const int32_t *ids, const int32_t *adapter_ids,
                 int32_t *sorted, int32_t *sorted_adapter, int32_t *bexp, int32_t *npp, int32_t *items,
                 int32_t *nitems, int32_t *tmp, int32_t *tiles, int32_t *ntiles,
                 hipStream_t st, int32_t *npp_copy = nullptr, int32_t *queue = nullptr,
                 const RouteParams *rp = nullptr) {
    std::call_once(g_attr_once, set_kernel_attributes);
    if (g_attr_err != hipSuccess) return hip_fail(g_attr_err, "hipFuncSetAttribute(align)");
    const AlignParams ap = align_params(pl, d, ids, adapter_ids, sorted, sorted_adapter, bexp, npp, items, nitems,
                                        tmp, tiles, ntiles, npp_copy, queue);
    const int NK = (int)(pl.Ep * (pl.La + 1));
    if (pl.multi) {
        const size_t klds = sizeof(int) * (size_t)NK;
        hipLaunchKernelGGL(align_hist_kernel, dim3((unsigned)pl.anb), dim3(256), klds, st, ap);
        hipLaunchKernelGGL(align_colscan_kernel, dim3((unsigned)((NK + 255) / 256)), dim3(256), 0, st, ap);
        hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(1024),
                           sizeof(int) * (size_t)align_scan_lds_ints((int)pl.Ep, (int)pl.La), st, ap);
        hipLaunchKernelGGL(align_scatter_kernel, dim3((unsigned)pl.anb), dim3(256), klds, st, ap);
        return MOE_LORA_OK;
    }
    if (pl.small_align && tiles == nullptr && pl.P <= 64) {
        // at most 64 pairs: one wavefront, no barriers
        const dim3 g1(1), w1(64);
        if (rp == nullptr) {
            hipLaunchKernelGGL((align_tiny_kernel<false, 1>), g1, w1, 0, st, ap, RouteParams{});
        } else {
            const int E = rp->E;
            if (E <= 64) hipLaunchKernelGGL((align_tiny_kernel<true, 1>), g1, w1, 0, st, ap, *rp);
            else if (E <= 128) hipLaunchKernelGGL((align_tiny_kernel<true, 2>), g1, w1, 0, st, ap, *rp);
            else if (E <= 256) hipLaunchKernelGGL((align_tiny_kernel<true, 4>), g1, w1, 0, st, ap, *rp);
            else if (E <= 512) hipLaunchKernelGGL((align_tiny_kernel<true, 8>), g1, w1, 0, st, ap, *rp);
            else hipLaunchKernelGGL((align_tiny_kernel<true, 16>), g1, w1, 0, st, ap, *rp);
        }
        return MOE_LORA_OK;
    }
    if (pl.small_align && tiles == nullptr) {
        const dim3 g1(1), blk((unsigned)(pl.align_small_nw * 64));
        if (rp == nullptr) {
            hipLaunchKernelGGL((align_small_kernel<false, 1>), g1, blk, pl.align_small_lds, st, ap, RouteParams{});
        } else {
            const int E = rp->E;
            if (E <= 64) hipLaunchKernelGGL((align_small_kernel<true, 1>), g1, blk, pl.align_small_lds, st, ap, *rp);
            else if (E <= 128) hipLaunchKernelGGL((align_small_kernel<true, 2>), g1, blk, pl.align_small_lds, st, ap, *rp);
            else if (E <= 256) hipLaunchKernelGGL((align_small_kernel<true, 4>), g1, blk, pl.align_small_lds, st, ap, *rp);
            else if (E <= 512) hipLaunchKernelGGL((align_small_kernel<true, 8>), g1, blk, pl.align_small_lds, st, ap, *rp);
            else hipLaunchKernelGGL((align_small_kernel<true, 16>), g1, blk, pl.align_small_lds, st, ap, *rp);
        }
        return MOE_LORA_OK;
    }
    const dim3 grid(1), block((unsigned)(pl.align_nw * 64));
    hipLaunchKernelGGL(align_kernel, grid, block, pl.align_lds, st, ap);
    return MOE_LORA_OK;
}

template <int NT>
void launch_shrink_nt(const ShrinkParams &sp, int r, int split, int max_items, hipStream_t st) {
    const dim3 grid((unsigned)max_items, (unsigned)split), block(256);
    if (r <= 16) hipLaunchKernelGGL((shrink_kernel<NT, 1, true>), grid, block, 0, st, sp);
    else if (r <= 32) hipLaunchKernelGGL((shrink_kernel<NT, 2, true>), grid, block, 0, st, sp);
    else if (r <= 64) hipLaunchKernelGGL((shrink_kernel<NT, 4, true>), grid, block, 0, st, sp);
    else hipLaunchKernelGGL((shrink_kernel<NT, 8, true>), grid, block, 0, st, sp);
}

template <int NT>
void launch_shrink_rows_nt(const ShrinkParams &sp, int r, int split, int max_items, hipStream_t st) {
    const dim3 grid((unsigned)max_items, (unsigned)split), block(256);
    if (r <= 16) hipLaunchKernelGGL((shrink_kernel<NT, 1, false>), grid, block, 0, st, sp);
    else if (r <= 32) hipLaunchKernelGGL((shrink_kernel<NT, 2, false>), grid, block, 0, st, sp);
    else if (r <= 64) hipLaunchKernelGGL((shrink_kernel<NT, 4, false>), grid, block, 0, st, sp);
    else hipLaunchKernelGGL((shrink_kernel<NT, 8, false>), grid, block, 0, st, sp);
}

template <int NT>
void launch_pack_shrink_nt(const PackXParams &xp, const ShrinkParams &sp, int r, int mi, unsigned groups,
                           hipStream_t st) {
    const dim3 grid((unsigned)mi + groups), block(256);
    if (r <= 16) hipLaunchKernelGGL((pack_x_shrink_kernel<NT, 1>), grid, block, 0, st, xp, sp, mi);
    else if (r <= 32) hipLaunchKernelGGL((pack_x_shrink_kernel<NT, 2>), grid, block, 0, st, xp, sp, mi);
    else if (r <= 64) hipLaunchKernelGGL((pack_x_shrink_kernel<NT, 4>), grid, block, 0, st, xp, sp, mi);
    else hipLaunchKernelGGL((pack_x_shrink_kernel<NT, 8>), grid, block, 0, st, xp, sp, mi);
}

// gate_up shrink and x pack in one launch (tiled path; the shrink is unsplit there)
void launch_pack_shrink(const Plan &pl, const PackXParams &xp, ShrinkParams sp, int r, hipStream_t st) {
    sp.chunks_per_split = (sp.Kdim + 31) / 32;
    const int mi = (int)pl.max_items;
    const unsigned groups = (unsigned)(pl.cap / 16);
    if (pl.lbm == 16) launch_pack_shrink_nt<1>(xp, sp, r, mi, groups, st);
    else launch_pack_shrink_nt<2>(xp, sp, r, mi, groups, st);
}

void launch_shrink(const Plan &pl, ShrinkParams sp, bool gather, int r, hipStream_t st) {
    const int nch = (sp.Kdim + 31) / 32;
    sp.chunks_per_split = (nch + pl.split - 1) / pl.split;
    const int mi = (int)pl.max_items;
    if (gather) {
        if (pl.lbm == 16) launch_shrink_nt<1>(sp, r, pl.split, mi, st);
        else launch_shrink_nt<2>(sp, r, pl.split, mi, st);
    } else {
        if (pl.lbm == 16) launch_shrink_rows_nt<1>(sp, r, pl.split, mi, st);
        else launch_shrink_rows_nt<2>(sp, r, pl.split, mi, st);
    }
}


template <int BW, int BT, bool GU, bool WP, bool MX>
void launch_tiled(const Plan &pl, const GemmParams &gp, const int32_t *tiles, const int32_t *ntiles,
                  const int32_t *xsplit, hipStream_t st) {
    const int n_wt = (gp.Nout + (GU ? BW / 2 : BW) - 1) / (GU ? BW / 2 : BW);
    // every XCD may take up to xcap items of the cost-balanced ranges, or
    // (skewed order) its panels of kSkewPanel token tiles x n_wt items
    const int64_t panels = (pl.max_tiles + kSkewPanel - 1) / kSkewPanel;
    const int64_t skew_blocks = 8 * ((panels + 7) / 8) * kSkewPanel * n_wt;
    const unsigned total = (unsigned)std::max<int64_t>(8 * tiled_xcap(pl, n_wt), skew_blocks);
    hipLaunchKernelGGL((gemm_tiled_kernel<BW, BT, GU, WP, MX>), dim3(total), dim3(256), 0, st, gp, tiles, ntiles,
                       n_wt, xsplit + (GU ? 0 : 16));
}

template <bool GU, bool WP, bool MX>
void launch_tiled_shape(const Plan &pl, const GemmParams &gp, const int32_t *tiles, const int32_t *ntiles,
                        const int32_t *queue, hipStream_t st) {
    const int bw = tiled_bw(gp.Nout, GU);
    if (pl.tile == 128) {
        if (bw == 256) launch_tiled<256, 128, GU, WP, MX>(pl, gp, tiles, ntiles, queue, st);
        else launch_tiled<128, 128, GU, WP, MX>(pl, gp, tiles, ntiles, queue, st);
    } else {
        if (bw == 256) launch_tiled<256, 256, GU, WP, MX>(pl, gp, tiles, ntiles, queue, st);
        else launch_tiled<128, 256, GU, WP, MX>(pl, gp, tiles, ntiles, queue, st);
    }
}

// The streaming GEMM (few rows per expert).  fr: gate_up routes and aligns
// inside its workgroups.
template <bool GU, bool WP, bool MX>
void launch_stream(const Plan &pl, const GemmParams &gp, const FusedRoute *fr, hipStream_t st) {
    const int tile = GU ? kStreamBW / 2 : kStreamBW;
    const dim3 grid((unsigned)((gp.Nout + tile - 1) / tile), (unsigned)pl.max_blocks), block(256);
    if constexpr (GU) {
        if (fr != nullptr) {
            if (pl.bm == 16)
                hipLaunchKernelGGL((gemm_stream_route_kernel<kStreamBW, 16, WP, MX>), grid, block, 0, st, gp, *fr);
            else
                hipLaunchKernelGGL((gemm_stream_route_kernel<kStreamBW, 32, WP, MX>), grid, block, 0, st, gp, *fr);
            return;
        }
    }
    if (pl.bm == 16) hipLaunchKernelGGL((gemm_stream_kernel<kStreamBW, 16, GU, WP, MX>), grid, block, 0, st, gp);
    else hipLaunchKernelGGL((gemm_stream_kernel<kStreamBW, 32, GU, WP, MX>), grid, block, 0, st, gp);
}

template <bool GU, bool MX>
void launch_stream_wp(const Plan &pl, const GemmParams &gp, const FusedRoute *fr, bool wp, hipStream_t st) {
    if (wp) launch_stream<GU, true, MX>(pl, gp, fr, st);
    else launch_stream<GU, false, MX>(pl, gp, fr, st);
}

template <bool GU>
void launch_gemm(const Plan &pl, const GemmParams &gp, const int32_t *tiles, const int32_t *ntiles,
                 const int32_t *queue, bool wp, hipStream_t st, const FusedRoute *fr = nullptr) {
    const bool mx = gp.Wscale != nullptr;
    if (pl.kind == 2) {
        // MXFP8 weights: H, I <= 32 kMxTiledMaxBlocks (checked by moe_lora_check_args)
        if (mx) {
            if (wp) launch_tiled_shape<GU, true, true>(pl, gp, tiles, ntiles, queue, st);
            else launch_tiled_shape<GU, false, true>(pl, gp, tiles, ntiles, queue, st);
        } else {
            if (wp) launch_tiled_shape<GU, true, false>(pl, gp, tiles, ntiles, queue, st);
            else launch_tiled_shape<GU, false, false>(pl, gp, tiles, ntiles, queue, st);
        }
        return;
    }
    // kind 1 (kind 0, the fp32 path, does not come here; MXFP8 with kind 0 is checked out)
    if (mx) launch_stream_wp<GU, true>(pl, gp, fr, wp, st);
    else launch_stream_wp<GU, false>(pl, gp, fr, wp, st);
}

}  // namespace

extern "C" {

int moe_lora_plan_query(const moe_lora_dims *dims, moe_lora_plan *plan) {
    Plan p;
    const int rc = make_plan(dims, &p);
    if (rc != MOE_LORA_OK) return rc;
    if (!plan) return MOE_LORA_EINVAL;
    plan->block_m = p.bm;
    plan->tile_m = p.tile;
    plan->lora_block_m = p.lbm;
    plan->split_k = p.split;
    plan->gemm_kind = p.kind;
    plan->max_blocks = p.max_blocks;
    plan->sorted_capacity = p.cap;
    plan->max_items = p.max_items;
    plan->workspace_bytes = p.total;
    plan->align_workspace_bytes = p.align_total;
    return MOE_LORA_OK;
}

size_t moe_lora_workspace_bytes(const moe_lora_dims *dims) {
    Plan p;
    return make_plan(dims, &p) == MOE_LORA_OK ? p.total : 0;
}

int moe_lora_check_args(const moe_lora_dims *d, const moe_lora_args *a) {
    Plan p;
    const int rc = make_plan(d, &p);
    if (rc != MOE_LORA_OK) return rc;
    if (!a) return MOE_LORA_EINVAL;
    if (d->T == 0) return MOE_LORA_OK;
    if (!a->hidden || !a->router_logits || !a->w13 || !a->w2 || !a->out || !a->workspace) return MOE_LORA_EINVAL;
    if (p.lora && (!a->adapter_ids || !a->a13 || !a->b13 || !a->a2 || !a->b2)) return MOE_LORA_EINVAL;
    const void *v16[] = {a->hidden, a->w13, a->w2, a->out};
    for (const void *ptr : v16)
        if (!aligned(ptr, 16)) return MOE_LORA_EINVAL;
    if (p.lora) {
        const void *l16[] = {a->a13, a->b13, a->a2, a->b2};
        for (const void *ptr : l16)
            if (!aligned(ptr, 16)) return MOE_LORA_EINVAL;
    }
    if (!aligned(a->workspace, 256)) return MOE_LORA_EINVAL;
    if (a->expert_bias && d->router == MOE_LORA_ROUTER_TOPK) return MOE_LORA_EINVAL;
    const void *outs[] = {a->sorted_ids_out, a->block_expert_out, a->num_post_pad_out, a->expert_bias};
    for (const void *ptr : outs)
        if (ptr && !aligned(ptr, 4)) return MOE_LORA_EINVAL;
    if (a->workspace_bytes < p.total) return MOE_LORA_EWORKSPACE;
    if (a->weights_packed != 0 && a->weights_packed != 1) return MOE_LORA_EINVAL;
    if (a->weights_packed && d->dtype != MOE_LORA_BF16) return MOE_LORA_EUNSUPPORTED;
    if (a->weights_mxfp8 != 0 && a->weights_mxfp8 != 1) return MOE_LORA_EINVAL;
    if (a->weights_mxfp8) {
        if (!a->w13_scale || !a->w2_scale || !aligned(a->w13_scale, 16) || !aligned(a->w2_scale, 16))
            return MOE_LORA_EINVAL;
        // the streaming GEMM holds a row's scales for K <= 32 kMxMaxBlocks, the
        // tiled one for K <= 32 kMxTiledMaxBlocks
        const int64_t kmax = 32 * (p.kind == 2 ? kMxTiledMaxBlocks : kMxMaxBlocks);
        if (d->dtype != MOE_LORA_BF16 || d->H % 32 != 0 || d->I % 32 != 0 || p.kind == 0 || d->H > kmax ||
            d->I > kmax)
            return MOE_LORA_EUNSUPPORTED;
    }
    return MOE_LORA_OK;
}

size_t moe_lora_packed_weight_bytes(const moe_lora_dims *d, int which) {
    Plan p;
    if (make_plan(d, &p) != MOE_LORA_OK || d->dtype != MOE_LORA_BF16) return 0;
    if (which == 0) return (size_t)p.Ep * packed_w13_groups(d->I) * ((d->H + 31) / 32) * 1024;
    if (which == 1) return (size_t)p.Ep * packed_w2_groups(d->H) * ((d->I + 31) / 32) * 1024;
    return 0;
}

int moe_lora_pack_weights(const moe_lora_dims *d, const void *w13, const void *w2, void *w13_packed,
                          void *w2_packed, void *stream) {
    Plan p;
    const int rc = make_plan(d, &p);
    if (rc != MOE_LORA_OK) return rc;
    if (d->dtype != MOE_LORA_BF16) return MOE_LORA_EUNSUPPORTED;
    if ((w13 == nullptr) != (w13_packed == nullptr) || (w2 == nullptr) != (w2_packed == nullptr))
        return MOE_LORA_EINVAL;
    const void *ptrs[] = {w13, w2, w13_packed, w2_packed};
    for (const void *ptr : ptrs)
        if (ptr && !aligned(ptr, 16)) return MOE_LORA_EINVAL;
    if (!w13 && !w2) return MOE_LORA_OK;
    hipStream_t st = (hipStream_t)stream;
    if (w13) {
        PackWParams pw;
        pw.src = (const uint16_t *)w13;
        pw.dst = (uint16_t *)w13_packed;
        pw.rows_src = 2 * d->I;
        pw.K = (int)d->H;
        pw.nslab = (int)((d->H + 31) / 32);
        pw.G = (int)packed_w13_groups(d->I);
        pw.N = (int)d->I;
        pw.gate_up = 1;
        hipLaunchKernelGGL(pack_w_kernel, dim3((unsigned)pw.G, (unsigned)p.Ep), dim3(256), 0, st, pw);
    }
    if (w2) {
        PackWParams pw;
        pw.src = (const uint16_t *)w2;
        pw.dst = (uint16_t *)w2_packed;
        pw.rows_src = d->H;
        pw.K = (int)d->I;
        pw.nslab = (int)((d->I + 31) / 32);
        pw.G = (int)packed_w2_groups(d->H);
        pw.N = (int)d->H;
        pw.gate_up = 0;
        hipLaunchKernelGGL(pack_w_kernel, dim3((unsigned)pw.G, (unsigned)p.Ep), dim3(256), 0, st, pw);
    }
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_LORA_OK : hip_fail(e, "pack launch");
}

size_t moe_lora_packed_mxfp8_bytes(const moe_lora_dims *d, int which) {
    Plan p;
    if (make_plan(d, &p) != MOE_LORA_OK || d->H % 32 != 0 || d->I % 32 != 0) return 0;
    if (which == 0) return (size_t)(p.Ep * 2 * d->I / 16) * packed_mx_chunks(d->H) * 2048;
    if (which == 1) return (size_t)(p.Ep * d->H / 16) * packed_mx_chunks(d->I) * 2048;
    return 0;
}

int moe_lora_pack_mxfp8_weights(const moe_lora_dims *d, const void *w13, const void *w2, void *w13_packed,
                                void *w2_packed, void *stream) {
    Plan p;
    const int rc = make_plan(d, &p);
    if (rc != MOE_LORA_OK) return rc;
    if (d->H % 32 != 0 || d->I % 32 != 0) return MOE_LORA_EUNSUPPORTED;
    if ((w13 == nullptr) != (w13_packed == nullptr) || (w2 == nullptr) != (w2_packed == nullptr))
        return MOE_LORA_EINVAL;
    const void *ptrs[] = {w13, w2, w13_packed, w2_packed};
    for (const void *ptr : ptrs)
        if (ptr && !aligned(ptr, 16)) return MOE_LORA_EINVAL;
    if (!w13 && !w2) return MOE_LORA_OK;
    hipStream_t st = (hipStream_t)stream;
    for (int which = 0; which < 2; ++which) {
        const void *src = which ? w2 : w13;
        if (!src) continue;
        PackMxParams pm;
        pm.src = (const uint8_t *)src;
        pm.dst = (uint8_t *)(which ? w2_packed : w13_packed);
        pm.K = (int)(which ? d->I : d->H);
        pm.nch = (int)packed_mx_chunks(pm.K);
        pm.pieces = (int64_t)moe_lora_packed_mxfp8_bytes(d, which) / 16;
        const int64_t blocks = (pm.pieces + 255) / 256;
        hipLaunchKernelGGL(pack_mx_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, st, pm);
    }
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_LORA_OK : hip_fail(e, "pack mxfp8 launch");
}

int moe_lora_check_inputs(const moe_lora_dims *d, const moe_lora_args *a, int32_t *status, void *stream) {
    const int rc = moe_lora_check_args(d, a);
    if (rc != MOE_LORA_OK) return rc;
    if (!status) return MOE_LORA_EINVAL;
    Plan p;
    make_plan(d, &p);
    hipStream_t st = (hipStream_t)stream;
    CheckParams cp{};
    cp.status = status;
    if (d->T > 0) {
        if (a->workspace_bytes < sizeof(int32_t) * kCheckBlocks) return MOE_LORA_EWORKSPACE;
        cp.partial = (int32_t *)a->workspace;
        cp.logits = a->router_logits;
        cp.n_logits = (int64_t)d->T * d->E;
        cp.bias = a->expert_bias;
        cp.n_bias = a->expert_bias ? d->E : 0;
        cp.adapter_ids = p.lora ? a->adapter_ids : nullptr;
        cp.n_adapters = p.lora ? d->T : 0;
        cp.L = (int)p.La;
        if (a->weights_mxfp8) {
            const int64_t Ep = p.Ep, H = d->H, I = d->I;
            cp.mx[0] = (const uint8_t *)a->w13;
            cp.n_mx[0] = a->weights_packed ? (int64_t)moe_lora_packed_mxfp8_bytes(d, 0) : Ep * 2 * I * H;
            cp.mx[1] = (const uint8_t *)a->w13_scale;
            cp.n_mx[1] = Ep * 2 * I * (H / 32);
            cp.mx[2] = (const uint8_t *)a->w2;
            cp.n_mx[2] = a->weights_packed ? (int64_t)moe_lora_packed_mxfp8_bytes(d, 1) : Ep * H * I;
            cp.mx[3] = (const uint8_t *)a->w2_scale;
            cp.n_mx[3] = Ep * H * (I / 32);
        }
        hipLaunchKernelGGL(check_inputs_kernel, dim3(kCheckBlocks), dim3(256), 0, st, cp);
    }
    // with T = 0 the reduction alone writes a zero status
    hipLaunchKernelGGL(check_inputs_reduce_kernel, dim3(1), dim3(256), 0, st, cp);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_LORA_OK : hip_fail(e, "check_inputs launch");
}

int moe_lora_route(const moe_lora_dims *d, const float *logits, const float *expert_bias, int32_t *topk_ids,
                   float *topk_weights, void *stream) {
    if (!d) return MOE_LORA_EINVAL;
    if (d->T < 0 || d->E <= 0 || d->K <= 0 || d->K > d->E || d->S < 0) return MOE_LORA_EINVAL;
    if (d->router < MOE_LORA_ROUTER_TOPK || d->router > MOE_LORA_ROUTER_BIAS_SIGMOID) return MOE_LORA_EINVAL;
    if (expert_bias && d->router == MOE_LORA_ROUTER_TOPK) return MOE_LORA_EINVAL;
    if (d->E > 1024 || d->K > 64 || d->S > 64) return MOE_LORA_EUNSUPPORTED;
    if (!(std::isfinite(d->routed_scaling_factor) && d->routed_scaling_factor > 0.0f)) return MOE_LORA_EINVAL;
    if (d->renormalize != 0 && d->renormalize != 1) return MOE_LORA_EINVAL;
    if (d->T == 0) return MOE_LORA_OK;
    if (!logits || !topk_ids || !topk_weights) return MOE_LORA_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    launch_route(d, logits, expert_bias, topk_ids, topk_weights, st);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_LORA_OK : hip_fail(e, "route launch");
}

int moe_lora_align(const moe_lora_dims *d, const int32_t *topk_ids, const int32_t *adapter_ids,
                   int32_t *sorted_ids, int32_t *block_expert, int32_t *num_post_pad, int32_t *lora_items,
                   int32_t *num_items, void *workspace, size_t workspace_bytes, void *stream) {
    Plan p;
    const int rc = make_plan(d, &p);
    if (rc != MOE_LORA_OK) return rc;
    if (d->T == 0) return MOE_LORA_OK;
    if (!topk_ids || !sorted_ids || !block_expert || !num_post_pad || !workspace) return MOE_LORA_EINVAL;
    if (p.lora && (!adapter_ids || !lora_items || !num_items)) return MOE_LORA_EINVAL;
    if (lora_items && !aligned(lora_items, 16)) return MOE_LORA_EINVAL;
    if (!aligned(workspace, 256)) return MOE_LORA_EINVAL;
    if (workspace_bytes < p.align_total) return MOE_LORA_EWORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    char *ws = (char *)workspace;
    int32_t *tmp = (int32_t *)ws;
    int32_t *cnt = (int32_t *)(ws + round_up(sizeof(int32_t) * p.tmp_ints, 256));
    int r2 = launch_align(p, d, topk_ids, adapter_ids, sorted_ids, nullptr, block_expert, num_post_pad, lora_items,
                          num_items ? num_items : cnt + 1, tmp, nullptr, nullptr, st);
    if (r2 != MOE_LORA_OK) return r2;
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_LORA_OK : hip_fail(e, "align launch");
}

int moe_lora_forward(const moe_lora_dims *d, const moe_lora_args *a, void *stream) {
    const int rc = moe_lora_check_args(d, a);
    if (rc != MOE_LORA_OK) return rc;
    if (d->T == 0) return MOE_LORA_OK;
    Plan p;
    make_plan(d, &p);
    hipStream_t st = (hipStream_t)stream;
    char *ws = (char *)a->workspace;
    int32_t *ids = a->topk_ids_out ? a->topk_ids_out : (int32_t *)(ws + p.o_ids);
    float *wts = a->topk_weights_out ? a->topk_weights_out : (float *)(ws + p.o_w);
    // the alignment goes to the caller's buffers when they are given
    int32_t *sorted = a->sorted_ids_out ? a->sorted_ids_out : (int32_t *)(ws + p.o_sorted);
    int32_t *sadp = (int32_t *)(ws + p.o_sadp);
    int32_t *bexp = a->block_expert_out ? a->block_expert_out : (int32_t *)(ws + p.o_bexp);
    int32_t *cnt = (int32_t *)(ws + p.o_cnt);
    int32_t *items = (int32_t *)(ws + p.o_items);
    int32_t *tmp = (int32_t *)(ws + p.o_tmp);
    float *s13 = (float *)(ws + p.o_s13);
    float *s2 = (float *)(ws + p.o_s2);
    void *h = (void *)(ws + p.o_h);
    void *y2 = (void *)(ws + p.o_y2);
    const int H = (int)d->H, I = (int)d->I, r = (int)d->r;

    void **ev = a->stage_events;
    auto mark = [&](int slot) {
        if (ev) (void)hipEventRecord((hipEvent_t)ev[slot], st);
    };
    int32_t *tiles = (int32_t *)(ws + p.o_tiles);
    int32_t *queue = (int32_t *)(ws + p.o_queue);
    // with route_in_gemm the gate_up launch routes and aligns (both stages empty)
    mark(2 * MOE_LORA_STAGE_ROUTE);
    if (p.row_shrink) launch_route_shrink(p, d, a, ids, wts, s13, st);
    else if (!p.route_in_align && !p.route_in_gemm) launch_route(d, a->router_logits, a->expert_bias, ids, wts, st);
    mark(2 * MOE_LORA_STAGE_ROUTE + 1);
    const RouteParams rp_align = route_params(d, a->router_logits, a->expert_bias, ids, wts);
    mark(2 * MOE_LORA_STAGE_ALIGN);
    FusedRoute fused;
    if (p.route_in_gemm) {
        fused.ap = align_params(p, d, ids, a->adapter_ids, sorted, nullptr, bexp, cnt, items, cnt + 1, tmp, nullptr,
                                cnt + 2, a->num_post_pad_out, queue);
        fused.rp = rp_align;
        const int64_t Ep = p.Ep, H = d->H, I = d->I;
        const int64_t es = a->weights_mxfp8 ? 1 : 2;  // bytes per weight element (MXFP8 codes: 1)
        const int64_t b13 = a->weights_packed ? (int64_t)(a->weights_mxfp8 ? moe_lora_packed_mxfp8_bytes(d, 0)
                                                                            : moe_lora_packed_weight_bytes(d, 0))
                                              : Ep * 2 * I * H * es;
        const int64_t b2 = a->weights_packed ? (int64_t)(a->weights_mxfp8 ? moe_lora_packed_mxfp8_bytes(d, 1)
                                                                           : moe_lora_packed_weight_bytes(d, 1))
                                             : Ep * H * I * es;
        fused.touch13 = (const unsigned char *)a->w13;
        fused.touch2 = (const unsigned char *)a->w2;
        fused.stride13 = b13 / Ep;
        fused.stride2 = b2 / Ep;
    } else {
        const int r2 = launch_align(p, d, ids, a->adapter_ids, sorted, p.kind == 2 ? sadp : nullptr, bexp, cnt,
                                    items, cnt + 1, tmp, p.kind == 2 ? tiles : nullptr, cnt + 2, st,
                                    a->num_post_pad_out, queue, p.route_in_align ? &rp_align : nullptr);
        if (r2 != MOE_LORA_OK) return r2;
    }
    // the tiled GEMM reads x gathered and packed per sorted row; with LoRA
    // the pack shares one launch with the gate_up shrink (stage SHRINK13)
    PackXParams xp;
    xp.x = (const uint16_t *)a->hidden;
    xp.sorted_ids = sorted;
    xp.counters = cnt;
    xp.xp = (uint16_t *)(ws + p.o_xp);
    xp.H = H;
    xp.P = (int)p.P;
    xp.Kp = (int)p.Kp;
    if (p.kind == 2 && !p.lora)
        hipLaunchKernelGGL(pack_x_kernel, dim3((unsigned)(p.cap / 16)), dim3(256), 0, st, xp);
    mark(2 * MOE_LORA_STAGE_ALIGN + 1);

    if (p.kind == 0) {
        // fp32 path
        mark(2 * MOE_LORA_STAGE_SHRINK13);
        if (p.lora)
            hipLaunchKernelGGL(shrink_f32_kernel, dim3((unsigned)p.max_items), dim3(256), 0, st,
                               (const float *)a->hidden, sorted, (const float *)a->a13, items, cnt, s13, H, r,
                               (int)p.Ep, (int)p.Kp, 1);
        mark(2 * MOE_LORA_STAGE_SHRINK13 + 1);
        F32Params fp;
        fp.sorted_ids = sorted;
        fp.block_expert = bexp;
        fp.counters = cnt;
        fp.adapter_ids = a->adapter_ids;
        fp.Kp = (int)p.Kp;
        fp.P = (int)p.P;
        fp.cap = (int)p.cap;
        fp.Ep = (int)p.Ep;
        fp.r = r;
        fp.L = (int)p.La;
        fp.lora = p.lora ? 1 : 0;
        fp.bt = p.bm;
        fp.in = (const float *)a->hidden;
        fp.W = (const float *)a->w13;
        fp.B = (const float *)a->b13;
        fp.s = s13;
        fp.out = (float *)h;
        fp.Kdim = H;
        fp.Nout = I;
        mark(2 * MOE_LORA_STAGE_GATE_UP);
        hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3((unsigned)((I + 63) / 64), (unsigned)p.max_blocks),
                           dim3(256), 0, st, fp);
        mark(2 * MOE_LORA_STAGE_GATE_UP + 1);
        mark(2 * MOE_LORA_STAGE_SHRINK2);
        if (p.lora)
            hipLaunchKernelGGL(shrink_f32_kernel, dim3((unsigned)p.max_items), dim3(256), 0, st,
                               (const float *)h, sorted, (const float *)a->a2, items, cnt, s2, I, r, (int)p.Ep,
                               (int)p.Kp, 0);
        mark(2 * MOE_LORA_STAGE_SHRINK2 + 1);
        fp.in = (const float *)h;
        fp.W = (const float *)a->w2;
        fp.B = (const float *)a->b2;
        fp.s = s2;
        fp.out = (float *)y2;
        fp.Kdim = I;
        fp.Nout = H;
        mark(2 * MOE_LORA_STAGE_DOWN);
        hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3((unsigned)((H + 63) / 64), (unsigned)p.max_blocks),
                           dim3(256), 0, st, fp);
        mark(2 * MOE_LORA_STAGE_DOWN + 1);
        mark(2 * MOE_LORA_STAGE_COMBINE);
        hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)((H / kCombineVec<false> + 255) / 256), (unsigned)d->T), dim3(256),
                           0, st, y2, wts, a->out, (int)d->T, H, (int)p.Kp, d->routed_scaling_factor);
        mark(2 * MOE_LORA_STAGE_COMBINE + 1);
    } else {
        ShrinkParams sp;
        sp.sorted_ids = sorted;
        sp.items = items;
        sp.counters = cnt;
        sp.r = r;
        sp.Ep = (int)p.Ep;
        sp.Kp = (int)p.Kp;
        sp.P = (int)p.P;
        sp.cap = (int)p.cap;
        sp.out_bf16 = p.kind == 2 ? 1 : 0;
        sp.in_packed = p.kind == 2 ? 1 : 0;  // the tiled GEMM keeps h packed
        mark(2 * MOE_LORA_STAGE_SHRINK13);
        if (p.lora && !p.row_shrink) {  // row_shrink: done in the router launch
            sp.in = (const uint16_t *)a->hidden;
            sp.A = (const uint16_t *)a->a13;
            sp.s_part = s13;
            sp.Kdim = H;
            if (p.kind == 2) launch_pack_shrink(p, xp, sp, r, st);
            else launch_shrink(p, sp, true, r, st);
        }
        mark(2 * MOE_LORA_STAGE_SHRINK13 + 1);
        GemmParams gp;
        gp.sorted_ids = sorted;
        gp.sorted_adapter = sadp;
        gp.block_expert = bexp;
        gp.counters = cnt;
        gp.adapter_ids = a->adapter_ids;
        gp.Kp = (int)p.Kp;
        gp.P = (int)p.P;
        gp.cap = (int)p.cap;
        gp.Ep = (int)p.Ep;
        gp.r = r;
        gp.L = (int)p.La;
        gp.split = p.row_shrink ? 1 : p.split;  // s13 by pair is unsplit
        gp.lora = p.lora ? 1 : 0;
        gp.in = (p.kind == 2) ? (const uint16_t *)(ws + p.o_xp) : (const uint16_t *)a->hidden;
        gp.W = (const uint16_t *)a->w13;
        gp.Wscale = a->weights_mxfp8 ? (const uint8_t *)a->w13_scale : nullptr;
        mark(2 * MOE_LORA_STAGE_GATE_UP);
        gp.B = (const uint16_t *)a->b13;
        gp.s_part = s13;
        gp.s_by_pair = p.row_shrink ? 1 : 0;
        gp.out = h;
        gp.Kdim = H;
        gp.Nout = I;
        launch_gemm<true>(p, gp, tiles, cnt + 2, queue, a->weights_packed != 0, st,
                          p.route_in_gemm ? &fused : nullptr);
        mark(2 * MOE_LORA_STAGE_GATE_UP + 1);
        mark(2 * MOE_LORA_STAGE_SHRINK2);
        if (p.lora) {
            sp.in = (const uint16_t *)h;
            sp.A = (const uint16_t *)a->a2;
            sp.s_part = s2;
            sp.Kdim = I;
            launch_shrink(p, sp, false, r, st);
        }
        mark(2 * MOE_LORA_STAGE_SHRINK2 + 1);
        gp.in = (const uint16_t *)h;
        gp.W = (const uint16_t *)a->w2;
        gp.Wscale = a->weights_mxfp8 ? (const uint8_t *)a->w2_scale : nullptr;
        gp.B = (const uint16_t *)a->b2;
        gp.s_part = s2;
        gp.s_by_pair = 0;
        gp.split = p.split;
        gp.out = y2;
        gp.Kdim = I;
        gp.Nout = H;
        mark(2 * MOE_LORA_STAGE_DOWN);
        launch_gemm<false>(p, gp, tiles, cnt + 2, queue, a->weights_packed != 0, st);
        mark(2 * MOE_LORA_STAGE_DOWN + 1);
        mark(2 * MOE_LORA_STAGE_COMBINE);
        hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)((H / kCombineVec<true> + 255) / 256), (unsigned)d->T), dim3(256),
                           0, st, y2, wts, a->out, (int)d->T, H, (int)p.Kp, d->routed_scaling_factor);
        mark(2 * MOE_LORA_STAGE_COMBINE + 1);
    }
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_LORA_OK : hip_fail(e, "forward launch");
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
int scratch_ptr(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return MOE_LORA_EUNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr || !aligned(ptr, 256)) return hip_fail(hipErrorInvalidSymbol, "scratch address");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MOE_LORA_OK;
}
}  // namespace

int moe_lora_forward_static(const moe_lora_dims *d, const moe_lora_args *a, void *stream) {
    Plan p;
    const int rc = make_plan(d, &p);
    if (rc != MOE_LORA_OK) return rc;
    if (!a) return MOE_LORA_EINVAL;
    if (d->T == 0) return MOE_LORA_OK;
    if (p.total > (size_t)MOE_LORA_STATIC_SCRATCH_BYTES) return MOE_LORA_EWORKSPACE;
    moe_lora_args b = *a;
    // argument checks first (pure host), with a stand-in for the scratch address
    b.workspace = (void *)(uintptr_t)256;
    b.workspace_bytes = MOE_LORA_STATIC_SCRATCH_BYTES;
    const int rc2 = moe_lora_check_args(d, &b);
    if (rc2 != MOE_LORA_OK) return rc2;
    const int rc3 = scratch_ptr(&b.workspace);
    if (rc3 != MOE_LORA_OK) return rc3;
    return moe_lora_forward(d, &b, stream);
}

const char *moe_lora_strerror(int code) {
    switch (code) {
        case MOE_LORA_OK: return "ok";
        case MOE_LORA_EINVAL: return "invalid argument (null pointer, bad size, K > E, rsf <= 0 or misaligned pointer)";
        case MOE_LORA_EUNSUPPORTED: return "unsupported configuration (dtype, H or I not a multiple of 8, or a size limit)";
        case MOE_LORA_EWORKSPACE: return "workspace too small";
        case MOE_LORA_EHIP: return g_errbuf[0] ? g_errbuf : "HIP error";
        default: return "unknown error code";
    }
}

}  // extern "C"
