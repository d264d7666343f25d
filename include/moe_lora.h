/*
 * moe_lora.h -- C ABI of the fused MoE-LoRA layer for MI355X (gfx950).
 *
 * One layer call computes, for T tokens with hidden size H:
 *   1. top-K routing over E routed experts from fp32 router logits, softmax
 *      weights over the selected logits, and S always-on shared experts
 *      appended as extra slots after the routed ones (ids E..E+S-1, weight
 *      1/routed_scaling_factor)                           [moe_lora_route]
 *   2. alignment of the T*(K+S) (token, slot) pairs by expert over the
 *      E+S stacked w13 rows, padded per expert to the GEMM block, with the
 *      pairs of each expert grouped by adapter           [moe_lora_align]
 *   3. per pair: g = W13[e] x (+ B13[a,e] A13[a,e] x), h = silu(g_gate) *
 *      g_up, y = W2[e] h (+ B2[a,e] A2[a,e] h), and out = rsf * sum_j w_j y_j
 *                                                       [moe_lora_forward]
 * Sources of the method:
 *   - aitrends.kr summary of the AWS post on multi-LoRA serving of MoE
 *     models in vLLM, "section details": routing and adapter choice are two
 *     sparsities at once; LoRA shrink and expand are fused into every expert
 *     projection; layers without LoRA exit at once; skinny LoRA products use
 *     split-K; the LoRA sum is folded into the expand step.  "Image
 *     analysis", diagram: an adapter path on gate_up and on down.
 *   - secrett2633 analysis of vLLM PR 46545 ("vLLM ROCm shared-expert
 *     fusion"), "code analysis" parts 1-2: shared slots appended after the
 *     routed top-k with ids from the routed expert count upward and one
 *     constant weight; the alignment expert count is the number of stacked
 *     w13 rows.  "Lessons" item 2: that weight is 1/routed_scaling_factor.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major and contiguous,
 *     16-byte aligned.  The caller owns every buffer; the library never
 *     allocates or frees device memory and keeps no state between calls.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued; no call synchronises the host or copies device data back,
 *     so a call can be captured into a HIP graph.  Inputs must stay alive
 *     until the stream reaches the call.
 *   - Return value: MOE_LORA_OK, or a negative code below.  Nothing is
 *     enqueued when argument checking fails.  Preconditions NOT checked on
 *     the device by the layer: router logits are finite; adapter ids lie in
 *     [-1, L) (moe_lora_check_inputs tests both on request).
 *   - T may be 0: the call is a no-op returning MOE_LORA_OK.
 *   - Concurrent calls are safe when they use distinct workspaces.
 */
#ifndef MOE_LORA_H
#define MOE_LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_LORA_OK 0
#define MOE_LORA_EINVAL (-1)       /* null pointer, bad size, K > E, rsf <= 0, misaligned pointer */
#define MOE_LORA_EUNSUPPORTED (-2) /* dtype, H or I not a multiple of 8, limits below exceeded */
#define MOE_LORA_EWORKSPACE (-3)   /* workspace smaller than moe_lora_workspace_bytes() */
#define MOE_LORA_EHIP (-4)         /* a HIP launch failed; moe_lora_strerror() has the text */

#define MOE_LORA_F32 0
#define MOE_LORA_BF16 1

/* Stages of moe_lora_forward, in launch order (for moe_lora_args.stage_events).
 * A stage launches nothing when its work runs in another stage's launch:
 * with the streaming GEMM (gemm_kind 1) and LoRA the gate_up shrink runs in
 * the router's launch (SHRINK13 empty); small calls otherwise route inside
 * the alignment's launch (ROUTE empty); tiny calls without LoRA (T <= 4, at
 * most 64 (token, slot) pairs, E <= 256) route and align inside the gate_up
 * launch (ROUTE and ALIGN empty).  With the LDS-tiled GEMM (gemm_kind 2) x
 * is gathered and packed into sorted-row order: in the same launch as the
 * gate_up shrink (stage SHRINK13) when LoRA is active, else as a second
 * launch of stage ALIGN.  ALIGN is one launch below 8192 pairs and four from
 * there on; every other stage is at most one kernel. */
#define MOE_LORA_STAGE_ROUTE 0
#define MOE_LORA_STAGE_ALIGN 1
#define MOE_LORA_STAGE_SHRINK13 2
#define MOE_LORA_STAGE_GATE_UP 3
#define MOE_LORA_STAGE_SHRINK2 4
#define MOE_LORA_STAGE_DOWN 5
#define MOE_LORA_STAGE_COMBINE 6
#define MOE_LORA_NUM_STAGES 7

/* Sizes and knobs of one layer call.
 *   T  tokens (>= 0)             H  hidden size (multiple of 8)
 *   I  expert intermediate size (multiple of 8); w13 holds 2I rows: gate
 *      rows [0, I) then up rows [I, 2I)
 *   E  routed experts (1..1024)  K  routed top-k (1..min(E, 64))
 *   S  shared experts appended as slots K..K+S-1 (0..64)
 *   L  LoRA adapters (>= 0)      r  LoRA rank (0..128); LoRA is active iff
 *      L > 0 and r > 0
 *   routed_scaling_factor  rsf > 0: shared slots get weight 1/rsf (fp32
 *      division) and the whole combine is multiplied by rsf
 *   renormalize  1: softmax over the K selected logits; 0: softmax over all
 *      E logits, taken at the K selected ones
 *   dtype  MOE_LORA_BF16 (bf16 tensors, fp32 accumulation) or MOE_LORA_F32
 *   block_m  token rows per GEMM tile; 0 = library choice from the
 *      average rows per expert.  16 or 32: streaming GEMM, experts padded to
 *      block_m rows.  128 or 256 (bf16 layers only, MOE_LORA_EUNSUPPORTED for
 *      fp32): LDS-tiled GEMM, experts padded to 32 rows and cut into tiles
 *      of at most block_m rows; it takes MXFP8 weights with H, I <= 3072
 *   lora_block_m  rows per LoRA shrink work item; 0 = library choice, else
 *      16 or 32 (32 needs r <= 64)
 *   router  MOE_LORA_ROUTER_TOPK (0): top-K of the logits, weights as under
 *      renormalize.  MOE_LORA_ROUTER_BIAS_SOFTMAX (1) / _SIGMOID (2): the
 *      biased top-k router.  The PR 46545 analysis ("code analysis" part 1)
 *      names a biased top-k router module without defining it; the reading
 *      implemented: fp64 score s_e per expert (softmax over all E logits,
 *      or the sigmoid of the logit), the K experts with the largest
 *      s_e + bias_e chosen (lower index on an exact tie, slot order =
 *      choice order), weights = the unbiased scores of the chosen experts,
 *      divided by their slot-order sum when renormalize = 1, rounded once
 *      to fp32.  The bias (moe_lora_args.expert_bias, may be NULL = 0)
 *      steers the choice only
 *   split_k  K-splits of the LoRA shrink; 0 = library choice, else 1..16.
 *      Applies to the streaming GEMM only: with the LDS-tiled GEMM the
 *      shrink runs unsplit (the plan reports 1).  With 0 on the streaming
 *      GEMM (and K+S <= 64, r <= 64) the gate_up shrink runs per pair inside
 *      the router's launch and only the down shrink uses the split
 * Limits: (E+S) * (La+1) <= 16384 where La = L if LoRA is active else 0;
 *   L <= 1024; T*(K+S) < 2^31 - 1. */
typedef struct moe_lora_dims {
    int64_t T, H, I, E, K, S, L, r;
    float routed_scaling_factor;
    int32_t renormalize;
    int32_t dtype;
    int32_t block_m;
    int32_t lora_block_m;
    int32_t split_k;
    int32_t router;
} moe_lora_dims;

#define MOE_LORA_ROUTER_TOPK 0
#define MOE_LORA_ROUTER_BIAS_SOFTMAX 1
#define MOE_LORA_ROUTER_BIAS_SIGMOID 2

/* What the library will do for a given moe_lora_dims (filled by
 * moe_lora_plan_query).  block_m / lora_block_m / max_blocks /
 * sorted_capacity / max_items also size the outputs of moe_lora_align. */
typedef struct moe_lora_plan {
    int32_t block_m;         /* alignment block: each expert group is padded to a multiple of it */
    int32_t tile_m;          /* token rows per GEMM tile */
    int32_t lora_block_m;    /* rows per LoRA work item */
    int32_t split_k;         /* LoRA shrink K-splits */
    int32_t gemm_kind;       /* 0 = fp32 path, 1 = bf16 streaming, 2 = bf16 LDS-tiled */
    int64_t max_blocks;      /* ceil(P/block_m) + min(E+S, P), P = T*(K+S) */
    int64_t sorted_capacity; /* max_blocks * block_m */
    int64_t max_items;       /* ceil(P/lora_block_m) + min(P, L*(E+S)); 0 without LoRA */
    size_t workspace_bytes;       /* for moe_lora_forward */
    size_t align_workspace_bytes; /* for moe_lora_align */
} moe_lora_plan;

/* Device buffers of one layer call.
 *   hidden [T,H] dtype;  router_logits [T,E] f32;  adapter_ids [T] i32
 *     (-1 = no LoRA for that token; may be NULL when LoRA is inactive)
 *   w13 [E+S, 2I, H] dtype;  w2 [E+S, H, I] dtype
 *   a13 [L, E+S, r, H];  b13 [L, E+S, 2I, r];  a2 [L, E+S, r, I];
 *   b2 [L, E+S, H, r]   (dtype; may all be NULL when LoRA is inactive)
 *   out [T, H] dtype (written)
 *   workspace: device scratch of at least moe_lora_workspace_bytes(),
 *     256-byte aligned; contents on entry do not matter
 *   topk_ids_out [T, K+S] i32, topk_weights_out [T, K+S] f32: optional
 *     (NULL = not written) copies of the routing decisions
 *   stage_events: optional (NULL = none) array of 2*MOE_LORA_NUM_STAGES
 *     hipEvent_t handles created by the caller; the call records
 *     stage_events[2s] on `stream` right before stage s and
 *     stage_events[2s+1] right after it (both back to back for a stage that
 *     launches nothing), so the caller can time each kernel on the stream it
 *     runs on.  Stages: see MOE_LORA_STAGE_*.
 *   weights_packed: 0 = w13 and w2 as above; 1 = w13 and w2 are the packed
 *     copies written by moe_lora_pack_weights (bf16), or with weights_mxfp8
 *     the packed codes written by moe_lora_pack_mxfp8_weights.
 *   weights_mxfp8: 0 = w13 and w2 in dtype as above; 1 = MXFP8 expert
 *     weights (MX block scaling, the precision of the ROCm shared-expert
 *     fusion path in the secrett2633 analysis of vLLM PR 46545, "code
 *     analysis" part 2): w13 [E+S, 2I, H] and w2 [E+S, H, I] hold one FP8
 *     E4M3 code per element (1 byte, 16-byte aligned), w13_scale
 *     [E+S, 2I, H/32] and w2_scale [E+S, H, I/32] (16-byte aligned) one
 *     E8M0 scale byte per 32 consecutive elements along the reduction;
 *     element = code *
 *     2^(scale - 127).  Activations, LoRA stacks and the output stay bf16,
 *     and the products run in bf16 on the exactly converted weights.
 *     Preconditions (not checked on the device): scale bytes in [1, 254],
 *     codes not NaN (0x7F, 0xFF).  Needs dtype bf16, H and I multiples
 *     of 32, and H, I at most 8192 on the streaming GEMM (plan gemm_kind 1)
 *     or at most 3072 on the LDS-tiled GEMM (gemm_kind 2, which converts
 *     each weight fragment in registers right before its products; pass
 *     block_m 16 or 32 for longer rows), else MOE_LORA_EUNSUPPORTED; NULL or
 *     misaligned scales give MOE_LORA_EINVAL.
 *   expert_bias [E] f32: the per-expert bias of the biased router
 *     (dims.router 1 or 2; NULL = all zero); must be NULL with router 0.
 *   sorted_ids_out [sorted_capacity], block_expert_out [max_blocks],
 *     num_post_pad_out [1] (i32, sizes from moe_lora_plan_query, 4-byte
 *     aligned): optional (NULL = kept in the workspace) outputs of the
 *     alignment step, in the layout moe_lora_align documents; the layer
 *     then uses these buffers in place of its workspace copies. */
typedef struct moe_lora_args {
    const void *hidden;
    const float *router_logits;
    const int32_t *adapter_ids;
    const void *w13;
    const void *w2;
    const void *a13;
    const void *b13;
    const void *a2;
    const void *b2;
    void *out;
    void *workspace;
    size_t workspace_bytes;
    int32_t *topk_ids_out;
    float *topk_weights_out;
    void **stage_events;
    int32_t weights_packed;
    int32_t weights_mxfp8;
    const void *w13_scale;
    const void *w2_scale;
    const float *expert_bias;
    int32_t *sorted_ids_out;
    int32_t *block_expert_out;
    int32_t *num_post_pad_out;
} moe_lora_args;

/* Validate dims and describe the plan.  Pure host code: touches no device
 * and may be called on a machine without a GPU.  Returns MOE_LORA_OK,
 * MOE_LORA_EINVAL or MOE_LORA_EUNSUPPORTED; `plan` is written only on OK. */
int moe_lora_plan_query(const moe_lora_dims *dims, moe_lora_plan *plan);

/* Workspace bytes moe_lora_forward needs for `dims`; 0 when dims are
 * invalid.  Pure host code. */
size_t moe_lora_workspace_bytes(const moe_lora_dims *dims);

/* Full argument check of a moe_lora_forward call (null pointers, sizes,
 * alignment, workspace size).  Pure host code: dereferences no pointer and
 * touches no device. */
int moe_lora_check_args(const moe_lora_dims *dims, const moe_lora_args *args);

/* Step 1 alone: top-K routing plus shared-slot append.
 *   logits [T,E] f32 in; expert_bias [E] f32 in (biased router only, may be
 *   NULL; must be NULL with router 0); topk_ids [T,K+S] i32 and
 *   topk_weights [T,K+S] f32 out.  Router 0: larger logit first, lower
 *   expert index on an exact tie (+0 == -0); slot order = selection order;
 *   weights: fp64 softmax rounded once to fp32.  Routers 1 and 2: see
 *   moe_lora_dims.router.  Only T, E, K, S, routed_scaling_factor,
 *   renormalize and router of `dims` are read. */
int moe_lora_route(const moe_lora_dims *dims, const float *logits, const float *expert_bias,
                   int32_t *topk_ids, float *topk_weights, void *stream);

/* Step 2 alone: alignment of the pairs f = t*(K+S) + j by expert.
 * The pages fix only the expert count (the number of stacked w13 rows, PR
 * 46545 analysis, "code analysis" part 2); the order inside an expert, the
 * padding and the LoRA work list are this library's layout, chosen so that
 * one sorted list serves the base GEMM (contiguous, padded expert groups)
 * and the LoRA shrink/expand (contiguous (adapter, expert) runs) at once.
 * In particular there are no separate LoRA-sorted arrays (a second sorted
 * id list, block adapter/expert maps and padded count per LoRA block): the
 * (adapter, expert) runs inside sorted_ids, listed by lora_items, take their
 * place.  moe_lora_forward can write the same sorted_ids, block_expert and
 * num_post_pad to caller buffers (moe_lora_args.*_out).
 *   topk_ids [T,K+S] i32 in (values in [0, E+S)); adapter_ids [T] i32 in
 *   (ignored when LoRA is inactive).
 *   sorted_ids [sorted_capacity]: pairs of expert 0, then expert 1, ...;
 *     inside an expert ordered by adapter (no-LoRA first) then by f; each
 *     expert group padded to a multiple of block_m with the sentinel
 *     P = T*(K+S); the tail after num_post_pad also holds P.
 *   block_expert [max_blocks]: expert of each block_m-row block, -1 after
 *     the last used block.
 *   num_post_pad [1]: padded row count.
 *   lora_items [max_items][4] (start row, rows, adapter, expert): the
 *     (adapter >= 0, expert) runs of sorted_ids in key order, cut into pieces
 *     of at most lora_block_m rows; tail (0, 0, -1, -1).  May be NULL when
 *     LoRA is inactive.  num_items [1]: item count (may be NULL likewise).
 *   workspace: at least align_workspace_bytes of the plan. */
int moe_lora_align(const moe_lora_dims *dims, const int32_t *topk_ids, const int32_t *adapter_ids,
                   int32_t *sorted_ids, int32_t *block_expert, int32_t *num_post_pad,
                   int32_t *lora_items, int32_t *num_items, void *workspace,
                   size_t workspace_bytes, void *stream);

/* The whole layer (steps 1-3), enqueued on `stream`. */
int moe_lora_forward(const moe_lora_dims *dims, const moe_lora_args *args, void *stream);

/* moe_lora_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc.  The layer's scratch is a fixed device array of
 * MOE_LORA_STATIC_SCRATCH_BYTES (64 MiB) inside the library, one per GPU,
 * created when the library is first used on that GPU and held until the
 * process ends; args->workspace and args->workspace_bytes are ignored.  The
 * call allocates nothing and otherwise behaves as moe_lora_forward (same
 * arguments, checks, kernels and bits).  The stream must belong to the
 * current device.  Returns MOE_LORA_EWORKSPACE when the plan's workspace
 * (moe_lora_workspace_bytes) exceeds the array, before anything is
 * enqueued.  Every call on one GPU uses the same array: calls that can run
 * at the same time on one GPU (other streams, other host threads without
 * ordering) race and must be serialised by the caller; a call may follow
 * another on the same stream freely. */
#define MOE_LORA_STATIC_SCRATCH_BYTES (64u << 20)
int moe_lora_forward_static(const moe_lora_dims *dims, const moe_lora_args *args, void *stream);

/* Check of the input preconditions moe_lora_forward does not check on the
 * device, for debugging a caller.  The logits feed the top-k softmax of step
 * 1 and each adapter id picks one of the L adapters (or none) of step 3
 * (sources above); the MXFP8 conditions are those of the weight format
 * under moe_lora_args.weights_mxfp8.  Checked: every router logit (and
 * every expert_bias value, when given) finite (MOE_LORA_BAD_LOGIT); with LoRA
 * active every adapter id in [-1, L); with weights_mxfp8 every scale byte in
 * [1, 254] and no NaN code (0x7F, 0xFF).  Reads the same `args` as
 * moe_lora_forward (only router_logits, adapter_ids, w13, w2 and the scale
 * pointers) and uses the first 2 KiB of args->workspace as scratch.
 * Enqueued on `stream` (two small launches, no host synchronisation, no
 * allocation, so it can be captured in a graph like the forward):
 * when the stream reaches it, *status (device int32, caller-owned) holds the
 * OR of MOE_LORA_BAD_LOGIT, MOE_LORA_BAD_ADAPTER and MOE_LORA_BAD_MXFP8
 * for the violations found, 0 when none.  Returns MOE_LORA_OK, or
 * MOE_LORA_EINVAL / MOE_LORA_EUNSUPPORTED / MOE_LORA_EWORKSPACE from the
 * same checks as moe_lora_check_args (a workspace of at least 2 KiB), or
 * MOE_LORA_EINVAL for a null `status`; MOE_LORA_EHIP on a launch failure.
 * T = 0 writes 0 to *status. */
#define MOE_LORA_BAD_LOGIT 1
#define MOE_LORA_BAD_ADAPTER 2
#define MOE_LORA_BAD_MXFP8 4
int moe_lora_check_inputs(const moe_lora_dims *dims, const moe_lora_args *args, int32_t *status, void *stream);

/* Packed MXFP8 codes.  An optional one-time re-layout of the E4M3 code
 * matrices of moe_lora_args.weights_mxfp8 (w13 [E+S,2I,H], w2 [E+S,H,I],
 * uint8): for every 16 consecutive rows of an expert and every 128-wide
 * chunk c of the reduction, one 2 KiB block whose byte 16*(64*q + 16*g + r)
 * starts the 16 codes 128c + 32g + 16q .. +15 of row r (q in {0,1}, g in
 * 0..3, zeros past the reduction length), the order in which the streaming
 * GEMM loads them.  With weights_packed = 1 and weights_mxfp8 = 1, w13 and
 * w2 point at these copies (the scales stay row-major); results are
 * bit-identical to the row-major codes.
 *   moe_lora_packed_mxfp8_bytes: bytes of the packed w13 (which = 0) or w2
 *   (which = 1); 0 when the shape has no MXFP8 form (H or I not a multiple
 *   of 32) or another value of `which`.
 *   moe_lora_pack_mxfp8_weights: enqueues the copy on `stream`; a NULL
 *   source with a NULL destination skips that matrix.  MOE_LORA_EINVAL for
 *   a source without a destination (or the reverse) or a pointer not 16-byte
 *   aligned, MOE_LORA_EUNSUPPORTED for H or I not a multiple of 32, the
 *   dims' own error codes, MOE_LORA_EHIP on a launch failure.  Buffers are
 *   caller-owned device memory. */
size_t moe_lora_packed_mxfp8_bytes(const moe_lora_dims *dims, int which);
int moe_lora_pack_mxfp8_weights(const moe_lora_dims *dims, const void *w13, const void *w2, void *w13_packed,
                                void *w2_packed, void *stream);

/* Packed expert weights (bf16 only).  An optional one-time re-layout of w13
 * and w2 (for example at model load) into the order the GEMM kernels read:
 * rows in groups of 16 and the reduction dimension in slabs of 32, one
 * 1 KiB block per (group, slab), so each load instruction of a wavefront
 * reads 1 KiB contiguously instead of 16 rows x 64 bytes.  The layer's
 * arithmetic does not change: moe_lora_forward with weights_packed = 1 gives
 * the same bits as with the row-major weights.
 *
 * Layout.  Inside a block, element (r, k), r in [0,16), k in [0,32), is at
 * element index (k/8)*128 + r*8 + k%8.  Blocks are ordered
 * [expert][group][slab]; elements past the matrix edge are zero.
 *   w13 (G = 16*ceil(I/128) groups, ceil(H/32) slabs): row r of group q
 *     holds feature f = 8q + 2*(r/4) + r%2 of the gate half (r%4 < 2, row f
 *     of w13[e]) or of the up half (r%4 >= 2, row I+f), so each group
 *     carries the gate and up rows of 8 features; K = H.
 *   w2 (G = 16*ceil(H/256) groups, ceil(I/32) slabs): row r of group q is
 *     row 16q + r of w2[e]; K = I.
 *   (G rounds the group count up to whole 256-row GEMM tiles; groups past
 *   the last feature or row are zero.)
 * The interleave of gate and up rows is a property of the layout only: the
 * packed w13 is read as w13, with the same meaning.
 *
 * moe_lora_packed_weight_bytes: size of the packed w13 (which = 0) or w2
 * (which = 1); 0 for invalid dims or a dtype other than bf16.  Pure host
 * code.
 * moe_lora_pack_weights: writes w13_packed from w13 and w2_packed from w2
 * (either pair may be NULL to skip it) on `stream`.  Buffers: device
 * memory, 16-byte aligned, sizes as above; the source and the packed copy
 * must not overlap.  Returns MOE_LORA_OK, MOE_LORA_EINVAL (bad pointers),
 * MOE_LORA_EUNSUPPORTED (dims or dtype) or MOE_LORA_EHIP. */
size_t moe_lora_packed_weight_bytes(const moe_lora_dims *dims, int which);
int moe_lora_pack_weights(const moe_lora_dims *dims, const void *w13, const void *w2, void *w13_packed,
                          void *w2_packed, void *stream);

/* Text for a return code.  For MOE_LORA_EHIP it includes the HIP error of
 * the failing call on this thread.  Never NULL. */
const char *moe_lora_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LORA_H */
