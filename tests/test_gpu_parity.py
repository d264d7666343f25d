"""GPU parity of the HIP path against the fp64 oracle, called through the C ABI.

Routing and alignment must match the oracle bit for bit; the layer output must
match within max-abs 2e-2 and relative L2 1e-2 (bf16) or 1e-5 (fp32); the
LoRA delta (output minus the no-LoRA output) is checked on its own so that a
missing LoRA term cannot hide inside the absolute tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import lora_expert_gemm_topk_amd as ml
from lora_expert_gemm_topk_amd import synth
from tests.gpu_util import LORA_DELTA_RELL2, assert_close, errs, inputs, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


# --------------------------------------------------------------------- route

ROUTE_CASES = [
    dict(T=16, E=4, K=2), dict(T=64, E=32, K=4), dict(T=4096, E=32, K=4),
    dict(T=128, E=64, K=8, S=1, rsf=2.5), dict(T=33, E=300, K=5), dict(T=3, E=1000, K=64, S=2),
    dict(T=50, E=12, K=3, renorm=0), dict(T=1, E=1, K=1), dict(T=8192, E=128, K=8, zipf=True),
    # K = E: every expert selected, in value order
    dict(T=20, E=8, K=8), dict(T=7, E=64, K=64, S=1, rsf=2.0), dict(T=9, E=40, K=40, renorm=0),
]


@pytest.mark.parametrize("c", ROUTE_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_route_bitexact(c):
    T, E, K, S = c["T"], c["E"], c["K"], c.get("S", 0)
    rsf, rn = c.get("rsf", 1.0), c.get("renorm", 1)
    g = torch.Generator().manual_seed(T * 7 + E)
    lg = torch.randn(T, E, generator=g)
    if c.get("zipf"):
        lg += -1.1 * torch.log(torch.randperm(E, generator=g).float() + 1.0)
    say("route", c)
    ids, w = ml.moe_lora_route(lg.to(DEV), K, S, rsf, rn)
    torch.cuda.synchronize()
    oids, ow = oracle.route(lg.numpy(), K, S, rsf, rn)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.array_equal(_bits(w), ow.view(np.int32))


def test_route_ties_bitexact():
    g = torch.Generator().manual_seed(5)
    lg = (torch.randint(-3, 4, (300, 40), generator=g).float() * 0.5)
    lg[::7] = 0.0
    lg[1::7] = -0.0
    say("route ties")
    ids, w = ml.moe_lora_route(lg.to(DEV), 6)
    torch.cuda.synchronize()
    oids, ow = oracle.route(lg.numpy(), 6)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.array_equal(_bits(w), ow.view(np.int32))


def test_route_signed_zero_ties_bitexact():
    """+0 and -0 mixed inside rows (they tie and the lower index goes first),
    two logits per lane (E = 100), with and without renormalisation."""
    g = torch.Generator().manual_seed(17)
    lg = torch.randint(-2, 3, (200, 100), generator=g).float() * 0.5
    neg = torch.rand(200, 100, generator=g) < 0.5
    lg[(lg == 0) & neg] = -0.0
    assert bool((torch.signbit(lg) & (lg == 0)).any()) and bool((~torch.signbit(lg) & (lg == 0)).any())
    for rn in (1, 0):
        say("route signed zeros", rn)
        ids, w = ml.moe_lora_route(lg.to(DEV), 7, 1, 2.5, rn)
        torch.cuda.synchronize()
        oids, ow = oracle.route(lg.numpy(), 7, 1, 2.5, rn)
        assert np.array_equal(ids.cpu().numpy(), oids)
        assert np.array_equal(_bits(w), ow.view(np.int32))


# --------------------------------------------------------------------- align

def _align_case(T, E, K, S, L, r, seed, bm=0, lbm=0, adapters="uniform_all", logits="normal", one_expert=False):
    shape = synth.LayerShape(T=T, H=64, I=64, E=E, K=K, S=S, L=L, r=r)
    inp = synth.make_inputs(shape, synth.Recipe(adapters=adapters, logits=logits), seed=seed)
    ids, _ = oracle.route(inp.logits.numpy(), K, S)
    if one_expert:
        ids[:, 0] = 0
    dims = ml.make_dims(T, 64, 64, E, K, S, L, r, block_m=bm, lora_block_m=lbm)
    return ids, inp.adapter_ids, dims


ALIGN_CASES = [
    dict(T=16, E=4, K=2, S=0, L=2, r=8), dict(T=64, E=32, K=4, S=0, L=8, r=16),
    dict(T=4096, E=32, K=4, S=0, L=32, r=32, adapters="runs"), dict(T=128, E=64, K=8, S=1, L=0, r=0),
    dict(T=1, E=64, K=8, S=1, L=0, r=0), dict(T=500, E=6, K=2, S=1, L=3, r=8, bm=32, lbm=32),
    dict(T=300, E=8, K=3, S=0, L=5, r=8, one_expert=True), dict(T=77, E=5, K=5, S=2, L=1, r=8, bm=16),
    dict(T=8192, E=128, K=8, S=0, L=64, r=64, adapters="zipf", logits="zipf_bias"),
    dict(T=200, E=16, K=2, S=0, L=4, r=16, adapters="none"),
    # pair counts at and just past the switch to the multi-workgroup alignment
    # (8192 pairs; the second leaves a last slice of 4 pairs)
    dict(T=2048, E=33, K=3, S=1, L=0, r=0), dict(T=2049, E=7, K=4, S=0, L=2, r=8),
    # 80000 pairs: slices of 1280 pairs, so each scatter wave walks two windows
    dict(T=10000, E=64, K=8, S=0, L=16, r=16, adapters="zipf", logits="zipf_bias"),
    dict(T=3000, E=128, K=8, S=1, L=0, r=0),
    # the largest router (1025 alignment experts x 9 adapter keys) in both forms
    dict(T=40, E=1024, K=64, S=1, L=8, r=8), dict(T=200, E=1024, K=64, S=1, L=8, r=8),
    # the one-pass form for small calls: at its limit (1024 pairs, 16 waves),
    # one pair past it, and with 1024 composite keys
    dict(T=128, E=40, K=8, S=0, L=6, r=8), dict(T=205, E=40, K=5, S=0, L=6, r=8),
    dict(T=64, E=64, K=8, S=0, L=15, r=8),
    # a few pairs over many mostly empty experts, and a key count whose LDS
    # need just exceeds what the one-pass form takes
    dict(T=16, E=1024, K=4, S=0, L=0, r=0), dict(T=12, E=700, K=3, S=1, L=2, r=8),
    # 65 to 256 pairs (just past one wavefront, mid-range, the top): the one-workgroup form
    dict(T=65, E=9, K=1, S=0, L=0, r=0), dict(T=33, E=12, K=3, S=1, L=5, r=8),
    dict(T=50, E=300, K=5, S=0, L=3, r=8, bm=32), dict(T=32, E=8, K=7, S=1, L=2, r=8, lbm=32),
]


@pytest.mark.parametrize("c", ALIGN_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_align_bitexact(c):
    c = dict(c)
    T, E, K, S, L, r = (c.pop(k) for k in ("T", "E", "K", "S", "L", "r"))
    ids, ad, dims = _align_case(T, E, K, S, L, r, seed=T + E, **c)
    say("align", T, E, K, S, L, r, c)
    g = ml.moe_lora_align(torch.from_numpy(ids).to(DEV), ad.to(DEV), dims)
    torch.cuda.synchronize()
    plan = g["plan"]
    La = L if (L > 0 and r > 0) else 0
    o = oracle.align(ids, ad.numpy(), E + S, La, plan["block_m"], plan["lora_block_m"])
    assert int(g["num_post_pad"].item()) == o["num_post_pad"]
    assert np.array_equal(g["sorted_ids"].cpu().numpy(), o["sorted_ids"])
    assert np.array_equal(g["block_expert"].cpu().numpy(), o["block_expert"])
    if La:
        assert int(g["num_items"].item()) == o["num_items"]
        assert np.array_equal(g["lora_items"].cpu().numpy(), o["items"])


# ------------------------------------------------------------ small forwards

SMALL = [
    # ragged K (H=200), ragged gate tiles (I=72), several experts/blocks
    dict(T=40, H=200, I=72, E=6, K=2, S=0, L=3, r=16, dtype="bf16"),
    dict(T=100, H=256, I=128, E=8, K=3, S=1, L=4, r=32, rsf=2.5, dtype="bf16"),
    dict(T=300, H=128, I=96, E=4, K=2, S=0, L=2, r=8, dtype="bf16", block_m=256),
    dict(T=64, H=192, I=160, E=16, K=4, S=0, L=5, r=64, dtype="bf16", block_m=32, lbm=32),
    dict(T=24, H=136, I=72, E=5, K=2, S=1, L=3, r=16, dtype="bf16", split=3),
    dict(T=40, H=200, I=72, E=6, K=2, S=0, L=3, r=4, dtype="f32"),
    dict(T=33, H=64, I=40, E=3, K=3, S=2, L=2, r=5, rsf=2.0, dtype="f32", block_m=32),
    dict(T=50, H=96, I=64, E=7, K=1, S=0, L=0, r=0, dtype="bf16"),
    # LDS-tiled MFMA kernel: ragged K (200 = 3*64 + 8), ragged weight tiles, r=24 (partial k-step)
    dict(T=300, H=200, I=200, E=4, K=2, S=0, L=3, r=24, dtype="bf16", block_m=128),
    dict(T=500, H=256, I=384, E=6, K=2, S=1, L=4, r=32, rsf=2.5, dtype="bf16", block_m=128),
    dict(T=260, H=192, I=96, E=3, K=2, S=0, L=2, r=16, dtype="bf16", block_m=256, split=2),
    dict(T=200, H=128, I=128, E=5, K=3, S=0, L=0, r=0, dtype="bf16", block_m=128),
    # tiled LoRA expand in 64-rank units: r=48 (ranks 48..63 of the unit
    # zero), r=96 (one 64-rank range, then a 32-rank one), ragged gate tiles
    dict(T=300, H=192, I=160, E=4, K=2, S=1, L=3, r=48, rsf=2.0, dtype="bf16", block_m=128),
    dict(T=260, H=128, I=136, E=3, K=2, S=0, L=3, r=96, dtype="bf16", block_m=256),
    # 64 slots per token: the most the router launch takes the gate_up shrink for
    dict(T=8, H=64, I=64, E=100, K=63, S=1, L=3, r=8, rsf=2.0, dtype="bf16"),
    # K = E: every pair of a token on a different expert, all experts on every token
    dict(T=12, H=64, I=64, E=4, K=4, S=0, L=2, r=8, dtype="bf16"),
    dict(T=300, H=128, I=96, E=3, K=3, S=1, L=2, r=16, rsf=2.5, dtype="bf16", block_m=128),
    # the largest rank (128, in 16-row LoRA items) on both GEMM kinds and on the fp32 path
    dict(T=40, H=256, I=192, E=6, K=2, S=1, L=3, r=128, rsf=2.5, dtype="bf16", block_m=16),
    dict(T=300, H=256, I=192, E=4, K=2, S=0, L=3, r=128, dtype="bf16", block_m=128),
    dict(T=24, H=128, I=64, E=4, K=2, S=0, L=2, r=128, dtype="f32"),
    # routed inside the small alignment's launch (no LoRA, or a split shrink;
    # at most one token per wave): E up to 1000, 64 slots
    dict(T=15, H=64, I=64, E=1000, K=63, S=1, L=0, r=0, rsf=2.0, dtype="bf16"),
    dict(T=4, H=96, I=64, E=300, K=7, S=0, L=2, r=8, dtype="bf16", split=2),
    dict(T=3, H=64, I=40, E=130, K=4, S=0, L=0, r=0, dtype="f32"),
    # one token more than the alignment has waves: routed in its own launch
    dict(T=5, H=64, I=40, E=130, K=4, S=0, L=0, r=0, dtype="bf16"),
    # tiny calls without LoRA: every gate_up workgroup routes and aligns
    # (one token; 64 slots with 256 experts in 32-row blocks; K = E with a
    # ragged hidden size); past 256 experts the alignment's launch routes
    dict(T=1, H=96, I=64, E=64, K=8, S=1, L=0, r=0, rsf=2.5, dtype="bf16"),
    dict(T=4, H=64, I=72, E=256, K=15, S=1, L=0, r=0, rsf=2.0, dtype="bf16", block_m=32),
    dict(T=2, H=200, I=40, E=3, K=3, S=0, L=0, r=0, dtype="bf16"),
    dict(T=4, H=64, I=40, E=257, K=4, S=0, L=0, r=0, dtype="bf16"),
    dict(T=1, H=64, I=40, E=1, K=1, S=0, L=0, r=0, dtype="bf16"),
    dict(T=1, H=64, I=40, E=1, K=1, S=1, L=0, r=0, rsf=2.0, dtype="bf16"),
    # a wide, ragged hidden size (12296 = 8 * 1537, not a multiple of 32) on both GEMM kinds
    dict(T=24, H=12296, I=64, E=4, K=2, S=0, L=2, r=16, dtype="bf16", block_m=16),
    dict(T=260, H=12296, I=64, E=4, K=2, S=0, L=2, r=16, dtype="bf16", block_m=128),
]


def _shape(c):
    return synth.LayerShape(T=c["T"], H=c["H"], I=c["I"], E=c["E"], K=c["K"], S=c["S"], L=c["L"], r=c["r"],
                            rsf=c.get("rsf", 1.0), dtype=c["dtype"])


def _kw(c):
    return dict(block_m=c.get("block_m", 0), lora_block_m=c.get("lbm", 0), split_k=c.get("split", 0))


@pytest.mark.parametrize("c", SMALL, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_forward_small_parity(c):
    shape = _shape(c)
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=c["T"])
    say("forward", c)
    ids = torch.empty((shape.T, shape.Kp), dtype=torch.int32, device=DEV)
    w = torch.empty((shape.T, shape.Kp), dtype=torch.float32, device=DEV)
    out = ml.forward_inputs(inp, routing_out=(ids, w), **_kw(c))
    torch.cuda.synchronize()
    ref = oracle.forward_inputs(inp)
    assert_close(out, ref, shape.dtype, f"forward {c}")
    oids, ow = oracle.route(inp.logits.cpu().numpy(), shape.K, shape.S, shape.rsf)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.array_equal(_bits(w), ow.view(np.int32))
    if shape.lora:
        base = ml.forward_inputs(inp, lora=False, **_kw(c))
        torch.cuda.synchronize()
        ref0 = oracle.forward_inputs(inp, lora=False)
        d_gpu = out.double() - base.double()
        _, rel = errs(d_gpu, ref - ref0)
        assert rel <= LORA_DELTA_RELL2, f"LoRA delta rel-L2 {rel:.3e}"


def test_forward_multi_workgroup_alignment_all_tokens():
    """8400 (token, slot) pairs: the multi-workgroup alignment, the x pack in
    one launch with the gate_up shrink, equal-size token tiles and the LoRA
    slab skipping of the tiled GEMMs, checked against the oracle on every
    token (small H and I keep the oracle fast)."""
    c = dict(T=2100, H=128, I=96, E=16, K=4, S=0, L=6, r=16, dtype="bf16", block_m=128)
    shape = _shape(c)
    inp = inputs(shape, synth.Recipe(adapters="zipf", none_frac=0.1), seed=21)
    say("forward multi-wg align", c)
    out = ml.forward_inputs(inp, **_kw(c))
    torch.cuda.synchronize()
    assert ml.moe_lora_plan_query(ml.make_dims(shape.T, shape.H, shape.I, shape.E, shape.K, shape.S, shape.L,
                                               shape.r, block_m=128))["gemm_kind"] == 2
    assert_close(out, oracle.forward_inputs(inp), shape.dtype, "multi-wg align forward")


@pytest.mark.parametrize("logits,want_skewed", [("zipf_bias", True), ("normal", False)])
def test_tiled_work_orders(logits, want_skewed):
    """The LDS-tiled GEMMs enumerate their work in one of two orders, chosen
    on the device from the tile counts per expert (skewed: most tiles of one
    expert > 2x the mean over experts with tiles).  Both orders against the
    oracle; the routing here is checked to select the intended order."""
    c = dict(T=1200, H=128, I=128, E=16, K=2, S=0, L=3, r=16, dtype="bf16", block_m=128)
    shape = _shape(c)
    inp = inputs(shape, synth.Recipe(adapters="uniform_all", logits=logits), seed=5)
    say("work order", logits)
    oids, _ = oracle.route(inp.logits.cpu().numpy(), shape.K, shape.S, shape.rsf)
    cnt = np.bincount(oids.reshape(-1), minlength=shape.Ep)
    nt = -(-(-(-cnt // 32) * 32) // 128)
    assert (2 * nt.sum() < nt.max() * (nt > 0).sum()) == want_skewed
    out = ml.forward_inputs(inp, **_kw(c))
    torch.cuda.synchronize()
    assert_close(out, oracle.forward_inputs(inp), shape.dtype, f"work order {logits}")


@pytest.mark.parametrize("bm", [0, 128])
def test_lora_off_is_bitwise_base(bm):
    """Zero B or every adapter -1 gives exactly the base layer (compared with ==)."""
    shape = synth.LayerShape(T=96, H=256, I=128, E=8, K=2, L=4, r=16)
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=3)
    say("lora-off bitwise", bm)
    base = ml.forward_inputs(inp, lora=False, block_m=bm).clone()
    zb = ml.moe_lora_forward(inp.x, inp.logits, inp.adapter_ids, inp.w13, inp.w2, inp.a13,
                             torch.zeros_like(inp.b13), inp.a2, torch.zeros_like(inp.b2), K=2,
                             block_m=bm).clone()
    none = ml.moe_lora_forward(inp.x, inp.logits, torch.full_like(inp.adapter_ids, -1), inp.w13, inp.w2,
                               inp.a13, inp.b13, inp.a2, inp.b2, K=2, block_m=bm).clone()
    torch.cuda.synchronize()
    assert torch.equal(zb, base)
    assert torch.equal(none, base)


@pytest.mark.parametrize("bm", [0, 128])
def test_run_to_run_bitwise(bm):
    shape = synth.LayerShape(T=256, H=512, I=256, E=16, K=4, S=1, L=6, r=16, rsf=2.5)
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=9)
    say("determinism", bm)
    a = ml.forward_inputs(inp, block_m=bm).clone()
    b = ml.forward_inputs(inp, block_m=bm).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_empty_and_single_token():
    shape = synth.LayerShape(T=0, H=64, I=64, E=4, K=2, L=2, r=8)
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"))
    say("T=0")
    out = ml.forward_inputs(inp)
    torch.cuda.synchronize()
    assert out.shape == (0, 64)
    shape = synth.LayerShape(T=1, H=64, I=64, E=4, K=2, S=1, L=2, r=8, rsf=2.0)
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=1)
    inp.adapter_ids.fill_(1)
    say("T=1")
    out = ml.forward_inputs(inp)
    torch.cuda.synchronize()
    assert_close(out, oracle.forward_inputs(inp), synth.BF16, "T=1")


@pytest.mark.parametrize("bm", [0, 128])
def test_largest_router_sizes(bm):
    """The plan's largest router: 1024 experts, top-64 plus a shared slot (65
    slots per token), with LoRA (9225 alignment keys); routing bit for bit and
    the layer against the oracle on every token."""
    shape = synth.LayerShape(T=40, H=64, I=64, E=1024, K=64, S=1, L=8, r=8, rsf=2.5)
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=3)
    say("largest router", bm)
    ids = torch.empty((shape.T, shape.Kp), dtype=torch.int32, device=DEV)
    w = torch.empty((shape.T, shape.Kp), dtype=torch.float32, device=DEV)
    out = ml.forward_inputs(inp, routing_out=(ids, w), block_m=bm)
    torch.cuda.synchronize()
    oids, ow = oracle.route(inp.logits.cpu().numpy(), shape.K, shape.S, shape.rsf)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.array_equal(_bits(w), ow.view(np.int32))
    assert_close(out, oracle.forward_inputs(inp), synth.BF16, f"largest router bm={bm}")


def test_all_tokens_one_expert():
    """Degenerate routing: every token's top-1 is expert 0 (one huge expert group)."""
    shape = synth.LayerShape(T=700, H=128, I=64, E=8, K=2, L=3, r=8)
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=4)
    inp.logits[:, 0] += 100.0
    say("one expert")
    out = ml.forward_inputs(inp)
    torch.cuda.synchronize()
    assert_close(out, oracle.forward_inputs(inp), synth.BF16, "one expert")


# -------------------------------------------------------- named workloads

def test_tiny_fp32_workload_full():
    inp = inputs("tiny_fp32_T16")
    say("tiny_fp32_T16")
    out = ml.forward_inputs(inp)
    torch.cuda.synchronize()
    assert_close(out, oracle.forward_inputs(inp), synth.F32, "tiny_fp32_T16")


def _sample_tokens(T, n, seed=0):
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    return np.sort(np.concatenate([[0, T - 1], rng.choice(np.arange(1, T - 1), n - 2, replace=False)]))


@pytest.mark.parametrize("name,nsample", [("gptoss_decode_T64", 64), ("gptoss_prefill_T4096", 48),
                                          ("shared_fused_T1", 1), ("shared_fused_T32", 32),
                                          ("shared_fused_T128", 32)])
def test_workload_full_size(name, nsample):
    """Full-size workload on the GPU: routing and alignment bit-exact over every
    token, layer output element by element on sampled tokens."""
    inp = inputs(name)
    s = inp.shape
    say("workload", name)
    ids = torch.empty((s.T, s.Kp), dtype=torch.int32, device=DEV)
    w = torch.empty((s.T, s.Kp), dtype=torch.float32, device=DEV)
    out = ml.forward_inputs(inp, routing_out=(ids, w))
    torch.cuda.synchronize()
    oids, ow = oracle.route(inp.logits.cpu().numpy(), s.K, s.S, s.rsf)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.array_equal(_bits(w), ow.view(np.int32))
    dims = ml.make_dims(s.T, s.H, s.I, s.E, s.K, s.S, s.L, s.r, s.rsf)
    g = ml.moe_lora_align(ids, inp.adapter_ids, dims)
    torch.cuda.synchronize()
    La = s.L if s.lora else 0
    o = oracle.align(oids, inp.adapter_ids.cpu().numpy(), s.Ep, La, g["plan"]["block_m"],
                     g["plan"]["lora_block_m"])
    assert np.array_equal(g["sorted_ids"].cpu().numpy(), o["sorted_ids"])
    assert np.array_equal(g["block_expert"].cpu().numpy(), o["block_expert"])
    tok = _sample_tokens(s.T, nsample)
    host = inp.to("cpu")
    ref = oracle.forward_inputs(host, tokens=tok)
    assert_close(out[torch.from_numpy(tok).to(DEV)], ref, s.dtype, name)
    if s.lora:
        base = ml.forward_inputs(inp, lora=False)
        torch.cuda.synchronize()
        ref0 = oracle.forward_inputs(host, tokens=tok, lora=False)
        sel = torch.from_numpy(tok).to(DEV)
        _, rel = errs(out[sel].double() - base[sel].double(), ref - ref0)
        assert rel <= LORA_DELTA_RELL2, f"LoRA delta rel-L2 {rel:.3e}"


def test_shared_fused_equals_unfused_on_gpu():
    """Shared slot fused into the grouped GEMM (weight 1/rsf, output x rsf) equals
    the routed layer times rsf plus a separate dense shared MLP, both on the GPU."""
    inp = inputs("shared_fused_T32")
    s = inp.shape
    say("shared fused vs unfused")
    fused = ml.forward_inputs(inp)
    routed = ml.moe_lora_forward(inp.x, inp.logits, None, inp.w13[:s.E].contiguous(), inp.w2[:s.E].contiguous(),
                                 K=s.K, S=0, rsf=s.rsf)
    ones = torch.zeros((s.T, 1), dtype=torch.float32, device=DEV)
    shared = ml.moe_lora_forward(inp.x, ones, None, inp.w13[s.E:].contiguous(), inp.w2[s.E:].contiguous(),
                                 K=1, S=0, rsf=1.0)
    torch.cuda.synchronize()
    host = inp.to("cpu")
    ref = oracle.forward_inputs(host)
    assert_close(fused, ref, s.dtype, "fused")
    unfused = routed.double() + shared.double()
    maxabs, rel = errs(unfused, ref)
    assert maxabs <= 2 * 2e-2 and rel <= 1e-2, (maxabs, rel)


@pytest.mark.parametrize("block_m", [32, 128])
def test_separate_gate_up_slices_as_rank_2r(block_m):
    """A LoRA given as separate gate and up slices runs as the single-adapter
    form of rank 2r: A13 = [A_g; A_u] and a block-diagonal B13 (the oracle
    pins this equivalence on the CPU).  Both GEMM kinds against the oracle,
    and the LoRA delta on its own."""
    from dataclasses import replace
    shape = synth.LayerShape(T=160, H=192, I=128, E=6, K=2, L=3, r=16)   # rank 2r = 16
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=11)
    g = torch.Generator(device=DEV).manual_seed(3)
    L, Ep, r, H, I = shape.L, shape.Ep, shape.r // 2, shape.H, shape.I
    nrm = lambda *s, std: (torch.randn(s, generator=g, device=DEV) * std).to(torch.bfloat16)
    Ag, Au = nrm(L, Ep, r, H, std=H ** -0.5), nrm(L, Ep, r, H, std=H ** -0.5)
    Bg, Bu = nrm(L, Ep, I, r, std=0.02), nrm(L, Ep, I, r, std=0.02)
    a13 = torch.cat([Ag, Au], dim=2).contiguous()
    b13 = torch.zeros((L, Ep, 2 * I, 2 * r), dtype=torch.bfloat16, device=DEV)
    b13[:, :, :I, :r] = Bg
    b13[:, :, I:, r:] = Bu
    inp = replace(inp, a13=a13, b13=b13.contiguous())
    say("separate gate/up slices", block_m)
    out = ml.forward_inputs(inp, block_m=block_m)
    base = ml.forward_inputs(inp, lora=False, block_m=block_m)
    torch.cuda.synchronize()
    ref = oracle.forward_inputs(inp)
    assert_close(out, ref, synth.BF16, "separate gate/up slices")
    _, rel = errs(out.double() - base.double(), ref - oracle.forward_inputs(inp, lora=False))
    assert rel <= LORA_DELTA_RELL2, f"LoRA delta rel-L2 {rel:.3e}"


# ------------------------------------------------ heavy skewed (many adapters)

def _adapter_cover_sample(adapter_ids: np.ndarray, ids: np.ndarray, hot: int, n_hot: int, n_adapters: int):
    """Tokens for an element-by-element check: the first and last token,
    `n_hot` tokens routed to expert `hot`, one token for each of the first
    `n_adapters` adapter ids present (ascending) and two without an adapter."""
    T = adapter_ids.shape[0]
    pick = {0, T - 1}
    hot_tok = np.nonzero((ids == hot).any(axis=1))[0]
    pick.update(hot_tok[np.linspace(0, hot_tok.size - 1, n_hot).astype(int)].tolist())
    for a in np.unique(adapter_ids)[:n_adapters + 1]:
        toks = np.nonzero(adapter_ids == a)[0]
        pick.update(toks[[0, -1]].tolist() if a < 0 else [int(toks[toks.size // 2])])
    return np.array(sorted(pick))


def test_heavy_skewed_full_size():
    """heavy_skewed_T8192 (T=8192, H=4096, I=1536, 128 experts top-8 with a
    Zipf-skewed router bias, 64 Zipf(1.1) adapters of rank 64, 10% of tokens
    without LoRA) at full size with the packed weights the benchmark uses:
    routing and alignment bit for bit over all 65536 pairs, the layer
    element by element on tokens of the hottest expert and of 24 distinct
    adapters, and the LoRA delta on those tokens."""
    inp = inputs("heavy_skewed_T8192")
    s = inp.shape
    pw = ml.PackedWeights(inp.w13, inp.w2)
    say("heavy_skewed_T8192 full size (packed weights)")
    ids = torch.empty((s.T, s.Kp), dtype=torch.int32, device=DEV)
    w = torch.empty((s.T, s.Kp), dtype=torch.float32, device=DEV)
    out = ml.forward_inputs(inp, packed=pw, routing_out=(ids, w))
    base = ml.forward_inputs(inp, packed=pw, lora=False)
    torch.cuda.synchronize()
    oids, ow = oracle.route(inp.logits.cpu().numpy(), s.K, s.S, s.rsf)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.array_equal(_bits(w), ow.view(np.int32))
    dims = ml.make_dims(s.T, s.H, s.I, s.E, s.K, s.S, s.L, s.r, s.rsf)
    g = ml.moe_lora_align(ids, inp.adapter_ids, dims)
    torch.cuda.synchronize()
    ad = inp.adapter_ids.cpu().numpy()
    o = oracle.align(oids, ad, s.Ep, s.L, g["plan"]["block_m"], g["plan"]["lora_block_m"])
    assert int(g["num_post_pad"].item()) == o["num_post_pad"]
    assert np.array_equal(g["sorted_ids"].cpu().numpy(), o["sorted_ids"])
    assert np.array_equal(g["block_expert"].cpu().numpy(), o["block_expert"])
    assert int(g["num_items"].item()) == o["num_items"]
    assert np.array_equal(g["lora_items"].cpu().numpy(), o["items"])
    hot = int(np.argmax(np.bincount(oids.reshape(-1), minlength=s.Ep)))
    tok = _adapter_cover_sample(ad, oids, hot, 16, 24)
    assert np.unique(ad[tok][ad[tok] >= 0]).size >= 16 and (oids[tok] == hot).any(axis=1).sum() >= 16
    del pw
    host = inp.to("cpu")
    ref = oracle.forward_inputs(host, tokens=tok)
    sel = torch.from_numpy(tok).to(DEV)
    assert_close(out[sel], ref, s.dtype, "heavy_skewed_T8192")
    ref0 = oracle.forward_inputs(host, tokens=tok, lora=False)
    _, rel = errs(out[sel].double() - base[sel].double(), ref - ref0)
    assert rel <= LORA_DELTA_RELL2, f"LoRA delta rel-L2 {rel:.3e}"


def test_heavy_skewed_reduced_all_tokens():
    """The heavy workload's structure at a size the oracle checks on every
    token: 2048 tokens, 32 experts top-8 with the Zipf router bias, 64
    Zipf(1.1) adapters of rank 64 (10% without LoRA), 256-row token tiles.
    Each tile then holds dozens of adapters, which drives the LoRA expand
    over a long adapter list in both tiled GEMMs."""
    shape = synth.LayerShape(T=2048, H=256, I=256, E=32, K=8, L=64, r=64)
    inp = inputs(shape, synth.Recipe(adapters="zipf", none_frac=0.10, logits="zipf_bias"), seed=8)
    say("heavy reduced, every token")
    dims = ml.make_dims(shape.T, shape.H, shape.I, shape.E, shape.K, 0, shape.L, shape.r, block_m=256)
    assert ml.moe_lora_plan_query(dims)["gemm_kind"] == 2
    out = ml.forward_inputs(inp, block_m=256)
    base = ml.forward_inputs(inp, lora=False, block_m=256)
    torch.cuda.synchronize()
    # the tiles really hold many adapters: adapters per expert group (upper bound of a tile's list)
    oids, _ = oracle.route(inp.logits.cpu().numpy(), shape.K)
    ad = np.repeat(inp.adapter_ids.cpu().numpy(), shape.K)
    per_expert = [np.unique(ad[(oids.reshape(-1) == e) & (ad >= 0)]).size for e in range(shape.E)]
    assert max(per_expert) >= 40
    ref = oracle.forward_inputs(inp)
    assert_close(out, ref, shape.dtype, "heavy reduced")
    _, rel = errs(out.double() - base.double(), ref - oracle.forward_inputs(inp, lora=False))
    assert rel <= LORA_DELTA_RELL2, f"LoRA delta rel-L2 {rel:.3e}"
