"""GPU parity of the biased top-k router and of the forward's optional
alignment outputs, through the C ABI.

The biased router is the reading of the router module that the PR 46545
analysis names ("code analysis" part 1): fp64 scores (sigmoid, or softmax
over all E), a per-expert bias for the choice only, weights from the
unbiased scores.  Ids and weights must match the oracle bit for bit; the
layer with that router must match it within the bf16 tolerances.
"""
import numpy as np
import pytest
import torch

import oracle
import lora_expert_gemm_topk_amd as ml
from lora_expert_gemm_topk_amd import synth
from tests.gpu_util import assert_close, inputs, say

pytestmark = pytest.mark.gpu

DEV = "cuda"
SCORING = {"bias_softmax": "softmax", "bias_sigmoid": "sigmoid"}


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


ROUTE_CASES = [
    dict(T=64, E=32, K=4, router="bias_sigmoid"), dict(T=64, E=32, K=4, router="bias_softmax"),
    dict(T=8192, E=128, K=8, router="bias_sigmoid", zipf=True), dict(T=4096, E=128, K=8, router="bias_softmax"),
    dict(T=33, E=300, K=5, S=1, rsf=2.5, router="bias_sigmoid", renorm=0),
    dict(T=3, E=1000, K=64, S=2, router="bias_softmax"), dict(T=17, E=7, K=7, router="bias_sigmoid"),
    dict(T=50, E=12, K=3, router="bias_softmax", renorm=0, nobias=True), dict(T=1, E=1, K=1, router="bias_sigmoid"),
]


@pytest.mark.parametrize("c", ROUTE_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_route_bias_bitexact(c):
    T, E, K, S = c["T"], c["E"], c["K"], c.get("S", 0)
    rsf, rn = c.get("rsf", 1.0), c.get("renorm", 1)
    g = torch.Generator().manual_seed(T * 5 + E)
    lg = torch.randn(T, E, generator=g) * 2
    if c.get("zipf"):
        lg += -1.1 * torch.log(torch.randperm(E, generator=g).float() + 1.0)
    bias = None if c.get("nobias") else (torch.randn(E, generator=g) * 0.1)
    say("route bias", c)
    ids, w = ml.moe_lora_route(lg.to(DEV), K, S, rsf, rn, router=c["router"],
                               expert_bias=None if bias is None else bias.to(DEV))
    torch.cuda.synchronize()
    oids, ow = oracle.route_bias(lg.numpy(), K, S, rsf, rn, SCORING[c["router"]],
                                 None if bias is None else bias.numpy())
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.array_equal(_bits(w), ow.view(np.int32))


def test_route_bias_ties_bitexact():
    """Logits and biases on a coarse grid: many exact key ties (+0 and -0
    among them), settled by the lower expert index on both sides."""
    g = torch.Generator().manual_seed(12)
    lg = torch.randint(-3, 4, (300, 40), generator=g).float() * 0.5
    lg[::7] = 0.0
    lg[1::7] = -0.0
    bias = torch.randint(-2, 3, (40,), generator=g).float() * 0.25
    for router in ("bias_sigmoid", "bias_softmax"):
        say("route bias ties", router)
        ids, w = ml.moe_lora_route(lg.to(DEV), 6, router=router, expert_bias=bias.to(DEV))
        torch.cuda.synchronize()
        oids, ow = oracle.route_bias(lg.numpy(), 6, 0, 1.0, 1, SCORING[router], bias.numpy())
        assert np.array_equal(ids.cpu().numpy(), oids)
        assert np.array_equal(_bits(w), ow.view(np.int32))


@pytest.mark.parametrize("E", [100, 300])
def test_route_bias_signed_zero_ties_bitexact(E):
    """+0 and -0 mixed inside rows and in the bias (equal keys: the lower
    index goes first), several logits per lane, both scorings."""
    g = torch.Generator().manual_seed(E)
    lg = torch.randint(-2, 3, (120, E), generator=g).float() * 0.5
    lg[(lg == 0) & (torch.rand(120, E, generator=g) < 0.5)] = -0.0
    bias = torch.randint(-1, 2, (E,), generator=g).float() * 0.25
    bias[(bias == 0) & (torch.rand(E, generator=g) < 0.5)] = -0.0
    for router in ("bias_sigmoid", "bias_softmax"):
        for rn in (1, 0):
            say("route bias signed zeros", E, router, rn)
            ids, w = ml.moe_lora_route(lg.to(DEV), 8, 1, 2.0, rn, router=router, expert_bias=bias.to(DEV))
            torch.cuda.synchronize()
            oids, ow = oracle.route_bias(lg.numpy(), 8, 1, 2.0, rn, SCORING[router], bias.numpy())
            assert np.array_equal(ids.cpu().numpy(), oids)
            assert np.array_equal(_bits(w), ow.view(np.int32))


FWD = [
    # streaming GEMM with the gate_up shrink in the router launch (decode form)
    dict(T=40, H=200, I=72, E=6, K=2, S=0, L=3, r=16, router="bias_sigmoid"),
    dict(T=24, H=136, I=72, E=5, K=2, S=1, L=3, r=16, rsf=2.5, router="bias_softmax"),
    # no LoRA: up to 4 tokens route inside each gate_up workgroup, more in their own launch
    dict(T=3, H=128, I=96, E=40, K=5, S=1, L=0, r=0, rsf=2.5, router="bias_softmax"),
    dict(T=4, H=128, I=96, E=200, K=6, S=0, L=0, r=0, router="bias_sigmoid"),
    dict(T=70, H=128, I=96, E=200, K=6, S=0, L=0, r=0, router="bias_sigmoid"),
    # LoRA with a split shrink: few tokens route inside the small alignment's launch
    dict(T=4, H=128, I=96, E=200, K=6, S=0, L=2, r=8, router="bias_softmax", split=2),
    # LDS-tiled GEMM
    dict(T=300, H=200, I=200, E=4, K=2, S=0, L=3, r=24, router="bias_softmax", block_m=128),
    dict(T=500, H=256, I=384, E=6, K=2, S=1, L=4, r=32, rsf=2.5, router="bias_sigmoid", block_m=128),
]


@pytest.mark.parametrize("c", FWD, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_forward_biased_router(c):
    shape = synth.LayerShape(T=c["T"], H=c["H"], I=c["I"], E=c["E"], K=c["K"], S=c["S"], L=c["L"], r=c["r"],
                             rsf=c.get("rsf", 1.0))
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=c["T"] + 1)
    bias = (torch.randn(shape.E, generator=torch.Generator().manual_seed(4)) * 0.2).to(DEV)
    say("forward biased router", c)
    ids = torch.empty((shape.T, shape.Kp), dtype=torch.int32, device=DEV)
    w = torch.empty((shape.T, shape.Kp), dtype=torch.float32, device=DEV)
    out = ml.forward_inputs(inp, routing_out=(ids, w), block_m=c.get("block_m", 0), split_k=c.get("split", 0),
                            router=c["router"], expert_bias=bias)
    torch.cuda.synchronize()
    sc = SCORING[c["router"]]
    oids, ow = oracle.route_bias(inp.logits.cpu().numpy(), shape.K, shape.S, shape.rsf, 1, sc, bias.cpu().numpy())
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.array_equal(_bits(w), ow.view(np.int32))
    assert_close(out, oracle.forward_inputs(inp, scoring=sc, bias=bias.cpu()), shape.dtype, f"biased {c}")


@pytest.mark.parametrize("bm,tiny", [(0, False), (128, False), (0, True)])
def test_forward_alignment_outputs(bm, tiny):
    """sorted_ids, block_expert and num_post_pad written by the forward to the
    caller's buffers equal the oracle's alignment, and the layer output is
    the same as with the alignment kept in the workspace (tiny: a call
    without LoRA whose gate_up launch routes and aligns)."""
    shape = (synth.LayerShape(T=3, H=128, I=96, E=40, K=5, S=1, L=0, r=0, rsf=2.5) if tiny else
             synth.LayerShape(T=300, H=128, I=96, E=8, K=3, S=1, L=4, r=16, rsf=2.5))
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=13)
    dims = ml.make_dims(shape.T, shape.H, shape.I, shape.E, shape.K, shape.S, shape.L, shape.r, shape.rsf,
                        block_m=bm)
    plan = ml.moe_lora_plan_query(dims)
    sid = torch.full((plan["sorted_capacity"],), -7, dtype=torch.int32, device=DEV)
    bex = torch.full((plan["max_blocks"],), -7, dtype=torch.int32, device=DEV)
    npp = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    say("forward alignment outputs", bm)
    out = ml.forward_inputs(inp, block_m=bm, align_out=(sid, bex, npp)).clone()
    ref_out = ml.forward_inputs(inp, block_m=bm)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    oids, _ = oracle.route(inp.logits.cpu().numpy(), shape.K, shape.S, shape.rsf)
    o = oracle.align(oids, inp.adapter_ids.cpu().numpy(), shape.Ep, shape.L, plan["block_m"], plan["lora_block_m"])
    assert int(npp.item()) == o["num_post_pad"]
    assert np.array_equal(sid.cpu().numpy(), o["sorted_ids"])
    assert np.array_equal(bex.cpu().numpy(), o["block_expert"])


def test_check_inputs_flags_a_nonfinite_bias():
    """moe_lora_check_inputs reads the biased router's expert bias with the
    logits: a NaN or infinite bias value is reported as MOE_LORA_BAD_LOGIT."""
    shape = synth.LayerShape(T=40, H=128, I=96, E=6, K=2, S=1, L=3, r=16, rsf=2.5)
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=3)
    for val, want in ((0.5, 0), (float("nan"), ml.MOE_LORA_BAD_LOGIT), (float("inf"), ml.MOE_LORA_BAD_LOGIT)):
        bias = torch.zeros(shape.E, dtype=torch.float32, device=DEV)
        bias[shape.E - 1] = val
        say("check_inputs bias", val)
        st = ml.moe_lora_check_inputs(inp.x, inp.logits, inp.adapter_ids, inp.w13, inp.w2, inp.a13, inp.b13,
                                      inp.a2, inp.b2, K=shape.K, S=shape.S, rsf=shape.rsf,
                                      router="bias_sigmoid", expert_bias=bias)
        torch.cuda.synchronize()
        assert int(st.item()) == want
