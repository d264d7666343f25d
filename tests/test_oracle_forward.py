"""Pins of the oracle's layer forward, CPU only."""
import json
from dataclasses import replace
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
from lora_expert_gemm_topk_amd import synth
from tests import bruteforce as bf

GOLDEN = Path(__file__).parent / "golden"


def _small(T=12, H=24, I=20, E=5, K=2, S=0, L=3, r=4, rsf=1.0, dtype=synth.F32, adapters="uniform_all",
           seed=0):
    shape = synth.LayerShape(T=T, H=H, I=I, E=E, K=K, S=S, L=L, r=r, rsf=rsf, dtype=dtype)
    return synth.make_inputs(shape, synth.Recipe(adapters=adapters), seed=seed)


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def test_golden_hand_example():
    spec = json.loads((GOLDEN / "hand_example.json").read_text())
    s = spec["shape"]
    inp = {k: torch.tensor(v, dtype=torch.float32) for k, v in spec["inputs"].items() if k != "adapter_ids"}
    ad = np.array(spec["inputs"]["adapter_ids"], np.int32)
    base = oracle.forward(inp["x"], inp["logits"], None, inp["w13"], inp["w2"], None, None, None, None,
                          K=s["K"], S=s["S"], rsf=s["rsf"])
    assert np.allclose(base[0], spec["expected_base"], rtol=1e-14, atol=1e-14)
    lora = oracle.forward(inp["x"], inp["logits"], ad, inp["w13"], inp["w2"], inp["a13"], inp["b13"],
                          inp["a2"], inp["b2"], K=s["K"], S=s["S"], rsf=s["rsf"])
    assert np.allclose(lora[0], spec["expected_lora"], rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("S,rsf", [(0, 1.0), (1, 2.5), (2, 1.0)])
def test_forward_vs_dense_bruteforce(dtype, S, rsf):
    inp = _small(T=10, H=24, I=20, E=6, K=3, S=S, L=3, r=4, rsf=rsf, dtype=dtype)
    s = inp.shape
    out = oracle.forward_inputs(inp)
    ids, w = bf.route(inp.logits.numpy(), s.K, s.S, s.rsf)
    G = bf.gate_matrix(ids, w, s.Ep)
    ref = bf.layer_dense(inp.x, inp.w13, inp.w2, G, inp.adapter_ids.numpy(), inp.a13, inp.b13,
                         inp.a2, inp.b2, rsf=s.rsf)
    assert _rel(out, ref) < 1e-12
    # and without LoRA
    out0 = oracle.forward_inputs(inp, lora=False)
    ref0 = bf.layer_dense(inp.x, inp.w13, inp.w2, G, rsf=s.rsf)
    assert _rel(out0, ref0) < 1e-12
    # the LoRA delta is not negligible at these sizes, so a dropped term would show
    assert _rel(out, out0) > 1e-3


def test_forward_token_subset_matches_full():
    inp = _small(T=9)
    full = oracle.forward_inputs(inp)
    sub = oracle.forward_inputs(inp, tokens=[8, 0, 3])
    assert np.array_equal(sub, full[[8, 0, 3]])


def test_dense_special_case_is_plain_swiglu_mlp():
    """E = K = 1, no shared, no LoRA: the layer is a plain SwiGLU MLP (torch fp64)."""
    inp = _small(T=7, H=16, I=12, E=1, K=1, L=0, r=0, rsf=1.75)
    out = oracle.forward_inputs(inp)
    x = inp.x.double()
    w1, w3 = inp.w13[0, :12].double(), inp.w13[0, 12:].double()
    ref = 1.75 * (torch.nn.functional.silu(x @ w1.T) * (x @ w3.T)) @ inp.w2[0].double().T
    assert _rel(out, ref.numpy()) < 1e-13


def test_lora_merged_weight_closed_form():
    """Every token on adapter a: equal to the base MoE with W13 + B13 A13 and W2 + B2 A2."""
    inp = _small(T=8, H=20, I=16, E=4, K=2, L=3, r=5)
    a = 2
    inp.adapter_ids[:] = a
    out = oracle.forward_inputs(inp)
    f = bf.to_f64
    W13m = f(inp.w13) + np.einsum("enk,ekh->enh", f(inp.b13[a]), f(inp.a13[a]))
    W2m = f(inp.w2) + np.einsum("enk,eki->eni", f(inp.b2[a]), f(inp.a2[a]))
    s = inp.shape
    ids, w = bf.route(inp.logits.numpy(), s.K)
    ref = bf.layer_dense(inp.x, W13m, W2m, bf.gate_matrix(ids, w, s.Ep), rsf=s.rsf)
    assert _rel(out, ref) < 1e-12


@pytest.mark.parametrize("how", ["rank0", "zeroB", "all_minus1"])
def test_lora_off_equals_base_exactly(how):
    inp = _small(T=10, dtype=synth.BF16)
    base = oracle.forward_inputs(inp, lora=False)
    if how == "rank0":
        out = oracle.forward(inp.x, inp.logits, inp.adapter_ids, inp.w13, inp.w2, None, None, None, None,
                             K=inp.shape.K)
    elif how == "zeroB":
        out = oracle.forward(inp.x, inp.logits, inp.adapter_ids, inp.w13, inp.w2, inp.a13,
                             torch.zeros_like(inp.b13), inp.a2, torch.zeros_like(inp.b2), K=inp.shape.K)
    else:
        out = oracle.forward(inp.x, inp.logits, torch.full_like(inp.adapter_ids, -1), inp.w13, inp.w2,
                             inp.a13, inp.b13, inp.a2, inp.b2, K=inp.shape.K)
    assert np.array_equal(out, base)


def test_lora_linear_in_b2():
    """With B13 = 0 the LoRA delta is linear in B2 (factor 2: exact in fp32)."""
    inp = _small(T=6)
    z = torch.zeros_like(inp.b13)
    base = oracle.forward_inputs(inp, lora=False)
    d1 = oracle.forward(inp.x, inp.logits, inp.adapter_ids, inp.w13, inp.w2, inp.a13, z, inp.a2, inp.b2,
                        K=inp.shape.K) - base
    d3 = oracle.forward(inp.x, inp.logits, inp.adapter_ids, inp.w13, inp.w2, inp.a13, z, inp.a2,
                        2 * inp.b2, K=inp.shape.K) - base
    assert _rel(d3, 2 * d1) < 1e-10


@pytest.mark.parametrize("rsf,tol", [(2.0, 1e-13), (2.5, 1e-7)])
def test_shared_slot_identity(rsf, tol):
    """S=1 with weight 1/rsf equals rsf * routed-only output plus a separate dense
    shared MLP (the fused and unfused forms agree; exact when 1/rsf is exact in fp32)."""
    inp = _small(T=9, H=16, I=12, E=6, K=2, S=1, L=0, r=0, rsf=rsf)
    fused = oracle.forward_inputs(inp)
    routed = oracle.forward(inp.x, inp.logits, None, inp.w13[:6].contiguous(), inp.w2[:6].contiguous(),
                            None, None, None, None, K=2, S=0, rsf=rsf)
    x = inp.x.double()
    w1, w3, w2 = inp.w13[6, :12].double(), inp.w13[6, 12:].double(), inp.w2[6].double()
    shared = ((torch.nn.functional.silu(x @ w1.T) * (x @ w3.T)) @ w2.T).numpy()
    assert _rel(fused, routed + shared) < tol


def test_top1_single_slot_is_expert_output():
    inp = _small(T=5, E=3, K=1, L=0, r=0, rsf=1.0)
    out = oracle.forward_inputs(inp)
    ids, _ = bf.route(inp.logits.numpy(), 1)
    G = np.zeros((5, 3))
    G[np.arange(5), ids[:, 0]] = 1.0
    ref = bf.layer_dense(inp.x, inp.w13, inp.w2, G)
    assert _rel(out, ref) < 1e-13


def test_token_permutation_equivariance():
    inp = _small(T=11, dtype=synth.BF16)
    perm = torch.randperm(11, generator=torch.Generator().manual_seed(1))
    out = oracle.forward_inputs(inp)
    inp2 = replace(inp)
    inp2.x, inp2.logits, inp2.adapter_ids = inp.x[perm].contiguous(), inp.logits[perm].contiguous(), \
        inp.adapter_ids[perm].contiguous()
    out2 = oracle.forward_inputs(inp2)
    assert np.array_equal(out2, out[perm.numpy()])


def test_oracle_rejects_bad_adapter():
    inp = _small(T=4)
    inp.adapter_ids[1] = 7
    with pytest.raises(ValueError):
        oracle.forward_inputs(inp)


def test_separate_gate_up_lora_as_rank_2r():
    """A LoRA with separate gate and up slices (A_g, B_g on rows [0, I), A_u,
    B_u on rows [I, 2I)) is the single-adapter form of rank 2r with
    A13 = [A_g; A_u] and the block-diagonal B13 = [[B_g, 0], [0, B_u]]: every
    token on one adapter, the oracle with those stacks equals the base MoE
    with the gate and up weights merged slice by slice."""
    rng = np.random.default_rng(7)
    inp = _small(T=8, H=20, I=16, E=4, K=2, L=2, r=3)
    s = inp.shape
    L, Ep, r, H, I = s.L, s.Ep, s.r, s.H, s.I
    Ag, Au = rng.normal(0, 0.3, (L, Ep, r, H)), rng.normal(0, 0.3, (L, Ep, r, H))
    Bg, Bu = rng.normal(0, 0.1, (L, Ep, I, r)), rng.normal(0, 0.1, (L, Ep, I, r))
    a13 = np.concatenate([Ag, Au], axis=2)
    b13 = np.zeros((L, Ep, 2 * I, 2 * r))
    b13[:, :, :I, :r] = Bg
    b13[:, :, I:, r:] = Bu
    # A2/B2 of rank 2r as well (one rank for both projections)
    a2 = rng.normal(0, 0.3, (L, Ep, 2 * r, I))
    b2 = rng.normal(0, 0.1, (L, Ep, H, 2 * r))
    t32 = lambda a: torch.from_numpy(a.astype(np.float32))
    a13, b13, a2, b2 = t32(a13), t32(b13), t32(a2), t32(b2)
    ad = 1
    inp.adapter_ids[:] = ad
    out = oracle.forward(inp.x, inp.logits, inp.adapter_ids, inp.w13, inp.w2, a13, b13, a2, b2, K=s.K)
    f = bf.to_f64
    W13m = f(inp.w13).copy()
    W13m[:, :I] += np.einsum("eik,ekh->eih", f(t32(Bg.astype(np.float32)))[ad], f(t32(Ag.astype(np.float32)))[ad])
    W13m[:, I:] += np.einsum("eik,ekh->eih", f(t32(Bu.astype(np.float32)))[ad], f(t32(Au.astype(np.float32)))[ad])
    W2m = f(inp.w2) + np.einsum("enk,eki->eni", f(b2[ad]), f(a2[ad]))
    ids, w = bf.route(inp.logits.numpy(), s.K)
    ref = bf.layer_dense(inp.x, W13m, W2m, bf.gate_matrix(ids, w, s.Ep), rsf=s.rsf)
    assert _rel(out, ref) < 1e-12


@pytest.mark.parametrize("scoring", ["sigmoid", "softmax"])
def test_forward_biased_router_vs_dense_bruteforce(scoring):
    """The layer with the biased router (the router module the PR 46545
    analysis names, read as in oracle.route_bias): the oracle's forward
    against the dense brute force gated by the brute-force biased routing."""
    inp = _small(T=10, H=24, I=20, E=6, K=3, S=1, L=3, r=4, rsf=2.5, dtype=synth.BF16)
    s = inp.shape
    bias = np.array([0.3, -0.2, 0.0, 0.5, -0.4, 0.1], np.float32)
    out = oracle.forward_inputs(inp, scoring=scoring, bias=bias)
    ids, w = bf.route_bias(inp.logits.numpy(), s.K, s.S, s.rsf, 1, scoring, bias)
    G = bf.gate_matrix(ids, w, s.Ep)
    ref = bf.layer_dense(inp.x, inp.w13, inp.w2, G, inp.adapter_ids.numpy(), inp.a13, inp.b13,
                         inp.a2, inp.b2, rsf=s.rsf)
    assert _rel(out, ref) < 1e-12
    # the bias changes the routing of some tokens here, so the output differs from the plain router's
    assert _rel(out, oracle.forward_inputs(inp)) > 1e-3
