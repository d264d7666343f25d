"""Packed expert weights (moe_lora_pack_weights) on the GPU.

* The packed bytes equal the layout the header documents, rebuilt here with
  numpy from that definition (rows in groups of 16, K in slabs of 32,
  element (r, k) of a block at (k/8)*128 + r*8 + k%8; w13 groups carry the
  gate and up rows of 8 features in quads; group counts padded to 256-row
  tiles; zeros past the edges).
* moe_lora_forward with the packed copies gives the same bits as with the
  row-major weights, for the streaming and the LDS-tiled GEMMs, with and
  without LoRA, with shared experts, ragged K and N, and at the full decode
  and prefill workload sizes.  (The row-major path itself is checked against
  the oracle in test_gpu_parity.py.)
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import lora_expert_gemm_topk_amd as ml
from lora_expert_gemm_topk_amd import synth

pytestmark = pytest.mark.gpu


def _bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _pack_reference(w: np.ndarray, gate_up: bool) -> np.ndarray:
    """Pack one weight tensor [E', rows, K] (uint16 bits) by the definition."""
    Ep, rows, K = w.shape
    if gate_up:
        N = rows // 2
        G = 16 * -(-N // 128)
    else:
        N = rows
        G = 16 * -(-N // 256)
    ns = -(-K // 32)
    out = np.zeros((Ep, G, ns, 512), np.uint16)
    for q in range(G):
        for r in range(16):
            if gate_up:
                f = 8 * q + 2 * (r // 4) + r % 2
                if f >= N:
                    continue
                src = w[:, f if r % 4 < 2 else N + f, :]
            else:
                if 16 * q + r >= N:
                    continue
                src = w[:, 16 * q + r, :]
            padded = np.zeros((Ep, ns * 32), np.uint16)
            padded[:, :K] = src
            for k in range(32):
                out[:, q, :, (k // 8) * 128 + r * 8 + k % 8] = padded[:, k::32]
    return out.reshape(-1)


@pytest.mark.parametrize("Ep,H,I", [(3, 136, 200), (2, 256, 128), (1, 64, 8)])
def test_pack_layout_matches_definition(Ep, H, I):
    g = torch.Generator().manual_seed(7)
    w13 = torch.randn(Ep, 2 * I, H, generator=g).to(torch.bfloat16).cuda()
    w2 = torch.randn(Ep, H, I, generator=g).to(torch.bfloat16).cuda()
    pw = ml.PackedWeights(w13, w2)
    torch.cuda.synchronize()
    got13 = pw.w13.cpu().numpy().view(np.uint16)
    got2 = pw.w2.cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got13, _pack_reference(_bf16_bits(w13), True))
    np.testing.assert_array_equal(got2, _pack_reference(_bf16_bits(w2), False))


SMALL = [
    dict(T=40, H=200, I=72, E=6, K=2, S=0, L=3, r=16),                  # streaming, ragged N
    dict(T=100, H=256, I=128, E=8, K=3, S=1, L=4, r=32, rsf=2.5),       # streaming, shared expert
    dict(T=64, H=192, I=160, E=16, K=4, S=0, L=5, r=64, block_m=32),    # streaming, 32-row blocks
    dict(T=300, H=200, I=200, E=4, K=2, S=0, L=3, r=24, block_m=128),   # tiled, ragged K/N, r=24
    dict(T=500, H=256, I=384, E=6, K=2, S=1, L=4, r=32, rsf=2.5, block_m=256),
    dict(T=260, H=136, I=96, E=3, K=2, S=0, L=2, r=16, block_m=256),    # tiled, H not a slab multiple
    dict(T=200, H=128, I=128, E=5, K=3, S=0, L=0, r=0, block_m=128),    # tiled, no LoRA
    dict(T=300, H=192, I=136, E=4, K=2, S=1, L=3, r=64, rsf=2.0, block_m=256),  # tiled, 64-rank units
    dict(T=260, H=128, I=96, E=3, K=2, S=0, L=2, r=96, block_m=128),    # tiled, 64 + 32 ranks
    dict(T=50, H=96, I=64, E=7, K=1, S=0, L=0, r=0),                    # streaming, no LoRA
    dict(T=1, H=96, I=64, E=64, K=8, S=1, L=0, r=0, rsf=2.5),           # routed inside gate_up
]


def _shape(c):
    return synth.LayerShape(T=c["T"], H=c["H"], I=c["I"], E=c["E"], K=c["K"], S=c["S"], L=c["L"], r=c["r"],
                            rsf=c.get("rsf", 1.0))


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_forward_packed_equals_row_major(case):
    shape = _shape(case)
    inp = synth.make_inputs(shape, synth.Recipe(adapters="uniform_all"), seed=11,
                            device="cuda")
    bm = case.get("block_m", 0)
    ref = ml.forward_inputs(inp, block_m=bm).clone()
    pw = ml.PackedWeights(inp.w13, inp.w2)
    got = ml.forward_inputs(inp, block_m=bm, packed=pw)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("name", ["gptoss_decode_T64", "gptoss_prefill_T4096"])
def test_forward_packed_equals_row_major_full_size(name):
    shape, recipe = synth.workload(name)
    inp = synth.make_inputs(shape, recipe, seed=0, device="cuda")
    ref = ml.forward_inputs(inp).clone()
    pw = ml.PackedWeights(inp.w13, inp.w2)
    got = ml.forward_inputs(inp, packed=pw)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    del pw
    torch.cuda.empty_cache()


def test_packed_rejects_f32_and_mismatch():
    shape = synth.LayerShape(T=8, H=64, I=64, E=4, K=2, dtype="f32")
    inp = synth.make_inputs(shape, synth.Recipe(), seed=1, device="cuda")
    with pytest.raises(ValueError):
        ml.PackedWeights(inp.w13, inp.w2)   # f32 tensors: bf16 only
    b = synth.make_inputs(synth.LayerShape(T=8, H=64, I=64, E=4, K=2), synth.Recipe(), seed=1, device="cuda")
    with pytest.raises(ValueError):
        ml.PackedWeights(b.w13, b.w2[:, :, :32].contiguous())
