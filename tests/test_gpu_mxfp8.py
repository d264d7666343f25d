"""GPU parity of the MXFP8 expert-weight path (streaming GEMM) against the
fp64 oracle run on the decoded weights, through the C ABI.

The weights are seeded bf16 draws turned into MXFP8 inputs by
synth.mxfp8_quantize on the CPU; the oracle decodes them (pinned in
test_oracle_mxfp8.py) and runs its unchanged layer forward.  Routing must
match bit for bit, the output within the bf16 bars.
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

CASES = [
    dict(T=64, H=256, I=192, E=8, K=2, S=0, L=3, r=16),
    dict(T=40, H=320, I=160, E=6, K=3, S=1, L=2, r=32, rsf=2.5),
    dict(T=33, H=128, I=96, E=5, K=2, S=0, L=0, r=0, block_m=32),
    dict(T=1, H=192, I=64, E=9, K=8, S=1, L=0, r=0, rsf=2.5),
    dict(T=7, H=64, I=64, E=4, K=1, S=0, L=2, r=8, block_m=16),   # one 128-wide chunk of K at most
    dict(T=9, H=8192, I=64, E=4, K=2, S=0, L=2, r=16),    # gate_up at the largest K (256 scale blocks per row)
    dict(T=9, H=64, I=8192, E=4, K=2, S=1, L=2, r=8),     # down at the largest K
]


def _mx(inp):
    c13, s13 = synth.mxfp8_quantize(inp.w13.cpu())
    c2, s2 = synth.mxfp8_quantize(inp.w2.cpu())
    mxw = ml.Mxfp8Weights(c13.to(DEV), s13.to(DEV), c2.to(DEV), s2.to(DEV))
    return mxw, oracle.mxfp8_to_bf16(c13, s13), oracle.mxfp8_to_bf16(c2, s2)


def _oracle(inp, w13, w2, lora=True):
    s = inp.shape
    use = lora and s.lora
    return oracle.forward(inp.x, inp.logits, inp.adapter_ids if use else None, w13, w2,
                          inp.a13 if use else None, inp.b13 if use else None,
                          inp.a2 if use else None, inp.b2 if use else None,
                          K=s.K, S=s.S, rsf=s.rsf, renormalize=s.renormalize)


@pytest.mark.parametrize("c", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_mxfp8_forward_parity(c):
    c = dict(c)
    bm = c.pop("block_m", 0)
    shape = synth.LayerShape(**c)
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=shape.T + shape.H)
    say("mxfp8 forward", c, bm)
    mxw, d13, d2 = _mx(inp)
    ids = torch.empty((shape.T, shape.Kp), dtype=torch.int32, device=DEV)
    w = torch.empty((shape.T, shape.Kp), dtype=torch.float32, device=DEV)
    out = ml.forward_inputs(inp, packed=mxw, routing_out=(ids, w), block_m=bm)
    torch.cuda.synchronize()
    ref = _oracle(inp, d13, d2)
    assert_close(out, ref, synth.BF16, f"mxfp8 forward {c}")
    oids, ow = oracle.route(inp.logits.cpu().numpy(), shape.K, shape.S, shape.rsf)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.array_equal(w.cpu().view(torch.int32).numpy(), ow.view(np.int32))
    if shape.lora:
        base = ml.forward_inputs(inp, packed=mxw, lora=False, block_m=bm)
        torch.cuda.synchronize()
        _, rel = errs(out.double() - base.double(), ref - _oracle(inp, d13, d2, lora=False))
        assert rel <= LORA_DELTA_RELL2, f"LoRA delta rel-L2 {rel:.3e}"


def test_mxfp8_gptoss_decode_full_size():
    """The GPT-OSS-20B-shaped decode layer (T=64, H=I=2880, 32 experts top-4,
    8 adapters of rank 16) with MXFP8 expert weights, every token against the
    oracle on the decoded weights."""
    shape, recipe = synth.workload("gptoss_decode_T64")
    inp = inputs(shape, recipe, seed=0)
    say("mxfp8 gptoss decode")
    mxw, d13, d2 = _mx(inp)
    out = ml.forward_inputs(inp, packed=mxw)
    torch.cuda.synchronize()
    assert_close(out, _oracle(inp, d13, d2), synth.BF16, "mxfp8 gptoss decode")


def test_mxfp8_rejects_the_tiled_path():
    shape = synth.LayerShape(T=512, H=128, I=128, E=4, K=2, L=2, r=8)
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=1)
    mxw, _, _ = _mx(inp)
    with pytest.raises(ml.MoeLoraError) as ei:
        ml.forward_inputs(inp, packed=mxw, block_m=128)
    assert ei.value.code == ml.MOE_LORA_EUNSUPPORTED


def _pack_by_definition(codes: np.ndarray) -> np.ndarray:
    """The packed code layout written out: per 16 rows and 128-wide chunk c,
    byte 16*(64q + 16g + r) + i holds code 128c + 32g + 16q + i of row r."""
    rows, K = codes.reshape(-1, codes.shape[-1]).shape
    nch = -(-K // 128)
    src = np.zeros((rows, nch * 128), np.uint8)
    src[:, :K] = codes.reshape(rows, K)
    out = src.reshape(rows // 16, 16, nch, 4, 2, 16)          # [grp][r][c][g][q][i]
    return out.transpose(0, 2, 4, 3, 1, 5).reshape(-1)        # [grp][c][q][g][r][i]


@pytest.mark.parametrize("c", CASES[:2] + CASES[5:], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_mxfp8_packed_codes_layout_and_forward(c):
    """Packed codes match the layout by definition byte for byte, and the
    forward over them equals the forward over the row-major codes bit for bit."""
    c = dict(c)
    bm = c.pop("block_m", 0)
    shape = synth.LayerShape(**c)
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=shape.T + 7)
    say("mxfp8 packed", c, bm)
    mxw, _, _ = _mx(inp)
    pk = mxw.pack()
    torch.cuda.synchronize()
    assert np.array_equal(pk.w13.cpu().numpy(), _pack_by_definition(mxw.w13.cpu().numpy()))
    assert np.array_equal(pk.w2.cpu().numpy(), _pack_by_definition(mxw.w2.cpu().numpy()))
    a = ml.forward_inputs(inp, packed=mxw, block_m=bm).clone()
    b = ml.forward_inputs(inp, packed=pk, block_m=bm)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_mxfp8_packed_gptoss_decode_full_size():
    inp = inputs("gptoss_decode_T64", seed=0)
    say("mxfp8 packed gptoss_decode_T64")
    mxw, _, _ = _mx(inp)
    pk = mxw.pack()
    a = ml.forward_inputs(inp, packed=mxw).clone()
    b = ml.forward_inputs(inp, packed=pk)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
