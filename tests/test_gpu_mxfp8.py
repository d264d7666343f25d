"""GPU parity of the MXFP8 expert-weight path (streaming and LDS-tiled
GEMMs) against the fp64 oracle run on the decoded weights, through the C ABI.

The weights are seeded bf16 draws turned into MXFP8 inputs by
synth.mxfp8_quantize on the CPU; the oracle decodes them (pinned in
test_oracle_mxfp8.py) and runs its unchanged layer forward.  Routing must
match bit for bit, the output within the bf16 bars.
"""
import dataclasses

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
    dict(T=3, H=128, I=96, E=40, K=5, S=1, L=0, r=0, rsf=2.5),  # routed inside gate_up
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


# The LDS-tiled GEMM (block_m 128/256) on MXFP8 weights: weight tiles of 128
# rows (2I or H <= 128) and 256 rows, ragged last tiles, 3 and 5 scale blocks
# per row (each tile's scale range starts off the dword grid), shared
# experts, no LoRA, and K at the tiled path's largest (3072, 96 blocks).
TILED = [
    dict(T=512, H=256, I=192, E=4, K=2, S=0, L=3, r=16, block_m=128),
    dict(T=600, H=96, I=160, E=3, K=2, S=1, L=2, r=32, rsf=2.5, block_m=256),
    dict(T=400, H=128, I=96, E=3, K=2, S=0, L=3, r=64, block_m=128),
    dict(T=700, H=160, I=64, E=4, K=3, S=0, L=0, r=0, block_m=128),
    dict(T=300, H=3072, I=64, E=2, K=1, S=0, L=2, r=8, block_m=128),
    dict(T=300, H=64, I=3072, E=2, K=2, S=1, L=2, r=8, block_m=256),
    dict(T=900, H=288, I=224, E=6, K=2, S=0, L=4, r=64, block_m=256),
]


@pytest.mark.parametrize("c", TILED, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_mxfp8_tiled_parity(c):
    """Every token of the layer on the tiled GEMM against the oracle on the
    decoded weights; packed codes give the same output bit for bit."""
    c = dict(c)
    bm = c.pop("block_m")
    shape = synth.LayerShape(**c)
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=shape.T + shape.I)
    say("mxfp8 tiled", c, bm)
    mxw, d13, d2 = _mx(inp)
    dims = ml.make_dims(shape.T, shape.H, shape.I, shape.E, shape.K, shape.S, shape.L, shape.r, shape.rsf,
                        block_m=bm)
    assert ml.moe_lora_plan_query(dims)["gemm_kind"] == 2
    out = ml.forward_inputs(inp, packed=mxw, block_m=bm).clone()
    torch.cuda.synchronize()
    ref = _oracle(inp, d13, d2)
    assert_close(out, ref, synth.BF16, f"mxfp8 tiled {c}")
    pk = ml.forward_inputs(inp, packed=mxw.pack(), block_m=bm)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), pk.view(torch.int16))
    if shape.lora:
        base = ml.forward_inputs(inp, packed=mxw, lora=False, block_m=bm)
        torch.cuda.synchronize()
        _, rel = errs(out.double() - base.double(), ref - _oracle(inp, d13, d2, lora=False))
        assert rel <= LORA_DELTA_RELL2, f"LoRA delta rel-L2 {rel:.3e}"


def test_mxfp8_tiled_matches_bf16_tiled_on_decoded_weights():
    """The MXFP8 tiled GEMM converts each code exactly, so on the same tiles it
    computes what the bf16 tiled GEMM computes on the decoded weights: equal
    bit for bit."""
    shape = synth.LayerShape(T=640, H=192, I=320, E=4, K=2, S=1, L=3, r=16, rsf=2.5)
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=11)
    say("mxfp8 tiled vs bf16 tiled")
    mxw, d13, d2 = _mx(inp)
    for bm in (128, 256):
        a = ml.forward_inputs(inp, packed=mxw, block_m=bm).clone()
        dec = dataclasses.replace(inp, w13=d13.to(DEV), w2=d2.to(DEV))
        b = ml.forward_inputs(dec, block_m=bm)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), bm


def test_mxfp8_tiled_rejects_long_rows():
    """K beyond 3072 (96 scale blocks per row) has no tiled MXFP8 form; the
    streaming GEMM (block_m 16/32) still takes it."""
    shape = synth.LayerShape(T=512, H=3104, I=64, E=4, K=2, L=2, r=8)
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=1)
    mxw, _, _ = _mx(inp)
    with pytest.raises(ml.MoeLoraError) as ei:
        ml.forward_inputs(inp, packed=mxw, block_m=128)
    assert ei.value.code == ml.MOE_LORA_EUNSUPPORTED
    ml.forward_inputs(inp, packed=mxw, block_m=32)
    torch.cuda.synchronize()


def test_mxfp8_gptoss_prefill_full_size():
    """The GPT-OSS-20B-shaped prefill (T=4096, 32 experts top-4, 32 adapters of
    rank 32) with MXFP8 expert weights on the tiled GEMM: routing over every
    token bit-exact, the output on sampled tokens against the oracle on the
    decoded weights, and packed codes equal to row-major ones bit for bit."""
    inp = inputs("gptoss_prefill_T4096", seed=0)
    s = inp.shape
    say("mxfp8 gptoss prefill")
    mxw, d13, d2 = _mx(inp)
    dims = ml.make_dims(s.T, s.H, s.I, s.E, s.K, s.S, s.L, s.r, s.rsf)
    assert ml.moe_lora_plan_query(dims)["gemm_kind"] == 2
    out = ml.forward_inputs(inp, packed=mxw).clone()
    pk = ml.forward_inputs(inp, packed=mxw.pack())
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), pk.view(torch.int16))
    rng = np.random.default_rng(3)
    tok = np.sort(np.concatenate([[0, s.T - 1], rng.choice(np.arange(1, s.T - 1), 30, replace=False)]))
    host = inp.to("cpu")
    ref = oracle.forward(host.x, host.logits, host.adapter_ids, d13, d2, host.a13, host.b13, host.a2, host.b2,
                         K=s.K, S=s.S, rsf=s.rsf, renormalize=s.renormalize, tokens=tok)
    assert_close(out[torch.from_numpy(tok).to(DEV)], ref, synth.BF16, "mxfp8 gptoss prefill")


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
