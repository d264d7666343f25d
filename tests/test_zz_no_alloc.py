"""moe_lora_forward_static (the entry point for callers that cannot
allocate: its scratch is the library's fixed per-GPU array) against
moe_lora_forward with a caller workspace, through the C ABI: bit-identical
outputs and routing on two calls in a row, the second smaller than the
first (the array keeps the first call's contents)."""
import pytest
import torch

import lora_expert_gemm_topk_amd as ml
from lora_expert_gemm_topk_amd import synth
from tests.gpu_util import inputs, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _both(inp, **kw):
    s = inp.shape
    ids_a = torch.empty((s.T, s.Kp), dtype=torch.int32, device=DEV)
    w_a = torch.empty((s.T, s.Kp), dtype=torch.float32, device=DEV)
    ids_b, w_b = torch.empty_like(ids_a), torch.empty_like(w_a)
    ref = ml.forward_inputs(inp, routing_out=(ids_a, w_a), **kw)
    use = s.lora
    out = torch.empty_like(ref)
    got = ml.moe_lora_forward_static(inp.x, inp.logits, inp.adapter_ids if use else None, inp.w13, inp.w2,
                                     inp.a13 if use else None, inp.b13 if use else None,
                                     inp.a2 if use else None, inp.b2 if use else None, K=s.K, S=s.S, rsf=s.rsf,
                                     out=out, routing_out=(ids_b, w_b), **kw)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(ids_a, ids_b) and torch.equal(w_a.view(torch.int32), w_b.view(torch.int32))


@pytest.mark.parametrize("name,small_T", [("gptoss_decode_T64", 9), ("shared_fused_T128", 3)])
def test_forward_static_matches_forward_twice(name, small_T):
    big = inputs(name)
    say("forward_static", name, big.shape.T)
    _both(big)
    shape, recipe = synth.workload(name, T=small_T)
    small = inputs(shape, recipe, seed=1)
    say("forward_static", name, small_T)
    _both(small)


def test_forward_static_tiled_and_fp32():
    """Both other GEMM kinds fit the array at small sizes: the LDS-tiled bf16
    kernel (block_m 128) and the fp32 path; then a smaller call again."""
    for shape, kw in ((synth.LayerShape(T=300, H=256, I=192, E=6, K=2, S=1, L=3, r=16, rsf=2.5), dict(block_m=128)),
                      (synth.LayerShape(T=40, H=128, I=64, E=4, K=2, L=2, r=8, dtype=synth.F32), {}),
                      (synth.LayerShape(T=20, H=256, I=192, E=6, K=2, S=1, L=3, r=16, rsf=2.5), dict(block_m=128))):
        inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=shape.T)
        say("forward_static", shape, kw)
        _both(inp, **kw)


def test_forward_static_too_large_is_refused():
    """A call whose plan needs more than the fixed array is refused with
    MOE_LORA_EWORKSPACE before anything is enqueued."""
    dims = ml.make_dims(2048, 2880, 2880, 32, 4)
    assert ml.moe_lora_workspace_bytes(dims) > ml.moe_lora.STATIC_SCRATCH_BYTES
    say("forward_static refusal")
    logits = torch.zeros((2048, 32), dtype=torch.float32, device=DEV)
    x = torch.zeros((2048, 2880), dtype=torch.bfloat16, device=DEV)
    w13 = torch.zeros((32, 5760, 2880), dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros((32, 2880, 2880), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ml.MoeLoraError) as ei:
        ml.moe_lora_forward_static(x, logits, None, w13, w2, K=4)
    assert ei.value.code == ml.MOE_LORA_EWORKSPACE
