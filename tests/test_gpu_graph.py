"""moe_lora_forward captured in a HIP graph (through torch.cuda.CUDAGraph).

The forward neither synchronises the host nor allocates, and clears its
counters with kernels (no memset nodes), so a captured call can be replayed.
Each replay is checked bit for bit against an eager call on the same inputs,
with eager work and host synchronisation between the replays, for the
streaming and the LDS-tiled plans, with packed weights, with MXFP8
weights, for calls routed inside gate_up, and for the fp32 layer.  The input check is captured too and replayed over changing
buffer contents.
"""
from __future__ import annotations

import pytest
import torch

import lora_expert_gemm_topk_amd as ml
from lora_expert_gemm_topk_amd import synth

pytestmark = pytest.mark.gpu


def _weights(inp, packed):
    if packed in ("mx", "mxp"):
        c13, s13 = synth.mxfp8_quantize(inp.w13.cpu())
        c2, s2 = synth.mxfp8_quantize(inp.w2.cpu())
        mxw = ml.Mxfp8Weights(c13.cuda(), s13.cuda(), c2.cuda(), s2.cuda())
        return mxw.pack() if packed == "mxp" else mxw
    return ml.PackedWeights(inp.w13, inp.w2) if packed else None


# L = 0 with T <= 4: the gate_up launch routes and aligns (three launches)
@pytest.mark.parametrize("T,bm,packed,L", [(48, 0, False, 3), (64, 0, True, 3), (600, 128, True, 3), (1, 0, False, 3),
                                           (64, 0, "mx", 3), (7, 32, "mx", 3), (64, 0, "mxp", 3),
                                           (1, 0, True, 0), (3, 32, "mxp", 0)])
def test_graph_replay_equals_eager(T, bm, packed, L):
    shape = synth.LayerShape(T=T, H=256, I=192, E=8, K=2, S=1, L=L, r=16 if L else 0, rsf=2.5)
    inp = synth.make_inputs(shape, synth.Recipe(adapters="uniform_all"), seed=T, device="cuda")
    pw = _weights(inp, packed)
    ws = ml.Workspace()
    out = torch.empty((T, shape.H), dtype=torch.bfloat16, device="cuda")
    ref = ml.forward_inputs(inp, block_m=bm, packed=pw).clone()   # eager, own workspace

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ml.forward_inputs(inp, block_m=bm, packed=pw, out=out, workspace=ws)   # sizes the workspace
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ml.forward_inputs(inp, block_m=bm, packed=pw, out=out, workspace=ws)
    for i in range(4):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        # eager work between replays, on the same workspace
        eager = ml.forward_inputs(inp, block_m=bm, packed=pw, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(eager.view(torch.int16), ref.view(torch.int16)), f"eager after replay {i}"


def test_graph_replay_equals_eager_fp32():
    """The fp32 layer (its own GEMM kernels) captured and replayed the same way."""
    shape = synth.LayerShape(T=16, H=128, I=256, E=4, K=2, S=1, L=2, r=8, rsf=2.5, dtype=synth.F32)
    inp = synth.make_inputs(shape, synth.Recipe(adapters="uniform_all"), seed=3, device="cuda")
    ws = ml.Workspace()
    out = torch.empty((shape.T, shape.H), dtype=torch.float32, device="cuda")
    ref = ml.forward_inputs(inp).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ml.forward_inputs(inp, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ml.forward_inputs(inp, out=out, workspace=ws)
    for i in range(4):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"replay {i}"
        eager = ml.forward_inputs(inp, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(eager.view(torch.int32), ref.view(torch.int32)), f"eager after replay {i}"


def test_graph_replay_of_the_input_check():
    """moe_lora_check_inputs captured once: each replay reports the values the
    buffers hold at that replay (bad values planted and removed between
    replays by eager copies)."""
    shape = synth.LayerShape(T=40, H=256, I=192, E=8, K=2, S=1, L=3, r=16, rsf=2.5)
    inp = synth.make_inputs(shape, synth.Recipe(adapters="uniform_all"), seed=5, device="cuda")
    ws = ml.Workspace()
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")

    def check():
        ml.moe_lora_check_inputs(inp.x, inp.logits, inp.adapter_ids, inp.w13, inp.w2, inp.a13, inp.b13, inp.a2,
                                 inp.b2, K=shape.K, S=shape.S, rsf=shape.rsf, workspace=ws, status=st)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        check()                                                     # sizes the workspace
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        check()
    lg0, ad0 = inp.logits.clone(), inp.adapter_ids.clone()
    for i, (plant, want) in enumerate([(None, 0), ("logit", 1), ("adapter", 2), ("both", 3), (None, 0)]):
        inp.logits.copy_(lg0)
        inp.adapter_ids.copy_(ad0)
        if plant in ("logit", "both"):
            inp.logits[3, 1] = float("nan")
        if plant in ("adapter", "both"):
            inp.adapter_ids[9] = shape.L
        st.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert int(st.item()) == want, f"replay {i} ({plant})"
