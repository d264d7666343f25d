"""GPU checks of moe_lora_check_inputs, the debug check of the inputs the
layer does not validate on the device: bad values are planted on the host
(numpy decides the expected flags) and the status word must name exactly
those violations."""
import numpy as np
import pytest
import torch

import lora_expert_gemm_topk_amd as ml
from lora_expert_gemm_topk_amd import synth
from tests.gpu_util import inputs, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _status(inp, packed=None, lora=True, **kw):
    s = inp.shape
    use = lora and s.lora
    w13, w2 = (packed, None) if packed is not None else (inp.w13, inp.w2)
    st = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    ml.moe_lora_check_inputs(inp.x, inp.logits, inp.adapter_ids if use else None, w13, w2,
                             inp.a13 if use else None, inp.b13 if use else None,
                             inp.a2 if use else None, inp.b2 if use else None,
                             K=s.K, S=s.S, rsf=s.rsf, status=st, **kw)
    torch.cuda.synchronize()
    return int(st.item())


def _expected(inp, mx=None, lora=True):
    f = 0
    if not np.isfinite(inp.logits.cpu().numpy()).all():
        f |= ml.MOE_LORA_BAD_LOGIT
    if lora and inp.shape.lora:
        a = inp.adapter_ids.cpu().numpy()
        if ((a < -1) | (a >= inp.shape.L)).any():
            f |= ml.MOE_LORA_BAD_ADAPTER
    if mx is not None:
        codes = np.concatenate([mx.w13.cpu().numpy().ravel(), mx.w2.cpu().numpy().ravel()])
        scales = np.concatenate([mx.w13_scale.cpu().numpy().ravel(), mx.w2_scale.cpu().numpy().ravel()])
        if ((codes & 0x7F) == 0x7F).any() or ((scales == 0) | (scales == 255)).any():
            f |= ml.MOE_LORA_BAD_MXFP8
    return f


SHAPE = synth.LayerShape(T=40, H=128, I=96, E=6, K=2, S=1, L=3, r=16, rsf=2.5)
# T*E above one grid stride of the check (512 workgroups x 256 threads)
BIG = synth.LayerShape(T=4100, H=64, I=64, E=64, K=4, S=0, L=4, r=8)


@pytest.mark.parametrize("plant", ["none", "nan_logit", "inf_logit", "adapter_L", "adapter_m2", "both",
                                   "last_logit_big", "last_adapter_big"])
def test_check_inputs_flags(plant):
    shape = BIG if plant.endswith("big") else SHAPE
    inp = inputs(shape, synth.Recipe(adapters="uniform_all"), seed=11)
    say("check_inputs", plant, shape)
    lg, ad = inp.logits.cpu(), inp.adapter_ids.cpu()
    if plant in ("nan_logit", "both"):
        lg[5, 3] = float("nan")
    if plant == "inf_logit":
        lg[0, 0] = float("-inf")
    if plant in ("adapter_L", "both"):
        ad[7] = shape.L
    if plant == "adapter_m2":
        ad[shape.T - 1] = -2
    if plant == "last_logit_big":
        lg[-1, -1] = float("inf")
    if plant == "last_adapter_big":
        ad[-1] = shape.L + 5
    inp.logits.copy_(lg)
    inp.adapter_ids.copy_(ad)
    want = _expected(inp)
    assert want == {"none": 0, "nan_logit": 1, "inf_logit": 1, "adapter_L": 2, "adapter_m2": 2, "both": 3,
                    "last_logit_big": 1, "last_adapter_big": 2}[plant]
    assert _status(inp) == want
    # without LoRA the adapter ids are not read
    assert _status(inp, lora=False) == want & ml.MOE_LORA_BAD_LOGIT


@pytest.mark.parametrize("plant", ["none", "scale255_w13", "scale0_w2", "nan_code_w13", "nan_code_w2_last"])
def test_check_inputs_mxfp8(plant):
    inp = inputs(SHAPE, synth.Recipe(adapters="uniform_all"), seed=12)
    say("check_inputs mxfp8", plant)
    c13, s13 = synth.mxfp8_quantize(inp.w13.cpu())
    c2, s2 = synth.mxfp8_quantize(inp.w2.cpu())
    if plant == "scale255_w13":
        s13[2, 5, 1] = 255
    if plant == "scale0_w2":
        s2[1, 0, 0] = 0
    if plant == "nan_code_w13":
        c13[0, 3, 17] = 0xFF
    if plant == "nan_code_w2_last":
        c2[-1, -1, -1] = 0x7F
    mxw = ml.Mxfp8Weights(c13.to(DEV), s13.to(DEV), c2.to(DEV), s2.to(DEV))
    want = _expected(inp, mxw)
    assert want == (0 if plant == "none" else ml.MOE_LORA_BAD_MXFP8)
    assert _status(inp, packed=mxw) == want
    # the packed codes carry the same codes (and zero padding past K, never
    # flagged): the check reads the packed buffer and reports the same
    packed = mxw.pack()
    torch.cuda.synchronize()
    assert _status(inp, packed=packed) == want


def test_check_inputs_empty_batch_writes_zero():
    inp = inputs(SHAPE, synth.Recipe(adapters="uniform_all"), seed=13)
    say("check_inputs T=0")
    st = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    ml.moe_lora_check_inputs(inp.x[:0], inp.logits[:0], inp.adapter_ids[:0], inp.w13, inp.w2, inp.a13, inp.b13,
                             inp.a2, inp.b2, K=SHAPE.K, S=SHAPE.S, rsf=SHAPE.rsf, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0


def test_binding_rejects_mismatched_shapes():
    inp = inputs(SHAPE, synth.Recipe(adapters="uniform_all"), seed=14)
    s = SHAPE
    say("binding shape checks")
    with pytest.raises(ValueError, match="w13"):
        ml.moe_lora_forward(inp.x, inp.logits[:, :-1].contiguous(), None, inp.w13, inp.w2, K=s.K, S=s.S)
    with pytest.raises(ValueError, match="b2"):
        ml.moe_lora_forward(inp.x, inp.logits, inp.adapter_ids, inp.w13, inp.w2, inp.a13, inp.b13, inp.a2,
                            inp.b2[:, :, :-8].contiguous(), K=s.K, S=s.S)
    with pytest.raises(ValueError, match="out"):
        ml.moe_lora_forward(inp.x, inp.logits, None, inp.w13, inp.w2, K=s.K, S=s.S,
                            out=torch.empty((s.T + 1, s.H), dtype=inp.x.dtype, device=DEV))
