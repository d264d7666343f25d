"""Seeded random layer shapes on the GPU against the oracle.

Each case draws T, H, I (multiples of 8, ragged against the 32-wide K slabs
and the weight tiles), E, K, S (0 or 1 shared slot, rsf != 1 with a shared
slot), L and r (bf16: r a multiple of 8), an adapter recipe, a logits
recipe and a block size that selects the streaming or the LDS-tiled GEMM,
then compares the whole layer with the oracle on every token to the
tolerance of its dtype, and the routing bit for bit.  The draw is fixed by
the case index, so a failure names a reproducible shape.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import lora_expert_gemm_topk_amd as ml
from lora_expert_gemm_topk_amd import synth
from tests.gpu_util import assert_close, inputs, say

pytestmark = pytest.mark.gpu

N_CASES = 48


def _draw(i: int) -> dict:
    rng = np.random.default_rng(1000 + i)
    dtype = "f32" if i % 6 == 5 else "bf16"
    E = int(rng.integers(2, 24))
    K = int(rng.integers(1, min(E, 8) + 1))
    S = int(rng.integers(0, 2))
    lora = rng.random() < 0.8
    L = int(rng.integers(1, 7)) if lora else 0
    r = (int(rng.integers(1, 9)) * 8 if dtype == "bf16" else int(rng.integers(1, 17))) if lora else 0
    if dtype == "bf16" and r > 64:
        r = 64
    c = dict(T=int(rng.integers(1, 700)), H=8 * int(rng.integers(2, 40)), I=8 * int(rng.integers(2, 40)),
             E=E, K=K, S=S, L=L, r=r, rsf=float(rng.choice([1.0, 2.5])) if S else 1.0, dtype=dtype,
             block_m=int(rng.choice([0, 16, 32, 128, 256] if dtype == "bf16" else [0, 16, 32])),
             adapters=str(rng.choice(["uniform_all", "fraction_none", "zipf", "runs"])) if lora else "none",
             logits=str(rng.choice(["normal", "zipf_bias"])))
    return c


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_parity(i):
    c = _draw(i)
    shape = synth.LayerShape(T=c["T"], H=c["H"], I=c["I"], E=c["E"], K=c["K"], S=c["S"], L=c["L"], r=c["r"],
                             rsf=c["rsf"], dtype=c["dtype"])
    recipe = synth.Recipe(adapters=c["adapters"], none_frac=0.2, run_len=64, logits=c["logits"])
    inp = inputs(shape, recipe, seed=i)
    say("random shape", i, c)
    ids = torch.empty((shape.T, shape.Kp), dtype=torch.int32, device="cuda")
    w = torch.empty((shape.T, shape.Kp), dtype=torch.float32, device="cuda")
    out = ml.forward_inputs(inp, routing_out=(ids, w), block_m=c["block_m"])
    torch.cuda.synchronize()
    oids, ow = oracle.route(inp.logits.cpu().numpy(), shape.K, shape.S, shape.rsf)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.array_equal(w.cpu().numpy().view(np.int32), ow.view(np.int32))
    assert_close(out, oracle.forward_inputs(inp), shape.dtype, f"random shape {i} {c}")
