"""Helpers shared by the GPU parity tests (comparison metrics, input staging)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from lora_expert_gemm_topk_amd import synth

# Tolerances of the layer output against the fp64 oracle.
BF16_MAXABS, BF16_RELL2 = 2e-2, 1e-2
F32_MAXABS, F32_RELL2 = 1e-5, 1e-5
LORA_DELTA_RELL2 = 5e-2


def say(*a):
    """Print and flush (names the case before each GPU step)."""
    print(*a, flush=True)
    sys.stdout.flush()


def errs(gpu: torch.Tensor, ref: np.ndarray):
    g = gpu.detach().float().cpu().double().numpy()
    d = g - ref
    maxabs = float(np.max(np.abs(d))) if d.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d) / den) if den > 0 else float(np.linalg.norm(d))
    return maxabs, rel


def assert_close(gpu: torch.Tensor, ref: np.ndarray, dtype: str, what: str = ""):
    maxabs, rel = errs(gpu, ref)
    if dtype == synth.F32:
        ok = maxabs <= F32_MAXABS and rel <= F32_RELL2
    else:
        ok = maxabs <= BF16_MAXABS and rel <= BF16_RELL2
    assert ok, f"{what}: max-abs {maxabs:.3e} rel-L2 {rel:.3e} ({dtype})"
    return maxabs, rel


def inputs(name_or_shape, recipe=None, seed=0, device="cuda"):
    """Seeded inputs on the GPU.  Small shapes are drawn on the CPU and copied;
    full-size workloads are drawn on the GPU directly."""
    if isinstance(name_or_shape, str):
        shape, recipe = synth.workload(name_or_shape)
    else:
        shape = name_or_shape
        recipe = recipe or synth.Recipe()
    big = shape.Ep * 3 * shape.H * shape.I > 50_000_000
    if big:
        return synth.make_inputs(shape, recipe, seed=seed, device=device)
    return synth.make_inputs(shape, recipe, seed=seed, device="cpu").to(device)
