"""Seeded synthetic inputs for the fused MoE-LoRA layer.

This module only draws inputs: hidden states, router logits, per-token
adapter ids, stacked expert weights and LoRA A/B stacks.  It holds none of
the layer's arithmetic (no routing, no alignment, no matmul), so both the
HIP path and the CPU oracle can be fed from it without sharing any of the
method.

Shapes follow the workloads that the pages describe only in outline:
  * a GPT-OSS-20B-shaped MoE layer served with many LoRA adapters
    (aitrends.kr summary of the AWS multi-LoRA MoE post, "key summary" and
    "section details"), and
  * a MiniMax-M3-style layer whose shared expert is fused into the routed
    grouped GEMM as one extra top-k slot (secrett2633 analysis of vLLM
    PR 46545, sections "code analysis" and "performance").
Neither page prints its inputs, so every tensor is a seeded draw:

  hidden x      ~ N(0, 1)
  logits        ~ N(0, 1)   (optionally plus a Zipf-shaped per-expert bias)
  w13, w2       ~ N(0, 0.02)            (second parameter = std deviation)
  LoRA A        ~ N(0, 1/sqrt(fan_in))  (fan_in = H for A13, I for A2)
  LoRA B        ~ N(0, 0.02)

Draw order is fixed: logits, x, w13, w2, a13, b13, a2, b2, adapter ids.
bf16 tensors are drawn in fp32 and rounded with ``.to(torch.bfloat16)``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class LayerShape:
    """Sizes of one MoE-LoRA layer call.

    T tokens, H hidden, I expert intermediate (w13 has 2I rows: gate then up),
    E routed experts, K routed top-k, S shared experts appended as extra
    slots, L adapters of rank r, rsf the routed scaling factor.
    """

    T: int
    H: int
    I: int
    E: int
    K: int
    S: int = 0
    L: int = 0
    r: int = 0
    rsf: float = 1.0
    renormalize: int = 1
    dtype: str = BF16

    @property
    def Ep(self) -> int:
        return self.E + self.S

    @property
    def Kp(self) -> int:
        return self.K + self.S

    @property
    def P(self) -> int:
        return self.T * self.Kp

    @property
    def lora(self) -> bool:
        return self.L > 0 and self.r > 0


@dataclass(frozen=True)
class Recipe:
    """How adapter ids and logits are drawn.

    adapters:
      "none"            every token -1 (no LoRA)
      "uniform_all"     uniform over {-1, 0, .., L-1}
      "fraction_none"   exactly round(none_frac*T) tokens -1 (seeded
                        permutation), the rest uniform over {0..L-1}
      "runs"            contiguous runs of `run_len` tokens, one adapter per
                        run drawn uniformly from {0..L-1}; no -1
      "zipf"            exactly round(none_frac*T) tokens -1, the rest draw
                        adapter rank k in 1..L with p ~ k^-zipf_s, id = k-1
    logits:
      "normal"          N(0, 1)
      "zipf_bias"       N(0, 1) + b_e, b_e = -zipf_s * ln(pi(e)+1) with pi a
                        seeded permutation of the experts
    """

    adapters: str = "none"
    none_frac: float = 0.0
    run_len: int = 512
    zipf_s: float = 1.1
    logits: str = "normal"


@dataclass
class LayerInputs:
    shape: LayerShape
    recipe: Recipe
    seed: int
    x: torch.Tensor
    logits: torch.Tensor
    adapter_ids: torch.Tensor
    w13: torch.Tensor
    w2: torch.Tensor
    a13: Optional[torch.Tensor]
    b13: Optional[torch.Tensor]
    a2: Optional[torch.Tensor]
    b2: Optional[torch.Tensor]
    extra: dict = field(default_factory=dict)

    def to(self, device) -> "LayerInputs":
        def mv(t):
            return None if t is None else t.to(device)
        return LayerInputs(self.shape, self.recipe, self.seed, mv(self.x), mv(self.logits),
                           mv(self.adapter_ids), mv(self.w13), mv(self.w2), mv(self.a13),
                           mv(self.b13), mv(self.a2), mv(self.b2), dict(self.extra))


def _tdtype(dtype: str) -> torch.dtype:
    return torch.bfloat16 if dtype == BF16 else torch.float32


def _normal(gen, shape, std, dtype, device):
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(_tdtype(dtype))


def _adapter_ids(gen, shape: LayerShape, recipe: Recipe, device) -> torch.Tensor:
    T, L = shape.T, shape.L
    ids = torch.full((T,), -1, dtype=torch.int32)
    mode = recipe.adapters if L > 0 else "none"
    cpu = torch.Generator().manual_seed(int(torch.randint(0, 2**62, (1,), generator=gen, device=device).item()))
    if mode == "none" or T == 0:
        pass
    elif mode == "uniform_all":
        ids = torch.randint(-1, L, (T,), generator=cpu, dtype=torch.int64).to(torch.int32)
    elif mode == "fraction_none":
        ids = torch.randint(0, L, (T,), generator=cpu, dtype=torch.int64).to(torch.int32)
        n_none = int(round(recipe.none_frac * T))
        perm = torch.randperm(T, generator=cpu)
        ids[perm[:n_none]] = -1
    elif mode == "runs":
        n_runs = (T + recipe.run_len - 1) // recipe.run_len
        run_ad = torch.randint(0, L, (n_runs,), generator=cpu, dtype=torch.int64).to(torch.int32)
        ids = run_ad.repeat_interleave(recipe.run_len)[:T].contiguous()
    elif mode == "zipf":
        k = torch.arange(1, L + 1, dtype=torch.float64)
        p = k.pow(-recipe.zipf_s)
        p = p / p.sum()
        ids = torch.multinomial(p, T, replacement=True, generator=cpu).to(torch.int32)
        n_none = int(round(recipe.none_frac * T))
        perm = torch.randperm(T, generator=cpu)
        ids[perm[:n_none]] = -1
    else:
        raise ValueError(f"unknown adapter recipe {mode!r}")
    return ids.to(device)


def make_inputs(shape: LayerShape, recipe: Recipe = Recipe(), seed: int = 0,
                device: str | torch.device = "cpu") -> LayerInputs:
    """Draw every input of one layer call from one seeded generator on `device`.

    The same (shape, recipe, seed, device type) always yields the same
    tensors.  Draws on "cuda" and on "cpu" differ from each other.
    """
    device = torch.device(device)
    gen = torch.Generator(device=device).manual_seed(seed)
    s = shape
    dt = s.dtype
    logits = torch.randn((s.T, s.E), generator=gen, device=device, dtype=torch.float32)
    extra = {}
    if recipe.logits == "zipf_bias":
        cpu = torch.Generator().manual_seed(seed + 7919)
        perm = torch.randperm(s.E, generator=cpu).to(torch.float64)
        bias = (-recipe.zipf_s * torch.log(perm + 1.0)).to(torch.float32).to(device)
        logits = logits + bias[None, :]
        extra["expert_bias"] = bias
    elif recipe.logits != "normal":
        raise ValueError(f"unknown logit recipe {recipe.logits!r}")
    x = _normal(gen, (s.T, s.H), 1.0, dt, device)
    w13 = _normal(gen, (s.Ep, 2 * s.I, s.H), 0.02, dt, device)
    w2 = _normal(gen, (s.Ep, s.H, s.I), 0.02, dt, device)
    if s.lora:
        a13 = _normal(gen, (s.L, s.Ep, s.r, s.H), 1.0 / math.sqrt(s.H), dt, device)
        b13 = _normal(gen, (s.L, s.Ep, 2 * s.I, s.r), 0.02, dt, device)
        a2 = _normal(gen, (s.L, s.Ep, s.r, s.I), 1.0 / math.sqrt(s.I), dt, device)
        b2 = _normal(gen, (s.L, s.Ep, s.H, s.r), 0.02, dt, device)
    else:
        a13 = b13 = a2 = b2 = None
    adapter_ids = _adapter_ids(gen, s, recipe, device)
    return LayerInputs(s, recipe, seed, x, logits.contiguous(), adapter_ids, w13, w2,
                       a13, b13, a2, b2, extra)


def mxfp8_quantize(w: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """Expert weights as MXFP8 inputs: blocks of 32 consecutive elements of
    the last axis share one E8M0 scale byte s, chosen as the smallest power
    of two 2^(s-127) with max|block| / 2^(s-127) <= 448 (the largest E4M3
    value), and every element becomes the E4M3 code of w / 2^(s-127)
    (torch's float8_e4m3fn rounding).  Returns (codes, scales) as uint8
    tensors on w's device, shapes [..., K] and [..., K/32].  This prepares
    inputs; the layer itself only ever decodes them."""
    K = w.shape[-1]
    if K % 32:
        raise ValueError("the last axis must be a multiple of 32")
    wb = w.float().reshape(*w.shape[:-1], K // 32, 32)
    amax = wb.abs().amax(dim=-1)
    e = torch.ceil(torch.log2(torch.clamp(amax, min=1e-30) / 448.0))
    e = torch.where(amax / torch.exp2(e) > 448.0, e + 1, e)  # guard log2 rounding
    e = torch.clamp(e, -126, 127)
    q = (wb / torch.exp2(e).unsqueeze(-1)).to(torch.float8_e4m3fn)
    codes = q.view(torch.uint8).reshape(w.shape).contiguous()
    scales = (e + 127).to(torch.uint8).contiguous()
    return codes, scales


# ---------------------------------------------------------------------------
# Named workloads.  Sizes are the ones the layer is measured and checked on.
# ---------------------------------------------------------------------------

WORKLOADS = {
    # tiny fp32 layer: parity at 1e-5
    "tiny_fp32_T16": (LayerShape(T=16, H=128, I=256, E=4, K=2, L=2, r=8, dtype=F32),
                      Recipe(adapters="uniform_all")),
    # GPT-OSS-20B-shaped decode step, 8 adapters of rank 16, 25% tokens without LoRA
    "gptoss_decode_T64": (LayerShape(T=64, H=2880, I=2880, E=32, K=4, L=8, r=16),
                          Recipe(adapters="fraction_none", none_frac=0.25)),
    # same layer at prefill, 32 adapters of rank 32 in runs of 512 tokens
    "gptoss_prefill_T4096": (LayerShape(T=4096, H=2880, I=2880, E=32, K=4, L=32, r=32),
                             Recipe(adapters="runs", run_len=512)),
    # heavy skewed prefill: 128 experts top-8, 64 Zipf adapters of rank 64
    "heavy_skewed_T8192": (LayerShape(T=8192, H=4096, I=1536, E=128, K=8, L=64, r=64),
                           Recipe(adapters="zipf", none_frac=0.10, logits="zipf_bias")),
}
for _t in (1, 32, 128):
    # shared-expert fusion decode sweep: 64 routed top-8 + 1 shared slot, weight 1/2.5
    WORKLOADS[f"shared_fused_T{_t}"] = (
        LayerShape(T=_t, H=3072, I=1536, E=64, K=8, S=1, rsf=2.5), Recipe(adapters="none"))


def workload(name: str, **overrides) -> tuple[LayerShape, Recipe]:
    shape, recipe = WORKLOADS[name]
    if overrides:
        shape = replace(shape, **overrides)
    return shape, recipe
