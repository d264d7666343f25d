"""Throughput of the fused MoE-LoRA layer on one MI355X.

One step = one full layer call (route, align, LoRA shrink, gate_up GEMM with
LoRA expand + SwiGLU, LoRA shrink, down GEMM with LoRA expand, combine) over
one batch of seeded synthetic inputs already resident in HBM.  Prints ONE JSON
line.  The default workload is the GPT-OSS-20B-shaped decode layer
(T=64, H=I=2880, 32 experts top-4, 8 LoRA adapters of rank 16, 25% tokens
without LoRA); the prefill layer (T=4096, 32 adapters of rank 32) is measured
beside it and reported under "prefill".  Expert weights are packed once with
moe_lora_pack_weights before timing (as a model would at load time);
--row-major times the row-major weights instead.  Reported beside them
(never as the headline value): the tiny fp32 layer, the shared-expert
fusion sweep against its unfused comparator, the heavy skewed prefill, and
the decode layer with its expert weights given as MXFP8.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--row-major]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

import numpy as np
import torch

import lora_expert_gemm_topk_amd as ml
from lora_expert_gemm_topk_amd import moe_lora as mm
from lora_expert_gemm_topk_amd import synth

METRIC = "MoE-LoRA layer tokens/s (decode T=64, prefill T=4096); % HBM/MFMA roofline"
HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # FLOP/s, MI355X dense bf16

ROOT = Path(__file__).resolve().parent
CSRC = ROOT / "lora_expert_gemm_topk_amd" / "csrc"
# the dominant kernels' sources and their launch code: a recorded counter
# reading stays valid only while these are unchanged
KERNEL_SOURCES = ("common.hpp", "align.hpp", "gemm_stream.hpp", "gemm_tiled.hpp", "pack.hpp", "moe_lora.hip")


def kernel_sources_sha256() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(name.encode())
        h.update((CSRC / name).read_bytes())
    return h.hexdigest()


def recorded_traffic(workload: str, kernel: str) -> float | None:
    """HBM bytes per launch (scaled FETCH_SIZE + WRITE_SIZE) recorded in the
    counter summary under profiles/, or None if there is none or the kernel's
    sources have changed since it was taken."""
    path = ROOT / "profiles" / f"hbm_counters_{workload}.md"
    if not path.exists():
        return None
    m = re.search(rf"^traffic {re.escape(workload)} {kernel} bytes=(\d+) sources_sha256=([0-9a-f]+)$",
                  path.read_text(), re.M)
    if not m or m.group(2) != kernel_sources_sha256():
        return None
    return float(m.group(1))


# ------------------------------------------------------------ work counting

def work(shape: synth.LayerShape, ids: np.ndarray, adapter_ids: np.ndarray) -> dict:
    """Algorithmic bytes and FLOPs of one layer call, counted from the actual
    routing: only touched experts and touched (adapter, expert) LoRA bins."""
    s = shape
    es = 2 if s.dtype == synth.BF16 else 4
    touched = np.unique(ids.reshape(-1))
    ad = np.repeat(adapter_ids.astype(np.int64), s.Kp) if s.lora else np.full(ids.size, -1)
    lora_pairs = ad >= 0
    bins = np.unique(ad[lora_pairs] * s.Ep + ids.reshape(-1)[lora_pairs]) if s.lora else np.array([])
    P, P_lora = ids.size, int(lora_pairs.sum())
    w13 = 2 * s.I * s.H * es
    w2 = s.H * s.I * es
    a13, b13, a2, b2 = (s.r * s.H * es, 2 * s.I * s.r * es, s.r * s.I * es, s.H * s.r * es) if s.lora else (0,) * 4
    act = s.T * s.H * es * 2 + s.T * s.E * 4 + s.T * 4
    flops_gu = 2.0 * P * 2 * s.I * s.H + 2.0 * P_lora * 2 * s.I * s.r
    flops_dn = 2.0 * P * s.H * s.I + 2.0 * P_lora * s.H * s.r
    flops_sh = 2.0 * P_lora * s.r * (s.H + s.I)
    return dict(
        experts=int(touched.size), bins=int(bins.size), P=P, P_lora=P_lora,
        bytes_layer=float(touched.size * (w13 + w2) + bins.size * (a13 + b13 + a2 + b2) + act),
        flops_layer=flops_gu + flops_dn + flops_sh,
        bytes_gate_up=float(touched.size * w13 + bins.size * b13 + s.T * s.H * es),
        flops_gate_up=flops_gu,
        bytes_down=float(touched.size * w2 + bins.size * b2),
        flops_down=flops_dn,
    )


# ------------------------------------------------------------ stage timing

class StageEvents:
    """2 x 7 HIP events per step, recorded by the library around each stage
    on the stream the kernels run on."""

    def __init__(self, steps: int):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        n = 2 * len(mm.STAGES)
        self.arrays = []
        for _ in range(steps):
            arr = (ctypes.c_void_p * n)()
            for i in range(n):
                ev = ctypes.c_void_p()
                rc = self.hip.hipEventCreate(ctypes.byref(ev))
                if rc != 0:
                    raise RuntimeError(f"hipEventCreate failed: {rc}")
                arr[i] = ev
            self.arrays.append(arr)

    def stage_ms(self) -> dict:
        out = {name: [] for name in mm.STAGES}
        f = ctypes.c_float()
        for arr in self.arrays:
            for s, name in enumerate(mm.STAGES):
                rc = self.hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(arr[2 * s]),
                                                  ctypes.c_void_p(arr[2 * s + 1]))
                if rc != 0:
                    raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
                out[name].append(f.value)
        return {k: float(np.mean(v)) for k, v in out.items()}

    def close(self):
        for arr in self.arrays:
            for ev in arr:
                self.hip.hipEventDestroy(ctypes.c_void_p(ev))


# ------------------------------------------------------------ measurement

def measure(name: str, steps: int, warmup: int, seed: int = 0, packed: bool = True) -> dict:
    """Time `steps` layer calls.  With `packed`, w13/w2 are re-laid out once by
    moe_lora_pack_weights before any timing (a model-load step, like loading
    the weights themselves) and every call reads the packed copies."""
    shape, recipe = synth.workload(name)
    inp = synth.make_inputs(shape, recipe, seed=seed, device="cuda")
    dev = inp.x.device
    out = torch.empty((shape.T, shape.H), dtype=inp.x.dtype, device=dev)
    ws = ml.Workspace()
    ids = torch.empty((shape.T, shape.Kp), dtype=torch.int32, device=dev)
    wts = torch.empty((shape.T, shape.Kp), dtype=torch.float32, device=dev)
    pw = ml.PackedWeights(inp.w13, inp.w2) if packed and shape.dtype == synth.BF16 else None

    def step(ev=None):
        ml.forward_inputs(inp, out=out, workspace=ws, routing_out=(ids, wts), stage_events=ev, packed=pw)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps

    # second timed pass with per-stage HIP events (kernel durations)
    se = StageEvents(steps)
    torch.cuda.synchronize()
    for i in range(steps):
        step(se.arrays[i])
    torch.cuda.synchronize()
    stage = se.stage_ms()
    se.close()

    # third pass: each step between its own events, for median / p10 / p90;
    # then the same step captured once in a HIP graph and replayed
    dist = per_iteration(step, steps, 0)
    gdist = graph_per_iteration(step, steps, 2)

    wk = work(shape, ids.cpu().numpy(), inp.adapter_ids.cpu().numpy())
    plan = ml.moe_lora_plan_query(ml.make_dims(shape.T, shape.H, shape.I, shape.E, shape.K, shape.S, shape.L,
                                               shape.r, shape.rsf, shape.renormalize, shape.dtype))
    return dict(name=name, shape=shape, inp=inp, ms=ms, stage=stage, work=wk, plan=plan, packed=pw is not None,
                dist=dist, gdist=gdist)


MALL_FLUSH_BYTES = 512 << 20   # > 2x the 256 MB MALL


def per_iteration(call, steps: int, warmup: int, flush_bytes: int = 0) -> dict:
    """Time `call` `steps` times, each between its own pair of HIP events on
    the current stream; with flush_bytes, a scratch buffer of that size is
    read between iterations (outside the events) so that a small footprint
    cannot stay resident in the MALL.  The flush only reads (a sum over the
    buffer, written once beforehand): a flush that writes would leave the
    MALL full of dirty lines whose write-back then lands inside the next
    timed call.  Returns mean, median, p10 and p90 in ms."""
    scratch = torch.ones(flush_bytes // 4, dtype=torch.float32, device="cuda") if flush_bytes else None
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        if scratch is not None:
            torch.sum(scratch, dim=0, out=sink)
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return {"mean_ms": float(t.mean()), "median_ms": float(np.median(t)), "p10_ms": float(np.percentile(t, 10)),
            "p90_ms": float(np.percentile(t, 90))}


def graph_per_iteration(call, steps: int, warmup: int, flush_bytes: int = 0) -> dict:
    """per_iteration over replays of `call` captured once in a HIP graph
    (torch.cuda.CUDAGraph); `call` must already have run once eagerly so its
    workspace exists."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    return per_iteration(g.replay, steps, warmup, flush_bytes)


def report_config(name: str, steps: int, warmup: int, packed: bool = True) -> dict:
    """One of the reported-only configurations: per-iteration median/p10/p90
    and roofline fractions of the whole layer, the MALL flushed between
    iterations when the working set is within about 2x of it."""
    shape, recipe = synth.workload(name)
    inp = synth.make_inputs(shape, recipe, seed=0, device="cuda")
    out = torch.empty((shape.T, shape.H), dtype=inp.x.dtype, device="cuda")
    ws = ml.Workspace()
    ids = torch.empty((shape.T, shape.Kp), dtype=torch.int32, device="cuda")
    wts = torch.empty((shape.T, shape.Kp), dtype=torch.float32, device="cuda")
    pw = ml.PackedWeights(inp.w13, inp.w2) if packed and shape.dtype == synth.BF16 else None

    def call():
        ml.forward_inputs(inp, out=out, workspace=ws, routing_out=(ids, wts), packed=pw)

    call()
    torch.cuda.synchronize()
    wk = work(shape, ids.cpu().numpy(), inp.adapter_ids.cpu().numpy())
    flush = MALL_FLUSH_BYTES if wk["bytes_layer"] < 2 * (256 << 20) else 0
    t = per_iteration(call, steps, warmup, flush)
    tg = graph_per_iteration(call, steps, warmup, flush)
    sec = t["median_ms"] * 1e-3
    res = {"tokens_per_s": shape.T / sec, **t, "mall_flushed": bool(flush),
           "weights": "packed" if pw is not None else "row-major", "dtype": shape.dtype,
           "hbm_frac": wk["bytes_layer"] / sec / HBM_PEAK, "mfma_frac": wk["flops_layer"] / sec / MFMA_BF16_PEAK,
           "bytes": wk["bytes_layer"], "flops": wk["flops_layer"], "experts": wk["experts"], "bins": wk["bins"],
           "graph_replay": {"tokens_per_s": shape.T / (tg["median_ms"] * 1e-3), **tg}}
    if shape.S > 0 and not shape.lora:
        # the unfused comparator: the routed experts alone (output x rsf) plus
        # the shared expert as a separate dense MLP through the same kernels
        # (E = 1, K = 1, weight 1), then the sum
        E = shape.E
        w13r, w2r = inp.w13[:E].contiguous(), inp.w2[:E].contiguous()
        w13s, w2s = inp.w13[E:].contiguous(), inp.w2[E:].contiguous()
        pr = ml.PackedWeights(w13r, w2r) if pw is not None else None
        ps = ml.PackedWeights(w13s, w2s) if pw is not None else None
        ones = torch.zeros((shape.T, 1), dtype=torch.float32, device="cuda")
        o1 = torch.empty_like(out)
        o2 = torch.empty_like(out)
        ws2 = ml.Workspace()

        def unfused():
            ml.moe_lora_forward(inp.x, inp.logits, None, pr if pr is not None else w13r, None if pr else w2r,
                                K=shape.K, S=0, rsf=shape.rsf, out=o1, workspace=ws)
            ml.moe_lora_forward(inp.x, ones, None, ps if ps is not None else w13s, None if ps else w2s,
                                K=1, S=0, rsf=1.0, out=o2, workspace=ws2)
            torch.add(o1, o2, out=out)

        tu = per_iteration(unfused, steps, warmup, flush)
        res["unfused"] = {"tokens_per_s": shape.T / (tu["median_ms"] * 1e-3), **tu,
                          "speedup_fused": tu["median_ms"] / t["median_ms"]}
    del inp, pw
    torch.cuda.empty_cache()
    return res


def report_mxfp8(name: str, steps: int, warmup: int) -> dict:
    """A bf16 workload with its expert weights given as MXFP8 (E4M3 codes and
    one E8M0 scale per 32 elements, drawn from the same seeded bf16 weights):
    per-iteration median/p10/p90, the layer's HBM fraction with the weights
    counted at 1 + 1/32 bytes per element and its matrix-core fraction (bf16
    products on the converted weights), the gate_up and down kernels timed by
    stage events, and the bf16 layer (packed weights) on the same inputs
    beside it, its kernels timed the same way."""
    shape, recipe = synth.workload(name)
    inp = synth.make_inputs(shape, recipe, seed=0, device="cuda")
    c13, s13 = synth.mxfp8_quantize(inp.w13.cpu())
    c2, s2 = synth.mxfp8_quantize(inp.w2.cpu())
    mxw = ml.Mxfp8Weights(c13.cuda(), s13.cuda(), c2.cuda(), s2.cuda()).pack()   # packed codes, as served
    del c13, s13, c2, s2
    torch.cuda.empty_cache()
    out = torch.empty((shape.T, shape.H), dtype=inp.x.dtype, device="cuda")
    ws = ml.Workspace()
    ids = torch.empty((shape.T, shape.Kp), dtype=torch.int32, device="cuda")
    wts = torch.empty((shape.T, shape.Kp), dtype=torch.float32, device="cuda")

    def call(ev=None):
        ml.forward_inputs(inp, out=out, workspace=ws, routing_out=(ids, wts), packed=mxw, stage_events=ev)

    call()
    torch.cuda.synchronize()
    wk = work(shape, ids.cpu().numpy(), inp.adapter_ids.cpu().numpy())
    wbf16 = wk["experts"] * 3 * shape.I * shape.H * 2          # touched w13 + w2 at 2 bytes per element
    bytes_layer = wk["bytes_layer"] - wbf16 + wbf16 / 2 * (1 + 1 / 32)
    t = per_iteration(call, steps, warmup)
    se = StageEvents(steps)
    for i in range(steps):
        call(se.arrays[i])
    torch.cuda.synchronize()
    stage = se.stage_ms()
    se.close()
    sec = t["median_ms"] * 1e-3
    gu_bytes = wk["bytes_gate_up"] - wk["experts"] * 2 * shape.I * shape.H * (2 - (1 + 1 / 32))
    pw = ml.PackedWeights(inp.w13, inp.w2)
    tb = per_iteration(lambda: ml.forward_inputs(inp, out=out, workspace=ws, packed=pw), steps, warmup)
    se = StageEvents(steps)
    for i in range(steps):
        ml.forward_inputs(inp, out=out, workspace=ws, packed=pw, stage_events=se.arrays[i])
    torch.cuda.synchronize()
    stage_b = se.stage_ms()
    se.close()
    dims = ml.make_dims(shape.T, shape.H, shape.I, shape.E, shape.K, shape.S, shape.L, shape.r, shape.rsf)
    res = {"tokens_per_s": shape.T / sec, **t, "weights": "mxfp8 (E4M3, E8M0 scale per 32), codes packed",
           "dtype": "bf16", "gemm_kind": ml.moe_lora_plan_query(dims)["gemm_kind"],
           "bytes": bytes_layer, "hbm_frac": bytes_layer / sec / HBM_PEAK,
           "mfma_frac": wk["flops_layer"] / sec / MFMA_BF16_PEAK,
           "gate_up_us": stage["gate_up"] * 1e3, "down_us": stage["down"] * 1e3,
           "gate_up_hbm_frac": gu_bytes / (stage["gate_up"] * 1e-3) / HBM_PEAK,
           "gate_up_mfma_frac": wk["flops_gate_up"] / (stage["gate_up"] * 1e-3) / MFMA_BF16_PEAK,
           "bf16_packed_median_ms": tb["median_ms"], "speedup_vs_bf16": tb["median_ms"] / t["median_ms"],
           "bf16_gate_up_us": stage_b["gate_up"] * 1e3, "bf16_down_us": stage_b["down"] * 1e3}
    del inp, mxw, pw
    torch.cuda.empty_cache()
    return res


REPORTED = ("tiny_fp32_T16", "shared_fused_T1", "shared_fused_T32", "shared_fused_T128", "heavy_skewed_T8192")


def roofline_obj(m: dict, bound: str) -> dict:
    st = m["stage"]["gate_up"] * 1e-3
    kern = ("gemm_tiled" if m["plan"]["gemm_kind"] == 2 else "gemm_stream") + \
        " gate_up (+LoRA expand13, SwiGLU)"
    traffic = recorded_traffic(m["name"], "gate_up")
    if bound == "hbm":
        ach = m["work"]["bytes_gate_up"] / st
        return {"kernel": kern, "bound": "hbm",
                "achieved": ach / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": ach / HBM_PEAK,
                "traffic": traffic, "kernel_us": st * 1e6,
                "algorithmic_bytes": m["work"]["bytes_gate_up"]}
    ach = m["work"]["flops_gate_up"] / st
    return {"kernel": kern, "bound": "mfma",
            "achieved": ach / 1e12, "peak": MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK,
            "traffic": traffic, "kernel_us": st * 1e6, "algorithmic_flops": m["work"]["flops_gate_up"],
            "algorithmic_bytes": m["work"]["bytes_gate_up"]}


def layer_roofline(m: dict) -> dict:
    wk = m["work"]
    t = m["ms"] * 1e-3
    t_roof = max(wk["bytes_layer"] / HBM_PEAK, wk["flops_layer"] / MFMA_BF16_PEAK)
    return {"bytes": wk["bytes_layer"], "flops": wk["flops_layer"],
            "hbm_frac": wk["bytes_layer"] / t / HBM_PEAK, "mfma_frac": wk["flops_layer"] / t / MFMA_BF16_PEAK,
            "roofline_us": t_roof * 1e6, "frac_of_roofline": t_roof / t}


def cpu_baseline(m: dict, budget_tokens: int, min_wall_s: float = 10.0, max_reps: int = 200) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the same layer call:
    the first `budget_tokens` tokens, repeated until about `min_wall_s` of wall time."""
    import oracle
    s = m["shape"]
    host = m["inp"].to("cpu")
    n = min(s.T, budget_tokens)
    tokens = np.arange(n)
    # every CPU thread this process may use (its affinity set), unless the
    # host's OpenMP setting gives it a smaller share (16 threads per GPU on
    # the measurement hosts)
    host_cpus = len(os.sched_getaffinity(0))
    omp = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(host_cpus, omp) if omp > 0 else host_cpus
    reps, wall = 0, 0.0
    while reps < max_reps and (reps == 0 or wall < min_wall_s):
        t0 = time.perf_counter()
        oracle.forward_inputs(host, tokens=tokens, nthreads=threads)
        wall += time.perf_counter() - t0
        reps += 1
    return {"value": n * reps / wall, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {s.T} tokens of one {m['name']} layer call, {reps} repetitions "
                      f"(fp64 oracle, OpenMP)", "wall_s": wall, "host_cpus": host_cpus,
            "omp_num_threads": omp or None, "cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_calibration(mib: int, reps: int) -> None:
    """A plain device-to-device copy of `mib` MiB, `reps` times: the reference
    kernel whose FETCH_SIZE / WRITE_SIZE counters scale the layer's counters."""
    n = mib * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "reps": reps}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gptoss_decode_T64")
    ap.add_argument("--prefill", default="gptoss_prefill_T4096", help="secondary workload ('' to skip)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-tokens", type=int, default=64)
    ap.add_argument("--no-reported", action="store_true",
                    help="skip the reported-only configurations (tiny fp32, shared sweep, heavy)")
    ap.add_argument("--row-major", action="store_true",
                    help="read w13/w2 row-major instead of packing them once before timing")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration) and exit")
    ap.add_argument("--mxfp8-only", default="",
                    help="only run the MXFP8-weight report on these comma-separated workloads (one JSON line each)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this layer is built and measured on one GPU only; "
              f"--gpus {args.gpus} (WORLD_SIZE={world}) is not supported", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1

    if args.copy_calib_mib:
        copy_calibration(args.copy_calib_mib, args.steps)
        return 0
    if args.mxfp8_only:
        for name in args.mxfp8_only.split(","):
            print(json.dumps({"workload": name, "mxfp8": report_mxfp8(name, args.steps, args.warmup)}), flush=True)
        return 0
    print(f"bench: {args.workload} steps={args.steps} warmup={args.warmup}", file=sys.stderr, flush=True)
    m = measure(args.workload, args.steps, args.warmup, packed=not args.row_major)
    s = m["shape"]
    result = {
        "metric": METRIC,
        "value": s.T / (m["ms"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms"],
        "step_ms": {k: m["dist"][k] for k in ("median_ms", "p10_ms", "p90_ms")},
        "graph_replay": {"tokens_per_s": s.T / (m["gdist"]["median_ms"] * 1e-3),
                         **{k: m["gdist"][k] for k in ("median_ms", "p10_ms", "p90_ms")}},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic (seeded)",
        "config": {"workload": args.workload, "T": s.T, "H": s.H, "I": s.I, "E": s.E, "K": s.K, "S": s.S,
                   "L": s.L, "r": s.r, "block_m": m["plan"]["block_m"], "split_k": m["plan"]["split_k"],
                   "weights": "packed once before timing" if m["packed"] else "row-major"},
        "roofline": roofline_obj(m, "hbm"),
        "layer": layer_roofline(m),
        "stage_us": {k: v * 1e3 for k, v in m["stage"].items()},
        "work": m["work"],
    }
    if not args.no_cpu:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(m, args.cpu_tokens)
    else:
        result["cpu_baseline"] = None
    del m
    torch.cuda.empty_cache()
    if args.prefill:
        print(f"bench: {args.prefill}", file=sys.stderr, flush=True)
        p = measure(args.prefill, max(20, args.steps // 2), max(5, args.warmup // 2), packed=not args.row_major)
        ps = p["shape"]
        result["prefill"] = {"workload": args.prefill, "tokens_per_s": ps.T / (p["ms"] * 1e-3),
                             "ms_per_step": p["ms"], "roofline": roofline_obj(p, "mfma"),
                             "step_ms": {k: p["dist"][k] for k in ("median_ms", "p10_ms", "p90_ms")},
                             "graph_replay": {"tokens_per_s": ps.T / (p["gdist"]["median_ms"] * 1e-3),
                                              **{k: p["gdist"][k] for k in ("median_ms", "p10_ms", "p90_ms")}},
                             "layer": layer_roofline(p), "stage_us": {k: v * 1e3 for k, v in p["stage"].items()},
                             "block_m": p["plan"]["block_m"], "work": p["work"]}
    if not args.no_reported:
        result["reported"] = {}
        for name in REPORTED:
            print(f"bench: reported {name}", file=sys.stderr, flush=True)
            result["reported"][name] = report_config(name, max(20, args.steps), max(5, args.warmup),
                                                     packed=not args.row_major)
        print("bench: reported gptoss_decode_T64 with MXFP8 weights", file=sys.stderr, flush=True)
        result["reported"]["gptoss_decode_T64_mxfp8"] = report_mxfp8("gptoss_decode_T64", max(20, args.steps),
                                                                     max(5, args.warmup))
        if args.prefill:
            print(f"bench: reported {args.prefill} with MXFP8 weights", file=sys.stderr, flush=True)
            result["reported"][f"{args.prefill}_mxfp8"] = report_mxfp8(args.prefill, max(20, args.steps // 2),
                                                                       max(5, args.warmup // 2))
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
