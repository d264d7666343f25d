"""CPU oracle of the fused MoE-LoRA layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  The product path (the HIP library and its binding) never
loads it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, fp64 accumulation); this file
builds it with gcc and marshals numpy arrays through ctypes.  bf16 tensors are
passed as their raw 16-bit patterns and widened exactly inside the C code.

Parity status of each function (what pins it, in ``tests/test_oracle_*.py``):
  route    pinned: brute-force sort on tiny inputs, library top-k/softmax,
           printed shared-slot layout, closed-form hand example
  route_bias  pinned: brute-force sort of fp64 keys on tiny inputs, library
           sigmoid/softmax + top-k, zero-bias reductions to the plain
           router, forced choice by a dominant bias, bias-free weights
  align    pinned: brute-force stable sort, counting invariants
  forward  pinned: dense all-experts brute force, plain SwiGLU MLP special
           case, merged-LoRA closed form, shared-slot identity, hand example
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
_LIB = _HERE / "liboracle.so"
# tests/test_oracle_mutations.py points this at a deliberately broken build
# of oracle.c to check that the pins catch the mistake
_LIB_OVERRIDE = os.environ.get("MOELORA_ORACLE_LIB")
_lib = None

F32 = 0
BF16 = 1


def build(force: bool = True) -> Path:
    """Compile oracle.c into liboracle.so with gcc -O2 -fopenmp (no fast-math)."""
    if force or not _LIB.exists():
        tmp = _LIB.with_suffix(".so.tmp")
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
               str(_SRC), "-o", str(tmp), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
            build()
        lib = ctypes.CDLL(str(_LIB))
    i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float
    vp = ctypes.c_void_p
    lib.oracle_route.argtypes = [i64, i64, i64, i64, f32, i32, vp, vp, vp]
    lib.oracle_route.restype = i32
    lib.oracle_max_blocks.argtypes = [i64, i64, i64]
    lib.oracle_max_blocks.restype = i64
    lib.oracle_max_items.argtypes = [i64, i64, i64, i64]
    lib.oracle_max_items.restype = i64
    lib.oracle_align.argtypes = [i64, i64, i64, i64, i64, i64, vp, vp, vp, i64, vp, i64, vp, vp,
                                 i64, vp]
    lib.oracle_align.restype = i32
    lib.oracle_route_bias.argtypes = [i64, i64, i64, i64, f32, i32, i32, vp, vp, vp, vp]
    lib.oracle_route_bias.restype = i32
    lib.oracle_forward.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, f32, i32, i32, i32, vp,
                                   vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, i32]
    lib.oracle_forward.restype = i32
    lib.oracle_mxfp8_decode.argtypes = [i64, i64, vp, vp, vp]
    lib.oracle_mxfp8_decode.restype = i32
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _np(t, dtype=None):
    """torch tensor or array -> C-contiguous numpy array on the host.

    bf16 torch tensors become uint16 arrays holding the raw bit patterns."""
    if t is None:
        return None
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().to("cpu").contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16)
            t = t.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(t)
    if dtype is not None:
        a = np.ascontiguousarray(a.astype(dtype, copy=False))
    return a


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def route(logits, K: int, S: int = 0, rsf: float = 1.0, renormalize: int = 1):
    """Top-K routing plus S shared slots -> (ids int32 [T, K+S], weights f32 [T, K+S])."""
    lg = _np(logits, np.float32)
    T, E = lg.shape
    ids = np.empty((T, K + S), np.int32)
    w = np.empty((T, K + S), np.float32)
    rc = _load().oracle_route(T, E, K, S, float(rsf), int(renormalize), _ptr(lg), _ptr(ids), _ptr(w))
    if rc != 0:
        raise ValueError(f"oracle_route failed: {rc}")
    return ids, w


SCORING = {None: -1, "softmax": 0, "sigmoid": 1}


def route_bias(logits, K: int, S: int = 0, rsf: float = 1.0, renormalize: int = 1, scoring: str = "sigmoid",
               bias=None):
    """Biased top-K routing: fp64 scores (sigmoid, or softmax over all E),
    choice by score + bias, weights from the unbiased scores of the chosen
    experts (renormalized over them when renormalize=1), S shared slots
    appended.  -> (ids int32 [T, K+S], weights f32 [T, K+S])."""
    lg = _np(logits, np.float32)
    T, E = lg.shape
    b = None if bias is None else _np(bias, np.float32)
    if b is not None and b.shape != (E,):
        raise ValueError("bias must have one fp32 value per routed expert")
    ids = np.empty((T, K + S), np.int32)
    w = np.empty((T, K + S), np.float32)
    rc = _load().oracle_route_bias(T, E, K, S, float(rsf), int(renormalize), SCORING[scoring], _ptr(lg), _ptr(b),
                                   _ptr(ids), _ptr(w))
    if rc != 0:
        raise ValueError(f"oracle_route_bias failed: {rc}")
    return ids, w


def max_blocks(P: int, Ep: int, bm: int) -> int:
    return int(_load().oracle_max_blocks(P, Ep, bm))


def max_items(P: int, Ep: int, La: int, lbm: int) -> int:
    return int(_load().oracle_max_items(P, Ep, La, lbm))


def align(topk_ids, adapter_ids, Ep: int, La: int, bm: int, lbm: int):
    """Canonical alignment.  Returns a dict with sorted_ids, block_expert,
    num_post_pad, items [n, 4] (start, rows, adapter, expert), num_items."""
    ids = _np(topk_ids, np.int32)
    T, Kp = ids.shape
    P = T * Kp
    ad = _np(adapter_ids, np.int32) if La > 0 else None
    mb = max_blocks(P, Ep, bm)
    cap = mb * bm
    mi = max_items(P, Ep, La, lbm) if La > 0 else 0
    sorted_ids = np.empty(cap, np.int32)
    block_expert = np.empty(mb, np.int32)
    npp = np.zeros(1, np.int32)
    items = np.empty((max(mi, 1), 4), np.int32)
    nit = np.zeros(1, np.int32)
    rc = _load().oracle_align(T, Kp, Ep, La, bm, lbm, _ptr(ids), _ptr(ad), _ptr(sorted_ids), cap,
                              _ptr(block_expert), mb, _ptr(npp), _ptr(items), mi, _ptr(nit))
    if rc != 0:
        raise ValueError(f"oracle_align failed: {rc}")
    return dict(sorted_ids=sorted_ids, block_expert=block_expert, num_post_pad=int(npp[0]),
                items=items[:mi], num_items=int(nit[0]))


def forward(x, logits, adapter_ids, w13, w2, a13, b13, a2, b2, *, K: int, S: int = 0,
            rsf: float = 1.0, renormalize: int = 1, tokens=None, nthreads: int = 0, scoring=None,
            bias=None):
    """Layer output in fp64, rows for `tokens` (all tokens if None).

    scoring=None routes with the plain router (route); "softmax" or
    "sigmoid" with the biased router (route_bias), `bias` [E] fp32 or None.

    x [T,H], w13 [E+S,2I,H], w2 [E+S,H,I] and the LoRA stacks
    a13 [L,E+S,r,H], b13 [L,E+S,2I,r], a2 [L,E+S,r,I], b2 [L,E+S,H,r] are all
    fp32 or all bf16.  Pass a13..b2 = None (or adapter_ids all -1) for no LoRA.
    """
    import torch
    is_bf16 = isinstance(x, torch.Tensor) and x.dtype == torch.bfloat16
    dt = BF16 if is_bf16 else F32
    conv = (lambda t: _np(t)) if is_bf16 else (lambda t: _np(t, np.float32))
    xa = conv(x)
    T, H = xa.shape
    lg = _np(logits, np.float32)
    E = lg.shape[1]
    w13a, w2a = conv(w13), conv(w2)
    Ep = w13a.shape[0]
    I = w13a.shape[1] // 2
    assert Ep == E + S, "w13 rows must equal routed + shared experts"
    if a13 is not None:
        L, _, r, _ = a13.shape
        a13a, b13a, a2a, b2a = conv(a13), conv(b13), conv(a2), conv(b2)
        ad = _np(adapter_ids, np.int32)
    else:
        L = r = 0
        a13a = b13a = a2a = b2a = ad = None
    if tokens is None:
        tk = None
        ntok = T
    else:
        tk = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        ntok = tk.shape[0]
    out = np.zeros((ntok, H), np.float64)
    b = None if bias is None else _np(bias, np.float32)
    if scoring is None and b is not None:
        raise ValueError("a bias needs scoring='softmax' or 'sigmoid'")
    rc = _load().oracle_forward(T, H, I, E, K, S, L, r, float(rsf), int(renormalize), dt, SCORING[scoring],
                                _ptr(b), _ptr(xa), _ptr(lg), _ptr(ad), _ptr(w13a), _ptr(w2a), _ptr(a13a),
                                _ptr(b13a), _ptr(a2a), _ptr(b2a), _ptr(tk), ntok, _ptr(out),
                                int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_forward failed: {rc}")
    return out


def forward_inputs(inp, tokens=None, lora: bool = True, nthreads: int = 0, scoring=None, bias=None):
    """oracle.forward over a synth.LayerInputs bundle."""
    s = inp.shape
    use = lora and s.lora
    return forward(inp.x, inp.logits, inp.adapter_ids if use else None, inp.w13, inp.w2,
                   inp.a13 if use else None, inp.b13 if use else None,
                   inp.a2 if use else None, inp.b2 if use else None,
                   K=s.K, S=s.S, rsf=s.rsf, renormalize=s.renormalize, tokens=tokens,
                   nthreads=nthreads, scoring=scoring, bias=bias)


def mxfp8_decode(codes, scales) -> np.ndarray:
    """MXFP8 weights -> fp64 (same shape as `codes`): FP8 E4M3 codes times
    2^(scale - 127), one E8M0 scale byte per 32 elements of the last axis."""
    c = _np(codes, np.uint8)
    sc = _np(scales, np.uint8)
    K = c.shape[-1]
    rows = c.size // K
    if K % 32 or sc.shape[-1] != K // 32 or sc.size != rows * (K // 32):
        raise ValueError("scales must hold one byte per 32 elements of the last axis")
    out = np.empty(c.shape, np.float64)
    rc = _load().oracle_mxfp8_decode(rows, K, _ptr(c), _ptr(sc), _ptr(out))
    if rc != 0:
        raise ValueError("MXFP8 decode: NaN code or scale byte outside [1, 254]")
    return out


def mxfp8_to_bf16(codes, scales):
    """mxfp8_decode rounded to bf16, checked to be exact (E4M3 has three
    mantissa bits, so every decoded weight of a normal range is a bf16)."""
    import torch
    v = mxfp8_decode(codes, scales)
    t = torch.from_numpy(v).to(torch.bfloat16)
    if not np.array_equal(t.to(torch.float64).numpy(), v):
        raise ValueError("MXFP8 weights outside the exact bf16 range")
    return t
