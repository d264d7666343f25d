"""Python binding of libmoelora.so (see include/moe_lora.h for the contract).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoelora.so.  PyTorch supplies device memory and the current stream.  When
the library has not been built this module raises instead of falling back to
anything else.
"""
from __future__ import annotations

import ctypes
from pathlib import Path
from typing import Optional

import torch

_LIB_PATH = Path(__file__).resolve().parent / "libmoelora.so"
_lib = None

MOE_LORA_OK = 0
MOE_LORA_EINVAL = -1
MOE_LORA_EUNSUPPORTED = -2
MOE_LORA_EWORKSPACE = -3
MOE_LORA_EHIP = -4
MOE_LORA_F32 = 0
MOE_LORA_BF16 = 1
MOE_LORA_BAD_LOGIT = 1
MOE_LORA_BAD_ADAPTER = 2
MOE_LORA_BAD_MXFP8 = 4
STAGES = ("route", "align", "shrink13", "gate_up", "shrink2", "down", "combine")
# dims.router: the plain top-k router, or the biased router with softmax or sigmoid scores
ROUTERS = {"topk": 0, "bias_softmax": 1, "bias_sigmoid": 2}

EXPORTED = ("moe_lora_plan_query", "moe_lora_workspace_bytes", "moe_lora_check_args", "moe_lora_route",
            "moe_lora_align", "moe_lora_forward", "moe_lora_packed_weight_bytes", "moe_lora_pack_weights",
            "moe_lora_strerror", "moe_lora_check_inputs",
            "moe_lora_packed_mxfp8_bytes", "moe_lora_pack_mxfp8_weights", "moe_lora_forward_static")
STATIC_SCRATCH_BYTES = 64 << 20


class MoeLoraDims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("I", ctypes.c_int64), ("E", ctypes.c_int64),
                ("K", ctypes.c_int64), ("S", ctypes.c_int64), ("L", ctypes.c_int64), ("r", ctypes.c_int64),
                ("routed_scaling_factor", ctypes.c_float), ("renormalize", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("block_m", ctypes.c_int32), ("lora_block_m", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("router", ctypes.c_int32)]


class MoeLoraPlan(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("lora_block_m", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("gemm_kind", ctypes.c_int32), ("max_blocks", ctypes.c_int64),
                ("sorted_capacity", ctypes.c_int64), ("max_items", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_size_t), ("align_workspace_bytes", ctypes.c_size_t)]


class MoeLoraArgs(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_void_p), ("router_logits", ctypes.c_void_p),
                ("adapter_ids", ctypes.c_void_p), ("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("a13", ctypes.c_void_p), ("b13", ctypes.c_void_p), ("a2", ctypes.c_void_p),
                ("b2", ctypes.c_void_p), ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("topk_ids_out", ctypes.c_void_p),
                ("topk_weights_out", ctypes.c_void_p), ("stage_events", ctypes.c_void_p),
                ("weights_packed", ctypes.c_int32), ("weights_mxfp8", ctypes.c_int32),
                ("w13_scale", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p), ("expert_bias", ctypes.c_void_p),
                ("sorted_ids_out", ctypes.c_void_p), ("block_expert_out", ctypes.c_void_p),
                ("num_post_pad_out", ctypes.c_void_p)]


class MoeLoraError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {moe_lora_strerror(code)} (code {code})")
        self.code = code


def library_path() -> Path:
    return _LIB_PATH


def lib():
    """Load libmoelora.so once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        raise RuntimeError(f"HIP library {_LIB_PATH} is missing; build it with "
                           "`python -m lora_expert_gemm_topk_amd.build`")
    L = ctypes.CDLL(str(_LIB_PATH))
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    L.moe_lora_plan_query.argtypes = [P(MoeLoraDims), P(MoeLoraPlan)]
    L.moe_lora_plan_query.restype = ctypes.c_int
    L.moe_lora_workspace_bytes.argtypes = [P(MoeLoraDims)]
    L.moe_lora_workspace_bytes.restype = ctypes.c_size_t
    L.moe_lora_check_args.argtypes = [P(MoeLoraDims), P(MoeLoraArgs)]
    L.moe_lora_check_args.restype = ctypes.c_int
    L.moe_lora_route.argtypes = [P(MoeLoraDims), vp, vp, vp, vp, vp]
    L.moe_lora_route.restype = ctypes.c_int
    L.moe_lora_align.argtypes = [P(MoeLoraDims), vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.moe_lora_align.restype = ctypes.c_int
    L.moe_lora_forward.argtypes = [P(MoeLoraDims), P(MoeLoraArgs), vp]
    L.moe_lora_forward.restype = ctypes.c_int
    L.moe_lora_forward_static.argtypes = [P(MoeLoraDims), P(MoeLoraArgs), vp]
    L.moe_lora_forward_static.restype = ctypes.c_int
    L.moe_lora_packed_weight_bytes.argtypes = [P(MoeLoraDims), ctypes.c_int]
    L.moe_lora_packed_weight_bytes.restype = ctypes.c_size_t
    L.moe_lora_pack_weights.argtypes = [P(MoeLoraDims), vp, vp, vp, vp, vp]
    L.moe_lora_pack_weights.restype = ctypes.c_int
    L.moe_lora_packed_mxfp8_bytes.argtypes = [P(MoeLoraDims), ctypes.c_int]
    L.moe_lora_packed_mxfp8_bytes.restype = ctypes.c_size_t
    L.moe_lora_pack_mxfp8_weights.argtypes = [P(MoeLoraDims), vp, vp, vp, vp, vp]
    L.moe_lora_pack_mxfp8_weights.restype = ctypes.c_int
    L.moe_lora_check_inputs.argtypes = [P(MoeLoraDims), P(MoeLoraArgs), vp, vp]
    L.moe_lora_check_inputs.restype = ctypes.c_int
    L.moe_lora_strerror.argtypes = [ctypes.c_int]
    L.moe_lora_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def make_dims(T, H, I, E, K, S=0, L=0, r=0, rsf=1.0, renormalize=1, dtype="bf16", block_m=0,
              lora_block_m=0, split_k=0, router="topk") -> MoeLoraDims:
    dt = {"bf16": MOE_LORA_BF16, "f32": MOE_LORA_F32, torch.bfloat16: MOE_LORA_BF16,
          torch.float32: MOE_LORA_F32}.get(dtype, dtype)
    return MoeLoraDims(int(T), int(H), int(I), int(E), int(K), int(S), int(L), int(r), float(rsf),
                       int(renormalize), int(dt), int(block_m), int(lora_block_m), int(split_k),
                       int(ROUTERS.get(router, router)))


def moe_lora_strerror(code: int) -> str:
    return lib().moe_lora_strerror(int(code)).decode()


def moe_lora_plan_query(dims: MoeLoraDims) -> dict:
    p = MoeLoraPlan()
    rc = lib().moe_lora_plan_query(ctypes.byref(dims), ctypes.byref(p))
    if rc != MOE_LORA_OK:
        raise MoeLoraError(rc, "moe_lora_plan_query")
    return {name: getattr(p, name) for name, _ in MoeLoraPlan._fields_}


def moe_lora_workspace_bytes(dims: MoeLoraDims) -> int:
    return int(lib().moe_lora_workspace_bytes(ctypes.byref(dims)))


def moe_lora_check_args(dims: MoeLoraDims, args: MoeLoraArgs) -> int:
    return int(lib().moe_lora_check_args(ctypes.byref(dims), ctypes.byref(args)))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dev_tensor(t, name, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def moe_lora_route(logits: torch.Tensor, K: int, S: int = 0, rsf: float = 1.0, renormalize: int = 1,
                   router: str = "topk", expert_bias: Optional[torch.Tensor] = None):
    """Top-K routing + shared-slot append on the GPU -> (topk_ids int32, topk_weights f32).
    router "bias_softmax" / "bias_sigmoid" selects the biased router (expert_bias [E] f32 or None)."""
    _dev_tensor(logits, "logits", torch.float32)
    _dev_tensor(expert_bias, "expert_bias", torch.float32)
    T, E = logits.shape
    if expert_bias is not None and tuple(expert_bias.shape) != (E,):
        raise ValueError(f"expert_bias has shape {tuple(expert_bias.shape)}, expected {(E,)}")
    dims = make_dims(T, 8, 8, E, K, S, 0, 0, rsf, renormalize, router=router)
    ids = torch.empty((T, K + S), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, K + S), dtype=torch.float32, device=logits.device)
    with torch.cuda.device(logits.device):
        rc = lib().moe_lora_route(ctypes.byref(dims), _ptr(logits), _ptr(expert_bias), _ptr(ids), _ptr(w),
                                  _stream(logits.device))
    if rc != MOE_LORA_OK:
        raise MoeLoraError(rc, "moe_lora_route")
    return ids, w


def moe_lora_align(topk_ids: torch.Tensor, adapter_ids: Optional[torch.Tensor], dims: MoeLoraDims) -> dict:
    """Alignment on the GPU.  Returns sorted_ids, block_expert, num_post_pad [1],
    lora_items [max_items, 4], num_items [1] and the plan, all device tensors."""
    _dev_tensor(topk_ids, "topk_ids", torch.int32)
    _dev_tensor(adapter_ids, "adapter_ids", torch.int32)
    if tuple(topk_ids.shape) != (dims.T, dims.K + dims.S):
        raise ValueError(f"topk_ids has shape {tuple(topk_ids.shape)}, expected {(dims.T, dims.K + dims.S)}")
    if adapter_ids is not None and tuple(adapter_ids.shape) != (dims.T,):
        raise ValueError(f"adapter_ids has shape {tuple(adapter_ids.shape)}, expected {(dims.T,)}")
    plan = moe_lora_plan_query(dims)
    dev = topk_ids.device
    sorted_ids = torch.empty(plan["sorted_capacity"], dtype=torch.int32, device=dev)
    block_expert = torch.empty(plan["max_blocks"], dtype=torch.int32, device=dev)
    npp = torch.zeros(1, dtype=torch.int32, device=dev)
    items = torch.empty((max(plan["max_items"], 1), 4), dtype=torch.int32, device=dev)
    nitems = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = torch.empty(max(plan["align_workspace_bytes"], 256), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        rc = lib().moe_lora_align(ctypes.byref(dims), _ptr(topk_ids), _ptr(adapter_ids), _ptr(sorted_ids),
                                  _ptr(block_expert), _ptr(npp), _ptr(items), _ptr(nitems), _ptr(ws),
                                  ctypes.c_size_t(ws.numel()), _stream(dev))
    if rc != MOE_LORA_OK:
        raise MoeLoraError(rc, "moe_lora_align")
    return dict(sorted_ids=sorted_ids, block_expert=block_expert, num_post_pad=npp,
                lora_items=items[:plan["max_items"]], num_items=nitems, plan=plan)


def moe_lora_packed_mxfp8_bytes(dims: MoeLoraDims, which: int) -> int:
    """Bytes of the packed MXFP8 codes of w13 (which=0) or w2 (which=1); 0 if none."""
    return int(lib().moe_lora_packed_mxfp8_bytes(ctypes.byref(dims), int(which)))


def moe_lora_packed_weight_bytes(dims: MoeLoraDims, which: int) -> int:
    """Bytes of the packed w13 (which=0) or w2 (which=1); 0 if unsupported."""
    return int(lib().moe_lora_packed_weight_bytes(ctypes.byref(dims), int(which)))


def _layout_dims(Ep: int, H: int, I: int) -> MoeLoraDims:
    """Dims that describe only the stacked weights' shapes (E+S = Ep expert
    slices): the routing fields do not affect the packed layouts, so one
    token and K = 1 stand in, with up to 1024 routed experts and the rest as
    shared slots (the largest router the layer takes, E = 1024 and S = 64)."""
    E = min(Ep, 1024)
    return make_dims(1, H, I, E, 1, Ep - E, 0, 0, 1.0, 1, "bf16")


class PackedWeights:
    """w13 and w2 re-laid out once by moe_lora_pack_weights (bf16 only).

    Pass an instance as `w13` (with `w2=None`) to moe_lora_forward; the layer
    then reads the packed copies and gives the same bits as with the
    row-major weights.  Holds the shapes the layout was made for."""

    def __init__(self, w13: torch.Tensor, w2: torch.Tensor):
        _dev_tensor(w13, "w13", torch.bfloat16)
        _dev_tensor(w2, "w2", torch.bfloat16)
        self.Ep, twoI, self.H = (int(v) for v in w13.shape)
        self.I = twoI // 2
        if tuple(w2.shape) != (self.Ep, self.H, self.I):
            raise ValueError(f"w2 shape {tuple(w2.shape)} does not match w13 {tuple(w13.shape)}")
        self.dims = _layout_dims(self.Ep, self.H, self.I)
        n13 = moe_lora_packed_weight_bytes(self.dims, 0)
        n2 = moe_lora_packed_weight_bytes(self.dims, 1)
        if n13 == 0 or n2 == 0:
            raise ValueError("weights cannot be packed for these shapes")
        self.w13 = torch.empty(n13, dtype=torch.uint8, device=w13.device)
        self.w2 = torch.empty(n2, dtype=torch.uint8, device=w13.device)
        self.device = w13.device
        with torch.cuda.device(w13.device):
            rc = lib().moe_lora_pack_weights(ctypes.byref(self.dims), w13.data_ptr(), w2.data_ptr(),
                                             self.w13.data_ptr(), self.w2.data_ptr(), _stream(w13.device))
        if rc != MOE_LORA_OK:
            raise MoeLoraError(rc, "moe_lora_pack_weights")


class Workspace:
    """A reusable device workspace: grows on demand, never shrinks."""

    def __init__(self):
        self.buf: Optional[torch.Tensor] = None

    def get(self, nbytes: int, device) -> torch.Tensor:
        nbytes = max(int(nbytes), 256)
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != torch.device(device):
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        return self.buf


class Mxfp8Weights:
    """MXFP8 expert weights for moe_lora_forward (moe_lora_args.weights_mxfp8):
    FP8 E4M3 codes w13 [E+S,2I,H] and w2 [E+S,H,I] (uint8) with one E8M0
    scale byte per 32 elements along the reduction, w13_scale [E+S,2I,H/32]
    and w2_scale [E+S,H,I/32] (uint8).  Pass it as w13 with w2=None."""

    def __init__(self, w13: torch.Tensor, w13_scale: torch.Tensor, w2: torch.Tensor, w2_scale: torch.Tensor):
        for name, t in (("w13", w13), ("w13_scale", w13_scale), ("w2", w2), ("w2_scale", w2_scale)):
            _dev_tensor(t, name, torch.uint8)
        Ep, twoI, H = w13.shape
        I = twoI // 2
        if tuple(w2.shape) != (Ep, H, I) or tuple(w13_scale.shape) != (Ep, twoI, H // 32) or \
                tuple(w2_scale.shape) != (Ep, H, I // 32) or H % 32 or I % 32:
            raise ValueError("MXFP8 weights: w13 [E',2I,H], w13_scale [E',2I,H/32], w2 [E',H,I], "
                             "w2_scale [E',H,I/32] with H and I multiples of 32")
        self.w13, self.w13_scale, self.w2, self.w2_scale = w13, w13_scale, w2, w2_scale
        self.Ep, self.I, self.H = Ep, I, H
        self.device = w13.device
        self.packed = False

    def pack(self) -> "Mxfp8Weights":
        """A copy whose codes are in the packed order of
        moe_lora_pack_mxfp8_weights (same scales, bit-identical results)."""
        dims = _layout_dims(self.Ep, self.H, self.I)
        n13, n2 = moe_lora_packed_mxfp8_bytes(dims, 0), moe_lora_packed_mxfp8_bytes(dims, 1)
        if not n13 or not n2:
            raise ValueError("no packed MXFP8 form for this shape")
        p13 = torch.empty(n13, dtype=torch.uint8, device=self.device)
        p2 = torch.empty(n2, dtype=torch.uint8, device=self.device)
        with torch.cuda.device(self.device):
            rc = lib().moe_lora_pack_mxfp8_weights(ctypes.byref(dims), _ptr(self.w13), _ptr(self.w2), _ptr(p13),
                                                   _ptr(p2), _stream(self.device))
        if rc != MOE_LORA_OK:
            raise MoeLoraError(rc, "moe_lora_pack_mxfp8_weights")
        out = Mxfp8Weights.__new__(Mxfp8Weights)
        out.w13, out.w13_scale, out.w2, out.w2_scale = p13, self.w13_scale, p2, self.w2_scale
        out.Ep, out.I, out.H, out.device, out.packed = self.Ep, self.I, self.H, self.device, True
        return out


def moe_lora_forward(x: torch.Tensor, logits: torch.Tensor, adapter_ids: Optional[torch.Tensor],
                     w13: torch.Tensor, w2: torch.Tensor, a13=None, b13=None, a2=None, b2=None, *,
                     K: int, S: int = 0, rsf: float = 1.0, renormalize: int = 1,
                     out: Optional[torch.Tensor] = None, workspace: Optional[Workspace] = None,
                     block_m: int = 0, lora_block_m: int = 0, split_k: int = 0,
                     routing_out: Optional[tuple] = None, stage_events=None, router: str = "topk",
                     expert_bias: Optional[torch.Tensor] = None, align_out: Optional[tuple] = None) -> torch.Tensor:
    """The fused MoE-LoRA layer on the GPU (enqueued on the current stream).

    Shapes: x [T,H], logits [T,E] f32, adapter_ids [T] i32 (-1 = none),
    w13 [E+S,2I,H], w2 [E+S,H,I] (or w13 = PackedWeights or Mxfp8Weights of
    both, w2 = None),
    a13 [L,E+S,r,H], b13 [L,E+S,2I,r],
    a2 [L,E+S,r,I], b2 [L,E+S,H,r]; x, weights and out share one dtype
    (bf16 or f32).  routing_out = (ids [T,K+S] i32, weights [T,K+S] f32)
    receives the routing decisions when given.  stage_events: optional
    ctypes array of 2*len(STAGES) hipEvent_t handles recorded around each
    stage on the launch stream.  router / expert_bias: see moe_lora_route.
    align_out = (sorted_ids, block_expert, num_post_pad) int32 device
    tensors of the plan's sizes receives the alignment when given."""
    dims, args, out, _ws = _layer_args(x, logits, adapter_ids, w13, w2, a13, b13, a2, b2, K=K, S=S, rsf=rsf,
                                       renormalize=renormalize, out=out, workspace=workspace, block_m=block_m,
                                       lora_block_m=lora_block_m, split_k=split_k, routing_out=routing_out,
                                       stage_events=stage_events, router=router, expert_bias=expert_bias,
                                       align_out=align_out)
    with torch.cuda.device(x.device):
        rc = lib().moe_lora_forward(ctypes.byref(dims), ctypes.byref(args), _stream(x.device))
    if rc != MOE_LORA_OK:
        raise MoeLoraError(rc, "moe_lora_forward")
    return out


def moe_lora_forward_static(x: torch.Tensor, logits: torch.Tensor, adapter_ids: Optional[torch.Tensor],
                            w13, w2, a13=None, b13=None, a2=None, b2=None, *, K: int, S: int = 0,
                            rsf: float = 1.0, renormalize: int = 1, out: Optional[torch.Tensor] = None,
                            **kw) -> torch.Tensor:
    """moe_lora_forward through the entry point that allocates nothing: the
    library's fixed per-GPU scratch array (STATIC_SCRATCH_BYTES) stands in for
    the workspace.  Same arguments as moe_lora_forward (no workspace).  `out`
    is allocated here when not given; pass it for a call that must not
    allocate."""
    if out is None:
        out = torch.empty((x.shape[0], x.shape[1]), dtype=x.dtype, device=x.device)
    dims, args, out, _ws = _layer_args(x, logits, adapter_ids, w13, w2, a13, b13, a2, b2, K=K, S=S, rsf=rsf,
                                       renormalize=renormalize, out=out, workspace=_NO_WORKSPACE, **kw)
    with torch.cuda.device(x.device):
        rc = lib().moe_lora_forward_static(ctypes.byref(dims), ctypes.byref(args), _stream(x.device))
    if rc != MOE_LORA_OK:
        raise MoeLoraError(rc, "moe_lora_forward_static")
    return out


class _NoWorkspace:
    """Workspace stand-in for moe_lora_forward_static: no buffer at all."""

    def get(self, nbytes, device):
        return None


_NO_WORKSPACE = _NoWorkspace()


def moe_lora_check_inputs(x: torch.Tensor, logits: torch.Tensor, adapter_ids: Optional[torch.Tensor],
                          w13: torch.Tensor, w2: torch.Tensor, a13=None, b13=None, a2=None, b2=None, *,
                          K: int, S: int = 0, rsf: float = 1.0, renormalize: int = 1,
                          workspace: Optional[Workspace] = None, status: Optional[torch.Tensor] = None,
                          **kw) -> torch.Tensor:
    """Checks the device-side preconditions of moe_lora_forward on the same
    arguments (finite logits, adapter ids in [-1, L), valid MXFP8 scales and
    codes).  Returns the device int32 status word (enqueued on the current
    stream): the OR of the MOE_LORA_BAD_* flags found, 0 when none."""
    # the check writes no output: x stands in for `out`, which only has to pass the argument checks
    dims, args, _out, _ws = _layer_args(x, logits, adapter_ids, w13, w2, a13, b13, a2, b2, K=K, S=S, rsf=rsf,
                                        renormalize=renormalize, out=x, workspace=workspace, **kw)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=x.device)
    _dev_tensor(status, "status", torch.int32)
    with torch.cuda.device(x.device):
        rc = lib().moe_lora_check_inputs(ctypes.byref(dims), ctypes.byref(args), _ptr(status), _stream(x.device))
    if rc != MOE_LORA_OK:
        raise MoeLoraError(rc, "moe_lora_check_inputs")
    return status


def _layer_args(x, logits, adapter_ids, w13, w2, a13, b13, a2, b2, *, K, S, rsf, renormalize, out, workspace,
                block_m=0, lora_block_m=0, split_k=0, routing_out=None, stage_events=None, router="topk",
                expert_bias=None, align_out=None):
    """Marshals the layer's tensors (shapes as for moe_lora_forward) into
    (dims, args, out, workspace tensor)."""
    dt = x.dtype
    packed = isinstance(w13, PackedWeights)
    mx = isinstance(w13, Mxfp8Weights)
    if packed or mx:
        if w2 is not None:
            raise ValueError("with PackedWeights or Mxfp8Weights as w13, pass w2=None")
        if w13.device != x.device:
            raise ValueError("the weights live on another device")
        Ep, I = w13.Ep, w13.I
    for name, t in (("x", x), ("a13", a13), ("b13", b13), ("a2", a2), ("b2", b2)) + \
            (() if packed or mx else (("w13", w13), ("w2", w2))):
        _dev_tensor(t, name, dt)
    _dev_tensor(logits, "logits", torch.float32)
    _dev_tensor(adapter_ids, "adapter_ids", torch.int32)
    _dev_tensor(expert_bias, "expert_bias", torch.float32)
    T, H = x.shape
    if (packed or mx) and w13.H != H:
        raise ValueError(f"the weights are for H={w13.H}, x has H={H}")
    if not (packed or mx):
        Ep, twoI, _ = w13.shape
        I = twoI // 2
    E = logits.shape[1]
    L, r = (a13.shape[0], a13.shape[2]) if a13 is not None else (0, 0)
    want = {"logits": (logits, (T, E)), "out": (out, (T, H)), "expert_bias": (expert_bias, (E,))}
    if not (packed or mx):
        want.update(w13=(w13, (E + S, 2 * I, H)), w2=(w2, (E + S, H, I)))
    elif Ep != E + S:
        raise ValueError(f"the weights hold {Ep} experts, E+S = {E + S}")
    if a13 is not None:
        want.update(adapter_ids=(adapter_ids, (T,)), a13=(a13, (L, E + S, r, H)), b13=(b13, (L, E + S, 2 * I, r)),
                    a2=(a2, (L, E + S, r, I)), b2=(b2, (L, E + S, H, r)))
    for name, (t, shp) in want.items():
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
    dims = make_dims(T, H, I, E, K, S, L, r, rsf, renormalize, dt, block_m, lora_block_m, split_k, router)
    if align_out is not None:
        plan = moe_lora_plan_query(dims)
        for name, t, n in zip(("sorted_ids", "block_expert", "num_post_pad"), align_out,
                              (plan["sorted_capacity"], plan["max_blocks"], 1)):
            _dev_tensor(t, name, torch.int32)
            if t.numel() != n:
                raise ValueError(f"{name} must hold {n} int32 values, got {t.numel()}")
    if out is None:
        out = torch.empty((T, H), dtype=dt, device=x.device)
    _dev_tensor(out, "out", dt)
    nbytes = moe_lora_workspace_bytes(dims)
    ws = (workspace or Workspace()).get(nbytes, x.device)
    ids_out, w_out = routing_out if routing_out is not None else (None, None)
    w13_ptr, w2_ptr = (w13.w13.data_ptr(), w13.w2.data_ptr()) if packed or mx else (w13.data_ptr(), w2.data_ptr())
    args = MoeLoraArgs(x.data_ptr(), logits.data_ptr(), adapter_ids.data_ptr() if adapter_ids is not None else None,
                       w13_ptr, w2_ptr,
                       *(t.data_ptr() if t is not None else None for t in (a13, b13, a2, b2)),
                       out.data_ptr(), ws.data_ptr() if ws is not None else None,
                       ws.numel() if ws is not None else 0,
                       ids_out.data_ptr() if ids_out is not None else None,
                       w_out.data_ptr() if w_out is not None else None,
                       ctypes.cast(stage_events, ctypes.c_void_p) if stage_events is not None else None,
                       1 if packed or (mx and w13.packed) else 0, 1 if mx else 0,
                       w13.w13_scale.data_ptr() if mx else None, w13.w2_scale.data_ptr() if mx else None,
                       expert_bias.data_ptr() if expert_bias is not None else None,
                       *((t.data_ptr() for t in align_out) if align_out is not None else (None,) * 3))
    return dims, args, out, ws


def forward_inputs(inp, *, lora: bool = True, packed=None, **kw) -> torch.Tensor:
    """moe_lora_forward over a synth.LayerInputs bundle already on the GPU
    (with `packed`, a PackedWeights or Mxfp8Weights, those weights are read
    instead of its w13 and w2)."""
    s = inp.shape
    use = lora and s.lora
    w13, w2 = (packed, None) if packed is not None else (inp.w13, inp.w2)
    return moe_lora_forward(inp.x, inp.logits, inp.adapter_ids if use else None, w13, w2,
                            inp.a13 if use else None, inp.b13 if use else None,
                            inp.a2 if use else None, inp.b2 if use else None,
                            K=s.K, S=s.S, rsf=s.rsf, renormalize=s.renormalize, **kw)
