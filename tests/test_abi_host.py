"""Host-only checks of the C ABI: the library loads without a GPU, exports every
symbol the header declares, and rejects bad arguments with the documented
codes before touching any device."""
import ctypes
import re
from pathlib import Path

import pytest

import lora_expert_gemm_topk_amd as ml
from lora_expert_gemm_topk_amd import moe_lora as mm

HEADER = Path(__file__).resolve().parent.parent / "include" / "moe_lora.h"


def _declared():
    txt = HEADER.read_text()
    return sorted(set(re.findall(r"^(?:int|size_t|const char \*)\s*(moe_lora_\w+)\s*\(", txt, re.M)))


def test_header_declares_the_entry_points():
    assert _declared() == sorted(mm.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(str(mm.library_path()))
    for name in _declared():
        assert hasattr(lib, name), name


def test_strerror_never_null():
    for c in (0, -1, -2, -3, -4, 17):
        assert isinstance(ml.moe_lora_strerror(c), str) and ml.moe_lora_strerror(c)


def _dims(**kw):
    base = dict(T=64, H=2880, I=2880, E=32, K=4, S=0, L=8, r=16)
    base.update(kw)
    return ml.make_dims(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(K=33), ml.MOE_LORA_EINVAL),            # K > E
    (dict(K=0), ml.MOE_LORA_EINVAL),
    (dict(T=-1), ml.MOE_LORA_EINVAL),
    (dict(H=0), ml.MOE_LORA_EINVAL),
    (dict(rsf=0.0), ml.MOE_LORA_EINVAL),
    (dict(rsf=float("nan")), ml.MOE_LORA_EINVAL),
    (dict(renormalize=2), ml.MOE_LORA_EINVAL),
    (dict(H=2884), ml.MOE_LORA_EUNSUPPORTED),    # H not a multiple of 8
    (dict(I=100), ml.MOE_LORA_EUNSUPPORTED),
    (dict(dtype=7), ml.MOE_LORA_EUNSUPPORTED),
    (dict(r=12), ml.MOE_LORA_EUNSUPPORTED),      # bf16 rank must be a multiple of 8
    (dict(r=256), ml.MOE_LORA_EUNSUPPORTED),
    (dict(E=2048, K=4), ml.MOE_LORA_EUNSUPPORTED),
    (dict(block_m=24), ml.MOE_LORA_EUNSUPPORTED),
    (dict(E=256, L=128), ml.MOE_LORA_EUNSUPPORTED),  # (E+S)*(L+1) over the align limit
])
def test_plan_rejects(kw, code):
    d = _dims(**kw)
    with pytest.raises(ml.MoeLoraError) as ei:
        ml.moe_lora_plan_query(d)
    assert ei.value.code == code
    assert ml.moe_lora_workspace_bytes(d) == 0


def test_plan_sizes_follow_the_bounds():
    for T, E, K, S, L, r in [(64, 32, 4, 0, 8, 16), (4096, 32, 4, 0, 32, 32), (1, 64, 8, 1, 0, 0),
                             (8192, 128, 8, 0, 64, 64), (16, 4, 2, 0, 2, 8)]:
        d = _dims(T=T, E=E, K=K, S=S, L=L, r=r)
        p = ml.moe_lora_plan_query(d)
        P, Ep = T * (K + S), E + S
        assert p["max_blocks"] == -(-P // p["block_m"]) + min(Ep, P)
        assert p["sorted_capacity"] == p["max_blocks"] * p["block_m"]
        if L and r:
            assert p["max_items"] == -(-P // p["lora_block_m"]) + min(P, L * Ep)
        else:
            assert p["max_items"] == 0
        assert p["workspace_bytes"] == ml.moe_lora_workspace_bytes(d) > 0


def test_align_workspace_covers_both_alignment_forms():
    """moe_lora_align's workspace holds the P-int scratch of the one-workgroup
    alignment and, from 8192 pairs on, the [slices][keys] + [keys] ints of the
    multi-workgroup form (slices of max(256, ceil(P/64) rounded up to 64)
    pairs)."""
    for T, E, K, S, L, r in [(64, 32, 4, 0, 8, 16), (2047, 7, 4, 0, 2, 8), (2048, 7, 4, 0, 2, 8),
                             (4096, 32, 4, 0, 32, 32), (8192, 128, 8, 0, 64, 64), (10000, 64, 8, 0, 16, 16)]:
        p = ml.moe_lora_plan_query(_dims(T=T, E=E, K=K, S=S, L=L, r=r))
        P, Ep = T * (K + S), E + S
        La = L if (L and r) else 0
        need = 4 * P
        if P >= 8192:
            chunk = max(256, -(-(-(-P // 64)) // 64) * 64)
            nb = -(-P // chunk)
            nk = Ep * (La + 1)
            need = max(need, 4 * (nb * nk + nk))
        assert p["align_workspace_bytes"] >= need + 64


def _args(**kw):
    a = ml.MoeLoraArgs()
    fields = dict(hidden=0x1000, router_logits=0x2000, adapter_ids=0x3000, w13=0x4000, w2=0x5000,
                  a13=0x6000, b13=0x7000, a2=0x8000, b2=0x9000, out=0xa000, workspace=0x10000,
                  workspace_bytes=1 << 40)
    fields.update(kw)
    for k, v in fields.items():
        setattr(a, k, v)
    return a


def test_check_args_codes_without_device():
    d = _dims()
    need = ml.moe_lora_workspace_bytes(d)
    assert ml.moe_lora_check_args(d, _args(workspace_bytes=need)) == ml.MOE_LORA_OK
    assert ml.moe_lora_check_args(d, _args(workspace_bytes=need - 1)) == ml.MOE_LORA_EWORKSPACE
    for name in ("hidden", "router_logits", "w13", "w2", "out", "workspace", "adapter_ids", "a13", "b2"):
        assert ml.moe_lora_check_args(d, _args(**{name: None})) == ml.MOE_LORA_EINVAL, name
    assert ml.moe_lora_check_args(d, _args(hidden=0x1008)) == ml.MOE_LORA_EINVAL     # misaligned
    assert ml.moe_lora_check_args(d, _args(workspace=0x10010)) == ml.MOE_LORA_EINVAL
    # without LoRA the adapter and LoRA pointers may be NULL
    d0 = _dims(L=0, r=0)
    assert ml.moe_lora_check_args(d0, _args(adapter_ids=None, a13=None, b13=None, a2=None, b2=None)) == 0
    # T = 0 is a no-op and needs no buffers
    assert ml.moe_lora_check_args(_dims(T=0), _args(hidden=None, out=None, workspace=None)) == 0


def test_check_args_weights_packed_flag():
    d = _dims()
    assert ml.moe_lora_check_args(d, _args(weights_packed=1)) == ml.MOE_LORA_OK
    assert ml.moe_lora_check_args(d, _args(weights_packed=2)) == ml.MOE_LORA_EINVAL
    assert ml.moe_lora_check_args(_dims(dtype="f32"), _args(weights_packed=1)) == ml.MOE_LORA_EUNSUPPORTED


def test_check_args_mxfp8_flag():
    d = _dims()                                   # decode shape: streaming GEMM, H = I = 2880
    sc = dict(w13_scale=0xb000, w2_scale=0xc000)
    assert ml.moe_lora_check_args(d, _args(weights_mxfp8=1, **sc)) == ml.MOE_LORA_OK
    assert ml.moe_lora_check_args(d, _args(weights_mxfp8=2, **sc)) == ml.MOE_LORA_EINVAL
    assert ml.moe_lora_check_args(d, _args(weights_mxfp8=1, w13_scale=0xb000)) == ml.MOE_LORA_EINVAL
    assert ml.moe_lora_check_args(d, _args(weights_mxfp8=1, w13_scale=0xb004, w2_scale=0xc000)) == ml.MOE_LORA_EINVAL
    assert ml.moe_lora_check_args(_dims(H=8224), _args(weights_mxfp8=1, **sc)) == ml.MOE_LORA_EUNSUPPORTED
    # bf16 only, H and I multiples of 32; packed codes allowed
    assert ml.moe_lora_check_args(_dims(dtype="f32"), _args(weights_mxfp8=1, **sc)) == ml.MOE_LORA_EUNSUPPORTED
    assert ml.moe_lora_check_args(d, _args(weights_mxfp8=1, weights_packed=1, **sc)) == ml.MOE_LORA_OK
    assert ml.moe_lora_check_args(_dims(H=2888), _args(weights_mxfp8=1, **sc)) == ml.MOE_LORA_EUNSUPPORTED
    assert ml.moe_lora_check_args(_dims(I=2888), _args(weights_mxfp8=1, **sc)) == ml.MOE_LORA_EUNSUPPORTED
    # the LDS-tiled GEMM takes K (H for gate_up, I for down) up to 3072, the
    # streaming one up to 8192
    big = _dims(T=4096, L=32, r=32)
    assert ml.moe_lora_plan_query(big)["gemm_kind"] == 2
    assert ml.moe_lora_check_args(big, _args(weights_mxfp8=1, **sc)) == ml.MOE_LORA_OK
    for H, I in ((3072, 3072), (3104, 2880), (2880, 3104)):
        want = ml.MOE_LORA_OK if max(H, I) <= 3072 else ml.MOE_LORA_EUNSUPPORTED
        assert ml.moe_lora_check_args(_dims(T=4096, H=H, I=I, L=32, r=32), _args(weights_mxfp8=1, **sc)) == want
        assert ml.moe_lora_check_args(_dims(T=4096, H=H, I=I, L=32, r=32, block_m=32),
                                      _args(weights_mxfp8=1, **sc)) == 0
    # the flag off ignores the scale pointers
    assert ml.moe_lora_check_args(d, _args()) == ml.MOE_LORA_OK


def test_packed_weight_bytes_formula():
    # w13: E+S experts x 16*ceil(I/128) groups x ceil(H/32) slabs x 1 KiB;
    # w2: E+S experts x 16*ceil(H/256) groups x ceil(I/32) slabs x 1 KiB
    for (H, I, E, S) in ((2880, 2880, 32, 0), (136, 200, 5, 1), (64, 8, 4, 0), (4096, 1536, 64, 1)):
        d = _dims(H=H, I=I, E=E, S=S)
        Ep = E + S
        assert mm.moe_lora_packed_weight_bytes(d, 0) == Ep * 16 * -(-I // 128) * -(-H // 32) * 1024
        assert mm.moe_lora_packed_weight_bytes(d, 1) == Ep * 16 * -(-H // 256) * -(-I // 32) * 1024
        assert mm.moe_lora_packed_weight_bytes(d, 2) == 0
    assert mm.moe_lora_packed_weight_bytes(_dims(dtype="f32"), 0) == 0
    assert mm.moe_lora_packed_weight_bytes(_dims(H=100), 0) == 0   # H not a multiple of 8


def test_pack_weights_rejects_without_device():
    L = mm.lib()
    d = _dims()
    vp = ctypes.c_void_p
    # a source without a destination (or the reverse), misaligned pointers, f32
    assert L.moe_lora_pack_weights(ctypes.byref(d), vp(0x1000), None, None, None, None) == ml.MOE_LORA_EINVAL
    assert L.moe_lora_pack_weights(ctypes.byref(d), None, None, None, vp(0x1000), None) == ml.MOE_LORA_EINVAL
    assert L.moe_lora_pack_weights(ctypes.byref(d), vp(0x1008), None, vp(0x2000), None, None) == ml.MOE_LORA_EINVAL
    assert L.moe_lora_pack_weights(ctypes.byref(_dims(dtype="f32")), vp(0x1000), None, vp(0x2000), None,
                                   None) == ml.MOE_LORA_EUNSUPPORTED
    # nothing to do is fine (no launch)
    assert L.moe_lora_pack_weights(ctypes.byref(d), None, None, None, None, None) == ml.MOE_LORA_OK


def test_check_inputs_rejects_without_device():
    L = mm.lib()
    d = _dims()
    st = ctypes.c_void_p(0x20000)
    # the same argument checks as moe_lora_check_args, then a null status
    assert L.moe_lora_check_inputs(ctypes.byref(d), ctypes.byref(_args(hidden=None)), st, None) == \
        ml.MOE_LORA_EINVAL
    assert L.moe_lora_check_inputs(ctypes.byref(_dims(r=12)), ctypes.byref(_args()), st, None) == \
        ml.MOE_LORA_EUNSUPPORTED
    need = ml.moe_lora_workspace_bytes(d)
    assert L.moe_lora_check_inputs(ctypes.byref(d), ctypes.byref(_args(workspace_bytes=need - 1)), st, None) == \
        ml.MOE_LORA_EWORKSPACE
    assert L.moe_lora_check_inputs(ctypes.byref(d), ctypes.byref(_args()), None, None) == ml.MOE_LORA_EINVAL


def test_packed_mxfp8_bytes_formula():
    # one 2 KiB block per 16 rows and 128-wide chunk of the reduction
    for (H, I, E, S) in ((2880, 2880, 32, 0), (64, 8192, 4, 1), (8192, 64, 128, 0), (96, 160, 5, 1)):
        d = _dims(H=H, I=I, E=E, S=S, K=1)
        Ep = E + S
        assert mm.moe_lora_packed_mxfp8_bytes(d, 0) == Ep * (2 * I // 16) * -(-H // 128) * 2048
        assert mm.moe_lora_packed_mxfp8_bytes(d, 1) == Ep * (H // 16) * -(-I // 128) * 2048
        assert mm.moe_lora_packed_mxfp8_bytes(d, 2) == 0
    assert mm.moe_lora_packed_mxfp8_bytes(_dims(H=2888), 0) == 0   # H not a multiple of 32


def test_pack_mxfp8_rejects_without_device():
    L = mm.lib()
    d = _dims()
    vp = ctypes.c_void_p
    assert L.moe_lora_pack_mxfp8_weights(ctypes.byref(d), vp(0x1000), None, None, None, None) == ml.MOE_LORA_EINVAL
    assert L.moe_lora_pack_mxfp8_weights(ctypes.byref(d), vp(0x1008), None, vp(0x2000), None, None) == \
        ml.MOE_LORA_EINVAL
    assert L.moe_lora_pack_mxfp8_weights(ctypes.byref(_dims(H=2888)), vp(0x1000), None, vp(0x2000), None,
                                         None) == ml.MOE_LORA_EUNSUPPORTED
    assert L.moe_lora_pack_mxfp8_weights(ctypes.byref(d), None, None, None, None, None) == ml.MOE_LORA_OK


def test_router_and_alignment_outputs_checked_on_host():
    d = _dims()
    # router outside {0, 1, 2}; a bias with the plain top-k router
    with pytest.raises(ml.MoeLoraError) as ei:
        ml.moe_lora_plan_query(_dims(router=3))
    assert ei.value.code == ml.MOE_LORA_EINVAL
    assert ml.moe_lora_check_args(d, _args(expert_bias=0xd000)) == ml.MOE_LORA_EINVAL
    for r in ("bias_softmax", "bias_sigmoid"):
        db = _dims(router=r)
        assert ml.moe_lora_check_args(db, _args(expert_bias=0xd000)) == ml.MOE_LORA_OK
        assert ml.moe_lora_check_args(db, _args()) == ml.MOE_LORA_OK         # no bias = zero bias
        assert ml.moe_lora_check_args(db, _args(expert_bias=0xd002)) == ml.MOE_LORA_EINVAL
    # optional alignment outputs: any 4-byte aligned buffer, misaligned rejected
    ok = dict(sorted_ids_out=0xe000, block_expert_out=0xf000, num_post_pad_out=0xf800)
    assert ml.moe_lora_check_args(d, _args(**ok)) == ml.MOE_LORA_OK
    for name in ok:
        assert ml.moe_lora_check_args(d, _args(**{**ok, name: ok[name] + 2})) == ml.MOE_LORA_EINVAL, name
    L = mm.lib()
    vp = ctypes.c_void_p
    assert L.moe_lora_route(ctypes.byref(d), vp(0x1000), vp(0x2000), vp(0x3000), vp(0x4000), None) == \
        ml.MOE_LORA_EINVAL
    assert L.moe_lora_route(ctypes.byref(_dims(router=5)), vp(0x1000), None, vp(0x3000), vp(0x4000), None) == \
        ml.MOE_LORA_EINVAL


def test_forward_static_rejects_on_host():
    """The no-allocation entry point checks sizes and arguments before it
    touches a device: a plan larger than the fixed scratch gives
    MOE_LORA_EWORKSPACE, a null input MOE_LORA_EINVAL, T = 0 is a no-op."""
    L = mm.lib()
    prefill = _dims(T=4096, L=32, r=32)
    assert ml.moe_lora_workspace_bytes(prefill) > mm.STATIC_SCRATCH_BYTES
    assert L.moe_lora_forward_static(ctypes.byref(prefill), ctypes.byref(_args()), None) == ml.MOE_LORA_EWORKSPACE
    d = _dims()
    assert ml.moe_lora_workspace_bytes(d) <= mm.STATIC_SCRATCH_BYTES
    assert L.moe_lora_forward_static(ctypes.byref(d), ctypes.byref(_args(hidden=None)), None) == ml.MOE_LORA_EINVAL
    assert L.moe_lora_forward_static(ctypes.byref(_dims(r=12)), ctypes.byref(_args()), None) == \
        ml.MOE_LORA_EUNSUPPORTED
    assert L.moe_lora_forward_static(ctypes.byref(_dims(T=0)), ctypes.byref(_args(hidden=None)), None) == 0
    # the workspace fields are ignored: no workspace pointer is needed
    assert L.moe_lora_forward_static(ctypes.byref(d), ctypes.byref(_args(workspace=None, workspace_bytes=0,
                                                                          hidden=None)), None) == ml.MOE_LORA_EINVAL


def test_packing_dims_cover_the_largest_router():
    """Packed layouts depend only on the weight shapes: stacks of more than
    1024 expert slices (1024 routed + shared slots) have a packed size."""
    for Ep in (1, 1024, 1025, 1088):
        d = mm._layout_dims(Ep, 64, 32)
        assert d.E + d.S == Ep and d.E <= 1024
        assert mm.moe_lora_packed_weight_bytes(d, 0) == Ep * 16 * 1 * 2 * 1024
        assert mm.moe_lora_packed_mxfp8_bytes(d, 1) == Ep * (64 // 16) * 1 * 2048
