"""Pins of the oracle's MXFP8 weight decode, CPU only.

The pages name the ROCm path's mxfp8 experts module (secrett2633 analysis of
vLLM PR 46545, "code analysis" part 2) but do not define the format; the
reading taken is the MX one: FP8 E4M3 elements, one E8M0 scale per block of
32.  The decoder is pinned against torch's own float8_e4m3fn conversion (an
independent library routine) on every code, against values that follow from
the E4M3 definition alone (largest finite 448, smallest normal 2^-6,
smallest subnormal 2^-9), and against exact power-of-two scaling.
"""
import numpy as np
import pytest
import torch

import oracle
from lora_expert_gemm_topk_amd import synth

NAN_CODES = (0x7F, 0xFF)


def _one_block(codes, scale):
    c = np.zeros(32, np.uint8)
    c[: len(codes)] = codes
    return c[None, :], np.array([[scale]], np.uint8)


def test_every_code_matches_torch_float8():
    codes = np.array([c for c in range(256) if c not in NAN_CODES], np.uint8)
    pad = (-len(codes)) % 32
    cc = np.concatenate([codes, np.zeros(pad, np.uint8)]).reshape(-1, 32)
    sc = np.full((cc.shape[0], 1), 127, np.uint8)               # scale 2^0
    got = oracle.mxfp8_decode(cc, sc).reshape(-1)[: len(codes)]
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("code,value", [(0x7E, 448.0), (0xFE, -448.0), (0x08, 2.0 ** -6), (0x01, 2.0 ** -9),
                                        (0x07, 7 * 2.0 ** -9), (0x38, 1.0), (0xC0, -2.0), (0x00, 0.0),
                                        (0x3F, 1.875)])
def test_definition_values(code, value):
    c, s = _one_block([code], 127)
    assert oracle.mxfp8_decode(c, s)[0, 0] == value


@pytest.mark.parametrize("scale", [1, 100, 120, 127, 140, 254])
def test_scale_is_an_exact_power_of_two(scale):
    rng = np.random.default_rng(scale)
    codes = rng.choice([c for c in range(256) if c not in NAN_CODES], size=(3, 64)).astype(np.uint8)
    sc = np.full((3, 2), scale, np.uint8)
    one = oracle.mxfp8_decode(codes, np.full((3, 2), 127, np.uint8))
    assert np.array_equal(oracle.mxfp8_decode(codes, sc), np.ldexp(one, scale - 127))


def test_each_block_takes_its_own_scale():
    codes = np.full((2, 96), 0x38, np.uint8)                   # 1.0 everywhere
    sc = np.array([[120, 127, 130], [1, 254, 127]], np.uint8)
    got = oracle.mxfp8_decode(codes, sc)
    want = np.repeat(np.ldexp(1.0, sc.astype(int) - 127), 32, axis=1)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("bad", ["nan_code", "scale0", "scale255"])
def test_rejects_outside_the_precondition(bad):
    c, s = _one_block([0x38], 127)
    if bad == "nan_code":
        c[0, 5] = 0x7F
    else:
        s[0, 0] = 0 if bad == "scale0" else 255
    with pytest.raises(ValueError):
        oracle.mxfp8_decode(c, s)


def test_quantized_inputs_round_trip_within_e4m3_precision():
    """The seeded MXFP8 inputs decode to within half an E4M3 step of the
    weights they were drawn from (relative to each block's scale)."""
    w = torch.randn(3, 16, 128, generator=torch.Generator().manual_seed(0)) * 0.02
    codes, scales = synth.mxfp8_quantize(w)
    d = oracle.mxfp8_decode(codes, scales)
    step = np.repeat(np.ldexp(1.0, scales.numpy().astype(int) - 127), 32, axis=-1)  # one unit of the scale
    # |w| <= 448 * unit; E4M3 spacing at magnitude m is <= m / 8, so the error is <= 28 units
    assert np.all(np.abs(d - w.double().numpy()) <= 28 * step)
    assert oracle.mxfp8_to_bf16(codes, scales).dtype == torch.bfloat16
