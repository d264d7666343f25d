"""Pins of the oracle's router (top-k + shared-slot append), CPU only."""
import json
import struct
from pathlib import Path

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from tests import bruteforce as bf

GOLDEN = Path(__file__).parent / "golden"


def _f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def test_golden_shared_slot_layout():
    """Printed layout: shared ids E..E+S-1 after the routed top-k, weight 1/rsf."""
    spec = json.loads((GOLDEN / "shared_slot_layout.json").read_text())
    rng = np.random.default_rng(0)
    for c in spec["cases"]:
        lg = rng.standard_normal((5, c["E"])).astype(np.float32)
        ids, w = oracle.route(lg, c["K"], c["S"], c["rsf"])
        assert ids.shape == (5, c["K"] + c["S"])
        for t in range(5):
            assert list(ids[t, c["K"]:]) == c["tail_ids"]
            for q in range(c["S"]):
                assert _f32_bits(w[t, c["K"] + q]) == int(c["tail_weight_f32_hex"], 16)
            # routed part untouched by the append
            assert set(ids[t, :c["K"]]) <= set(range(c["E"]))


def test_golden_hand_example_route():
    spec = json.loads((GOLDEN / "hand_example.json").read_text())
    s = spec["shape"]
    ids, w = oracle.route(np.array(spec["inputs"]["logits"], np.float32), s["K"], s["S"], s["rsf"])
    assert ids.tolist() == spec["route_expected"]["topk_ids"]
    assert w.tolist() == spec["route_expected"]["topk_weights"]


@pytest.mark.parametrize("renorm", [1, 0])
@pytest.mark.parametrize("T,E,K", [(7, 5, 2), (16, 32, 4), (9, 64, 8), (3, 6, 6), (4, 130, 7)])
def test_route_vs_bruteforce(T, E, K, renorm):
    rng = np.random.default_rng(T * 1000 + E * 10 + K)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = oracle.route(lg, K, 0, 1.0, renorm)
    bids, bw = bf.route(lg, K, 0, 1.0, renorm)
    assert np.array_equal(ids, bids)
    # same math, different summation code: allow one fp32 ulp
    ulp = np.spacing(np.abs(bw).astype(np.float32))
    assert np.all(np.abs(w - bw) <= ulp)


def test_route_ties_lower_index_wins():
    lg = np.array([[1.0, 3.0, 3.0, 2.0, 3.0],
                   [0.0, -0.0, 0.0, -1.0, -0.0],
                   [5.0, 5.0, 5.0, 5.0, 5.0]], np.float32)
    ids, w = oracle.route(lg, 3)
    assert ids.tolist() == [[1, 2, 4], [0, 1, 2], [0, 1, 2]]
    # exact ties give exactly equal weights, 1/3 rounded once
    assert w[0, 0] == w[0, 1] == w[0, 2]
    assert w[2, 0] == np.float32(1.0 / 3.0)


def test_route_matches_torch_topk_softmax():
    """Library special case: on tie-free logits the ids equal torch.topk's and the
    weights equal torch's fp64 softmax of the selected logits."""
    g = torch.Generator().manual_seed(3)
    lg = torch.randn(64, 32, generator=g)
    ids, w = oracle.route(lg.numpy(), 4)
    v, i = torch.topk(lg, 4, dim=1)
    assert np.array_equal(ids, i.numpy())
    ref = torch.softmax(v.double(), dim=1).float().numpy()
    assert np.all(np.abs(w - ref) <= np.spacing(ref))


def test_route_invariants():
    rng = np.random.default_rng(11)
    lg = rng.standard_normal((50, 20)).astype(np.float32) * 4
    ids, w = oracle.route(lg, 5)
    for t in range(50):
        assert len(set(ids[t])) == 5
        # weights follow slot order (descending logits) and sum to one
        assert np.all(np.diff(w[t]) <= 0)
        assert abs(float(np.sum(w[t].astype(np.float64))) - 1.0) <= 5 * 2**-24
    # K = E selects every expert
    ids, _ = oracle.route(lg[:, :6], 6)
    assert all(sorted(r) == list(range(6)) for r in ids.tolist())


def test_route_renorm0_is_full_softmax():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((10, 12)).astype(np.float32)
    ids, w = oracle.route(lg, 3, renormalize=0)
    full = torch.softmax(torch.from_numpy(lg).double(), dim=1).numpy()
    ref = np.take_along_axis(full, ids.astype(np.int64), 1).astype(np.float32)
    assert np.all(np.abs(w - ref) <= np.spacing(ref))
    assert np.all(w.sum(1) < 1.0)


@settings(max_examples=60, deadline=None)
@given(T=st.integers(0, 6), E=st.integers(1, 12), data=st.data())
def test_route_hypothesis(T, E, data):
    K = data.draw(st.integers(1, E))
    S = data.draw(st.integers(0, 2))
    vals = data.draw(st.lists(st.sampled_from([-2.0, -0.5, -0.0, 0.0, 0.5, 1.0, 3.0]),
                              min_size=T * E, max_size=T * E))
    lg = np.array(vals, np.float32).reshape(T, E)
    ids, w = oracle.route(lg, K, S, 2.0)
    bids, bw = bf.route(lg, K, S, 2.0)
    assert np.array_equal(ids, bids)
    assert np.all(np.abs(w - bw) <= np.spacing(np.abs(bw).astype(np.float32)))
