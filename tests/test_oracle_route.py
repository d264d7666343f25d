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


# ------------------------------------------------------------- biased router
# Reading of the biased top-k router the PR 46545 analysis names ("code
# analysis" part 1): fp64 expert scores (sigmoid, or softmax over all E), a
# per-expert bias added for the choice only, weights from the unbiased
# scores of the chosen experts.


@pytest.mark.parametrize("scoring", ["sigmoid", "softmax"])
@pytest.mark.parametrize("renorm", [1, 0])
@pytest.mark.parametrize("T,E,K,S", [(7, 5, 2, 0), (16, 32, 4, 1), (9, 64, 8, 0), (3, 6, 6, 2), (4, 130, 7, 0)])
def test_route_bias_vs_bruteforce(T, E, K, S, renorm, scoring):
    rng = np.random.default_rng(T * 1000 + E * 10 + K)
    lg = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.3).astype(np.float32)
    ids, w = oracle.route_bias(lg, K, S, 2.5, renorm, scoring, bias)
    bids, bw = bf.route_bias(lg, K, S, 2.5, renorm, scoring, bias)
    assert np.array_equal(ids, bids)
    assert np.all(np.abs(w - bw) <= np.spacing(np.abs(bw).astype(np.float32)))


def test_route_bias_zero_bias_softmax_equals_plain_router():
    """With no bias and softmax scores, choosing by the full-softmax score is
    choosing by logit, and the renormalized weights are the plain router's
    softmax over the chosen logits (to one fp32 ulp: a different rounding
    path for the same value)."""
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((40, 24)).astype(np.float32)
    for renorm in (1, 0):
        ids, w = oracle.route_bias(lg, 5, 1, 2.5, renorm, "softmax", None)
        pids, pw = oracle.route(lg, 5, 1, 2.5, renorm)
        assert np.array_equal(ids, pids)
        assert np.all(np.abs(w - pw) <= np.spacing(pw))


def test_route_bias_sigmoid_library_case():
    """Library special case: sigmoid is increasing, so with no bias the chosen
    experts are torch.topk of the logits (tie-free, moderate logits) and the
    weights are torch's fp64 sigmoid of them, renormalized or not."""
    g = torch.Generator().manual_seed(8)
    lg = torch.randn(64, 48, generator=g) * 3
    v, i = torch.topk(lg, 6, dim=1)
    sg = torch.sigmoid(v.double())
    for renorm, ref in ((0, sg), (1, sg / sg.sum(dim=1, keepdim=True))):
        ids, w = oracle.route_bias(lg.numpy(), 6, 0, 1.0, renorm, "sigmoid", None)
        assert np.array_equal(ids, i.numpy())
        r = ref.float().numpy()
        assert np.all(np.abs(w - r) <= np.spacing(r))


@pytest.mark.parametrize("scoring", ["sigmoid", "softmax"])
def test_route_bias_dominant_bias_forces_choice(scoring):
    """A bias larger than any score difference decides the choice: experts
    with bias +10 (and only they) are chosen first, in order of their bias
    when the biases differ; the weights still come from the unbiased scores."""
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((20, 16)).astype(np.float32)
    bias = np.zeros(16, np.float32)
    bias[[11, 3]] = [20.0, 10.0]
    ids, w = oracle.route_bias(lg, 3, 0, 1.0, 0, scoring, bias)
    assert (ids[:, 0] == 11).all() and (ids[:, 1] == 3).all()
    # third slot: the best remaining expert by score alone
    l64 = lg.astype(np.float64)
    ex = np.exp(l64 - l64.max(1, keepdims=True))
    sc = 1 / (1 + np.exp(-l64)) if scoring == "sigmoid" else ex / ex.sum(1, keepdims=True)
    rest = sc.copy()
    rest[:, [11, 3]] = -1
    assert np.array_equal(ids[:, 2], rest.argmax(1))
    ref = np.take_along_axis(sc, ids.astype(np.int64), 1).astype(np.float32)
    assert np.all(np.abs(w - ref) <= np.spacing(ref))


def test_route_bias_weights_ignore_the_bias():
    """Two biases that lead to the same choice give bit-identical weights:
    the bias steers the choice only."""
    rng = np.random.default_rng(6)
    lg = rng.standard_normal((30, 10)).astype(np.float32)
    b1 = (rng.standard_normal(10) * 1e-3).astype(np.float32)
    ids0, w0 = oracle.route_bias(lg, 4, 0, 1.0, 1, "sigmoid", None)
    ids1, w1 = oracle.route_bias(lg, 4, 0, 1.0, 1, "sigmoid", b1)
    same = (ids0 == ids1).all(axis=1)
    assert same.sum() >= 20
    assert np.array_equal(w0[same].view(np.int32), w1[same].view(np.int32))


def test_route_bias_ties_and_invariants():
    """Exact key ties go to the lower index (+0 == -0), ids are distinct, and
    renormalized weights sum to one."""
    lg = np.array([[0.5, 0.5, 0.5, -0.5], [0.0, -0.0, 1.0, 1.0]], np.float32)
    ids, w = oracle.route_bias(lg, 2, 0, 1.0, 1, "sigmoid", np.zeros(4, np.float32))
    assert ids.tolist() == [[0, 1], [2, 3]]
    assert w[0, 0] == w[0, 1] == np.float32(0.5)
    rng = np.random.default_rng(9)
    lg = rng.standard_normal((50, 20)).astype(np.float32)
    ids, w = oracle.route_bias(lg, 5, 0, 1.0, 1, "softmax", rng.standard_normal(20).astype(np.float32) * 0.05)
    assert all(len(set(r)) == 5 for r in ids.tolist())
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 5 * 2**-24)


@settings(max_examples=60, deadline=None)
@given(T=st.integers(0, 5), E=st.integers(1, 10), data=st.data())
def test_route_bias_hypothesis(T, E, data):
    K = data.draw(st.integers(1, E))
    S = data.draw(st.integers(0, 2))
    scoring = data.draw(st.sampled_from(["sigmoid", "softmax"]))
    vals = data.draw(st.lists(st.sampled_from([-2.0, -0.5, -0.0, 0.0, 0.5, 1.0, 3.0]),
                              min_size=T * E, max_size=T * E))
    bias = np.array(data.draw(st.lists(st.sampled_from([0.0, 0.125, -0.25, 1.0]), min_size=E, max_size=E)),
                    np.float32)
    lg = np.array(vals, np.float32).reshape(T, E)
    ids, w = oracle.route_bias(lg, K, S, 2.0, 1, scoring, bias)
    bids, bw = bf.route_bias(lg, K, S, 2.0, 1, scoring, bias)
    assert np.array_equal(ids, bids)
    assert np.all(np.abs(w - bw) <= np.spacing(np.abs(bw).astype(np.float32)))
