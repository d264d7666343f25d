"""Pins of the oracle's expert/adapter alignment, CPU only."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from tests import bruteforce as bf


def _random_ids(rng, T, K, E, S):
    ids = np.zeros((T, K + S), np.int32)
    for t in range(T):
        ids[t, :K] = rng.choice(E, K, replace=False)
        ids[t, K:] = np.arange(E, E + S)
    return ids


def _check_vs_bruteforce(ids, ad, Ep, La, bm, lbm):
    o = oracle.align(ids, ad, Ep, La, bm, lbm)
    b = bf.align(ids, ad, Ep, La, bm, lbm)
    P = ids.size
    n = o["num_post_pad"]
    assert n == b["num_post_pad"]
    assert np.array_equal(o["sorted_ids"][:n], b["sorted_ids"])
    assert np.all(o["sorted_ids"][n:] == P)
    nb = n // bm
    assert np.array_equal(o["block_expert"][:nb], b["block_expert"])
    assert np.all(o["block_expert"][nb:] == -1)
    if La > 0:
        assert o["num_items"] == len(b["items"])
        assert np.array_equal(o["items"][:o["num_items"]], b["items"])
        assert np.all(o["items"][o["num_items"]:] == np.array([0, 0, -1, -1]))
    return o


@pytest.mark.parametrize("T,K,E,S,L,bm,lbm", [
    (8, 2, 4, 0, 0, 4, 4), (16, 2, 4, 0, 2, 16, 8), (13, 3, 6, 1, 3, 2, 2),
    (40, 4, 8, 0, 5, 16, 4), (5, 1, 3, 1, 1, 4, 16), (64, 4, 32, 0, 8, 32, 16)])
def test_align_vs_bruteforce(T, K, E, S, L, bm, lbm):
    rng = np.random.default_rng(T + 7 * E + L)
    ids = _random_ids(rng, T, K, E, S)
    ad = rng.integers(-1, L, T).astype(np.int32) if L > 0 else None
    _check_vs_bruteforce(ids, ad, E + S, L, bm, lbm)


def test_align_invariants():
    rng = np.random.default_rng(2)
    T, K, E, S, L, bm, lbm = 300, 4, 16, 1, 6, 16, 8
    ids = _random_ids(rng, T, K, E, S)
    ad = rng.integers(-1, L, T).astype(np.int32)
    o = oracle.align(ids, ad, E + S, L, bm, lbm)
    P = T * (K + S)
    n = o["num_post_pad"]
    s = o["sorted_ids"][:n]
    real = s[s < P]
    assert np.array_equal(np.sort(real), np.arange(P))          # every pair exactly once
    cnt = np.bincount(ids.reshape(-1), minlength=E + S)
    assert n == int(np.sum((cnt + bm - 1) // bm * bm))           # padded count formula
    be = o["block_expert"][: n // bm]
    assert np.all(np.diff(be) >= 0)                              # non-decreasing experts
    for b, e in enumerate(be):                                   # each block holds one expert
        rows = s[b * bm:(b + 1) * bm]
        assert np.all((rows == P) | (ids.reshape(-1)[np.minimum(rows, P - 1)] == e))
    # items cover exactly the LoRA pairs, each at most lbm rows, one (a, e) each
    covered = []
    for st_, ln, a, e in o["items"][:o["num_items"]]:
        assert 1 <= ln <= lbm
        for p in range(st_, st_ + ln):
            f = s[p]
            assert f < P and ids.reshape(-1)[f] == e and ad[f // (K + S)] == a
            covered.append(f)
    lora_pairs = [f for f in range(P) if ad[f // (K + S)] >= 0]
    assert sorted(covered) == lora_pairs


def test_align_empty_and_degenerate():
    # T = 0: nothing but sentinels
    o = oracle.align(np.zeros((0, 3), np.int32), np.zeros(0, np.int32), 5, 2, 4, 4)
    assert o["num_post_pad"] == 0 and o["num_items"] == 0
    # all pairs on one expert, no LoRA
    ids = np.zeros((10, 1), np.int32)
    o = oracle.align(ids, None, 3, 0, 4, 4)
    assert o["num_post_pad"] == 12
    assert o["sorted_ids"][:12].tolist() == list(range(10)) + [10, 10]
    assert o["block_expert"][:3].tolist() == [0, 0, 0]
    # all adapters -1: no items
    ids = _random_ids(np.random.default_rng(0), 6, 2, 4, 0)
    o = oracle.align(ids, np.full(6, -1, np.int32), 4, 3, 4, 4)
    assert o["num_items"] == 0


@settings(max_examples=80, deadline=None)
@given(T=st.integers(0, 12), data=st.data())
def test_align_hypothesis(T, data):
    E = data.draw(st.integers(1, 7))
    K = data.draw(st.integers(1, E))
    S = data.draw(st.integers(0, 2))
    L = data.draw(st.integers(0, 3))
    bm = data.draw(st.sampled_from([1, 2, 4, 16]))
    lbm = data.draw(st.sampled_from([1, 2, 4, 16]))
    seed = data.draw(st.integers(0, 10**6))
    rng = np.random.default_rng(seed)
    ids = _random_ids(rng, T, K, E, S)
    ad = rng.integers(-1, L, T).astype(np.int32) if L > 0 else None
    _check_vs_bruteforce(ids, ad, E + S, L, bm, lbm)
