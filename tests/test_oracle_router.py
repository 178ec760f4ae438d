"""Pins for the oracle's router (the gate's top-k in front of the expert path).

Reading: the k largest logits in descending order, ties to the lower expert id; probabilities =
softmax over the k selected logits (= the softmax over all E experts renormalised over the k).  The
gate step is part of the step breakdown on the page 'MC2 通算融合'; the router top-k distribution is
one of the checks listed on the page 'NPU Training Operators - MC2', section 验证项.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "router_worked_example.json")


def _f(v):
    return np.array([[float(x) for x in row] for row in v], np.float32)


def test_worked_examples():
    for case in json.load(open(GOLDEN))["cases"]:
        ids, probs = oracle.router(_f(case["logits"]), case["k"])
        assert ids.tolist() == case["ids"]
        np.testing.assert_allclose(probs, np.array(case["probs"]), rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("T,E,k,seed", [(200, 8, 2, 0), (100, 128, 8, 1), (50, 32, 4, 2), (30, 5, 5, 3),
                                        (40, 100, 1, 4)])
def test_selection_matches_a_stable_sort(T, E, k, seed):
    """The selection scan against numpy's stable sort of the negated logits (another algorithm)."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    # force ties: round half the rows to a coarse grid
    logits[::2] = np.round(logits[::2] * 2) / 2
    ids, _ = oracle.router(logits, k)
    ref = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    assert np.array_equal(ids, ref)


@pytest.mark.parametrize("E,k", [(8, 2), (128, 8), (16, 16)])
def test_probs_are_the_renormalised_full_softmax(E, k):
    """scipy's softmax over all E experts, restricted to the selected ones and renormalised."""
    rng = np.random.default_rng(E + k)
    logits = (3 * rng.standard_normal((64, E))).astype(np.float32)
    ids, probs = oracle.router(logits, k)
    full = softmax(logits.astype(np.float64), axis=1)
    sel = np.take_along_axis(full, ids, axis=1)
    np.testing.assert_allclose(probs, sel / sel.sum(axis=1, keepdims=True), rtol=1e-12)
    np.testing.assert_allclose(probs.sum(axis=1), 1.0, rtol=1e-14)
    assert np.all(np.diff(probs, axis=1) <= 0)          # descending logits, descending shares
    if k == E:
        np.testing.assert_allclose(np.take_along_axis(probs, np.argsort(ids, axis=1), axis=1), full,
                                   rtol=1e-12)


def test_shift_invariance_and_minus_infinity():
    rng = np.random.default_rng(9)
    # logits on a grid of 1/64 below 8 in magnitude, so adding 8 is exact in float32
    logits = (np.round(rng.standard_normal((32, 16)) * 64) / 64).clip(-7.9, 7.9).astype(np.float32)
    ids, probs = oracle.router(logits, 4)
    ids2, probs2 = oracle.router(logits + np.float32(8.0), 4)
    assert np.array_equal(ids, ids2)
    np.testing.assert_allclose(probs, probs2, rtol=1e-12)
    # experts with -inf logits are never picked while finite ones remain, and then get 0
    logits[:, :12] = -np.inf
    ids, probs = oracle.router(logits, 6)
    assert np.all(ids[:, :4] >= 12) and np.all(ids[:, 4:] == np.array([0, 1]))
    assert np.all(probs[:, 4:] == 0.0)


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.router(np.zeros((2, 4), np.float32), 5)
