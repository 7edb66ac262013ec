"""Pins for the oracle's router front end (CPU only): hand-worked cases, brute force on tiny
inputs, closed forms and invariants."""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import router as RT

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "router_worked.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    logits = np.array(case["logits"], dtype=np.float32)
    ids, w = RT.route(logits, case["k"], case["scoring"], case["renormalize"])
    assert ids.tolist() == case["ids"]
    np.testing.assert_allclose(w, np.array(case["weights"]), rtol=2e-7, atol=1e-9)


def _brute_topk(row, k):
    """The k-subset maximising the sum of logits, the tie rule as a lexicographic choice:
    among maximal subsets the one whose sorted (value desc, id asc) list is smallest."""
    e = len(row)
    best = None
    for sub in itertools.combinations(range(e), k):
        key = sorted(((-float(row[i]), i) for i in sub))
        score = -sum(float(row[i]) for i in sub)
        cand = (score, key)
        if best is None or cand < best:
            best = cand
    return [i for _, i in best[1]]


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    e = int(rng.integers(1, 7))
    k = int(rng.integers(1, e + 1))
    # few distinct values, so ties are common
    logits = rng.integers(-2, 3, size=(3, e)).astype(np.float32) * np.float32(0.5)
    ids, _ = RT.route(logits, k, "softmax")
    for r in range(3):
        assert ids[r].tolist() == _brute_topk(logits[r], k)


@pytest.mark.parametrize("scoring", RT.SCORINGS)
def test_invariants_random(scoring):
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((200, 128)).astype(np.float32)
    ids, w = RT.route(logits, 8, scoring, True)
    assert ids.dtype == np.int32 and ids.shape == (200, 8)
    for r in range(200):
        assert len(set(ids[r].tolist())) == 8                              # distinct experts
        sel = logits[r, ids[r]]
        rest = np.delete(logits[r], ids[r])
        assert sel.min() >= rest.max()                                      # the largest logits
        assert np.all(np.diff(sel) <= 0)                                    # largest first
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-12)              # renormalised
    assert np.all(w > 0) and np.all(np.diff(w, axis=1) <= 1e-15)            # positive, non-increasing


def test_softmax_closed_form_against_full_softmax():
    """Renormalised top-k softmax equals the full softmax restricted to the k experts and
    divided by their share: the full denominator cancels."""
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((50, 64)).astype(np.float32)
    ids, w = RT.route(logits, 6, "softmax", True)
    l = logits.astype(np.float64)
    full = np.exp(l) / np.exp(l).sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-12)
    _, wr = RT.route(logits, 6, "softmax", False)
    np.testing.assert_allclose(wr, sel, rtol=1e-12)


def test_sigmoid_closed_form():
    x = np.array([[math.log(9.0), 0.0, -math.log(4.0)]], dtype=np.float32)   # sigmoid 0.9, 0.5, 0.2
    ids, w = RT.route(x, 3, "sigmoid", False)
    assert ids.tolist() == [[0, 1, 2]]
    np.testing.assert_allclose(w, [[0.9, 0.5, 0.2]], rtol=1e-7)


def test_same_selection_for_both_scorings():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((100, 32)).astype(np.float32)
    assert np.array_equal(RT.route(logits, 5, "softmax")[0], RT.route(logits, 5, "sigmoid")[0])


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        RT.route(np.zeros((1, 4), np.float32), 5)
    with pytest.raises(ValueError):
        RT.route(np.zeros((1, 4), np.float32), 2, "relu")
    with pytest.raises(ValueError):
        RT.route(np.array([[0.0, np.inf]], np.float32), 1)
