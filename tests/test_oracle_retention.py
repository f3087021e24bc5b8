"""Pins of the oracle's keep/evict stream (no GPU)."""
import json
import os

import numpy as np
import pytest

from oracle import retained_set, retention_ends, visible_indices
from tests.bruteforce import closed_form_retained

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "retention_hand.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_trace(case):
    r = np.array(case["scores"], np.float32)
    T, s, w, C = case["T"], case["s"], case["w"], case["C"]
    end = retention_ends(r, s, w, C, T)
    assert end.tolist() == case["ends"]
    for i in range(T):
        assert retained_set(end, w, i).tolist() == case["retained"][i], i
        assert visible_indices(i, s, w, end).tolist() == case["visible"][i], i


def _rand_scores(rng, T, levels):
    if levels:   # coarse values force exact ties
        return rng.choice(np.linspace(0.3, 0.9, levels), size=T).astype(np.float32)
    return rng.uniform(0.2, 1.0, size=T).astype(np.float32)


@pytest.mark.parametrize("seed", range(40))
def test_stream_equals_closed_form(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 70))
    s = int(rng.integers(0, 5))
    w = int(rng.integers(1, 12))
    C = int(rng.integers(0, 9))
    r = _rand_scores(rng, T, levels=[0, 3, 5][seed % 3])
    end = retention_ends(r, s, w, C, T)
    for i in range(T):
        got = retained_set(end, w, i).tolist()
        assert got == closed_form_retained(r, s, w, C, i), (i, got)
        assert len(got) <= C
        assert len(visible_indices(i, s, w, end)) <= s + w + C


def test_evicted_never_returns():
    rng = np.random.default_rng(7)
    r = rng.uniform(0.4, 1.0, 300).astype(np.float32)
    s, w, C, T = 2, 10, 8, 300
    end = retention_ends(r, s, w, C, T)
    member = np.zeros((T, T), bool)
    for i in range(T):
        member[i, retained_set(end, w, i)] = True
    for j in range(T):
        steps = np.nonzero(member[:, j])[0]
        if len(steps):   # one contiguous interval starting when j leaves the window
            assert steps[0] == j + w
            assert np.all(np.diff(steps) == 1)


def test_exact_half_is_not_kept():
    r = np.full(50, 0.5, np.float32)
    end = retention_ends(r, 1, 4, 10, 50)
    assert np.all(end == -1)
    r2 = np.full(50, np.nextafter(np.float32(0.5), np.float32(1)), np.float32)
    assert np.all(retention_ends(r2, 1, 4, 10, 50)[1:46] >= 0)


def test_all_equal_scores_keep_earliest():
    # equal scores: lower index wins, so the first C eligible tokens stay forever
    T, s, w, C = 60, 2, 5, 7
    r = np.full(T, 0.75, np.float32)
    end = retention_ends(r, s, w, C, T)
    assert retained_set(end, w, T - 1).tolist() == list(range(s, s + C))
