"""Pins of the oracle's A-plus-column attention (no GPU).

* brute force: dense float64 masked softmax with the closed-form mask;
* library special cases via torch's scaled_dot_product_attention (float64, CPU):
  every token kept with C >= T is full causal attention, retention 0 is
  sink + sliding window, w >= T is full causal;
* closed forms: o_0 = v_0; q = 0 gives the mean of the visible values, which
  with v_j = 2^j spells out the visible set (checked against the hand trace);
  outputs lie in the convex hull of the visible values.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import all_ends, attention, prefill, visible_indices
from tests.bruteforce import dense_attention, dense_mask


def _rand_qkv(rng, B, T, Hq, Hkv, D):
    q = rng.standard_normal((B, T, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, T, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((B, T, Hkv, D)).astype(np.float32)
    return q, k, v


@pytest.mark.parametrize("seed", range(12))
def test_matches_dense_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 96))
    s = int(rng.integers(0, 5))
    w = int(rng.integers(5, 17))
    C = int(rng.integers(0, 9))
    G = [1, 2, 4][seed % 3]
    Hkv, D, B = 2, 8, 1
    q, k, v = _rand_qkv(rng, B, T, Hkv * G, Hkv, D)
    scores = rng.choice([0.3, 0.55, 0.7, 0.9, rng.uniform(0.4, 1)], size=(B, Hkv, T)).astype(np.float32)
    got = prefill(q, k, v, s, w, C, scores=scores)["o"]
    masks = np.stack([np.stack([dense_mask(scores[b, g], s, w, C, T) for g in range(Hkv)])
                      for b in range(B)])
    want = dense_attention(q, k, v, masks)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def _sdpa(q, k, v, mask=None, causal=False):
    qt = torch.as_tensor(q, dtype=torch.float64).transpose(1, 2)   # [B, H, T, D]
    kt = torch.as_tensor(k, dtype=torch.float64).transpose(1, 2)
    vt = torch.as_tensor(v, dtype=torch.float64).transpose(1, 2)
    G = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(G, dim=1)
    vt = vt.repeat_interleave(G, dim=1)
    m = None if mask is None else torch.as_tensor(mask)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=causal)
    return o.transpose(1, 2).numpy()


def test_everything_kept_is_full_causal():
    rng = np.random.default_rng(1)
    B, T, Hq, Hkv, D = 2, 40, 4, 2, 16
    q, k, v = _rand_qkv(rng, B, T, Hq, Hkv, D)
    scores = rng.uniform(0.6, 1.0, (B, Hkv, T)).astype(np.float32)
    got = prefill(q, k, v, 2, 6, T, scores=scores)["o"]
    np.testing.assert_allclose(got, _sdpa(q, k, v, causal=True), rtol=1e-10, atol=1e-12)


def test_nothing_kept_is_sink_plus_window():
    rng = np.random.default_rng(2)
    B, T, Hq, Hkv, D, s, w = 1, 50, 4, 4, 16, 3, 7
    q, k, v = _rand_qkv(rng, B, T, Hq, Hkv, D)
    scores = rng.uniform(0.0, 0.5, (B, Hkv, T)).astype(np.float32)
    got = prefill(q, k, v, s, w, 8, scores=scores)["o"]
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    mask = (j <= i) & ((j < s) | (j > i - w))
    np.testing.assert_allclose(got, _sdpa(q, k, v, mask=mask), rtol=1e-10, atol=1e-12)


def test_window_covering_everything_is_full_causal():
    rng = np.random.default_rng(3)
    B, T, Hq, Hkv, D = 1, 33, 2, 1, 8
    q, k, v = _rand_qkv(rng, B, T, Hq, Hkv, D)
    scores = rng.uniform(0, 1, (B, Hkv, T)).astype(np.float32)
    got = prefill(q, k, v, 1, T, 4, scores=scores)["o"]
    np.testing.assert_allclose(got, _sdpa(q, k, v, causal=True), rtol=1e-10, atol=1e-12)


def test_first_row_is_v0_and_outputs_are_convex():
    rng = np.random.default_rng(4)
    B, T, Hq, Hkv, D, s, w, C = 1, 64, 4, 2, 8, 2, 9, 5
    q, k, v = _rand_qkv(rng, B, T, Hq, Hkv, D)
    scores = rng.uniform(0.3, 1, (B, Hkv, T)).astype(np.float32)
    res = prefill(q, k, v, s, w, C, scores=scores)
    o, ends = res["o"], res["ends"]
    G = Hq // Hkv
    for h in range(Hq):
        np.testing.assert_allclose(o[0, 0, h], v[0, 0, h // G], rtol=0, atol=1e-12)
    for i in range(T):
        for g in range(Hkv):
            idx = visible_indices(i, s, w, ends[0, g])
            lo = v[0, idx, g].min(axis=0)
            hi = v[0, idx, g].max(axis=0)
            for h in range(g * G, (g + 1) * G):
                assert np.all(o[0, i, h] >= lo - 1e-12) and np.all(o[0, i, h] <= hi + 1e-12)


def test_zero_queries_spell_out_the_visible_set():
    path = os.path.join(os.path.dirname(__file__), "golden", "retention_hand.json")
    with open(path) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        T, s, w, C = case["T"], case["s"], case["w"], case["C"]
        q = np.zeros((1, T, 2, 1), np.float32)             # 2 query heads, 1 KV head
        k = np.ones((1, T, 1, 1), np.float32)
        v = (2.0 ** np.arange(T)).astype(np.float32).reshape(1, T, 1, 1)
        scores = np.array(case["scores"], np.float32).reshape(1, 1, T)
        ends = all_ends(scores, s, w, C, T)
        o = attention(q, k, v, s, w, ends)
        for i in range(T):
            n = len(case["visible"][i])
            bits = int(round(o[0, i, 0, 0] * n))
            assert bits == sum(1 << j for j in case["visible"][i]), i
            assert o[0, i, 1, 0] == o[0, i, 0, 0]


@pytest.mark.parametrize("seed", range(6))
def test_attention_on_a_given_set(seed):
    """attention_on_set (the oracle's softmax over sink U window U a given retained set)
    equals the dense float64 brute force with that mask, for arbitrary sets, and equals
    ``attention`` when the set is the oracle's own R_i."""
    from oracle import attention_on_set, retained_set
    rng = np.random.default_rng(500 + seed)
    T, s, w, C = int(rng.integers(20, 80)), int(rng.integers(0, 4)), int(rng.integers(5, 12)), 6
    G = [1, 2, 4][seed % 3]
    Hkv, D, B = 2, 8, 2
    q, k, v = _rand_qkv(rng, B, T, Hkv * G, Hkv, D)
    scores = rng.uniform(0.3, 1.0, size=(B, Hkv, T)).astype(np.float32)
    full = prefill(q, k, v, s, w, C, scores=scores)
    for b in range(B):
        for g in range(Hkv):
            for i in rng.integers(0, T, 6).tolist():
                R = retained_set(full["ends"][b, g], w, i)
                np.testing.assert_array_equal(
                    attention_on_set(q, k, v, s, w, b, i, g, R),
                    full["o"][b, i, g * G:(g + 1) * G])
                # an arbitrary set of earlier tokens, outside any keep rule
                Rx = sorted(set(rng.integers(0, i + 1, 5).tolist()))
                mask = np.zeros((T, T), bool)
                mask[i, :min(s, i + 1)] = True
                mask[i, max(0, i - w + 1):i + 1] = True
                mask[i, Rx] = True
                others = np.arange(T) != i                   # other rows: any valid mask
                mask[others, others] = True
                masks = np.broadcast_to(np.eye(T, dtype=bool), (B, Hkv, T, T)).copy()
                masks[b, g] = mask
                want = dense_attention(q, k, v, masks)[b, i, g * G:(g + 1) * G]
                np.testing.assert_allclose(attention_on_set(q, k, v, s, w, b, i, g, Rx), want,
                                           rtol=1e-10, atol=1e-12)
