"""Pins of the oracle's scoring CNN (no GPU).

The library pin re-computes the same two-layer network with torch's Conv1d
(cross-correlation, zero padding 1), exact GELU and sigmoid on the CPU in
float64.  The hand pins check tap orientation, channel order, and that zero
weights give z = b2 exactly.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import cnn_logits, cnn_scores


def _torch_logits(k, v, W1, b1, W2, b2):
    k = torch.as_tensor(np.asarray(k), dtype=torch.float64)
    v = torch.as_tensor(np.asarray(v), dtype=torch.float64)
    B, T, Hkv, D = k.shape
    out = torch.zeros((B, Hkv, T), dtype=torch.float64)
    for g in range(Hkv):
        x = torch.cat([k[:, :, g, :], v[:, :, g, :]], dim=2).transpose(1, 2)   # [B, 2D, T]
        h = F.conv1d(x, torch.as_tensor(W1[g], dtype=torch.float64),
                     torch.as_tensor(b1[g], dtype=torch.float64), padding=1)
        a = F.gelu(h, approximate="none")
        z = F.conv1d(a, torch.as_tensor(W2[g][None], dtype=torch.float64),
                     torch.as_tensor(b2[g:g + 1], dtype=torch.float64), padding=1)
        out[:, g, :] = z[:, 0, :]
    return out.numpy()


@pytest.mark.parametrize("seed", range(6))
def test_cnn_matches_torch_conv1d(seed):
    rng = np.random.default_rng(seed)
    B, T, Hkv, D, hidden = 2, int(rng.integers(1, 40)), 3, 8, 32
    k = rng.standard_normal((B, T, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((B, T, Hkv, D)).astype(np.float32)
    W1 = (rng.standard_normal((Hkv, hidden, 2 * D, 3)) * 0.3).astype(np.float32)
    b1 = rng.standard_normal((Hkv, hidden)).astype(np.float32)
    W2 = (rng.standard_normal((Hkv, hidden, 3)) * 0.3).astype(np.float32)
    b2 = rng.standard_normal((Hkv,)).astype(np.float32)
    ours = cnn_logits(k, v, W1, b1, W2, b2)
    ref = _torch_logits(k, v, W1, b1, W2, b2)
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-12)
    r = cnn_scores(k, v, W1, b1, W2, b2)
    assert r.dtype == np.float32
    np.testing.assert_allclose(r, 1 / (1 + np.exp(-ref)), rtol=1e-6, atol=1e-7)


def _gelu(x):
    return 0.5 * x * (1 + math.erf(x / math.sqrt(2)))


def test_tap_zero_reads_the_previous_token():
    # hidden 0 = key channel 0 of token t-1; z = hidden 0 of token t-1
    # => z[t] = gelu(k0[t-2]), with zero padding at the sequence start.
    T, D, hidden = 9, 4, 32
    k = np.zeros((1, T, 1, D), np.float32)
    v = np.zeros((1, T, 1, D), np.float32)
    k[0, :, 0, 0] = np.arange(1, T + 1, dtype=np.float32) / 4
    W1 = np.zeros((1, hidden, 2 * D, 3), np.float32)
    W1[0, 0, 0, 0] = 1.0
    W2 = np.zeros((1, hidden, 3), np.float32)
    W2[0, 0, 0] = 1.0
    z = cnn_logits(k, v, W1, np.zeros((1, hidden), np.float32), W2, np.zeros(1, np.float32))
    want = [0.0, 0.0] + [_gelu(float(k[0, t - 2, 0, 0])) for t in range(2, T)]
    np.testing.assert_allclose(z[0, 0], want, rtol=0, atol=1e-15)


def test_tap_two_reads_the_next_token_and_value_channels_follow_keys():
    T, D, hidden = 7, 3, 32
    k = np.zeros((1, T, 1, D), np.float32)
    v = np.zeros((1, T, 1, D), np.float32)
    v[0, :, 0, 1] = np.linspace(-1, 1, T).astype(np.float32)
    W1 = np.zeros((1, hidden, 2 * D, 3), np.float32)
    W1[0, 5, D + 1, 2] = 1.0        # hidden 5 = value channel 1 of token t+1
    W2 = np.zeros((1, hidden, 3), np.float32)
    W2[0, 5, 1] = 2.0               # centre tap
    z = cnn_logits(k, v, W1, np.zeros((1, hidden), np.float32), W2, np.zeros(1, np.float32))
    want = [2 * _gelu(float(v[0, t + 1, 0, 1])) for t in range(T - 1)] + [0.0]
    np.testing.assert_allclose(z[0, 0], want, rtol=0, atol=1e-15)


def test_zero_weights_give_the_bias():
    T, D, hidden = 5, 4, 32
    rng = np.random.default_rng(0)
    k = rng.standard_normal((2, T, 2, D)).astype(np.float32)
    z = cnn_logits(k, k, np.zeros((2, hidden, 2 * D, 3), np.float32),
                   np.zeros((2, hidden), np.float32), np.zeros((2, hidden, 3), np.float32),
                   np.array([0.25, -3.0], np.float32))
    assert np.all(z[:, 0] == 0.25) and np.all(z[:, 1] == -3.0)
    r = cnn_scores(k, k, np.zeros((2, hidden, 2 * D, 3), np.float32),
                   np.zeros((2, hidden), np.float32), np.zeros((2, hidden, 3), np.float32),
                   np.zeros(2, np.float32))
    assert np.all(r == np.float32(0.5))


def test_sigmoid_matches_library():
    """Library pin of the score's last step: r = sigmoid(z) stored as fp32 equals torch's
    float64 sigmoid rounded to fp32 (within one fp32 ulp where float64 rounding orders
    differ), and scipy's expit; the orientation is fixed by sigmoid(2) > 1/2 > sigmoid(-2)."""
    from scipy.special import expit

    from oracle import sigmoid_to_f32
    z = np.concatenate([np.linspace(-30.0, 30.0, 6001), [0.0, -0.0, 1e-8, -1e-8, 0.4, -0.4]])
    ours = sigmoid_to_f32(z)
    assert ours.dtype == np.float32
    ref = torch.sigmoid(torch.as_tensor(z, dtype=torch.float64)).to(torch.float32).numpy()
    ulps = np.abs(ours.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1
    assert (ulps == 0).mean() > 0.999
    np.testing.assert_allclose(ours, expit(z), rtol=1e-7, atol=0)
    assert np.all(np.diff(ours[:6001]) >= 0)                 # increasing in z
    two = sigmoid_to_f32(np.array([2.0, 0.0, -2.0]))
    assert two[0] > 0.5 and two[1] == np.float32(0.5) and two[2] < 0.5
    np.testing.assert_allclose(two[0], 0.8807970779778823, rtol=1e-7)
    # the fp32 evaluation (oracle dtype float32) against torch's fp32 sigmoid
    z32 = np.linspace(-20.0, 20.0, 4001).astype(np.float32)
    ours32 = sigmoid_to_f32(z32)
    ref32 = torch.sigmoid(torch.as_tensor(z32)).numpy()
    ulps32 = np.abs(ours32.view(np.int32).astype(np.int64) - ref32.view(np.int32).astype(np.int64))
    assert ulps32.max() <= 4
