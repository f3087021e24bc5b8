"""Pins of the linear-attention oracle (CPU): closed forms of the recurrence
S_t = a_t S_{t-1} + v_t k_t^T, o_t = S_t q_t ("Sparse Linear Attention: Viewing
SWA from the Perspective of Linear Attention", section "Background: Linear
attention"; A_t = a_t I), a hand-computed scalar case, the literal matrix form
S_{t-1} A_t, state resets and continuation from a saved state."""
import numpy as np
import pytest

import oracle


def _rand(seed, B=2, T=23, H=3, D=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, D))
    k = rng.standard_normal((B, T, H, D))
    v = rng.standard_normal((B, T, H, D))
    log_a = np.log(rng.uniform(0.3, 1.0, (B, T, H)))
    return q, k, v, log_a


def test_hand_computed_scalar_case():
    # D = 1: S_t = a_t S_{t-1} + v_t k_t, o_t = S_t q_t
    # S_1 = 1, o_1 = 1; S_2 = 0.5 + 2 = 2.5, o_2 = 2.5; S_3 = 1.25 + 2 = 3.25, o_3 = 6.5
    q = np.array([1.0, 1.0, 2.0]).reshape(1, 3, 1, 1)
    k = np.array([1.0, 2.0, 1.0]).reshape(1, 3, 1, 1)
    v = np.array([1.0, 1.0, 2.0]).reshape(1, 3, 1, 1)
    log_a = np.log(np.array([1.0, 0.5, 0.5])).reshape(1, 3, 1)
    o, S = oracle.linear_recurrent(q, k, v, log_a)
    assert np.allclose(o.ravel(), [1.0, 2.5, 6.5])
    assert np.isclose(S.item(), 3.25)


def test_no_decay_is_causal_linear_attention():
    q, k, v, _ = _rand(1)
    o, _ = oracle.linear_recurrent(q, k, v, np.zeros(q.shape[:3]))
    T = q.shape[1]
    mask = np.tril(np.ones((T, T)))
    for b in range(q.shape[0]):
        for h in range(q.shape[2]):
            ref = (q[b, :, h] @ k[b, :, h].T * mask) @ v[b, :, h]
            assert np.allclose(o[b, :, h], ref)


@pytest.mark.parametrize("a", [0.9, 0.5])
def test_constant_decay_closed_form(a):
    q, k, v, _ = _rand(2)
    T = q.shape[1]
    o, _ = oracle.linear_recurrent(q, k, v, np.full(q.shape[:3], np.log(a)))
    t = np.arange(T)
    M = np.where(t[:, None] >= t[None, :], a ** (t[:, None] - t[None, :]).astype(float), 0.0)
    for b in range(q.shape[0]):
        for h in range(q.shape[2]):
            ref = (q[b, :, h] @ k[b, :, h].T * M) @ v[b, :, h]
            assert np.allclose(o[b, :, h], ref)


def test_varying_decay_unrolled_sum_and_state():
    # o_t = sum_{j<=t} (prod_{l=j+1..t} a_l) (q_t . k_j) v_j ;
    # S_T = sum_j (prod_{l=j+1..T-1} a_l) v_j k_j^T
    q, k, v, log_a = _rand(3, B=1, T=9, H=2, D=4)
    a = np.exp(log_a)
    o, S = oracle.linear_recurrent(q, k, v, log_a)
    T = q.shape[1]
    for h in range(q.shape[2]):
        for t in range(T):
            acc = np.zeros(4)
            for j in range(t + 1):
                acc += np.prod(a[0, j + 1:t + 1, h]) * (q[0, t, h] @ k[0, j, h]) * v[0, j, h]
            assert np.allclose(o[0, t, h], acc)
        ref = sum(np.prod(a[0, j + 1:, h]) * np.outer(v[0, j, h], k[0, j, h]) for j in range(T))
        assert np.allclose(S[0, h], ref)


def test_literal_matrix_form():
    # S_{t-1} A_t with A_t = a_t I as a full matrix product, one step at a time
    q, k, v, log_a = _rand(4, B=1, T=7, H=1, D=3)
    o, S_end = oracle.linear_recurrent(q, k, v, log_a)
    S = np.zeros((3, 3))
    for t in range(7):
        S, ot = oracle.linear_step(S, np.exp(log_a[0, t, 0]), q[0, t, 0], k[0, t, 0], v[0, t, 0])
        assert np.allclose(ot, o[0, t, 0])
    assert np.allclose(S, S_end[0, 0])


def test_zero_decay_resets_the_state():
    q, k, v, log_a = _rand(5)
    t0 = 11
    log_a[:, t0] = -np.inf                      # a = 0: the state before t0 is dropped
    o, S = oracle.linear_recurrent(q, k, v, log_a)
    o2, S2 = oracle.linear_recurrent(q[:, t0:], k[:, t0:], v[:, t0:], log_a[:, t0:])
    assert np.allclose(o[:, t0:], o2) and np.allclose(S, S2)
    # and at the reset step itself o = (q . k) v
    assert np.allclose(o[:, t0], np.einsum("bhd,bhd->bh", q[:, t0], k[:, t0])[..., None]
                       * v[:, t0])


def test_continuation_from_saved_state():
    q, k, v, log_a = _rand(6, T=30)
    o, S = oracle.linear_recurrent(q, k, v, log_a)
    T1 = 13
    o1, S1 = oracle.linear_recurrent(q[:, :T1], k[:, :T1], v[:, :T1], log_a[:, :T1])
    o2, S2 = oracle.linear_recurrent(q[:, T1:], k[:, T1:], v[:, T1:], log_a[:, T1:], state=S1)
    assert np.allclose(np.concatenate([o1, o2], axis=1), o) and np.allclose(S2, S)
