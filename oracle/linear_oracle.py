"""Plain CPU oracle of the linear-attention layer of the hybrid -- TEST INFRASTRUCTURE.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares no code with the HIP path and imports nothing from it.

Source: "Sparse Linear Attention: Viewing SWA from the Perspective of Linear
Attention", section "Background: Linear attention": a fixed-size state matrix S_t
is decayed by A_t, written with the outer product of the current value and key,
and read with the query:  S_t = S_{t-1} A_t + v_t k_t^T,  o_t = S_t q_t.
The LTE summary page (TL;DR, Abstract) interleaves such layers with the LTE layer
("laLTE").

Readings where the pages are silent (each restated where used):

L1  A_t = a_t I: one decay factor a_t in [0, 1] per head and step, given as an
    input (as log a_t).  a_t = 1 everywhere is naive linear attention, which the
    page names as the case without decay.
L2  S_t is D_v x D_k, v_t k_t^T its write, o_t = S_t q_t its read; no scaling,
    feature map or normalisation of q and k (those belong to the model).
L3  Heads are independent; q, k, v have the same head count and head size D.
L4  S_0 is zero unless an initial state is given (a prefix already processed).
"""
from __future__ import annotations

import numpy as np

__all__ = ["linear_recurrent", "linear_step"]


def linear_step(S, a, q, k, v):
    """One step of the recurrence for a single head (L1, L2):
    S <- S A + v k^T with A = a I, then o = S q.  S [Dv, Dk] float64, a scalar,
    q, k [Dk], v [Dv].  Returns (S, o)."""
    S = S @ (a * np.eye(S.shape[1])) + np.outer(v, k)
    return S, S @ q


def linear_recurrent(q, k, v, log_a, state=None, dtype=np.float64):
    """The layer over a whole sequence, step by step, for every (batch, head).

    q, k [B, T, H, D]; v [B, T, H, D]; log_a [B, T, H] (a_t = exp(log_a));
    state [B, H, Dv, Dk] or None (L4).  Returns (o [B, T, H, D], S_T [B, H, Dv, Dk]).
    """
    q = np.asarray(q, dtype)
    k = np.asarray(k, dtype)
    v = np.asarray(v, dtype)
    a = np.exp(np.asarray(log_a, dtype))
    B, T, H, D = q.shape
    Dv = v.shape[-1]
    S = np.zeros((B, H, Dv, D), dtype) if state is None else np.array(state, dtype)
    o = np.zeros((B, T, H, Dv), dtype)
    for t in range(T):
        # S_t = S_{t-1} a_t + v_t k_t^T ; o_t = S_t q_t   (batched over b, h)
        S = S * a[:, t, :, None, None] + v[:, t, :, :, None] * k[:, t, :, None, :]
        o[:, t] = np.einsum("bhvk,bhk->bhv", S, q[:, t])
    return o, S
