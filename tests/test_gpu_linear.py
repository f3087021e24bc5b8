"""Linear-attention layer parity (needs an MI355X): the chunked MFMA prefill and the
decode step against the oracle's step-by-step recurrence in float64.

Tolerance, from the arithmetic.  bf16 keeps 8 significant bits: unit roundoff
u = 2^-8, a rounding error uniform in +-u of the value, standard deviation u/sqrt(3).
The kernel rounds to bf16 the decayed scores P, the weighted keys w K and, for the
inter-chunk product, the carried state; each output or state element is a sum of
many such terms with independent errors, so its error has a standard deviation of
about u/sqrt(3) = 0.23% of the element's typical size (rms), and the maximum over
~10^5 elements stays below 5 sigma, 1.1%.  The output's own bf16 rounding adds up
to u |o| with |o| up to about 4 rms.  Bounds, with about 2x margin:
  outputs  max |o - ref| <= 4e-2 rms(ref),  mean <= 4e-3 rms(ref);
  state    max |S - ref| <= 2.5e-2 rms(S_ref).
"""
import numpy as np
import pytest
import torch

import oracle
from learnable_kv_cache_amd import lte, synth

pytestmark = pytest.mark.gpu


def _check(o, ref, what):
    o = np.asarray(o, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    d = np.abs(o - ref)
    assert d.max() <= 4e-2 * rms and d.mean() <= 4e-3 * rms, (what, d.max(), d.mean(), rms)


def _check_state(S, ref, what):
    S = np.asarray(S, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    assert np.abs(S - ref).max() <= 2.5e-2 * rms, (what, np.abs(S - ref).max(), rms)


def _run(B, T, H, D, seed, state_in=False, resets=(), gate_mean=4.0):
    q, k, v, log_a = synth.linear_inputs(seed, B, T, H, D, gate_mean)
    for t in resets:
        log_a[:, t] = -float("inf")
    S0 = None
    if state_in:
        g = torch.Generator().manual_seed(seed + 1)
        S0 = torch.randn((B, H, D, D), generator=g) * 0.3
    layer = lte.LinearLayer(B, H, D)
    dev = torch.device("cuda")
    o, S = layer.prefill(q.to(dev), k.to(dev), v.to(dev), log_a.to(dev),
                         state_in=S0.to(dev) if S0 is not None else None)
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.linear_recurrent(q.float().numpy(), k.float().numpy(),
                                           v.float().numpy(), log_a.numpy(),
                                           state=None if S0 is None else S0.numpy())
    return o.float().cpu().numpy(), S.cpu().numpy(), ref_o, ref_S


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 64, 65, 200])
def test_linear_prefill(T, D):
    """Whole chunks, a one-row chunk and a ragged last chunk (200 = 3 x 64 + 8)."""
    o, S, ref_o, ref_S = _run(2, T, 3, D, seed=100 + T + D)
    _check(o, ref_o, "out")
    _check_state(S, ref_S, "state")


@pytest.mark.parametrize("seed", range(6))
def test_linear_random_shapes(seed):
    """Seeded random batch, length, head count and size, decay strength, an initial
    state or not, and a reset or not."""
    rng = np.random.default_rng(3000 + seed)
    B = int(rng.integers(1, 4))
    T = int(rng.integers(1, 400))
    H = int(rng.integers(1, 5))
    D = int(rng.choice([64, 128]))
    gate = float(rng.choice([1.0, 4.0, 8.0]))
    resets = (int(rng.integers(0, T)),) if rng.random() < 0.5 else ()
    o, S, ref_o, ref_S = _run(B, T, H, D, seed=4000 + seed, state_in=bool(rng.random() < 0.5),
                              resets=resets, gate_mean=gate)
    _check(o, ref_o, "out")
    _check_state(S, ref_S, "state")


def test_linear_prefill_state_in_and_resets():
    """A nonzero initial state, and resets (a = 0) inside a chunk and on a chunk edge."""
    o, S, ref_o, ref_S = _run(2, 300, 4, 128, seed=7, state_in=True, resets=(37, 128, 131))
    _check(o, ref_o, "out")
    _check_state(S, ref_S, "state")


def test_linear_no_decay():
    """a = 1 everywhere (naive linear attention: the state only accumulates)."""
    B, T, H, D = 1, 256, 2, 64
    q, k, v, _ = synth.linear_inputs(8, B, T, H, D)
    log_a = torch.zeros((B, T, H), dtype=torch.float32)
    layer = lte.LinearLayer(B, H, D)
    o, S = layer.prefill(q.cuda(), k.cuda(), v.cuda(), log_a.cuda())
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.linear_recurrent(q.float().numpy(), k.float().numpy(),
                                           v.float().numpy(), log_a.numpy())
    _check(o.float().cpu().numpy(), ref_o, "out")
    _check_state(S.cpu().numpy(), ref_S, "state")


@pytest.mark.parametrize("D", [64, 128])
def test_linear_decode_continues_prefill(D):
    """Prefill 150 tokens, then 40 decode steps on the same state buffer (in place),
    against one recurrence over all 190 tokens."""
    B, T1, n, H = 2, 150, 40, 3
    q, k, v, log_a = synth.linear_inputs(9 + D, B, T1 + n, H, D)
    dev = torch.device("cuda")
    qd, kd, vd, ad = q.to(dev), k.to(dev), v.to(dev), log_a.to(dev)
    layer = lte.LinearLayer(B, H, D)
    state = layer.alloc_state()
    o1, _ = layer.prefill(qd[:, :T1].contiguous(), kd[:, :T1].contiguous(),
                          vd[:, :T1].contiguous(), ad[:, :T1].contiguous(), state_in=state,
                          state_out=state)
    outs = [layer.decode_step(qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(),
                              ad[:, t].contiguous(), state) for t in range(T1, T1 + n)]
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.linear_recurrent(q.float().numpy(), k.float().numpy(),
                                           v.float().numpy(), log_a.numpy())
    _check(o1.float().cpu().numpy(), ref_o[:, :T1], "prefill out")
    _check(torch.stack(outs, 1).float().cpu().numpy(), ref_o[:, T1:], "decode out")
    _check_state(state.cpu().numpy(), ref_S, "state")


def test_linear_full_size():
    """B32, 4096 tokens, H16, D128 (the bench shape); batches 0 and 21 checked."""
    B, T, H, D = 32, 4096, 16, 128
    q, k, v, log_a = synth.linear_inputs(11, B, T, H, D)
    layer = lte.LinearLayer(B, H, D)
    o, S = layer.prefill(q.cuda(), k.cuda(), v.cuda(), log_a.cuda())
    torch.cuda.synchronize()
    sel = [0, 21]
    ref_o, ref_S = oracle.linear_recurrent(q[sel].float().numpy(), k[sel].float().numpy(),
                                           v[sel].float().numpy(), log_a[sel].numpy())
    _check(o[sel].float().cpu().numpy(), ref_o, "out")
    _check_state(S[sel].cpu().numpy(), ref_S, "state")
