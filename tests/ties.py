"""Inputs whose retention scores tie exactly (tests only).

The keep rule breaks ties between equal scores by the lower index, and a token
leaving the window displaces the weakest retained entry only when its score is
strictly higher.  With CNN inputs drawn from N(0, 1) two tokens practically never
share a score, so these cases build scores that tie by construction, identically
on any path that evaluates the CNN:

* ``flat_case``: W1 = W2 = 0, so every token's logit is b2 and every score is
  sigmoid(b2) -- one level for the whole sequence;
* ``level_case``: the only non-zero weights are W1[o=0][key channel 0][centre
  tap] = 1 and W2[o=0][centre tap] = 1, so z_j = b2 + GELU(k_j[0]).  Key channel 0
  is set to one of a few bf16-exact values per token, so the scores take a few
  levels, equal within a level: layer 1 sums one product with zeros, layer 2 one
  activation with zeros, both exact in any order.

The levels sit far from 0.5 and far from each other (more than 1e-3 apart), so
no token lies in the exemption band around the keep threshold, and ties inside
a level are exact: the keep sets must agree exactly, including which of the
tied tokens are kept.
"""
import numpy as np
import torch

from learnable_kv_cache_amd import synth

HIDDEN = 32
LEVELS = (-1.0, 0.5, 2.0)     # key channel 0 values; with b2 = -0.2 the scores are about
                              # 0.411 (not kept), 0.536 and 0.853


def _zero_cnn(Hkv, D, b2):
    return {"W1": np.zeros((Hkv, HIDDEN, 2 * D, 3), np.float32),
            "b1": np.zeros((Hkv, HIDDEN), np.float32),
            "W2": np.zeros((Hkv, HIDDEN, 3), np.float32),
            "b2": np.full((Hkv,), b2, np.float32)}


def flat_case(seed, B, T, Hq, Hkv, D, b2=0.4):
    """q, k, v (bf16, N(0,1)) and a CNN that scores every token sigmoid(b2)."""
    q, k, v = synth.make_qkv(B, T, Hq, Hkv, D, seed)
    return q, k, v, _zero_cnn(Hkv, D, b2)


def level_case(seed, B, T, Hq, Hkv, D, b2=-0.2, levels=LEVELS, probs=(0.45, 0.45, 0.1)):
    """q, k, v (bf16) with k[..., 0] drawn from ``levels`` (with probabilities ``probs``:
    the top level is rare, so a full segment of middle-level entries keeps being
    displaced by it), and a CNN whose score of token j is sigmoid(b2 + GELU(k_j[0]))."""
    q, k, v = synth.make_qkv(B, T, Hq, Hkv, D, seed)
    rng = np.random.default_rng(seed + 13)
    lv = rng.choice(np.asarray(levels, np.float32), size=(B, T, Hkv), p=probs)
    k = k.clone()
    k[..., 0] = torch.as_tensor(lv).to(torch.bfloat16)
    assert torch.equal(k[..., 0].float(), torch.as_tensor(lv)), "levels must be bf16-exact"
    cnn = _zero_cnn(Hkv, D, b2)
    cnn["W1"][:, 0, 0, 1] = 1.0
    cnn["W2"][:, 0, 1] = 1.0
    return q, k, v, cnn
