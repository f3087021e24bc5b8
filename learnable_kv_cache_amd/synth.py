"""Seeded synthetic inputs for the LTE sparse-attention layer.

This module only draws random numbers and arranges them into the shapes of the
workloads below.  It holds none of the layer's arithmetic, so both the CPU oracle
(under ``oracle/``) and the HIP path are fed from here without sharing any code
of the method itself.

Every tensor is drawn on the CPU with a seeded ``torch.Generator``:

* q, k, v ~ N(0, 1), drawn in fp32 and rounded to bf16 (round-to-nearest-even)
  before either side sees them, so the oracle and the GPU read identical values.
* CNN weights W1, W2 ~ N(0, 0.02^2) (0.02 is the standard deviation), b1 = 0,
  and the output bias b2 as each workload states.  They stay fp32.
* The "artificial KV cache" of the kernel-only workload is a Bernoulli(p) draw
  per (batch, KV head, token) over the tokens that can leave the window; it is
  handed to the layer as an explicit score (1.0 selected, 0.0 not).

Workload table (sizes as the LTE paper's Figure 4 setting: batch 32, 4K prompt):

====  ==========================================================================
 1    tiny layer: B1 T256 Hq4 Hkv2 D64 s2 w32 C16, CNN with b2 = 0
 2    attention only: B8 T4096 Hq16 Hkv4 D128 s4 w512 C512, 10% random retention
 3    full prefill: B32 T4096 Hq16 Hkv4 D128 s4 w512 C512, CNN, b2 ~ U(-2, 1)
 4    decode: config 3's shapes and CNN, prompt 4096 then 512 decode tokens
 5    long decode: B4 T32768 Hq32 Hkv8 D128 s4 w1024 C2048, then 256 decode
      tokens; b2 set per run to reach a target retention rate
====  ==========================================================================
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

HIDDEN = 32  # width of the scoring CNN's hidden layer


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int            # prompt length
    Hq: int
    Hkv: int
    D: int
    sink: int
    window: int
    capacity: int
    seed: int
    cnn: bool = True            # False: scores come from a Bernoulli override
    b2: str = "zero"            # "zero" | "uniform" (U(-2, 1) per KV head) | "given"
    override_rate: float = 0.0  # Bernoulli rate of the artificial KV cache
    decode_steps: int = 0
    cnn_seed: int | None = None

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {
    1: Workload("tiny-layer", B=1, T=256, Hq=4, Hkv=2, D=64, sink=2, window=32,
                capacity=16, seed=1001),
    2: Workload("attention-artificial-cache", B=8, T=4096, Hq=16, Hkv=4, D=128,
                sink=4, window=512, capacity=512, seed=1002, cnn=False,
                override_rate=0.1),
    3: Workload("prefill-b32-t4096", B=32, T=4096, Hq=16, Hkv=4, D=128, sink=4,
                window=512, capacity=512, seed=1003, b2="uniform"),
    4: Workload("decode-b32-t4096", B=32, T=4096, Hq=16, Hkv=4, D=128, sink=4,
                window=512, capacity=512, seed=1004, b2="uniform", decode_steps=512,
                cnn_seed=1103),
    5: Workload("long-decode-b4-t32768", B=4, T=32768, Hq=32, Hkv=8, D=128, sink=4,
                window=1024, capacity=2048, seed=1005, b2="given", decode_steps=256),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def bf16_values(x: torch.Tensor) -> torch.Tensor:
    """fp32 tensor whose values are the bf16 (RNE) roundings of ``x``."""
    return x.to(torch.bfloat16).to(torch.float32)


def make_qkv(B: int, T: int, Hq: int, Hkv: int, D: int, seed: int):
    """q [B,T,Hq,D], k and v [B,T,Hkv,D] as bf16 CPU tensors (N(0,1) rounded)."""
    g = _gen(seed)
    q = torch.randn((B, T, Hq, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((B, T, Hkv, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((B, T, Hkv, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v


def make_cnn(Hkv: int, D: int, seed: int, b2: str | np.ndarray = "zero",
             hidden: int = HIDDEN, std: float = 0.02):
    """Scoring-CNN parameters as fp32 numpy arrays.

    W1 [Hkv, hidden, 2D, 3], b1 [Hkv, hidden], W2 [Hkv, hidden, 3], b2 [Hkv].
    Channel order of the 2D input channels: the D key channels, then the D value
    channels.  Tap index 0..2 of a kernel-3 filter.
    """
    g = _gen(seed)
    W1 = (torch.randn((Hkv, hidden, 2 * D, 3), generator=g) * std).numpy().astype(np.float32)
    W2 = (torch.randn((Hkv, hidden, 3), generator=g) * std).numpy().astype(np.float32)
    b1 = np.zeros((Hkv, hidden), np.float32)
    if isinstance(b2, np.ndarray):
        b2v = b2.astype(np.float32).reshape(Hkv)
    elif b2 == "zero" or b2 == "given":
        b2v = np.zeros((Hkv,), np.float32)
    elif b2 == "uniform":
        b2v = (torch.rand((Hkv,), generator=g) * 3.0 - 2.0).numpy().astype(np.float32)
    else:
        raise ValueError(f"unknown b2 recipe {b2!r}")
    return {"W1": W1, "b1": b1, "W2": W2, "b2": b2v}


def make_override(B: int, Hkv: int, T: int, sink: int, window: int, rate: float,
                  seed: int) -> np.ndarray:
    """Artificial KV cache: fp32 scores [B,Hkv,T], 1.0 for a retained token, else 0.0.

    Only tokens j in [sink, T-1-window] ever leave the window during a T-token
    prefill, so only they are drawn; every other score is 0.0.
    """
    g = _gen(seed + 7)
    u = torch.rand((B, Hkv, T), generator=g)
    sel = (u < rate).numpy()
    j = np.arange(T)
    sel &= ((j >= sink) & (j <= T - 1 - window))[None, None, :]
    return sel.astype(np.float32)


def workload_inputs(n: int, T: int | None = None, B: int | None = None,
                    decode_steps: int | None = None, b2: np.ndarray | None = None):
    """Inputs of workload ``n`` (optionally cut to a smaller T / B / step count).

    Returns a dict with the ``Workload`` record, bf16 CPU tensors q,k,v holding
    the prompt followed by the decode tokens, the CNN parameters (or None) and
    the score override (or None).
    """
    wl = WORKLOADS[n]
    T = wl.T if T is None else T
    B = wl.B if B is None else B
    steps = wl.decode_steps if decode_steps is None else decode_steps
    q, k, v = make_qkv(B, T + steps, wl.Hq, wl.Hkv, wl.D, wl.seed)
    cnn = None
    override = None
    if wl.cnn:
        cseed = wl.cnn_seed if wl.cnn_seed is not None else wl.seed + 100
        cnn = make_cnn(wl.Hkv, wl.D, cseed, b2 if b2 is not None else wl.b2)
    else:
        override = make_override(B, wl.Hkv, T, wl.sink, wl.window, wl.override_rate, wl.seed)
    return {"workload": wl, "T": T, "B": B, "steps": steps, "q": q, "k": k, "v": v,
            "cnn": cnn, "override": override}


def random_case(seed: int, B: int, T: int, Hq: int, Hkv: int, D: int, cnn_std: float = 0.02,
                b2: float = 0.0):
    """Small random case for parity sweeps: bf16 q,k,v plus a CNN with a shared b2."""
    q, k, v = make_qkv(B, T, Hq, Hkv, D, seed)
    cnn = make_cnn(Hkv, D, seed + 100, np.full((Hkv,), b2, np.float32), std=cnn_std)
    return q, k, v, cnn


def linear_inputs(seed: int, B: int, T: int, H: int, D: int, gate_mean: float = 4.0):
    """Inputs of the linear-attention layer as CPU tensors: q, k [B,T,H,D] bf16 with
    std D^-1/4 (so q.k is of order 1), v [B,T,H,D] bf16 N(0,1), and the per-step
    decay as log a [B,T,H] fp32 with a = sigmoid(N(gate_mean, 1)) (mean about 0.98
    for gate_mean 4: a memory of some tens of tokens)."""
    g = _gen(seed)
    s = float(D) ** -0.25
    q = (torch.randn((B, T, H, D), generator=g) * s).to(torch.bfloat16)
    k = (torch.randn((B, T, H, D), generator=g) * s).to(torch.bfloat16)
    v = torch.randn((B, T, H, D), generator=g).to(torch.bfloat16)
    x = torch.randn((B, T, H), generator=g) + gate_mean
    log_a = torch.nn.functional.logsigmoid(x).to(torch.float32)
    return q, k, v, log_a
