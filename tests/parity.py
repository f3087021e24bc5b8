"""Helpers that compare the HIP path's results with the oracle's (tests only).

Keep/evict sets: the HIP path reports, per (batch, KV head), rank[j] and
thr[m]; token j is retained at query i iff j <= i-w and rank[j] <= thr[i-w].
These helpers turn that into the oracle's ``ends`` form (first step at which
a token is no longer retained) and check the two agree except for tokens
whose ORACLE score lies within ``band`` (1e-3) of a threshold:
  * the 0.5 keep threshold, or
  * the score of the weakest retained token at a step where the oracle's set
    is full (the top-C cut).
Several keep sets are correct for such tokens, so only the rest must agree.
"""
import numpy as np

NOT_CAND = 0x7FFFFFFF
BAND = 1e-3


def gpu_ends(rank: np.ndarray, thr: np.ndarray, w: int, steps: int) -> np.ndarray:
    """ends[j] of one (b, g) from rank [T] and thr [T] (thr non-increasing past its head)."""
    T = rank.shape[0]
    ends = np.full(T, -1, np.int64)
    last = steps - 1 - w                      # last prefix end reached by the queries
    if last < 0:
        return ends
    th = thr[:last + 1].astype(np.int64)
    for j in np.nonzero(rank != NOT_CAND)[0]:
        if j > last:
            continue
        rj = int(rank[j])
        ok = th[j:] >= rj                     # retained at prefix m = j .. last
        # retained steps form a prefix of [j + w, steps)
        n = int(np.argmin(ok)) if not ok.all() else ok.shape[0]
        ends[j] = j + w + n
    return ends


def normalize_ends(ends: np.ndarray, w: int) -> np.ndarray:
    """Maps empty retention intervals (end == j + w) to -1, leaving the set semantics."""
    e = np.array(ends, np.int64, copy=True)
    j = np.arange(e.shape[-1])
    e[e == j + w] = -1
    return e


def retained_at(ends: np.ndarray, w: int, i: int) -> np.ndarray:
    j = np.arange(ends.shape[0])
    return np.nonzero((ends >= 0) & (j + w <= i) & (i < ends))[0]


def _cut(r_or: np.ndarray, ends_or: np.ndarray, w: int, C: int, i: int):
    """Score of the weakest token the oracle retains at step i if its set is full."""
    R = retained_at(ends_or, w, i)
    if C == 0 or len(R) < C:
        return None
    return float(r_or[R].min())


def keep_set_mismatches(r_or, ends_or, ends_gpu, w, C, band=BAND, steps=None):
    """Non-exempt (token, step) disagreements between the oracle's and the GPU's sets."""
    r_or = np.asarray(r_or, np.float32)
    T = ends_or.shape[0]
    steps = T if steps is None else steps
    bad = []
    for j in np.nonzero(ends_or != ends_gpu)[0]:
        a, b = int(ends_or[j]), int(ends_gpu[j])
        start = j + w
        lo_end = a if a >= 0 else start
        hi_end = b if b >= 0 else start
        lo, hi = min(lo_end, hi_end), max(lo_end, hi_end)
        lo = max(lo, start)
        if lo >= hi:
            continue                          # both empty intervals
        if abs(float(r_or[j]) - 0.5) <= band:
            continue
        # every differing step must sit at a full set whose cut is within band
        ok = True
        for i in (lo, hi - 1):
            cut = _cut(r_or, ends_or, w, C, min(i, steps - 1))
            if cut is None or abs(float(r_or[j]) - cut) > band:
                ok = False
        if not ok:
            bad.append((int(j), lo, hi, float(r_or[j])))
    return bad


def output_errors(o_gpu: np.ndarray, o_ref: np.ndarray):
    d = np.abs(o_gpu.astype(np.float64) - o_ref.astype(np.float64))
    return float(d.max()), float(d.mean())


MAX_ABS = 2e-2      # bf16 inputs/outputs, fp32 accumulation
MEAN_ABS = 1e-3


def bf16_round(x: np.ndarray) -> np.ndarray:
    """x rounded to bfloat16 (round to nearest even), returned as float64."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.bfloat16).double().numpy()


def spiked_keys(k, every: int, top: float):
    """k (bf16 [B, T, Hkv, D]) with the rows of every ``every``-th token scaled by a factor
    growing linearly from 1 at token 0 to ``top`` at token T-1, rounded to bf16: later
    keys carry ever larger logits (of either sign), so a query row keeps meeting keys that
    beat everything it has seen so far."""
    import torch
    kk = k.float().clone()
    T = kk.shape[1]
    js = np.arange(0, T, every)
    f = 1.0 + (top - 1.0) * js / max(T - 1, 1)
    kk[:, js] *= torch.tensor(f, dtype=torch.float32)[None, :, None, None]
    return kk.to(torch.bfloat16)


def late_key_gain(q: np.ndarray, k: np.ndarray, w: int, rows) -> float:
    """Largest, over the given rows (batch 0, query head 0, KV head 0), of the row's best
    logit in its window minus its best logit over the first 32 keys of that window, in
    log2 units: above 8, a kernel that walks the window from its oldest keys and keeps a
    reference maximum must move that reference."""
    D = q.shape[-1]
    best = -np.inf
    for i in rows:
        lo = max(0, i - w + 1)
        lg = (k[0, lo:i + 1, 0].astype(np.float64) @ q[0, i, 0].astype(np.float64)) / np.sqrt(D)
        best = max(best, (lg.max() - lg[:32].max()) * np.log2(np.e))
    return float(best)
