"""Plain CPU oracle of the Learnable Token Eviction (LTE) sparse-attention layer.

TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It is slow on purpose: every step is
the definition written out, so a reader can check it against the sources by eye.
It shares no code with the HIP path and imports nothing from it.

Sources (cited by page title and the part of the page):

[LTE]  "Alleviating Forgetfulness of Linear Attention by Hybrid Sparse Attention
       and Contextualized Learnable Token Eviction" (He & Garner, arXiv
       2510.20787), summary page: TL;DR, Abstract, Figure 2 caption (eviction
       scheme, sink s and window w, per-token per-head score r_{j,h} from past
       and future neighbours, "A-plus-column" pattern), Figure 3 caption (cache
       layout: circular window segment, capped out-of-window segment holding
       the retained KVs and the sink; scoring batched and deferred).
[SWA]  "Sparse Linear Attention: Viewing SWA from the Perspective of Linear
       Attention", section "Viewing SWA from the linear-state perspective":
       the window is a FIFO of slots, one slot overwritten per token.

What the pages leave open is fixed here by these readings (each restated where
it is used):

R1  Window of query i = the w most recent positions including i: [i-w+1, i].
    Token j leaves the window at step j+w.
R2  Sink = the first s positions: always visible (causally), never scored or
    evicted, stored outside the capped segment.
R3  Scores, retention and the cache are per KV head; the query heads of a GQA
    group share them.
R4  Scoring CNN per KV head: x = concat(k, v) (2D channels, keys first);
    h = GELU(conv1d_{2D->32, kernel 3}(x) + b1); z = conv1d_{32->1, kernel 3}(h)
    + b2; r = sigmoid(z).  conv1d is cross-correlation with zero padding of 1
    on each layer (tap t reads offset t-1).  GELU is the exact erf form.
    Receptive field: tokens j-2 .. j+2 (past and future neighbours).
R5  Keep rule: token j >= s is a candidate iff r_j > 0.5 (strict, on the fp32
    score).  The retained set never exceeds C; on overflow the C best by
    (score descending, index ascending) stay, so among equal scores the lower
    index wins, and a newcomer only displaces the weakest entry when it ranks
    above it.  Decisions are causal: query i sees the set R_i built from the
    tokens that left the window by step i.
R6  Attention: o_i = sum_{j in V(i)} softmax_j(q_i.k_j / sqrt(D)) v_j over
    V(i) = sink U window U R_i (a set union); no bias, no RoPE.
R7  Deferred scoring in decode: a score is computed once tokens j-2..j+2 are
    all present, in batches, as late as the ring still holds the left
    neighbour j-2: when token t is appended and t = u + w - 3 for the oldest
    unscored token u, tokens u .. t-2 are scored from the ring.
"""
from __future__ import annotations

import heapq
import math

import numpy as np
from scipy.special import erf

__all__ = [
    "cnn_logits", "cnn_scores", "retention_ends", "retained_set", "visible_set",
    "visible_indices", "attention", "attention_on_set", "prefill", "LayerCache",
]


# --------------------------------------------------------------------------
# Scoring CNN  ([LTE] Figure 2 caption; reading R4)
# --------------------------------------------------------------------------

def _gelu(h: np.ndarray) -> np.ndarray:
    """Exact GELU: 0.5 h (1 + erf(h / sqrt 2))."""
    return 0.5 * h * (1.0 + erf(h / math.sqrt(2.0)))


def cnn_logits_seq(k_seq: np.ndarray, v_seq: np.ndarray, W1, b1, W2, b2,
                   dtype=np.float64) -> np.ndarray:
    """Logits z[t] of one KV head over one token sequence.

    k_seq, v_seq: [T, D]; W1 [hidden, 2D, 3], b1 [hidden], W2 [hidden, 3], b2 scalar.
    Both convolution layers pad the sequence ends with zeros (one token each).
    """
    T = k_seq.shape[0]
    x = np.concatenate([k_seq, v_seq], axis=1).astype(dtype)          # [T, 2D]
    hidden = W1.shape[0]
    xp = np.zeros((T + 2, x.shape[1]), dtype)
    xp[1:T + 1] = x                                                    # x[-1] = x[T] = 0
    h = np.zeros((T, hidden), dtype) + np.asarray(b1, dtype)[None, :]
    for tap in range(3):                                               # tap reads x[t + tap - 1]
        h += xp[tap:tap + T] @ np.asarray(W1[:, :, tap], dtype).T
    a = _gelu(h)
    ap = np.zeros((T + 2, hidden), dtype)
    ap[1:T + 1] = a                                                    # a[-1] = a[T] = 0
    z = np.zeros((T,), dtype) + dtype(b2)
    for tap in range(3):
        z += ap[tap:tap + T] @ np.asarray(W2[:, tap], dtype)
    return z


def cnn_logits(k, v, W1, b1, W2, b2, dtype=np.float64) -> np.ndarray:
    """z[b, g, t] for k, v [B, T, Hkv, D] and per-KV-head weights (reading R3/R4)."""
    k = np.asarray(k)
    v = np.asarray(v)
    B, T, Hkv, _ = k.shape
    z = np.zeros((B, Hkv, T), dtype)
    for b in range(B):
        for g in range(Hkv):
            z[b, g] = cnn_logits_seq(k[b, :, g, :], v[b, :, g, :], W1[g], b1[g], W2[g],
                                     b2[g], dtype)
    return z


def sigmoid_to_f32(z: np.ndarray) -> np.ndarray:
    """r = 1 / (1 + exp(-z)), evaluated in z's precision and stored as fp32."""
    one = z.dtype.type(1.0)
    return (one / (one + np.exp(-z))).astype(np.float32)


def cnn_scores(k, v, W1, b1, W2, b2, dtype=np.float64) -> np.ndarray:
    """Retention scores r[b, g, t] (fp32) of every token of a sequence."""
    return sigmoid_to_f32(cnn_logits(k, v, W1, b1, W2, b2, dtype))


# --------------------------------------------------------------------------
# Eviction under a budget  ([LTE] TL;DR, Figure 2 caption; readings R1, R2, R5)
# --------------------------------------------------------------------------

def retention_ends(r: np.ndarray, s: int, w: int, C: int, steps: int) -> np.ndarray:
    """Stream the keep/evict decisions of one (batch, KV head) over ``steps`` queries.

    At step i the token j = i - w leaves the window.  If j >= s and r_j > 0.5 it
    joins the retained set; if the set then holds more than C tokens the
    weakest one -- lowest score, and among equal scores the highest index --
    is evicted (possibly j itself).  R_i is the set after step i.

    Returns end[j]: -1 if token j never joins within ``steps`` steps; otherwise
    the first step at which j is no longer retained (``steps`` if it still is
    after the last step).  Token j is in R_i iff end[j] >= 0 and
    j + w <= i < end[j].
    """
    r = np.asarray(r, np.float32)
    end = np.full(r.shape[0], -1, np.int64)
    heap: list[tuple[float, int]] = []      # min-heap on (score, -index): the weakest on top
    for i in range(steps):
        j = i - w
        if j >= s and r[j] > np.float32(0.5):
            heapq.heappush(heap, (float(r[j]), -j))
            end[j] = steps
            if len(heap) > C:
                _, neg = heapq.heappop(heap)
                end[-neg] = i
    return end


def retained_set(end: np.ndarray, w: int, i: int) -> np.ndarray:
    """Sorted token indices of R_i from an ``end`` array."""
    j = np.arange(end.shape[0])
    return np.nonzero((end >= 0) & (j + w <= i) & (i < end))[0]


def visible_set(i: int, s: int, w: int, R) -> np.ndarray:
    """V(i) = sink U window U R as sorted unique indices, for a retained set R (R6)."""
    sink = np.arange(0, min(s, i + 1))
    window = np.arange(max(0, i - w + 1), i + 1)
    return np.union1d(np.union1d(sink, window), np.asarray(list(R), np.int64))


def visible_indices(i: int, s: int, w: int, end: np.ndarray) -> np.ndarray:
    """V(i) = sink U window U R_i as sorted unique indices (reading R6)."""
    return visible_set(i, s, w, retained_set(end, w, i))


# --------------------------------------------------------------------------
# A-plus-column attention  ([LTE] Figure 2 caption, right panel; reading R6)
# --------------------------------------------------------------------------

def attention(q, k, v, s: int, w: int, ends: np.ndarray, dtype=np.float64,
              rows=None, pairs=None) -> np.ndarray:
    """o[b, i, h] = softmax over V(i) of q.k / sqrt(D), applied to v.

    q [B, T, Hq, D]; k, v [B, T, Hkv, D]; ends [B, Hkv, T] from retention_ends.
    ``rows`` restricts the computed query rows (others stay NaN); ``pairs``
    restricts the (b, g) pairs.  Each row gathers its visible keys, exactly as
    the definition reads.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    out = np.full((B, T, Hq, D), np.nan, dtype)
    rows = range(T) if rows is None else rows
    pairs = [(b, g) for b in range(B) for g in range(Hkv)] if pairs is None else pairs
    for (b, g) in pairs:
        for i in rows:
            idx = visible_indices(int(i), s, w, ends[b, g])
            out[b, i, g * G:(g + 1) * G, :] = _softmax_rows(q[b, i, g * G:(g + 1) * G, :],
                                                           k[b, idx, g, :], v[b, idx, g, :],
                                                           dtype)
    return out


def _softmax_rows(Q, K, V, dtype) -> np.ndarray:
    """softmax(Q K^T / sqrt(D)) V for the query rows Q [G, D] over the keys K, V [n, D]."""
    Q = np.asarray(Q).astype(dtype)
    K = np.asarray(K).astype(dtype)
    V = np.asarray(V).astype(dtype)
    logits = (Q @ K.T) * dtype(1.0 / math.sqrt(Q.shape[-1]))      # [G, n]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    return (p @ V) / p.sum(axis=1, keepdims=True)


def attention_on_set(q, k, v, s: int, w: int, b: int, i: int, g: int, R,
                     dtype=np.float64) -> np.ndarray:
    """o of query row i of KV head g in sequence b ([G, D]) when the retained set at
    that step is R: the same softmax as ``attention`` over sink U window U R.

    Used to check a keep set realised elsewhere (the GPU's), where several sets are
    correct for tokens scored at a threshold; q [B, T, Hq, D], k, v [B, T, Hkv, D].
    """
    q = np.asarray(q)
    G = q.shape[2] // np.asarray(k).shape[2]
    idx = visible_set(int(i), s, w, R)
    return _softmax_rows(q[b, i, g * G:(g + 1) * G, :], np.asarray(k)[b, idx, g, :],
                         np.asarray(v)[b, idx, g, :], dtype)


def all_ends(scores: np.ndarray, s: int, w: int, C: int, steps: int) -> np.ndarray:
    B, Hkv, T = scores.shape
    ends = np.empty((B, Hkv, T), np.int64)
    for b in range(B):
        for g in range(Hkv):
            ends[b, g] = retention_ends(scores[b, g], s, w, C, steps)
    return ends


def prefill(q, k, v, s: int, w: int, C: int, cnn: dict | None = None,
            scores: np.ndarray | None = None, dtype=np.float64, rows=None, pairs=None):
    """The LTE layer over a whole prompt: score, evict, attend.

    Exactly one of ``cnn`` (parameters W1, b1, W2, b2) or ``scores`` (an
    explicit fp32 [B, Hkv, T] score array) is given.
    Returns dict(o, scores, ends).
    """
    k = np.asarray(k)
    T = k.shape[1]
    if scores is None:
        scores = cnn_scores(k, v, cnn["W1"], cnn["b1"], cnn["W2"], cnn["b2"], dtype)
    scores = np.asarray(scores, np.float32)
    ends = all_ends(scores, s, w, C, T)
    o = attention(q, k, v, s, w, ends, dtype, rows=rows, pairs=pairs)
    return {"o": o, "scores": scores, "ends": ends}


# --------------------------------------------------------------------------
# Explicit KV cache, stepped one token at a time
# ([LTE] Figure 3 caption; [SWA] FIFO slot write; readings R1, R2, R5, R7)
# --------------------------------------------------------------------------

class LayerCache:
    """The LTE cache of one layer for B sequences of equal length and Hkv heads.

    Per (b, g): a sink list (tokens 0..s-1), a ring of w slots where token j
    sits in slot j mod w, a capped list of at most C retained (token, score,
    key, value) entries, and per ring slot the token's score (NaN until
    scored).  ``pos`` is the number of tokens ingested; ``next_unscored`` the
    oldest token that still lacks a score.
    """

    def __init__(self, B, Hkv, D, s, w, C, cnn=None, dtype=np.float64):
        self.B, self.Hkv, self.D = B, Hkv, D
        self.s, self.w, self.C = s, w, C
        self.cnn = cnn
        self.dtype = dtype
        self.pos = 0
        self.next_unscored = s
        self.sink = [[[] for _ in range(Hkv)] for _ in range(B)]          # (j, k, v)
        self.ring_tok = np.full((B, Hkv, w), -1, np.int64)
        self.ring_k = np.zeros((B, Hkv, w, D), np.float32)
        self.ring_v = np.zeros((B, Hkv, w, D), np.float32)
        self.ring_score = np.full((B, Hkv, w), np.nan, np.float32)
        self.ret = [[[] for _ in range(Hkv)] for _ in range(B)]           # [j, r, k, v]

    # -- construction from a prefill -------------------------------------
    @classmethod
    def from_prefill(cls, k, v, scores, ends, s, w, C, cnn=None, dtype=np.float64):
        """Cache state after a T-token prompt: sink, last w tokens in the ring,
        R_{T-1} in the capped segment; scores are final for tokens <= T-3."""
        k = np.asarray(k)
        v = np.asarray(v)
        B, T, Hkv, D = k.shape
        c = cls(B, Hkv, D, s, w, C, cnn, dtype)
        for b in range(B):
            for g in range(Hkv):
                for j in range(min(s, T)):
                    c.sink[b][g].append((j, k[b, j, g].copy(), v[b, j, g].copy()))
                for j in range(max(0, T - w), T):
                    slot = j % w
                    c.ring_tok[b, g, slot] = j
                    c.ring_k[b, g, slot] = k[b, j, g]
                    c.ring_v[b, g, slot] = v[b, j, g]
                    if j >= s and j <= T - 3:
                        c.ring_score[b, g, slot] = scores[b, g, j]
                for j in retained_set(ends[b, g], w, T - 1):
                    c.ret[b][g].append([int(j), np.float32(scores[b, g, j]),
                                        k[b, j, g].copy(), v[b, j, g].copy()])
        c.pos = T
        c.next_unscored = max(T - 2, s)
        return c

    # -- one decode step ----------------------------------------------------
    def _insert(self, b, g, j, r, kj, vj):
        """Top-C insertion of a token that left the window with r > 0.5 (R5)."""
        lst = self.ret[b][g]
        if len(lst) < self.C:
            lst.append([j, r, kj, vj])
            return
        if self.C == 0:
            return
        # weakest entry: lowest score, then highest index
        wi = min(range(len(lst)), key=lambda x: (lst[x][1], -lst[x][0]))
        wr, wj = lst[wi][1], lst[wi][0]
        if (r, -j) > (wr, -wj):          # newcomer ranks above the weakest entry
            lst[wi] = [j, r, kj, vj]

    def _score_batch(self, b, g, u, t):
        """Score tokens u..t-2 from the ring contents (tokens u-2..t present)."""
        lo = max(0, u - 2)
        toks = list(range(lo, t + 1))
        ks = np.stack([self.ring_k[b, g, j % self.w] for j in toks])
        vs = np.stack([self.ring_v[b, g, j % self.w] for j in toks])
        for j in toks:
            assert self.ring_tok[b, g, j % self.w] == j
        cnn = self.cnn
        z = cnn_logits_seq(ks, vs, cnn["W1"][g], cnn["b1"][g], cnn["W2"][g], cnn["b2"][g],
                           self.dtype)
        r = sigmoid_to_f32(z)
        for j in range(u, t - 1):
            self.ring_score[b, g, j % self.w] = r[j - lo]

    def ingest(self, k_t, v_t):
        """Evict the token leaving the window, append token t, score if due."""
        t = self.pos
        s, w = self.s, self.w
        j = t - w
        slot = t % w
        for b in range(self.B):
            for g in range(self.Hkv):
                if j >= s:
                    assert self.ring_tok[b, g, slot] == j
                    r = self.ring_score[b, g, slot]
                    assert not np.isnan(r), "token left the window unscored"
                    if r > np.float32(0.5):
                        self._insert(b, g, j, np.float32(r), self.ring_k[b, g, slot].copy(),
                                     self.ring_v[b, g, slot].copy())
                self.ring_tok[b, g, slot] = t
                self.ring_k[b, g, slot] = k_t[b, g]
                self.ring_v[b, g, slot] = v_t[b, g]
                self.ring_score[b, g, slot] = np.nan
                if t < s:
                    self.sink[b][g].append((t, k_t[b, g].copy(), v_t[b, g].copy()))
        if t == self.next_unscored + w - 3:
            for b in range(self.B):
                for g in range(self.Hkv):
                    self._score_batch(b, g, self.next_unscored, t)
            self.next_unscored = t - 1
        self.pos = t + 1

    def visible(self, b, g):
        """(indices, K, V) of every key a query at position pos-1 attends to."""
        t = self.pos - 1
        idx, ks, vs = [], [], []
        for (j, kj, vj) in self.sink[b][g]:
            idx.append(j); ks.append(kj); vs.append(vj)
        for (j, _, kj, vj) in self.ret[b][g]:
            idx.append(j); ks.append(kj); vs.append(vj)
        for slot in range(self.w):
            j = int(self.ring_tok[b, g, slot])
            if j >= max(self.s, t - self.w + 1) and j <= t:
                idx.append(j); ks.append(self.ring_k[b, g, slot]); vs.append(self.ring_v[b, g, slot])
        return np.array(idx, np.int64), np.stack(ks), np.stack(vs)

    def attend(self, q_t):
        """o [B, Hq, D] of the newest token's queries over the cache."""
        q_t = np.asarray(q_t)
        B, Hq, D = q_t.shape
        G = Hq // self.Hkv
        out = np.zeros((B, Hq, D), self.dtype)
        scale = self.dtype(1.0 / math.sqrt(D))
        for b in range(B):
            for g in range(self.Hkv):
                _, K, V = self.visible(b, g)
                K = K.astype(self.dtype)
                V = V.astype(self.dtype)
                Q = q_t[b, g * G:(g + 1) * G].astype(self.dtype)
                logits = (Q @ K.T) * scale
                m = logits.max(axis=1, keepdims=True)
                p = np.exp(logits - m)
                out[b, g * G:(g + 1) * G] = (p @ V) / p.sum(axis=1, keepdims=True)
        return out

    def step(self, q_t, k_t, v_t):
        """One decode step: ingest token pos, then attend with its queries."""
        self.ingest(k_t, v_t)
        return self.attend(q_t)

    def retained_indices(self, b, g) -> np.ndarray:
        return np.array(sorted(e[0] for e in self.ret[b][g]), np.int64)
