"""Chunked prefill onto an existing cache (needs an MI355X).

A chunk of n tokens appended to a cache must give, for every sequence, what one
prefill over that sequence's whole history gives: its rows' outputs within
2e-2 max-abs / 1e-3 mean-abs of the oracle's attention on the GPU's realised
visible sets, those sets equal to the oracle's except for tokens whose oracle
score is within 1e-3 of 0.5 or of the top-C cut, and a cache equal to the
oracle's explicit cache after the same tokens (segment membership under the
same exemptions, ring scores within 5e-4, pos, next_unscored).  Decode steps
after a chunk are then checked like the decode tests.

The realised sets of the chunk's queries come from the call's workspace views
(rank/thr over the extended sequence: sink, segment sorted by token, ring,
chunk), mapped back to tokens with the cache's positions and segment as they
stood before the call.
"""
import numpy as np
import pytest
import torch

import oracle
from learnable_kv_cache_amd import lte, synth
from tests.parity import BAND, MAX_ABS, MEAN_ABS, NOT_CAND
from tests.test_gpu_decode import SCORE_TOL

pytestmark = pytest.mark.gpu


class Stream:
    """A layer over B independent token streams; each sequence's position advances
    through prefill, chunks and decode steps and is checked after each."""

    def __init__(self, B, Hq, Hkv, D, s, w, C, total=None, seed=None, b2=None, inputs=None,
                 check_b=None, every=1, exact=False):
        self.B, self.Hq, self.Hkv, self.D, self.s, self.w, self.C = B, Hq, Hkv, D, s, w, C
        # exact: scores tie exactly and lie far from every threshold, so no token is
        # exempt and every set must equal the oracle's
        self.exact = exact
        self.G = Hq // Hkv
        if inputs is None:
            inputs = synth.random_case(seed, B, total, Hq, Hkv, D, b2=b2)
        self.q, self.k, self.v, self.cnn = inputs
        self.check_b = list(range(B)) if check_b is None else check_b
        self.every = every                 # chunk query rows checked: every n-th and the last
        self.qn, self.kn, self.vn = (x[self.check_b].float().numpy()
                                     for x in (self.q, self.k, self.v))
        self.r_all = oracle.cnn_scores(self.kn, self.vn, self.cnn["W1"], self.cnn["b1"],
                                       self.cnn["W2"], self.cnn["b2"])
        self.dev = torch.device("cuda")
        self.qd, self.kd, self.vd = (x.to(self.dev) for x in (self.q, self.k, self.v))
        self.layer = lte.Layer(lte.Config(B, Hq, Hkv, D, s, w, C))
        self.dcnn = lte.CNN(self.cnn)
        self.cache = self.layer.alloc_cache()
        self.views = self.layer.cache_views(self.cache)
        self.pos = [0] * B
        self.dws = self.layer.alloc_workspace(0)

    # -- driving ---------------------------------------------------------------
    def prefill(self, lens):
        T = max(lens)
        ws = self.layer.alloc_workspace(T)
        sl = torch.tensor(lens, dtype=torch.int32, device=self.dev)
        self.layer.prefill(self.qd[:, :T].contiguous(), self.kd[:, :T].contiguous(),
                           self.vd[:, :T].contiguous(), cnn=self.dcnn, cache=self.cache,
                           workspace=ws, seq_lens=sl)
        torch.cuda.synchronize()
        self.pos = list(lens)
        self.check_cache()

    def _rows(self, x, n):
        idx = torch.tensor([[p + i for i in range(n)] for p in self.pos], device=self.dev)
        return x[torch.arange(self.B, device=self.dev)[:, None], idx].contiguous()

    def chunk(self, n):
        before = {nm: self.views[nm].cpu().numpy().copy() for nm in ("ret_idx", "count", "pos")}
        ws = self.layer.alloc_chunk_workspace(n)
        out = self.layer.prefill_chunk(self._rows(self.qd, n), self._rows(self.kd, n),
                                       self._rows(self.vd, n), self.dcnn, self.cache, ws)
        torch.cuda.synchronize()
        s, w, C = self.s, self.w, self.C
        E = s + C + w + n
        ev = {nm: x.cpu().numpy() for nm, x in self.layer.workspace_views(ws, E).items()}
        o = out.float().cpu().numpy()
        rows = sorted(set(range(0, n, self.every)) | {n - 1})
        for bi, b in enumerate(self.check_b):
            P = self.pos[b]
            Tn = P + n
            warm = P >= s + w
            q_lo = s + C + w if warm else P
            pre = oracle.prefill(self.qn[bi:bi + 1, :Tn], self.kn[bi:bi + 1, :Tn],
                                 self.vn[bi:bi + 1, :Tn], s, w, C, cnn=self.cnn, rows=[])
            for g in range(self.Hkv):
                bg_scores = self.r_all[bi, g]
                # row -> token of the extended sequence
                tokmap = np.arange(E, dtype=np.int64)
                if warm:
                    cnt = int(before["count"][b, g])
                    tokmap[s:s + C] = -1
                    tokmap[s:s + cnt] = np.sort(before["ret_idx"][b, g, :cnt])
                    tokmap[s + C:] += P - w - s - C
                rank, thr = ev["rank"][b, g].astype(np.int64), ev["thr"][b, g].astype(np.int64)
                sl = slice(g * self.G, (g + 1) * self.G)
                errs = []
                for qi in rows:
                    i = P + qi
                    m = q_lo + qi - w
                    R = set()
                    if m >= 0:
                        sel = np.nonzero((rank[:m + 1] != NOT_CAND) & (rank[:m + 1] <= thr[m]))[0]
                        assert np.all(tokmap[sel] >= 0), (b, g, sel)
                        R = set(tokmap[sel].tolist())
                    Ro = set(oracle.retained_set(pre["ends"][0, g], w, i).tolist())
                    cut = min(float(bg_scores[j]) for j in Ro) if C > 0 and len(Ro) == C else None
                    for j in R ^ Ro:
                        rj = float(bg_scores[j])
                        ok = abs(rj - 0.5) <= BAND or (cut is not None and abs(rj - cut) <= BAND)
                        assert ok and not self.exact, ("chunk set", b, g, i, j, rj, cut)
                    ref = oracle.attention_on_set(self.qn, self.kn, self.vn, s, w, bi, i, g, R)
                    errs.append(np.abs(o[b, qi, sl] - ref))
                d = np.stack(errs)
                assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS, ("chunk out", b, g, d.max(),
                                                                    d.mean())
        self.pos = [p + n for p in self.pos]
        self.check_cache()

    def decode(self, m):
        for _ in range(m):
            qt, kt, vt = self._rows(self.qd, 1)[:, 0], self._rows(self.kd, 1)[:, 0], \
                self._rows(self.vd, 1)[:, 0]
            o_t = self.layer.decode_step(qt.contiguous(), kt.contiguous(), vt.contiguous(),
                                         self.dcnn, self.cache, self.dws)
            torch.cuda.synchronize()
            og = o_t.float().cpu().numpy()
            ret_idx = self.views["ret_idx"].cpu().numpy()
            count = self.views["count"].cpu().numpy()
            for bi, b in enumerate(self.check_b):
                t = self.pos[b]
                for g in range(self.Hkv):
                    gset = set(ret_idx[b, g, :count[b, g]].tolist())
                    sl = slice(g * self.G, (g + 1) * self.G)
                    ref = oracle.attention_on_set(self.qn, self.kn, self.vn, self.s, self.w, bi,
                                                  t, g, gset)
                    d = np.abs(og[b, sl] - ref)
                    assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS, ("decode", t, b, g)
            self.pos = [p + 1 for p in self.pos]
        self.check_cache(fresh=False)

    # -- the cache against the oracle's explicit cache after the same tokens ------
    def check_cache(self, fresh=True):
        """fresh: after a prefill or chunk (no deferred scoring pending)."""
        s, w, C = self.s, self.w, self.C
        v = {nm: x.cpu().numpy() for nm, x in self.views.items() if nm not in ("k", "v")}
        # the exported bookkeeping is the cache's own
        ex = self.layer.cache_export(self.cache)
        for nm in ("count", "pos"):
            assert np.array_equal(ex[nm].numpy(), v[nm]), nm
        for b in range(self.B):
            for g in range(self.Hkv):
                cnt = int(v["count"][b, g])
                assert np.array_equal(ex["ret_idx"][b, g, :cnt].numpy(), v["ret_idx"][b, g, :cnt])
                assert np.array_equal(ex["ret_score"][b, g, :cnt].numpy(),
                                      v["ret_score"][b, g, :cnt])
        assert int(v["flags"].max()) == 0, "a token left the window unscored"
        kc = self.views["k"].float().cpu().numpy()
        for b in range(self.B):
            assert np.all(v["pos"][b] == self.pos[b]), (b, v["pos"][b], self.pos[b])
        for bi, b in enumerate(self.check_b):
            T = self.pos[b]
            nu = int(v["next_unscored"][b, 0])
            assert np.all(v["next_unscored"][b] == nu)
            if fresh:
                assert nu == max(T - 2, s), (b, nu, T)
            assert s <= nu <= max(T - 2, s)
            pre = oracle.prefill(self.qn[bi:bi + 1, :T], self.kn[bi:bi + 1, :T],
                                 self.vn[bi:bi + 1, :T], s, w, C, cnn=self.cnn, rows=[])
            oc = oracle.LayerCache.from_prefill(self.kn[bi:bi + 1, :T], self.vn[bi:bi + 1, :T],
                                                pre["scores"], pre["ends"], s, w, C, cnn=self.cnn)
            for g in range(self.Hkv):
                cnt = int(v["count"][b, g])
                gset = set(v["ret_idx"][b, g, :cnt].tolist())
                assert len(gset) == cnt <= C
                oset = set(oc.retained_indices(0, g).tolist())
                cut = None
                if C > 0 and len(oset) == C:
                    cut = min(float(self.r_all[bi, g, j]) for j in oset)
                for j in gset ^ oset:
                    rj = float(self.r_all[bi, g, j])
                    ok = abs(rj - 0.5) <= BAND or (cut is not None and abs(rj - cut) <= BAND)
                    assert ok and not self.exact, ("cache set", T, b, g, j, rj, cut)
                # retained entries carry their tokens' scores
                for x in range(cnt):
                    j = int(v["ret_idx"][b, g, x])
                    assert abs(float(v["ret_score"][b, g, x]) - float(self.r_all[bi, g, j])) <= \
                        SCORE_TOL, (b, g, x, j)
                # retained K rows hold their tokens' keys
                for x in range(cnt):
                    j = int(v["ret_idx"][b, g, x])
                    assert np.array_equal(kc[b, g, s + x], self.kn[bi, j, g]), (b, g, x, j)
                # ring: slot of token j holds its key; scores of scored tokens match
                for j in range(max(0, T - w), T):
                    slot = s + C + j % w
                    assert np.array_equal(kc[b, g, slot], self.kn[bi, j, g]), (b, g, j)
                    sc = v["ring_score"][b, g, j % w]
                    if s <= j < nu:
                        assert abs(sc - self.r_all[bi, g, j]) <= SCORE_TOL, (b, g, j, sc)
                    else:
                        assert np.isnan(sc), (b, g, j, sc)


def test_chunk_after_prefill():
    """B2 Hq8 Hkv2 D128 s4 w32 C16: prefill 200, a 40-token chunk (its first tokens leave
    the window within the chunk), a 7-token chunk, then 20 decode steps."""
    st = Stream(2, 8, 2, 128, 4, 32, 16, 280, seed=51, b2=0.05)
    st.prefill([200, 200])
    st.chunk(40)
    st.chunk(7)
    st.decode(20)


def test_chunk_from_short_history():
    """The cache still holds the whole history (3 tokens, sink 4): the chunk is laid out as
    the plain sequence; a second chunk then meets a cache that has lost tokens."""
    st = Stream(2, 4, 2, 64, 4, 8, 5, 120, seed=52, b2=0.1)
    st.prefill([3, 3])
    st.chunk(30)
    st.chunk(20)
    st.decode(10)


def test_chunk_mixed_positions():
    """Ragged prefill (100 and 5 tokens, w 32): one sequence in each layout; a 50-token
    chunk, a single-token chunk, decode."""
    st = Stream(2, 8, 2, 128, 4, 32, 16, 220, seed=53, b2=0.05)
    st.prefill([100, 5])
    st.chunk(50)
    st.chunk(1)
    st.decode(10)


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 8, 64), (16, 2, 128)])
def test_chunk_after_decode_steps(Hq, Hkv, D):
    """Decode steps first leave the segment out of token order (replacements in place);
    the chunk must sort it.  C 24 overflows (b2 small)."""
    st = Stream(1, Hq, Hkv, D, 2, 16, 24, 300, seed=54, b2=0.02)
    st.prefill([120])
    st.decode(37)
    st.chunk(64)
    st.decode(5)


def test_chunk_full_size():
    """B32, 4096-token prompt, Hq16 Hkv4 D128 s4 w512 C512 (the bench layer): a 504-token
    chunk, then 8 decode steps; sequences 0 and 21 checked, every 5th chunk row."""
    inp = synth.workload_inputs(4)
    wl = inp["workload"]
    st = Stream(wl.B, wl.Hq, wl.Hkv, wl.D, wl.sink, wl.window, wl.capacity,
                inputs=(inp["q"], inp["k"], inp["v"], inp["cnn"]), check_b=[0, 21], every=5)
    st.prefill([inp["T"]] * wl.B)
    st.chunk(504)
    st.decode(8)


@pytest.mark.parametrize("s,C", [(0, 12), (3, 0)])
def test_chunk_no_sink_or_no_segment(s, C):
    """No sink (the CNN's left padding is reached) or capacity 0 (no segment rows)."""
    st = Stream(2, 4, 2, 64, s, 16, C, 200, seed=55 + s, b2=0.05)
    st.prefill([60, 90])
    st.chunk(37)
    st.decode(6)
    st.chunk(25)


@pytest.mark.parametrize("seed", range(4))
def test_chunk_random_streams(seed):
    """Seeded random streams: ragged prefill lengths, then four operations, each a chunk
    or a run of decode steps, over random group size, head size, sink, window and
    capacity."""
    rng = np.random.default_rng(5000 + seed)
    G = [1, 2, 4, 8][seed]
    Hkv = int(rng.choice([1, 2]))
    D = int(rng.choice([64, 128]))
    s = int(rng.integers(0, 5))
    w = int(rng.integers(5, 32))
    C = int(rng.integers(0, 20))
    B = int(rng.integers(1, 3))
    lens = [int(rng.integers(1, 60)) for _ in range(B)]
    ops, total = [], max(lens)
    for _ in range(4):
        if rng.random() < 0.5:
            n = int(rng.integers(1, 80))
            ops.append(("chunk", n))
        else:
            n = int(rng.integers(1, 30))
            ops.append(("decode", n))
        total += n
    st = Stream(B, G * Hkv, Hkv, D, s, w, C, total + 1, seed=6000 + seed,
                b2=float(rng.choice([0.02, 0.3])))
    st.prefill(lens)
    for op, n in ops:
        getattr(st, op)(n)


def test_long_chunk():
    """A chunk of 300 tokens, far longer than w + C: most of it leaves the window inside the
    call and the segment overflows repeatedly (G1, D64)."""
    st = Stream(1, 2, 2, 64, 2, 24, 10, 500, seed=57, b2=0.02)
    st.prefill([90])
    st.chunk(300)
    st.decode(5)


@pytest.mark.parametrize("kind", ["flat", "level"])
def test_chunk_exact_ties(kind):
    """Scores that tie exactly (see tests/ties.py): after a prefill, chunks and decode steps
    the chunk queries' retained sets and the cache's segment must equal the oracle's
    exactly, ties resolved by the lower index (B2 Hq8 Hkv2 D128 s3 w24 C9, overflowing)."""
    from tests import ties
    make = ties.flat_case if kind == "flat" else ties.level_case
    st = Stream(2, 8, 2, 128, 3, 24, 9, inputs=make(77, 2, 420, 8, 2, 128), exact=True)
    st.prefill([150, 97])
    st.chunk(60)
    st.decode(31)
    st.chunk(120)
    st.decode(12)
