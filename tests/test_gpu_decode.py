"""Decode parity: the HIP cache stepped in lockstep with the oracle's explicit
cache (needs an MI355X).

Per step: the retained segment's membership must equal the oracle's except
for tokens whose oracle score is within 1e-3 of 0.5 or of the weakest
retained score of a full segment; the output must be within 2e-2 max-abs /
1e-3 mean-abs of the oracle's softmax over the GPU's realised visible set
(sink U retained segment U window); ring scores within 5e-4 of the oracle's;
no token may leave the window unscored (flags == 0).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from learnable_kv_cache_amd import lte, synth
from tests.parity import BAND, MAX_ABS, MEAN_ABS

pytestmark = pytest.mark.gpu

SCORE_TOL = 5e-4


def _attend_on_set(q_t, k, v, idx, G):
    """float64 softmax of q_t [Hq, D] over keys idx of one KV head's k, v [T, D]."""
    K = k[idx].astype(np.float64)
    V = v[idx].astype(np.float64)
    Q = q_t.astype(np.float64)
    logits = Q @ K.T / math.sqrt(Q.shape[-1])
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    return (p @ V) / p.sum(axis=1, keepdims=True)


def run_decode_parity(B, T, n, Hq, Hkv, D, s, w, C, q, k, v, cnn, check_b=None, every=1):
    """Prefill T tokens, then n decode steps; compare with the oracle on batches check_b."""
    check_b = list(range(B)) if check_b is None else check_b
    G = Hq // Hkv
    layer = lte.Layer(lte.Config(B, Hq, Hkv, D, s, w, C))
    dev = torch.device("cuda")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    dcnn = lte.CNN(cnn)
    ws = layer.alloc_workspace(T)
    cache = layer.alloc_cache()
    layer.prefill(qd[:, :T].contiguous(), kd[:, :T].contiguous(), vd[:, :T].contiguous(),
                  cnn=dcnn, cache=cache, workspace=ws)
    views = layer.cache_views(cache)

    qn = q.float().numpy()[check_b]
    kn = k.float().numpy()[check_b]
    vn = v.float().numpy()[check_b]
    r_all = oracle.cnn_scores(kn, vn, cnn["W1"], cnn["b1"], cnn["W2"], cnn["b2"])
    pre = oracle.prefill(qn[:, :T], kn[:, :T], vn[:, :T], s, w, C, cnn=cnn, rows=[])
    oc = oracle.LayerCache.from_prefill(kn[:, :T], vn[:, :T], pre["scores"], pre["ends"], s, w,
                                        C, cnn=cnn)
    worst = (0.0, 0.0)
    for t in range(T, T + n):
        o_t = layer.decode_step(qd[:, t].contiguous(), kd[:, t].contiguous(),
                                vd[:, t].contiguous(), dcnn, cache, ws)
        oc.ingest(kn[:, t], vn[:, t])
        if (t - T) % every != 0 and t != T + n - 1:
            continue
        torch.cuda.synchronize()
        o_g = o_t.float().cpu().numpy()
        count = views["count"].cpu().numpy()
        ret_idx = views["ret_idx"].cpu().numpy()
        assert int(views["flags"].cpu().numpy().max()) == 0, "a token left the window unscored"
        assert np.all(views["pos"].cpu().numpy() == t + 1)
        ring_sc = views["ring_score"].cpu().numpy()
        for bi, b in enumerate(check_b):
            for g in range(Hkv):
                gset = set(ret_idx[b, g, :count[b, g]].tolist())
                assert len(gset) == count[b, g] <= C
                oset = set(oc.retained_indices(bi, g).tolist())
                cut = None
                if C > 0 and len(oset) == C:
                    cut = min(float(r_all[bi, g, j]) for j in oset)
                for j in gset ^ oset:
                    rj = float(r_all[bi, g, j])
                    ok = abs(rj - 0.5) <= BAND or (cut is not None and abs(rj - cut) <= BAND)
                    assert ok, (t, b, g, j, rj, cut)
                # ring scores that are set must match the oracle's scores
                for slot in range(w):
                    x = t - ((t - slot) % w)
                    if x >= s and not np.isnan(ring_sc[b, g, slot]):
                        assert abs(ring_sc[b, g, slot] - r_all[bi, g, x]) <= SCORE_TOL, (t, x)
                # output on the GPU's realised visible set
                sink = list(range(min(s, t + 1)))
                window = list(range(max(0, t - w + 1), t + 1))
                idx = np.array(sorted(set(sink) | set(window) | gset), np.int64)
                assert len(idx) <= s + w + C
                ref = _attend_on_set(qn[bi, t, g * G:(g + 1) * G], kn[bi, :, g], vn[bi, :, g],
                                     idx, G)
                d = np.abs(o_g[b, g * G:(g + 1) * G] - ref)
                worst = (max(worst[0], float(d.max())), max(worst[1], float(d.mean())))
                assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS, (t, b, g, d.max(), d.mean())
    return worst


@pytest.mark.parametrize("T,n,s,w,C,b2", [
    (40, 40, 2, 8, 4, 0.02),      # overflow of the capped segment, deferred scoring fires
    (12, 50, 4, 6, 3, 0.5),       # short prompt
    (3, 30, 4, 5, 2, 0.0),        # prompt shorter than the sink
    (25, 40, 0, 7, 5, 0.1),       # no sink: the CNN's left padding is reached
    (30, 30, 1, 5, 0, 1.0),       # C = 0
])
def test_small_decode(T, n, s, w, C, b2):
    B, Hq, Hkv, D = 2, 4, 2, 64
    q, k, v, cnn = synth.random_case(31 + T, B, T + n, Hq, Hkv, D, b2=b2)
    run_decode_parity(B, T, n, Hq, Hkv, D, s, w, C, q, k, v, cnn)


def test_decode_d128_gqa8():
    B, T, n, Hq, Hkv, D, s, w, C = 1, 150, 120, 16, 2, 128, 4, 32, 16
    q, k, v, cnn = synth.random_case(9, B, T + n, Hq, Hkv, D, b2=0.05)
    run_decode_parity(B, T, n, Hq, Hkv, D, s, w, C, q, k, v, cnn)


def test_decode_split_workgroups():
    """Few (batch, KV head) pairs and a 304-slot cache: each pair's rows are split over three
    workgroups merged by the last to finish; the segment overflows and a deferred batch
    fires at t = 495."""
    B, T, n, Hq, Hkv, D, s, w, C = 1, 300, 220, 8, 2, 128, 4, 200, 100
    q, k, v, cnn = synth.random_case(17, B, T + n, Hq, Hkv, D, b2=0.05)
    run_decode_parity(B, T, n, Hq, Hkv, D, s, w, C, q, k, v, cnn, every=3)


def test_decode_full_size():
    """Decode at B32, 4096-token prompt, Hq16 Hkv4 D128 s4 w512 C512, 512 steps (one deferred
    scoring batch fires at t = 4603); batches 0 and 21 checked against the oracle."""
    inp = synth.workload_inputs(4)
    wl = inp["workload"]
    run_decode_parity(wl.B, inp["T"], inp["steps"], wl.Hq, wl.Hkv, wl.D, wl.sink, wl.window,
                      wl.capacity, inp["q"], inp["k"], inp["v"], inp["cnn"], check_b=[0, 21],
                      every=7)


@pytest.mark.parametrize("seed", range(6))
def test_random_shape_decode(seed):
    """Seeded random decode configurations: group size, head size, sink, window,
    capacity (overflowing or not), prompt length and step count."""
    rng = np.random.default_rng(2000 + seed)
    G = [1, 2, 4, 8, 16, 4][seed]
    Hkv = int(rng.choice([1, 2]))
    D = int(rng.choice([64, 128]))
    s = int(rng.integers(0, 6))
    w = int(rng.integers(5, 40))
    C = int(rng.integers(1, 24))
    T = int(rng.integers(1, 90))
    n = int(rng.integers(20, 70))
    b2 = float(rng.choice([0.0, 0.05, 0.5]))
    B = int(rng.integers(1, 3))
    q, k, v, cnn = synth.random_case(500 + seed, B, T + n, G * Hkv, Hkv, D, b2=b2)
    run_decode_parity(B, T, n, G * Hkv, Hkv, D, s, w, C, q, k, v, cnn)


@pytest.mark.parametrize("rho", [0.05, 0.2, 0.5])
def test_long_context_decode(rho):
    """B4, 32768-token prompt, Hq32 Hkv8 D128 s4 w1024 C2048, 256 decode steps, with b2 set
    from the bias-free logits so that a fraction rho of the tokens is kept (20% and 50%
    overflow C); batch 0 checked against the oracle."""
    wl = synth.WORKLOADS[5]
    T, n = wl.T, wl.decode_steps
    q, k, v = synth.make_qkv(wl.B, T + n, wl.Hq, wl.Hkv, wl.D, wl.seed)
    cnn0 = synth.make_cnn(wl.Hkv, wl.D, wl.seed + 100, "zero")
    z0 = oracle.cnn_logits(k[:1, :T].float().numpy(), v[:1, :T].float().numpy(), cnn0["W1"],
                           cnn0["b1"], cnn0["W2"], cnn0["b2"])
    b2 = -float(np.quantile(z0[:, :, wl.sink:], 1.0 - rho))
    cnn = dict(cnn0, b2=np.full((wl.Hkv,), b2, np.float32))
    run_decode_parity(wl.B, T, n, wl.Hq, wl.Hkv, wl.D, wl.sink, wl.window, wl.capacity, q, k,
                      v, cnn, check_b=[0], every=5)


def test_fused_step_equals_evict_then_attend():
    """lte_decode_step (one fused kernel) == lte_score_evict then lte_decode_attend, bitwise,
    including across a deferred-scoring step and segment overflow."""
    B, T, n, Hq, Hkv, D, s, w, C = 2, 60, 40, 8, 2, 128, 2, 9, 5
    q, k, v, cnn = synth.random_case(21, B, T + n, Hq, Hkv, D, b2=0.05)
    layer = lte.Layer(lte.Config(B, Hq, Hkv, D, s, w, C))
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    dcnn = lte.CNN(cnn)
    ws = layer.alloc_workspace(T)
    ca, cb = layer.alloc_cache(), layer.alloc_cache()
    for cache in (ca, cb):
        layer.prefill(qd[:, :T].contiguous(), kd[:, :T].contiguous(), vd[:, :T].contiguous(),
                      cnn=dcnn, cache=cache, workspace=ws)
    for t in range(T, T + n):
        qt, kt, vt = qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous()
        oa = layer.decode_step(qt, kt, vt, dcnn, ca, ws)
        layer.score_evict(kt, vt, dcnn, cb)
        ob = layer.decode_attend(qt, cb, ws)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), t
    va, vb = layer.cache_views(ca), layer.cache_views(cb)
    for name in ("ret_idx", "ret_score", "count", "pos", "next_unscored", "flags", "weak",
                 "nx_slot", "nx_score"):
        assert torch.equal(va[name], vb[name]), name
    # ring scores: NaN where unscored on both sides
    assert torch.equal(torch.nan_to_num(va["ring_score"], nan=-1.0),
                       torch.nan_to_num(vb["ring_score"], nan=-1.0))


def test_decode_from_empty_cache():
    """No prefill: a freshly initialised cache stepped from pos 0 (sink, ring and segment
    filled by decode alone; deferred batches fire from the first tokens on)."""
    B, n, Hq, Hkv, D, s, w, C = 2, 60, 4, 2, 64, 3, 8, 4
    q, k, v, cnn = synth.random_case(41, B, n, Hq, Hkv, D, b2=0.05)
    G = Hq // Hkv
    layer = lte.Layer(lte.Config(B, Hq, Hkv, D, s, w, C))
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    dcnn = lte.CNN(cnn)
    ws = layer.alloc_workspace(0)
    cache = layer.alloc_cache()
    views = layer.cache_views(cache)
    qn, kn, vn = q.float().numpy(), k.float().numpy(), v.float().numpy()
    r_all = oracle.cnn_scores(kn, vn, cnn["W1"], cnn["b1"], cnn["W2"], cnn["b2"])
    oc = oracle.LayerCache(B, Hkv, D, s, w, C, cnn=cnn)
    for t in range(n):
        o_t = layer.decode_step(qd[:, t].contiguous(), kd[:, t].contiguous(),
                                vd[:, t].contiguous(), dcnn, cache, ws)
        oc.ingest(kn[:, t], vn[:, t])
        torch.cuda.synchronize()
        assert np.all(views["pos"].cpu().numpy() == t + 1)
        assert int(views["flags"].cpu().numpy().max()) == 0
        o_g = o_t.float().cpu().numpy()
        count = views["count"].cpu().numpy()
        ret_idx = views["ret_idx"].cpu().numpy()
        for b in range(B):
            for g in range(Hkv):
                gset = set(ret_idx[b, g, :count[b, g]].tolist())
                oset = set(oc.retained_indices(b, g).tolist())
                cut = min(float(r_all[b, g, j]) for j in oset) if len(oset) == C else None
                for j in gset ^ oset:
                    rj = float(r_all[b, g, j])
                    assert abs(rj - 0.5) <= BAND or (cut is not None and abs(rj - cut) <= BAND)
                idx = np.array(sorted(set(range(min(s, t + 1))) | set(range(max(0, t - w + 1), t + 1))
                                      | gset), np.int64)
                ref = _attend_on_set(qn[b, t, g * G:(g + 1) * G], kn[b, :, g], vn[b, :, g], idx, G)
                d = np.abs(o_g[b, g * G:(g + 1) * G] - ref)
                # over the first few keys the output is not averaged down to a small
                # magnitude, so its bf16 rounding (unit roundoff 2^-8, on the output and
                # on the probabilities) adds a term proportional to the output itself
                mean_tol = MEAN_ABS + 2.0 ** -8 * float(np.abs(ref).mean())
                assert d.max() <= MAX_ABS and d.mean() <= mean_tol, (t, b, g, d.mean())
