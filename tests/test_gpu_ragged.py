"""Ragged batches (needs an MI355X): one prefill over prompts of different
lengths, padded to T rows, then decode steps in which every sequence advances
from its own position.

Each sequence must match the oracle run on that sequence alone (its first T_b
rows, then its own token stream), to the bars of the equal-length tests:
scores within 5e-4, keep sets equal outside the 1e-3 bands, outputs within
2e-2 max-abs / 1e-3 mean-abs of the oracle's attention on the realised sets.
Padding rows of q, k and v hold NaN, so a kernel that read one would put NaN
into some output; output rows at or past T_b must keep what they held.
"""
import numpy as np
import pytest
import torch

import oracle
from learnable_kv_cache_amd import lte, synth
from tests.parity import BAND, MAX_ABS, MEAN_ABS, gpu_ends, keep_set_mismatches, output_errors
from tests.test_gpu_decode import SCORE_TOL

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def _pad_nan(x, lens):
    x = x.clone()
    for b, n in enumerate(lens):
        x[b, n:] = float("nan")
    return x


def _check_prefill_seq(b, Tb, out, views, qn, kn, vn, s, w, C, Hkv, G, cnn=None, override=None):
    """Sequence b of a ragged prefill against the oracle on its first Tb rows."""
    sc = None if override is None else override[b:b + 1, :, :Tb]
    ref = oracle.prefill(qn[b:b + 1, :Tb], kn[b:b + 1, :Tb], vn[b:b + 1, :Tb], s, w, C, cnn=cnn,
                         scores=sc, rows=[])
    if override is None:
        err = float(np.abs(views["scores"][b, :, :Tb] - ref["scores"][0]).max())
        assert err <= SCORE_TOL, (b, err)
    ends_g = np.stack([gpu_ends(views["rank"][b, g, :Tb], views["thr"][b, g, :Tb], w, Tb)
                       for g in range(Hkv)])
    for g in range(Hkv):
        bad = keep_set_mismatches(ref["scores"][0, g], ref["ends"][0, g], ends_g[g], w, C)
        assert not bad, (b, g, bad[:5])
    o_ref = oracle.attention(qn[b:b + 1, :Tb], kn[b:b + 1, :Tb], vn[b:b + 1, :Tb], s, w,
                             ends_g[None], rows=list(range(Tb)))
    for g in range(Hkv):
        sl = slice(g * G, (g + 1) * G)
        mx, mean = output_errors(out[b, :Tb, sl], o_ref[0, :Tb, sl])
        assert mx <= MAX_ABS and mean <= MEAN_ABS, (b, g, mx, mean)
    assert np.all(out[b, Tb:] == SENTINEL), f"padding rows of sequence {b} were written"
    return ref


def test_ragged_prefill_then_decode():
    """B4 padded to T=300 (Hq8 Hkv2 D128 s4 w32 C16, CNN): lengths 300, 1 (shorter than the
    sink), 137 (mid-tile) and 45; then 40 decode steps per sequence from its own position,
    crossing deferred scoring batches and segment overflow."""
    B, T, n, Hq, Hkv, D, s, w, C = 4, 300, 40, 8, 2, 128, 4, 32, 16
    G = Hq // Hkv
    lens = [300, 1, 137, 45]
    q, k, v, cnn = synth.random_case(77, B, T + n, Hq, Hkv, D, b2=0.05)
    dev = torch.device("cuda")
    layer = lte.Layer(lte.Config(B, Hq, Hkv, D, s, w, C))
    ws = layer.alloc_workspace(T)
    cache = layer.alloc_cache()
    dcnn = lte.CNN(cnn)
    qp = _pad_nan(q[:, :T], lens).to(dev)
    kp = _pad_nan(k[:, :T], lens).to(dev)
    vp = _pad_nan(v[:, :T], lens).to(dev)
    out = torch.full_like(qp, SENTINEL)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    layer.prefill(qp, kp, vp, cnn=dcnn, cache=cache, workspace=ws, out=out, seq_lens=sl)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    views = {nm: x.cpu().numpy() for nm, x in layer.workspace_views(ws, T).items()}
    qn, kn, vn = q.float().numpy(), k.float().numpy(), v.float().numpy()
    ocs = []
    for b, Tb in enumerate(lens):
        ref = _check_prefill_seq(b, Tb, o, views, qn, kn, vn, s, w, C, Hkv, G, cnn=cnn)
        ocs.append(oracle.LayerCache.from_prefill(kn[b:b + 1, :Tb], vn[b:b + 1, :Tb],
                                                  ref["scores"], ref["ends"], s, w, C, cnn=cnn))
    r_all = oracle.cnn_scores(kn, vn, cnn["W1"], cnn["b1"], cnn["W2"], cnn["b2"])

    cv = layer.cache_views(cache)
    assert [int(x) for x in cv["pos"].cpu().numpy()[:, 0]] == lens
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    ar = torch.arange(B, device=dev)
    for step in range(n):
        pos = [Tb + step for Tb in lens]
        idx = torch.tensor(pos, device=dev)
        qt = qd[ar, idx].contiguous()
        kt = kd[ar, idx].contiguous()
        vt = vd[ar, idx].contiguous()
        o_t = layer.decode_step(qt, kt, vt, dcnn, cache, ws)
        for b in range(B):
            ocs[b].ingest(kn[b:b + 1, pos[b]], vn[b:b + 1, pos[b]])
        torch.cuda.synchronize()
        og = o_t.float().cpu().numpy()
        count = cv["count"].cpu().numpy()
        ret_idx = cv["ret_idx"].cpu().numpy()
        assert int(cv["flags"].cpu().numpy().max()) == 0, "a token left the window unscored"
        assert np.all(cv["pos"].cpu().numpy()[:, 0] == np.array(pos) + 1)
        for b in range(B):
            t = pos[b]
            for g in range(Hkv):
                gset = set(ret_idx[b, g, :count[b, g]].tolist())
                oset = set(ocs[b].retained_indices(0, g).tolist())
                cut = None
                if len(oset) == C:
                    cut = min(float(r_all[b, g, j]) for j in oset)
                for j in gset ^ oset:
                    rj = float(r_all[b, g, j])
                    ok = abs(rj - 0.5) <= BAND or (cut is not None and abs(rj - cut) <= BAND)
                    assert ok, (step, b, g, j, rj, cut)
                ref = oracle.attention_on_set(qn, kn, vn, s, w, b, t, g, gset)
                d = np.abs(og[b, g * G:(g + 1) * G] - ref)
                assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS, (step, b, g, d.max())


def test_ragged_prefill_with_score_override():
    """Explicit scores (B3 padded to T=520, Hq16 Hkv4 D64 s2 w64 C24): keep sets must equal the
    oracle's exactly (no CNN rounding), lengths 520, 64 (one window) and 333."""
    B, T, Hq, Hkv, D, s, w, C = 3, 520, 16, 4, 64, 2, 64, 24
    G = Hq // Hkv
    lens = [520, 64, 333]
    q, k, v, _ = synth.random_case(78, B, T, Hq, Hkv, D)
    rng = np.random.default_rng(78)
    scores = rng.uniform(0.0, 1.0, (B, Hkv, T)).astype(np.float32)
    ov = scores.copy()
    for b, Tb in enumerate(lens):
        ov[b, :, Tb:] = np.nan
    dev = torch.device("cuda")
    layer = lte.Layer(lte.Config(B, Hq, Hkv, D, s, w, C))
    ws = layer.alloc_workspace(T)
    cache = layer.alloc_cache()
    qp, kp, vp = (_pad_nan(x, lens).to(dev) for x in (q, k, v))
    out = torch.full_like(qp, SENTINEL)
    layer.prefill(qp, kp, vp, score_override=torch.from_numpy(ov).to(dev), cache=cache,
                  workspace=ws, out=out, seq_lens=torch.tensor(lens, dtype=torch.int32,
                                                               device=dev))
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    views = {nm: x.cpu().numpy() for nm, x in layer.workspace_views(ws, T).items()}
    qn, kn, vn = q.float().numpy(), k.float().numpy(), v.float().numpy()
    cv = layer.cache_views(cache)
    count = cv["count"].cpu().numpy()
    ret_idx = cv["ret_idx"].cpu().numpy()
    for b, Tb in enumerate(lens):
        ref = _check_prefill_seq(b, Tb, o, views, qn, kn, vn, s, w, C, Hkv, G, override=scores)
        for g in range(Hkv):
            ends_g = gpu_ends(views["rank"][b, g, :Tb], views["thr"][b, g, :Tb], w, Tb)
            assert np.array_equal(oracle.retained_set(ends_g, w, Tb - 1),
                                  oracle.retained_set(ref["ends"][0, g], w, Tb - 1)), (b, g)
            assert sorted(ret_idx[b, g, :count[b, g]].tolist()) == \
                oracle.retained_set(ref["ends"][0, g], w, Tb - 1).tolist(), (b, g)
