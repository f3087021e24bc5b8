"""lte_decode_step_static, the decode step that allocates nothing (needs an MI355X).

Its kernels are lte_decode_step's; only the split partials move from the caller's
workspace to the library's static device array.  So on the same cache and tokens
the two entry points must agree bit for bit, step after step, and both must match
the oracle like every decode step.  Two configurations run in a row on one device
-- the second with fewer (batch, KV head) pairs and a smaller cache, so it reuses a
smaller part of the array after the first call left it full -- and a third with
enough pairs that no split (and no partial) is used at all.
"""
import numpy as np
import pytest
import torch

import oracle
from learnable_kv_cache_amd import lte, synth
from tests.parity import MAX_ABS, MEAN_ABS

pytestmark = pytest.mark.gpu


def _run(B, T, n, Hq, Hkv, D, s, w, C, seed):
    q, k, v, cnn = synth.random_case(seed, B, T + n, Hq, Hkv, D, b2=0.05)
    layer = lte.Layer(lte.Config(B, Hq, Hkv, D, s, w, C))
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    dcnn = lte.CNN(cnn)
    ws = layer.alloc_workspace(T)
    # zeroed blobs: slots a cache never wrote compare equal too
    ca, cb = (torch.zeros(layer.cache_bytes(), dtype=torch.uint8, device="cuda") for _ in range(2))
    for cache in (ca, cb):
        layer.cache_init(cache)
    for cache in (ca, cb):
        layer.prefill(qd[:, :T].contiguous(), kd[:, :T].contiguous(), vd[:, :T].contiguous(),
                      cnn=dcnn, cache=cache, workspace=ws)
    qn, kn, vn = q.float().numpy(), k.float().numpy(), v.float().numpy()
    views = layer.cache_views(cb)
    G = Hq // Hkv
    out_b = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    for t in range(T, T + n):
        qt, kt, vt = qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous()
        oa = layer.decode_step(qt, kt, vt, dcnn, ca, ws)
        layer.decode_step_static(qt, kt, vt, dcnn, cb, out_b)
        torch.cuda.synchronize()
        assert torch.equal(oa, out_b), (t, float((oa.float() - out_b.float()).abs().max()))
        if t % 7 == 0 or t == T + n - 1:
            o_g = out_b.float().cpu().numpy()
            count = views["count"].cpu().numpy()
            ret_idx = views["ret_idx"].cpu().numpy()
            for b in range(B):
                for g in range(Hkv):
                    gset = set(ret_idx[b, g, :count[b, g]].tolist())
                    ref = oracle.attention_on_set(qn, kn, vn, s, w, b, t, g, gset)
                    d = np.abs(o_g[b, g * G:(g + 1) * G] - ref)
                    assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS, (t, b, g)
    assert torch.equal(torch.nan_to_num(ca.view(torch.float32), nan=-1.0),
                       torch.nan_to_num(cb.view(torch.float32), nan=-1.0))


def test_static_decode_matches_workspace_decode():
    # 4 (b, g) pairs, 1036-slot caches: 9 splits per pair, 36 partials of 8320 bytes
    _run(2, 600, 40, 32, 2, 128, 4, 512, 520, seed=71)
    # then fewer pairs and a smaller cache on the same device: 2 pairs x 3 splits
    _run(1, 300, 40, 8, 2, 128, 4, 200, 100, seed=72)
    # 128 pairs of 26 slots: one workgroup each, no partials
    _run(32, 64, 12, 8, 4, 64, 2, 16, 8, seed=73)
    # 128 pairs of 132 slots: 2 splits each, 256 partials
    _run(32, 150, 12, 16, 4, 128, 4, 64, 64, seed=74)
