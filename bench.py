"""Benchmark of the LTE sparse-attention layer on one MI355X.

One step = one pass of the whole hot path on synthetic inputs:
  * prefill of a B=32 x 4096-token bf16 prompt (Hq16 Hkv4 D128, sink 4, window
    512, capacity 512, scoring CNN with per-head b2 ~ U(-2, 1)): score, select,
    attend, build the cache;
  * 512 decode steps on that cache shape, each step run on L independent layer
    caches in rotation (L chosen so the caches exceed twice the 256 MB
    Infinity Cache, like consecutive layers of a model), replayed from a HIP
    graph.
Reported: prefill tokens/s (``value``) and decode microseconds per layer-step,
each with the roofline of its dominant kernel, next to the CPU oracle timed on
this host.

Beside it, the same engine as the two comparators of the LTE paper's Figure 4
(sink + sliding-window attention with no retained segment, and full causal
attention as a window covering the whole sequence), timed on the same inputs,
a chunked prefill of the next 512 tokens onto the prompt's cache, the
hybrid's linear-attention layer (B32, 4096 tokens, 16 heads of 128): chunked
prefill and decode steps, Figure 4(a)'s attention kernel with an artificial KV
cache (B8, 10% retention), and the long-context shape (B4, 32768-token prompt,
Hq32 Hkv8, w1024 C2048) at 5%, 20% and 50% retention: prefill and decode.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps N]
                       [--no-cpu-baseline] [--no-decode] [--no-comparators]
                       [--no-chunk] [--no-linear] [--no-artificial] [--no-long]
                       [--copy-calibration MIB]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LTE layer prefill tokens/s and decode µs/step, B=32, 4K prompt; % of roofline"
PEAK_BF16_FLOPS = 2.5e15      # MI355X dense bf16 MFMA
PEAK_HBM_BPS = 8.0e12         # MI355X HBM3E
MALL_BYTES = 256 * 2**20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


# A spin kernel queued ahead of a timed region's first event lets the host
# enqueue every launch of the region while the GPU waits, so the events time the
# GPU's work, not the host's launch latency after an idle queue.
GATE_CYCLES = 400_000          # about 170 us of the GPU clock counter


def gate():
    import torch
    torch.cuda._sleep(GATE_CYCLES)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=512)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-comparators", action="store_true")
    ap.add_argument("--no-chunk", action="store_true")
    ap.add_argument("--no-linear", action="store_true")
    ap.add_argument("--no-artificial", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="sequences the oracle runs for the CPU baseline (0: one per core)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (counter calibration)")
    return ap.parse_args()


def copy_calibration(mib: int):
    """Five device-to-device copies of a known size: the reference dispatches that
    scale the FETCH_SIZE / WRITE_SIZE counters of a profiled kernel to bytes."""
    import torch
    n = mib * 2**20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "copies": 5}), flush=True)


# ---------------------------------------------------------------------------
# algorithmic work from the realised masks
# ---------------------------------------------------------------------------

def visible_counts(rank: np.ndarray, T: int, s: int, w: int, C: int) -> np.ndarray:
    """|V(i)| per (b, g, i) from the GPU's candidate ranks.

    |R_i| = min(C, N(i - w)) with N(m) the number of candidates <= m (R_i is the
    top-C of those); the sink adds the tokens [0, s) that are not in the window.
    """
    cand = (rank != 0x7FFFFFFF)
    N = np.cumsum(cand, axis=-1)                             # N(m)
    i = np.arange(T)
    Rn = np.zeros(rank.shape, np.int64)
    m = i - w
    ok = m >= 0
    Rn[..., ok] = np.minimum(C, N[..., m[ok]])
    win = np.minimum(i + 1, w)
    sink_extra = np.maximum(0, np.minimum(s, i + 1) - np.maximum(0, i - w + 1))
    return Rn + (win + sink_extra)[None, None, :]


def kernel_sha(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(name: str, src: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(name)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != kernel_sha(src):
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on this host's cores
# ---------------------------------------------------------------------------

def _oracle_worker(args):
    import threadpoolctl
    with threadpoolctl.threadpool_limits(1):
        import oracle
        q, k, v, cnn, s, w, C = args
        t0 = time.perf_counter()
        oracle.prefill(q, k, v, s, w, C, cnn=cnn)
        return time.perf_counter() - t0


def _oracle_decode_worker(args):
    import threadpoolctl
    with threadpoolctl.threadpool_limits(1):
        import oracle
        q, k, v, cnn, s, w, C, T, n = args
        pre = oracle.prefill(q[:, :T], k[:, :T], v[:, :T], s, w, C, cnn=cnn, rows=[])
        cache = oracle.LayerCache.from_prefill(k[:, :T], v[:, :T], pre["scores"], pre["ends"],
                                               s, w, C, cnn=cnn)
        t0 = time.perf_counter()
        for t in range(T, T + n):
            cache.step(q[:, t], k[:, t], v[:, t])
        return (time.perf_counter() - t0) / n


def cpu_baseline(inp, wl, T, sample):
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(cores, 16))
    nseq = sample if sample > 0 else workers
    nseq = min(nseq, wl.B)
    nseq0 = min(max(sample, workers), wl.B)
    q = inp["q"][:nseq0].float().numpy()
    k = inp["k"][:nseq0].float().numpy()
    v = inp["v"][:nseq0].float().numpy()
    cnn = inp["cnn"]
    jobs = [(q[b:b + 1, :T], k[b:b + 1, :T], v[b:b + 1, :T], cnn, wl.sink, wl.window,
             wl.capacity) for b in range(nseq)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(min(workers, nseq)) as pool:
        pool.map(_oracle_worker, jobs)
    wall = time.perf_counter() - t0
    used = min(workers, nseq)
    # decode: a few steps of one sequence per worker
    ndec = 8
    djobs = [(q[b:b + 1], k[b:b + 1], v[b:b + 1], cnn, wl.sink, wl.window, wl.capacity, T, ndec)
             for b in range(used)]
    with ctx.Pool(used) as pool:
        per_seq_step = pool.map(_oracle_decode_worker, djobs)
    # one decode step of the full batch, spread over the same workers
    dec_us = float(np.mean(per_seq_step)) * math.ceil(wl.B / used) * 1e6
    return {
        "value": nseq * T / wall, "unit": "tokens/s", "cores": used, "kind": "oracle",
        "host_cores": cores,
        "sample": f"prefill of {nseq} of the {wl.B} sequences (all {wl.Hkv} KV heads, "
                  f"T={T}), one process per sequence; decode: {ndec} steps of {used} sequences, "
                  f"scaled to the full batch",
        "decode_us_per_step": dec_us,
        "cpu": _cpu_model(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------------------
# Figure 4 comparators: the same engine with no retained segment
# ---------------------------------------------------------------------------

def _graph_us_per_step(layer, caches, qs, ks, vs, cnn, ws, reps=3):
    """Decode microseconds per layer-step of a HIP-graph replay over caches."""
    import torch
    out = torch.empty_like(qs[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in caches:
            layer.decode_step(qs[0], ks[0], vs[0], cnn, c, ws, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(len(qs)):
            for c in caches:
                layer.decode_step(qs[t], ks[t], vs[t], cnn, c, ws, out)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gate()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e3 / (len(qs) * len(caches)))
    return best


def comparators(inp, wl, T, dev, ndec=64):
    """Sink + SWA (capacity 0) and full causal attention (window = T + ndec, capacity 0)
    run through the same kernels on the same q, k, v: prefill attention time and
    decode time per layer-step (caches rotated past the last-level cache)."""
    import torch
    from learnable_kv_cache_amd import lte
    B, s = wl.B, wl.sink
    G = wl.Hq // wl.Hkv
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    qp, kp, vp = (x[:, :T].contiguous() for x in (q, k, v))
    dq = [q[:, T + t].contiguous() for t in range(ndec)]
    dk = [k[:, T + t].contiguous() for t in range(ndec)]
    dv = [v[:, T + t].contiguous() for t in range(ndec)]
    cnn = lte.CNN(inp["cnn"], dev)
    zero_scores = torch.zeros((B, wl.Hkv, T), dtype=torch.float32, device=dev)
    res = {}
    for name, w in (("swa", wl.window), ("full", T + ndec)):
        layer = lte.Layer(lte.Config(B, wl.Hq, wl.Hkv, wl.D, s, w, 0))
        ws = layer.alloc_workspace(T, dev)
        out = torch.empty_like(qp)
        cache = layer.alloc_cache(dev)
        layer.prefill(qp, kp, vp, score_override=zero_scores, cache=cache, workspace=ws, out=out)
        times = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            gate()
            e0.record()
            layer.prefill_attend(qp, kp, vp, ws, out)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        att_ms = float(np.median(times))
        i = np.arange(T, dtype=np.float64)
        # window keys plus the sink tokens that lie below the window
        keys = np.minimum(i + 1, w) + np.minimum(np.minimum(s, i + 1), np.maximum(0, i - w + 1))
        flops = 4.0 * wl.D * G * B * wl.Hkv * float(keys.sum())
        L = math.ceil(2 * MALL_BYTES / layer.cache_bytes()) + 1
        caches = [cache] + [cache.clone() for _ in range(L - 1)]
        us = _graph_us_per_step(layer, caches, dq, dk, dv, cnn, ws)
        nvis = min(T + ndec // 2, w) + (s if w < T else 0)
        step_bytes = B * wl.Hkv * nvis * wl.D * 2 * 2 + 4 * B * wl.Hq * wl.D
        res[name] = {"window": w, "capacity": 0, "prefill_attend_ms": att_ms,
                     "prefill_attend_tflops": flops / (att_ms * 1e-3) / 1e12,
                     "decode_us_per_step": us, "decode_layers_rotated": L,
                     "decode_GBps": step_bytes / (us * 1e-6) / 1e9}
        del caches, cache, ws, out
        torch.cuda.empty_cache()
    return res


def linear_layer(dev, B=32, T=4096, H=16, D=128, ndec=64):
    """The hybrid's linear-attention layer on the same batch and prompt: chunked prefill
    (timed by events) and decode steps on the state (replayed from a graph).  Algorithmic
    flops of the prefill per head and 64-token chunk: the causal half of q.k and of p.v
    (L(L+1)/2 D multiply-adds each), q S (L D^2) and the state update (L D^2)."""
    import torch
    from learnable_kv_cache_amd import lte, synth
    q, k, v, log_a = (x.to(dev) for x in synth.linear_inputs(11, B, T + ndec, H, D))
    qp, kp, vp, ap = (x[:, :T].contiguous() for x in (q, k, v, log_a))
    layer = lte.LinearLayer(B, H, D)
    state = layer.alloc_state(dev)
    out = torch.empty_like(qp)
    layer.prefill(qp, kp, vp, ap, state_out=state, out=out)
    times = []
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gate()
        e0.record()
        layer.prefill(qp, kp, vp, ap, state_out=state, out=out)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times[1:]))
    L = 64
    nch = T / L
    flops = 2.0 * B * H * nch * (2 * (L * (L + 1) / 2) * D + 2 * L * D * D)
    pre_bytes = 4.0 * B * T * H * D * 2 + B * T * H * 4 + B * H * D * D * 4
    dq, dk, dv, da = ([x[:, T + t].contiguous() for t in range(ndec)] for x in (q, k, v, log_a))
    dout = torch.empty_like(dq[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.decode_step(dq[0], dk[0], dv[0], da[0], state, dout)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(ndec):
            layer.decode_step(dq[t], dk[t], dv[t], da[t], state, dout)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gate()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / ndec
    step_bytes = 2.0 * B * H * D * D * 4 + 4 * B * H * D * 2 + B * H * 4
    return {"shape": {"B": B, "T": T, "H": H, "D": D},
            "prefill_ms": ms, "prefill_tokens_per_s": B * T / (ms * 1e-3),
            # the prefill streams q, k, v and writes o (4 B T H D bf16) plus log a and the
            # final state: at 8 TB/s that takes longer than its flops at 2.5 PFLOP/s, so
            # HBM bounds it; the MFMA fraction is kept beside it
            "prefill_roofline": {"bound": "hbm", "achieved": pre_bytes / (ms * 1e-3) / 1e9,
                                 "peak": PEAK_HBM_BPS / 1e9, "unit": "GB/s",
                                 "frac": pre_bytes / (ms * 1e-3) / PEAK_HBM_BPS,
                                 "bytes_per_launch": pre_bytes,
                                 "mfma_tflops": flops / (ms * 1e-3) / 1e12,
                                 "mfma_frac": flops / (ms * 1e-3) / PEAK_BF16_FLOPS},
            "decode_us_per_step": us,
            "decode_roofline": {"bound": "hbm", "achieved": step_bytes / (us * 1e-6) / 1e9,
                                "peak": PEAK_HBM_BPS / 1e9, "unit": "GB/s",
                                "frac": step_bytes / (us * 1e-6) / PEAK_HBM_BPS,
                                "bytes_per_step": step_bytes}}


def _attend_ms(layer, q, k, v, ws, out, reps=7):
    """Median of event-timed lte_prefill_attend launches (each behind the gate)."""
    import torch
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gate()
        e0.record()
        layer.prefill_attend(q, k, v, ws, out)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return float(np.median(times[1:]))


def artificial_cache(dev):
    """Figure 4(a)'s kernel with an artificial KV cache: B8 T4096 Hq16 Hkv4 D128 s4 w512
    C512, each out-of-window token retained with probability 0.1 (given as scores), the
    attention alone; its MFMA fraction counted from the realised ranks."""
    import torch
    from learnable_kv_cache_amd import lte, synth
    inp = synth.workload_inputs(2)
    wl = inp["workload"]
    B, T = wl.B, inp["T"]
    layer = lte.Layer(lte.Config(B, wl.Hq, wl.Hkv, wl.D, wl.sink, wl.window, wl.capacity))
    q, k, v = (inp[x].to(dev).contiguous() for x in ("q", "k", "v"))
    ws = layer.alloc_workspace(T, dev)
    out = torch.empty_like(q)
    layer.prefill_select(T, ws, torch.as_tensor(inp["override"]).to(dev))
    ms = _attend_ms(layer, q, k, v, ws, out)
    rank = layer.workspace_views(ws, T)["rank"].cpu().numpy()
    vis = visible_counts(rank, T, wl.sink, wl.window, wl.capacity)
    flops = 4.0 * wl.D * (wl.Hq // wl.Hkv) * float(vis.sum())
    return {"workload": f"attention-artificial-cache-b{B}-t{T} (10% Bernoulli retention)",
            "attend_ms": ms, "tokens_per_s": B * T / (ms * 1e-3),
            "mean_visible_keys_per_row": float(vis.mean()),
            "roofline": {"bound": "mfma", "kernel": "attend_prefill_kernel<128,4>",
                         "achieved": flops / (ms * 1e-3) / 1e12, "peak": PEAK_BF16_FLOPS / 1e12,
                         "unit": "TFLOP/s", "frac": flops / (ms * 1e-3) / PEAK_BF16_FLOPS,
                         "flops_per_launch": flops}}


def long_context(dev, rhos=(0.05, 0.2, 0.5)):
    """The long-context stress shape: B4, 32768-token prompt, Hq32 Hkv8 D128 s4 w1024 C2048,
    with one output bias per run chosen so that a fraction rho of the prompt's tokens
    scores above 1/2 (from the quantile of the bias-free scores, computed by the library's
    own scorer); per rho the whole prefill (tokens/s, the attention's MFMA fraction) and
    256 decode steps over L rotating layer caches (us per layer-step, HBM fraction)."""
    import torch
    from learnable_kv_cache_amd import lte, synth
    inp = synth.workload_inputs(5)
    wl = inp["workload"]
    B, T, ndec = wl.B, inp["T"], inp["steps"]
    s, w, C, G = wl.sink, wl.window, wl.capacity, wl.Hq // wl.Hkv
    layer = lte.Layer(lte.Config(B, wl.Hq, wl.Hkv, wl.D, s, w, C))
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    qp, kp, vp = (x[:, :T].contiguous() for x in (q, k, v))
    dq = [q[:, T + t].contiguous() for t in range(ndec)]
    dk = [k[:, T + t].contiguous() for t in range(ndec)]
    dv = [v[:, T + t].contiguous() for t in range(ndec)]
    ws = layer.alloc_workspace(T, dev)
    out = torch.empty_like(qp)
    layer.prefill_score(kp, vp, lte.CNN(inp["cnn"], dev), ws)      # b2 = 0
    r0 = layer.workspace_views(ws, T)["scores"][:, :, s:].double().flatten()
    cache_bytes = layer.cache_bytes()
    L = math.ceil(2 * MALL_BYTES / cache_bytes) + 1
    caches = [layer.alloc_cache(dev) for _ in range(L)]
    res = {"workload": f"long-context-b{B}-t{T}", "B": B, "T": T, "Hq": wl.Hq, "Hkv": wl.Hkv,
           "D": wl.D, "sink": s, "window": w, "capacity": C, "decode_steps": ndec,
           "decode_layers": L, "runs": []}
    for rho in rhos:
        rq = float(torch.quantile(r0[:: max(1, r0.numel() // 4_000_000)], 1.0 - rho))
        b2 = -math.log(rq / (1.0 - rq))
        cnn = lte.CNN(dict(inp["cnn"], b2=np.full((wl.Hkv,), b2, np.float32)), dev)
        times = []
        for _ in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            gate()
            e0.record()
            layer.prefill(qp, kp, vp, cnn=cnn, cache=caches[0], workspace=ws, out=out)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        pf_ms = float(np.median(times[1:]))
        att_ms = _attend_ms(layer, qp, kp, vp, ws, out, reps=4)
        views = layer.workspace_views(ws, T)
        rank = views["rank"].cpu().numpy()
        vis = visible_counts(rank, T, s, w, C)
        flops = 4.0 * wl.D * G * float(vis.sum())
        rate = float(views["ncand"].double().mean()) / (T - s)
        # decode: every cache from this prefill, then a graph of ndec steps x L caches
        for c in caches[1:]:
            c.copy_(caches[0])
        seed = caches[0].clone()
        dout = torch.empty_like(dq[0])
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in caches:
                layer.decode_step(dq[0], dk[0], dv[0], cnn, c, ws, dout)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for t in range(ndec):
                for c in caches:
                    layer.decode_step(dq[t], dk[t], dv[t], cnn, c, ws, dout)
        flush = torch.empty(2 * MALL_BYTES, dtype=torch.uint8, device=dev)
        us = []
        for _ in range(3):
            for c in caches:
                c.copy_(seed)
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            us.append(e0.elapsed_time(e1) * 1e3 / (ndec * L))
        us_step = float(np.median(us))
        cnt = layer.cache_views(caches[-1])["count"].double().mean().item()
        step_bytes = (B * wl.Hkv * (s + cnt + w) * wl.D * 2 * 2 + 2 * B * wl.Hq * wl.D * 2
                      + 2 * B * wl.Hkv * wl.D * 2 + B * wl.Hkv * C * 4)
        res["runs"].append({
            "rho": rho, "b2": b2, "realised_candidate_rate": rate,
            "prefill_ms": pf_ms, "prefill_tokens_per_s": B * T / (pf_ms * 1e-3),
            "attend_ms": att_ms,
            "attend_roofline": {"bound": "mfma", "achieved": flops / (att_ms * 1e-3) / 1e12,
                                "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                                "frac": flops / (att_ms * 1e-3) / PEAK_BF16_FLOPS},
            "decode_us_per_step": us_step, "mean_segment_count": cnt,
            "decode_roofline": {"bound": "hbm", "achieved": step_bytes / (us_step * 1e-6) / 1e9,
                                "peak": PEAK_HBM_BPS / 1e9, "unit": "GB/s",
                                "frac": step_bytes / (us_step * 1e-6) / PEAK_HBM_BPS,
                                "bytes_per_step": step_bytes}})
        del g, flush, seed
        torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(batch and KV-head sharding need no communication and are described in the "
              "design notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch
    from learnable_kv_cache_amd import lte, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ndec = args.decode_steps
    inp = synth.workload_inputs(4, decode_steps=ndec)
    wl = inp["workload"]
    B, T = wl.B, inp["T"]
    cfg = lte.Config(B, wl.Hq, wl.Hkv, wl.D, wl.sink, wl.window, wl.capacity)
    layer = lte.Layer(cfg)
    q = inp["q"].to(dev)
    k = inp["k"].to(dev)
    v = inp["v"].to(dev)
    qp, kp, vp = (x[:, :T].contiguous() for x in (q, k, v))
    dq = [q[:, T + t].contiguous() for t in range(ndec)]
    dk = [k[:, T + t].contiguous() for t in range(ndec)]
    dv = [v[:, T + t].contiguous() for t in range(ndec)]
    cnn = lte.CNN(inp["cnn"], dev)
    ws = layer.alloc_workspace(T, dev)
    out = torch.empty_like(qp)
    cache0 = layer.alloc_cache(dev)
    cache_bytes = layer.cache_bytes()
    L = math.ceil(2 * MALL_BYTES / cache_bytes) + 1
    stream = torch.cuda.current_stream()

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]

    # The cache build needs only select's outputs and k/v, and writes only the
    # cache: it runs on a second stream beside the attention, which leaves LDS,
    # registers and HBM bandwidth to spare (the ABI allows this pairing).  Its
    # background form copies the rows on a few workgroups, so that the copy does
    # not crowd the attention's latency-bound phases with a burst of traffic.
    side_stream = torch.cuda.Stream()

    # Instrumented, the prefill records events between its stages (the per-stage times);
    # otherwise only at its ends (the prefill time), since each timing event adds a
    # few microseconds to the stream.
    def prefill_staged(instrumented=True):
        gate()
        ev[0].record(stream)
        layer.prefill_score(kp, vp, cnn, ws)
        if instrumented:
            ev[1].record(stream)
        layer.prefill_select(T, ws)
        if instrumented:
            ev[2].record(stream)
            side_stream.wait_event(ev[2])
        else:
            side_stream.wait_stream(stream)
        with torch.cuda.stream(side_stream):
            layer.prefill_build_cache_background(kp, vp, ws, cache0)
        layer.prefill_attend(qp, kp, vp, ws, out)
        if instrumented:
            ev[3].record(stream)
        stream.wait_stream(side_stream)
        ev[4].record(stream)

    prefill_staged()
    torch.cuda.synchronize()

    caches = [cache0] + [cache0.clone() for _ in range(L - 1)] if not args.no_decode else []
    dec_out = torch.empty_like(dq[0])

    def decode_loop(cs):
        for t in range(ndec):
            for c in cs:
                layer.decode_step(dq[t], dk[t], dv[t], cnn, c, ws, dec_out)

    graphs = {}
    if not args.no_decode:
        warm_caches = [caches[0]]
        for name, cs in (("rotating", caches), ("warm", warm_caches)):
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for c in cs:
                    layer.decode_step(dq[0], dk[0], dv[0], cnn, c, ws, dec_out)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                decode_loop(cs)
            torch.cuda.synchronize()
            graphs[name] = g

    dev_ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    stage_ms = {"score": [], "select": [], "attend": [], "build_cache": []}
    prefill_ms, dec_rot_ms, dec_warm_ms, step_ms = [], [], [], []
    if not args.no_decode:
        seed = torch.empty_like(cache0)
        flush_buf = torch.empty(2 * MALL_BYTES, dtype=torch.uint8, device=dev)
    for it in range(args.warmup + args.steps):
        timed = it >= args.warmup
        # timed steps alternate: the prefill time from uninstrumented prefills, the
        # stage times from instrumented ones (each step runs one prefill either way)
        instrumented = (it - args.warmup) % 2 == 1 or args.steps == 1
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        prefill_staged(instrumented)
        if not args.no_decode:
            # every decode replay starts from this prefill's cache (positions T .. T+ndec-1),
            # untimed: the rotating caches are re-seeded, then the last-level cache is
            # overwritten so that they start cold
            seed.copy_(cache0)
            for c in caches[1:]:
                c.copy_(seed)
            flush_buf.zero_()
            dev_ev[0].record(stream)
            graphs["rotating"].replay()
            dev_ev[1].record(stream)
            caches[0].copy_(seed)
            dev_ev[2].record(stream)
            graphs["warm"].replay()
            dev_ev[3].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if timed:
            step_ms.append((t1 - t0) * 1e3)
            if instrumented:
                stage_ms["score"].append(ev[0].elapsed_time(ev[1]))
                stage_ms["select"].append(ev[1].elapsed_time(ev[2]))
                stage_ms["attend"].append(ev[2].elapsed_time(ev[3]))
                stage_ms["build_cache"].append(ev[3].elapsed_time(ev[4]))
            if not instrumented or args.steps == 1:
                prefill_ms.append(ev[0].elapsed_time(ev[4]))
            if not args.no_decode:
                dec_rot_ms.append(dev_ev[0].elapsed_time(dev_ev[1]))
                dec_warm_ms.append(dev_ev[2].elapsed_time(dev_ev[3]))

    # realised masks of the last prefill -> algorithmic work
    views = layer.workspace_views(ws, T)
    rank = views["rank"].cpu().numpy()
    vis = visible_counts(rank, T, wl.sink, wl.window, wl.capacity)       # [B, Hkv, T]
    G = wl.Hq // wl.Hkv
    attn_flops = 4.0 * wl.D * G * float(vis.sum())
    cnn_flops = 2.0 * (3 * 2 * wl.D * 32 + 3 * 32) * B * T * wl.Hkv
    ncand = views["ncand"].cpu().numpy()
    cand_rate = ncand / max(1, T - wl.window - wl.sink)

    # medians over the timed steps
    pf_ms = float(np.median(prefill_ms))
    att_ms = float(np.median(stage_ms["attend"]))
    achieved = attn_flops / (att_ms * 1e-3)
    attend_src = os.path.join(ROOT, "learnable_kv_cache_amd", "csrc", "attend.hip")
    traffic = measured_traffic("attend_prefill", attend_src)
    roofline = {"bound": "mfma", "kernel": "attend_prefill_kernel<128,4>",
                "achieved": achieved / 1e12, "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_FLOPS, "traffic": traffic,
                "flops_per_launch": attn_flops, "ms_per_launch": att_ms}
    kv_bytes = 2 * B * T * wl.Hkv * wl.D * 2
    score_ms = float(np.median(stage_ms["score"]))
    stages = {
        "score": {"ms": score_ms, "bound": "hbm",
                  "achieved_GBps": kv_bytes / (score_ms * 1e-3) / 1e9,
                  "frac": kv_bytes / (score_ms * 1e-3) / PEAK_HBM_BPS},
        "select": {"ms": float(np.median(stage_ms["select"]))},
        "attend": {"ms": att_ms, "frac_mfma": achieved / PEAK_BF16_FLOPS},
        # runs beside attend on a second stream: ms is the part left after attend ends
        "build_cache": {"ms": float(np.median(stage_ms["build_cache"])),
                        "beside_attend": True},
    }
    result = {
        "metric": METRIC,
        "value": B * T / (pf_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": float(np.mean(step_ms)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"prefill-b32-t4096 then decode-b32 (positions {T}-{T + ndec - 1})",
                   "B": B, "T": T,
                   "Hq": wl.Hq, "Hkv": wl.Hkv, "D": wl.D, "sink": wl.sink, "window": wl.window,
                   "capacity": wl.capacity, "decode_steps": ndec, "decode_layers": L},
        "prefill_ms": pf_ms,
        "roofline": roofline,
        "stages": stages,
        "retention": {"candidate_rate_per_head": [float(x) for x in cand_rate.mean(axis=0)],
                      "mean_visible_keys_per_row": float(vis.mean()),
                      "prefill_flops": attn_flops + cnn_flops},
    }
    if not args.no_decode:
        # algorithmic bytes of one layer-step: K and V of every visible key (once per KV
        # head), q, o, the new k/v, the score scan of a full retained segment
        cv = layer.cache_views(caches[-1])
        counts = cv["count"].cpu().numpy()
        pos = int(cv["pos"].cpu().numpy().max())
        assert pos == T + ndec, (pos, T + ndec)        # re-seeded before every replay
        nvis = float(counts.mean()) + wl.window + wl.sink
        step_bytes = (B * wl.Hkv * nvis * wl.D * 2 * 2 + 2 * B * wl.Hq * wl.D * 2
                      + 2 * B * wl.Hkv * wl.D * 2 + B * wl.Hkv * wl.capacity * 4)
        us_rot = float(np.median(dec_rot_ms)) * 1e3 / (ndec * L)
        us_warm = float(np.median(dec_warm_ms)) * 1e3 / ndec
        achieved_b = step_bytes / (us_rot * 1e-6)
        result["decode"] = {
            "us_per_step": us_rot, "warm_single_cache_us_per_step": us_warm,
            "layers_rotated": L, "cache_bytes": cache_bytes, "positions": [T, T + ndec - 1],
            "roofline": {"bound": "hbm", "achieved": achieved_b / 1e9,
                         "peak": PEAK_HBM_BPS / 1e9, "unit": "GB/s",
                         "frac": achieved_b / PEAK_HBM_BPS, "bytes_per_step": step_bytes,
                         "traffic": measured_traffic(
                             "decode_step", os.path.join(ROOT, "learnable_kv_cache_amd", "csrc",
                                                         "decode.hip"))},
        }
    if not args.no_chunk and ndec > 0:
        # chunked prefill: the prompt's cache extended by the next n tokens in one call
        n = min(512, ndec)
        prefill_staged()
        torch.cuda.synchronize()
        qc, kc, vc = (x[:, T:T + n].contiguous() for x in (q, k, v))
        cws = layer.alloc_chunk_workspace(n, dev)
        cout = torch.empty_like(qc)
        times = []
        for _ in range(6):
            c = cache0.clone()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            gate()
            e0.record(stream)
            layer.prefill_chunk(qc, kc, vc, cnn, c, cws, cout)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
            del c
        ch_ms = float(np.median(times[1:]))
        result["chunk"] = {"n": n, "onto_position": T, "ms": ch_ms,
                           "tokens_per_s": B * n / (ch_ms * 1e-3)}
        del cws, cout
    if not args.no_linear:
        result["linear"] = linear_layer(dev)
    if not args.no_artificial:
        result["artificial_cache"] = artificial_cache(dev)
    if not args.no_comparators and not args.no_decode:
        cmp = comparators(inp, wl, T, dev, ndec=min(64, ndec))
        cmp["lte"] = {"window": wl.window, "capacity": wl.capacity, "prefill_attend_ms": att_ms,
                      "prefill_attend_tflops": achieved / 1e12,
                      "decode_us_per_step": result["decode"]["us_per_step"]}
        result["comparators"] = cmp
    if not args.no_long:
        del caches, graphs
        torch.cuda.empty_cache()
        result["long_context"] = long_context(dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, wl, T, args.cpu_sample)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
