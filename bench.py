#!/usr/bin/env python3
"""Verify-pass benchmark on one MI355X.

One step = one pass of the whole hot path over one batch: vq_decode_pass streams every
weight of the 27B-class stack once (64 layers of hidden 5120, kv 1024, ffn 17408, plus a
151936-row lm_head; 4-bit block-32 codes with fp16 scale and fp16 min, 13,698,252,800
bytes) for a K-wide window, then vq_verify_accept turns the logits into tokens.  The
headline line is K = 1 (plain decode; the bonus token sampled with temperature 0.6,
top-p 0.95, min-p 0.05).  K = 4 (greedy, drafts agreeing with the target argmax at
alpha 0.7), K = 8 (the sampling path over 1,000 synthetic windows) and K = 16 (MXFP4
stack) are reported in the same JSON line under "sweep".

Inputs are synthetic and seeded (synth): weights are generated on the host, copied to
HBM and tiled before timing.  Timed steps replay a captured HIP graph of the step; the
weight stream is HBM-bound, so "value" is weight bytes per pass / seconds per step.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--sweep 4,8,16] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E peak
STREAM_CEILING_GBPS = 7150.0    # one launch streaming-reading the stack's 13.7 GB on this GPU
METRIC = "verify-pass weight GB/s (% of ~8 TB/s HBM) and passes/s at K=1,4,8,16"
SAMPLER = dict(T=0.6, top_p=0.95, min_p=0.05)
ALPHAS = (0.5, 0.7, 0.9)
PROFILE = os.path.join(ROOT, "profiles", "k_flow_q4min_k1_27b_decode.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "speculative_decoding_verification_bit_amd", "csrc", f)
                  for f in ("flow.hip", "vq_device.h", "vq_internal.h", "steps.h", "api.hip")]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def tau(alpha: float, k: int) -> float:
    """Expected tokens per pass with k drafts each accepted independently with prob. alpha."""
    return (1 - alpha ** (k + 1)) / (1 - alpha)


def source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def profiled_traffic():
    """HBM bytes per launch of k_flow<Q4_MIN, K 1> from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a copy of known size), or None when the
    kernel sources have changed since the counters were taken."""
    try:
        fields = dict(line.split(": ", 1) for line in open(PROFILE).read().splitlines()
                      if line.startswith(("traffic_bytes_per_launch: ", "source_sha256: ")))
    except OSError:
        return None
    if fields.get("source_sha256") != source_hash():
        return None
    return int(fields["traffic_bytes_per_launch"])


def upload_stack(vq, synth, fmt, seed, threads):
    shape = synth.SHAPE_27B
    t0 = time.time()
    layers = []
    for l in range(shape.n_layers):
        L = {}
        for mid, name in enumerate(synth.LAYER_MATS):
            r, c = shape.mat_shape(mid)
            L[name] = vq.DeviceMatrix.from_host(synth.weight_matrix(fmt, seed, l, mid, r, c, threads=threads))
        layers.append(L)
    r, c = shape.mat_shape(synth.MAT_LM_HEAD)
    lm = vq.DeviceMatrix.from_host(synth.weight_matrix(fmt, seed, shape.n_layers, synth.MAT_LM_HEAD, r, c,
                                                       threads=threads))
    model = vq.DeviceModel(layers, lm)
    del layers, lm
    log(f"stack fmt {fmt}: {model.nbytes} bytes tiled on the device in {time.time() - t0:.1f} s")
    return model


def time_graph(torch, step, steps, warmup):
    """Capture step() into a HIP graph, replay warmup times, then time `steps` replays."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, g


def launch_times(torch, vq, model, x0, logits, ws, passes):
    """Durations of the pass kernel's launches (one cooperative launch per 16 layers, the
    last with the lm_head), from HIP events that the library records on the stream it
    launches on, and the weight bytes each launch streams."""
    events = [torch.cuda.Event(enable_timing=True) for _ in range(16)]
    for ev in events:
        ev.record()                     # creates the HIP event handles
    torch.cuda.synchronize()
    tot, n = None, 0
    for _ in range(passes):
        _, _, n = vq.decode_pass_launch(model, x0, logits, ws, vq.LAUNCH_AUTO, events)
        torch.cuda.synchronize()
        ms = np.array([events[2 * i].elapsed_time(events[2 * i + 1]) for i in range(n)])
        tot = ms if tot is None else tot + ms
    b = []
    for i in range(n):
        layers = model.tiled[16 * i:16 * (i + 1)]
        nb = sum(m.nbytes for L in layers for m in L.values())
        if i == n - 1:
            nb += model.lm_head.nbytes
        b.append(nb)
    return tot / passes, np.array(b, dtype=np.float64)


def cpu_baseline(synth, oracle_mod, budget_s: float):
    """The fp64 oracle on the host's cores (test infrastructure, timed as a baseline).

    Linear: whole layers of the 27B stack at K = 1 on all threads until budget_s of oracle
    time, scaled to the pass; the same on one thread for one o matrix; one layer at K =
    4, 8, 16 on all threads.  Acceptance: a few windows of the K = 8 sampling workload."""
    threads = min(16, len(os.sched_getaffinity(0)))
    model_name = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model_name = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    shape = synth.SHAPE_27B
    total_w = shape.n_weights()
    bpw = synth.bytes_per_weight(synth.FMT_Q4_MIN)
    mats = {}

    def mat(l, mid):
        key = (l, mid)
        if key not in mats:
            r, c = shape.mat_shape(mid)
            mats[key] = synth.weight_matrix(synth.FMT_Q4_MIN, 0, l, mid, r, c, threads=threads)
        return mats[key]

    x = {c: synth.activations(0, 1, c) for c in (shape.hidden, shape.ffn)}
    weights, spent, layers = 0, 0.0, 0
    for l in range(shape.n_layers):
        for mid in range(7):
            m = mat(l, mid)
            t0 = time.time()
            oracle_mod.linear(m, x[m.cols], threads=threads)
            spent += time.time() - t0
            weights += m.rows * m.cols
        layers += 1
        if spent >= budget_s:
            break
    w_per_s = weights / spent
    m = mat(0, synth.MAT_O)
    t0 = time.time()
    oracle_mod.linear(m, x[m.cols], threads=1)
    one_thread = m.rows * m.cols / (time.time() - t0)
    per_k = {}
    layer_w = sum(r * c for r, c in (shape.mat_shape(mid) for mid in range(7)))
    for K in (4, 8, 16):
        xk = synth.activations(0, K, m.cols)
        t0 = time.time()
        oracle_mod.linear(m, xk, threads=threads)
        per_k[f"K{K}_one_layer_s"] = round((time.time() - t0) * layer_w / (m.rows * m.cols), 3)
    mats.clear()
    c4 = synth.C4
    nwin = 4
    t, d = synth.logits_batch(c4["logits"], 0, nwin, threads=threads)
    f32 = lambda v: float(np.float32(v))
    t0 = time.time()
    r = oracle_mod.accept(oracle_mod.MODE_SAMPLE, t, d, None, oracle_mod.DRAFT_Q_SAMPLE, f32(c4["T"]),
                          f32(c4["top_p"]), f32(c4["min_p"]), 0.0, c4["philox_seed"], 0, threads=threads)
    acc_s = time.time() - t0
    return {
        "value": round(w_per_s * bpw / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "cpu_model": model_name,
        "passes_per_s": w_per_s / total_w,
        "single_thread_gbps": round(one_thread * bpw / 1e9, 4),
        "sample": (f"{layers} of 64 layers (7 matrices each, {weights} weights) of the 27B stack at "
                   f"K=1, {spent:.1f} s of fp64 oracle time on {threads} threads, scaled to the "
                   f"{total_w}-weight pass; one 5120x5120 matrix on 1 thread; one layer at K=4/8/16 on "
                   f"{threads} threads (the o matrix timed, scaled by weights); {nwin} C4 acceptance windows (K 8, V 151936)"),
        **per_k,
        "accept_windows_per_s": round(nwin / acc_s, 3),
        "accept_near_threshold_windows": int(np.count_nonzero(r["near"])),
        "accept_windows_checked": nwin,
    }


def bench_depth(torch, vq, model, dev, H, V, args):
    """Adaptive draft depth on this GPU's own pass times.  t_pass[k] = the measured verify pass
    with k drafts (K = k + 1 columns, graph replays of vq_decode_pass on the 27B stack); a
    draft step costs c of a K = 1 pass (the drafter is outside this build: c = 0.05, an MTP
    head, and c = 0.25, a small draft model, are stated, not measured).  Reported: the depth
    vq_depth_choose picks at fixed acceptance, and a synthetic trace (acceptance 0.85, 0.3,
    0.65 for 2,000 windows each; per window 15 seeded uniforms decide the drafts for every
    policy alike) run with the controller (observe each window, decay 0.98, prior 0.5 of
    weight 2) against every fixed depth; tokens/s = tokens / (passes + drafts)."""
    kmax = 8
    t = []
    for k in range(kmax + 1):
        K = k + 1
        x0 = torch.from_numpy(__import__("synth").activations(0, K, H)).to(dev)
        logits = torch.empty((K, V), dtype=torch.float32, device=dev)
        ws = torch.empty(model.workspace_bytes(K), dtype=torch.uint8, device=dev)
        ms, g = time_graph(torch, lambda: vq.decode_pass(model, x0, logits, ws=ws), max(5, args.steps // 2), 2)
        del g
        assert model.barrier_error(K, ws) == 0
        t.append(ms)
        del x0, logits, ws
    t = np.array(t)
    res = {"t_pass_ms": [round(float(x), 4) for x in t], "k_max": kmax}
    # the K columns as a batch of independent one-token sequences: tokens per second
    tb = {K: float(t[K - 1]) for K in range(1, kmax + 2)}
    for K in (12, 16):
        x0 = torch.from_numpy(__import__("synth").activations(0, K, H)).to(dev)
        logits = torch.empty((K, V), dtype=torch.float32, device=dev)
        ws = torch.empty(model.workspace_bytes(K), dtype=torch.uint8, device=dev)
        ms, g = time_graph(torch, lambda: vq.decode_pass(model, x0, logits, ws=ws), max(5, args.steps // 2), 2)
        del g
        assert model.barrier_error(K, ws) == 0
        tb[K] = ms
        del x0, logits, ws
    res["batch"] = {"note": "K independent sequences per pass (no speculation): tokens/s = K / t_pass(K)",
                    "per_K": {f"K{K}": {"ms": round(v, 4), "tok_per_s": round(K / v * 1e3, 1)}
                              for K, v in sorted(tb.items())}}
    rng = np.random.default_rng(11)
    segs = [(0.85, 2000), (0.3, 2000), (0.65, 2000)]
    U = rng.random((sum(n for _, n in segs), 15))
    A = np.concatenate([np.full(n, a) for a, n in segs])
    first_rej = lambda w, k: int(np.argmax(U[w, :k] >= A[w])) if k > 0 and (U[w, :k] >= A[w]).any() else k
    import time as _time
    for c in (0.05, 0.25):
        td = c * t[0]
        fixed_alpha = {}
        for a in (0.35, 0.5, 0.7, 0.9):
            st = vq.VqDepthStats(a * 1e6, (1 - a) * 1e6)
            k, _, r = vq.depth_choose(st, t, td)
            fixed_alpha[f"alpha_{a}"] = {"k": k, "tok_per_s": round(r * 1e3, 1),
                                         "tok_per_s_k3": round(1e3 * (1 - a ** 4) / (1 - a) / (t[3] + 3 * td), 1),
                                         "tok_per_s_k7": round(1e3 * (1 - a ** 8) / (1 - a) / (t[7] + 7 * td), 1)}
        # the trace: controller against every fixed depth, same uniforms
        st = vq.VqDepthStats(0.0, 0.0)
        k, tok, tim, ks = 3, 0, 0.0, []
        t0 = _time.perf_counter()
        for w in range(len(A)):
            n = first_rej(w, k)
            tok += n + 1
            tim += t[k] + k * td
            ks.append(k)
            vq.depth_observe(st, [n], [k], 0.98)
            k = vq.depth_choose(st, t, td, 0.5, 2.0)[0]
        ctl_us = (_time.perf_counter() - t0) / len(A) * 1e6
        fixed = {}
        for kf in range(kmax + 1):
            tk = sum(first_rej(w, kf) + 1 for w in range(len(A)))
            fixed[kf] = tk / (len(A) * (t[kf] + kf * td)) * 1e3
        best = max(fixed, key=fixed.get)
        ks = np.array(ks)
        res[f"c_{c}"] = {"fixed_alpha": fixed_alpha,
                         "trace_adaptive_tok_per_s": round(tok / tim * 1e3, 1),
                         "trace_best_fixed": {"k": best, "tok_per_s": round(fixed[best], 1)},
                         "trace_fixed_tok_per_s": {str(kf): round(v, 1) for kf, v in fixed.items()},
                         "trace_mean_depth_per_segment": [round(float(ks[i:i + 2000].mean()), 2)
                                                          for i in (0, 2000, 4000)],
                         "controller_us_per_window": round(ctl_us, 2)}
    return res


def bench_q4k(torch, vq, synth, dev, args):
    """The decode pass over the 27B-class stack with Q4_K super-block weights (4.625 bits per
    weight in the tiled layout) at K = 1 and 8: one graph-replayed pass, as the headline."""
    shape = synth.SHAPE_27B
    H, V = shape.hidden, shape.vocab
    model = upload_stack(vq, synth, synth.FMT_Q4_K, 0, args.threads)
    nbytes = model.nbytes
    assert nbytes == shape.n_weights() * 37 // 64
    res = {"workload": "27b-q4k-decode", "format": "q4_k: 256-weight super-blocks, 6-bit sub-block "
           "scale and min, fp16 d and dmin", "weight_bytes": nbytes}
    for K in (1, 8):
        x0 = torch.from_numpy(synth.activations(0, K, H)).to(dev)
        logits = torch.empty((K, V), dtype=torch.float32, device=dev)
        ws = torch.empty(model.workspace_bytes(K), dtype=torch.uint8, device=dev)
        ms = time_graph(torch, lambda: vq.decode_pass(model, x0, logits, ws=ws), args.steps, args.warmup)[0]
        assert model.barrier_error(K, ws) == 0, "a grid wait of the pass timed out"
        gbps = nbytes / ms / 1e6
        res[f"K{K}"] = {"ms_per_step": round(ms, 4), "gbps": round(gbps, 2),
                        "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "passes_per_s": round(1000 / ms, 2)}
        del ws, logits, x0
    res["k8_over_k1"] = round(res["K8"]["ms_per_step"] / res["K1"]["ms_per_step"], 3)
    del model
    torch.cuda.empty_cache()
    return res


def bench_ngram(vq, synth, t_pass=None, n_tokens=100000, max_drafts=8):
    """The n-gram map drafter on a synthetic code-like stream (synth.token_stream, 100,000
    tokens) replayed as the target's output: per window the map proposes up to 8 drafts,
    the accepted drafts are the prefix that equals the stream's next tokens, and the
    accepted drafts plus one token are appended.  Per key length: tokens per window (tau),
    the fraction of windows with a proposal, and the library's cost per window (append +
    propose through the binding).  With the measured pass times t_pass[k], the implied
    tokens/s when each window is verified with exactly the proposed drafts."""
    import time as _time
    s = synth.token_stream(0, n_tokens)
    res = {"stream": "synth.token_stream(seed 0, 100000 tokens)", "max_drafts": max_drafts, "per_key_len": {}}
    for k in (12, 6, 4, 2):
        m = vq.NgramMap(k)
        prompt = 2000
        m.append(s[:prompt])
        i, windows, hits, acc_sum, t_sec = prompt, 0, 0, 0, 0.0
        pass_ms = 0.0
        while i < s.size:
            t0 = _time.perf_counter()
            d = m.propose(max_drafts)
            t_sec += _time.perf_counter() - t0
            a = 0
            while a < len(d) and i + a < s.size and d[a] == s[i + a]:
                a += 1
            emit = s[i:i + a + 1]
            t0 = _time.perf_counter()
            m.append(emit)
            t_sec += _time.perf_counter() - t0
            i += emit.size
            windows += 1
            hits += len(d) > 0
            acc_sum += a
            if t_pass is not None:
                pass_ms += t_pass[min(len(d), len(t_pass) - 1)]
        r = {"tokens_per_window": round((s.size - prompt) / windows, 4), "hit_rate": round(hits / windows, 4),
             "accepted_per_hit": round(acc_sum / max(hits, 1), 3),
             "us_per_window": round(t_sec / windows * 1e6, 2)}
        if t_pass is not None:
            r["implied_tok_per_s"] = round((s.size - prompt) / pass_ms * 1e3, 1)
        res["per_key_len"][f"k{k}"] = r
    return res


def bench_attention(torch, vq, synth, dev, args):
    """The window's attention over one layer's q8_0 / q4_0 cache of the 27B model at 32768
    positions (40 query heads, 8 kv heads, head dim 128), K = 1, 4, 8, 16: time per call
    (both kernels) from a captured graph of 10 calls replayed, as the pass is (the eager
    time, which adds the binding's per-call cost and launch gaps, beside it), and the cache
    bytes over that time."""
    c = synth.ATTN
    Hkv, Hq, L = c["n_kv_heads"], c["n_q_heads"], c["length"]
    kc, ks = synth.kv_cache(c["kfmt"], c["seed"], 0, 0, Hkv, L, threads=args.threads)
    vc, vs = synth.kv_cache(c["vfmt"], c["seed"], 0, 1, Hkv, L, threads=args.threads)
    C = vq.DeviceKV.from_host(c["kfmt"], kc, ks, c["vfmt"], vc, vs, Hq, dev)
    cache = kc.nbytes + ks.nbytes + vc.nbytes + vs.nbytes
    res = {"workload": c["name"], "cache_bytes": cache, "per_K": {}}
    for K in (1, 4, 8, 16):
        q = torch.from_numpy(synth.queries(c["seed"], K, Hq)).to(dev)
        o = torch.empty(q.shape, dtype=torch.float32, device=dev)
        ws = torch.empty(C.workspace_bytes(K), dtype=torch.uint8, device=dev)
        for _ in range(max(2, args.warmup)):
            vq.verify_attention(C, q, out=o, ws=ws)
        torch.cuda.synchronize()
        n = max(50, 5 * args.steps)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            vq.verify_attention(C, q, out=o, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        us_eager = e0.elapsed_time(e1) * 1e3 / n
        per_graph = 10
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                vq.verify_attention(C, q, out=o, ws=ws)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        reps = max(5, n // per_graph)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * per_graph)
        del g
        algo = cache + q.numel() * 2 + o.numel() * 4
        res["per_K"][f"K{K}"] = {"us_per_call": round(us, 2), "gbps": round(algo / us / 1e3, 1),
                                 "frac_of_hbm_peak": round(algo / us / 1e3 / HBM_PEAK_GBPS, 4),
                                 "us_per_pass_64_layers": round(64 * us, 1),
                                 "us_per_call_eager": round(us_eager, 2)}
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--sweep", default="4,8,16", help="other K values to time ('' for none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-budget", type=float, default=8.0, help="seconds of oracle time to sample")
    ap.add_argument("--threads", type=int, default=16, help="host threads for input generation")
    ap.add_argument("--no-compare", action="store_true", help="skip timing the staged launch mode")
    ap.add_argument("--no-attn", action="store_true", help="skip timing the attention over the KV cache")
    ap.add_argument("--no-depth", action="store_true", help="skip the adaptive draft depth measurement")
    ap.add_argument("--no-ngram", action="store_true", help="skip the n-gram drafter measurement")
    ap.add_argument("--no-q4k", action="store_true", help="skip the pass over Q4_K super-block weights")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first copy 1 GiB with torch (the known-size kernel that scales HBM counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the verify pass on one GPU: runs on more than one GPU are not part "
              "of this benchmark (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import speculative_decoding_verification_bit_amd as vq
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    shape = synth.SHAPE_27B
    H, V = shape.hidden, shape.vocab

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # ---------------------------------------------------------------- K = 1
    model = upload_stack(vq, synth, synth.FMT_Q4_MIN, 0, args.threads)
    wbytes = model.nbytes
    assert wbytes == shape.n_weights() * 5 // 8

    def make_step(model, K, accept_fn):
        x0 = torch.from_numpy(synth.activations(0, K, H)).to(dev)
        logits = torch.empty((K, V), dtype=torch.float32, device=dev)
        ws = torch.empty(model.workspace_bytes(K), dtype=torch.uint8, device=dev)
        acc = accept_fn(logits)

        def step():
            vq.decode_pass(model, x0, logits, ws=ws)
            acc()
        return step, x0, logits, ws

    def sampled_bonus(logits):
        t = logits.view(1, 1, V)
        empty = torch.empty((1, 0, V), dtype=torch.float32, device=dev)
        probe = vq.verify_accept(vq.MODE_SAMPLE, t, empty, T=SAMPLER["T"], top_p=SAMPLER["top_p"],
                                 min_p=SAMPLER["min_p"], seed=0)
        aws = torch.empty(vq.workspace_bytes(vq.OP_ACCEPT, vq.accept_desc(1, t, empty), 1) or 1,
                          dtype=torch.uint8, device=dev)

        def acc():
            vq.verify_accept(vq.MODE_SAMPLE, t, empty, T=SAMPLER["T"], top_p=SAMPLER["top_p"],
                             min_p=SAMPLER["min_p"], seed=0, ws=aws, out=probe)
        return acc

    step1, x0_1, logits1, ws1 = make_step(model, 1, sampled_bonus)
    log("K=1: capture and time")
    ms1, g1 = time_graph(torch, step1, args.steps, args.warmup)
    del g1
    assert model.barrier_error(1, ws1) == 0, "a grid wait of the pass timed out"
    per_launch_ms, per_launch_bytes = launch_times(torch, vq, model, x0_1, logits1, ws1, args.steps)
    assert model.barrier_error(1, ws1) == 0, "a grid wait of the pass timed out"
    achieved = float(per_launch_bytes.sum() / (per_launch_ms.sum() * 1e-3) / 1e9)
    value = wbytes / (ms1 * 1e-3) / 1e9
    log(f"K=1 step {ms1:.3f} ms ({value:.0f} GB/s); launches "
        + ", ".join(f"{m * 1e3:.0f} us" for m in per_launch_ms) + f"; kernel {achieved:.0f} GB/s")
    staged1 = None
    if not args.no_compare:
        staged1 = time_graph(torch, lambda: vq.decode_pass_launch(model, x0_1, logits1, ws1, vq.LAUNCH_STAGED),
                             max(3, args.steps // 4), 1)[0]
        log(f"K=1 pass with one launch per stage: {staged1:.3f} ms")
    traffic = profiled_traffic()
    pps1 = 1000.0 / ms1
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms1, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16xf16->f32 (4-bit codes widened exactly to f16)",
        "data": "synthetic",
        "config": {"workload": synth.C2["name"], "layers": shape.n_layers, "hidden": H,
                   "kv": shape.kv_dim, "ffn": shape.ffn, "vocab": V, "K": 1,
                   "format": "q4 block-32 + fp16 scale + fp16 min", "weight_bytes": wbytes,
                   "accept": "sample T 0.6 top-p 0.95 min-p 0.05"},
        "passes_per_s": round(pps1, 2),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "frac_of_stream_ceiling": round(value / STREAM_CEILING_GBPS, 4),
        "implied_tok_s": {f"alpha_{a}": round(pps1 * tau(a, 0), 2) for a in ALPHAS},
        "staged_pass_ms": staged1 and round(staged1, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "traffic_over_algorithmic": None if traffic is None else round(traffic / per_launch_bytes.mean(), 4),
                     "kernel": "k_flow<Q4_MIN, K 1> (persistent, 16 layers per launch)",
                     "launches_per_pass": len(per_launch_ms),
                     "avg_launch_us": round(float(per_launch_ms.mean()) * 1e3, 3),
                     "bytes_per_launch": round(float(per_launch_bytes.mean()))},
    }

    # ------------------------------------------------------------------ sweep
    sweep = {}
    Ks = [int(k) for k in args.sweep.split(",") if k.strip()]
    if 4 in Ks:
        alpha = synth.C3["alpha"]

        def agree(logits):
            t = logits.view(1, 4, V)
            probe = vq.verify_accept(vq.MODE_GREEDY, t, draft_mode=vq.DRAFT_AGREE, alpha=alpha, seed=0)

            def acc():
                vq.verify_accept(vq.MODE_GREEDY, t, draft_tokens=probe["draft_tokens"],
                                 draft_mode=vq.DRAFT_AGREE, alpha=alpha, seed=0, out=probe)
            return acc

        step4, x0_4, logits4, ws4 = make_step(model, 4, agree)
        ms4, g4 = time_graph(torch, step4, args.steps, args.warmup)
        del g4
        assert model.barrier_error(4, ws4) == 0
        # measured acceptance on the pass's own logits, fresh Philox windows
        t = logits4.view(1, 4, V).expand(2000, 4, V).contiguous()
        r = vq.verify_accept(vq.MODE_GREEDY, t, draft_mode=vq.DRAFT_AGREE, alpha=alpha, seed=0)
        am = torch.argmax(logits4, dim=1)[:3]
        agree_rate = float((r["draft_tokens"] == am.view(1, 3)).float().mean())
        tau_meas = float((r["n_accepted"] + 1).float().mean())
        del t, r
        pps = 1000 / ms4
        sweep["K4"] = {"workload": synth.C3["name"], "ms_per_step": round(ms4, 4),
                       "gbps": round(wbytes / ms4 / 1e6, 2), "passes_per_s": round(pps, 2),
                       "frac_of_hbm_peak": round(wbytes / ms4 / 1e6 / HBM_PEAK_GBPS, 4),
                       "ratio_to_K1_pass": round(ms4 / ms1, 4),
                       "accept": "greedy, drafts agree with the target argmax at alpha 0.7",
                       "measured_alpha": round(agree_rate, 4), "measured_tau": round(tau_meas, 4),
                       "implied_tok_s": {f"alpha_{a}": round(pps * tau(a, 3), 2) for a in ALPHAS},
                       "implied_tok_s_measured": round(pps * tau_meas, 2)}
        log("K=4", sweep["K4"])
        del ws4
    if 8 in Ks:
        x0_8 = torch.from_numpy(synth.activations(0, 8, H)).to(dev)
        logits8 = torch.empty((8, V), dtype=torch.float32, device=dev)
        ws8 = torch.empty(model.workspace_bytes(8), dtype=torch.uint8, device=dev)
        ms8 = time_graph(torch, lambda: vq.decode_pass(model, x0_8, logits8, ws=ws8), args.steps, args.warmup)[0]
        assert model.barrier_error(8, ws8) == 0
        del ws8
        # the sampling path over the C4 windows
        c4 = synth.C4
        spec = c4["logits"]
        W = c4["windows"]
        td = torch.empty((W, spec.K, spec.vocab), dtype=torch.float32, device=dev)
        dd = torch.empty((W, spec.K - 1, spec.vocab), dtype=torch.float32, device=dev)
        for w0 in range(0, W, 100):
            t, d = synth.logits_batch(spec, w0, w0 + 100, threads=args.threads)
            td[w0:w0 + 100].copy_(torch.from_numpy(t))
            dd[w0:w0 + 100].copy_(torch.from_numpy(d))
        kw = dict(draft_mode=vq.DRAFT_Q_SAMPLE, T=c4["T"], top_p=c4["top_p"], min_p=c4["min_p"],
                  seed=c4["philox_seed"])
        r = vq.verify_accept(vq.MODE_SAMPLE, td, dd, **kw)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            vq.verify_accept(vq.MODE_SAMPLE, td, dd, out=r, **kw)
        e1.record()
        torch.cuda.synchronize()
        acc_ms = e0.elapsed_time(e1) / 3
        n_acc = r["n_accepted"].cpu().numpy()
        beta = [float((n_acc >= i).mean()) for i in range(1, 8)]
        tau8 = float((n_acc + 1).mean())
        del td, dd, r
        torch.cuda.empty_cache()
        pps = 1000 / ms8
        sweep["K8"] = {"workload": synth.C4["name"], "ms_per_step": round(ms8, 4),
                       "gbps": round(wbytes / ms8 / 1e6, 2), "passes_per_s": round(pps, 2),
                       "frac_of_hbm_peak": round(wbytes / ms8 / 1e6 / HBM_PEAK_GBPS, 4),
                       "ratio_to_K1_pass": round(ms8 / ms1, 4),
                       "accept_ms_1000_windows": round(acc_ms, 4),
                       "accept_us_per_window": round(acc_ms * 1000 / W, 3),
                       "measured_tau": round(tau8, 4),
                       "reach_position": [round(b, 4) for b in beta],
                       "implied_tok_s": {f"alpha_{a}": round(pps * tau(a, 7), 2) for a in ALPHAS},
                       "implied_tok_s_measured": round(pps * tau8, 2)}
        log("K=8", sweep["K8"])
    if not args.no_depth:
        out["adaptive_depth"] = bench_depth(torch, vq, model, dev, H, V, args)
        log("adaptive depth", {k: v for k, v in out["adaptive_depth"].items() if k != "trace"})
    if not args.no_ngram:
        tp = out["adaptive_depth"]["t_pass_ms"] if "adaptive_depth" in out else None
        out["ngram_drafter"] = bench_ngram(vq, synth, tp)
        log("n-gram drafter", out["ngram_drafter"])
    if 16 in Ks:
        del model
        torch.cuda.empty_cache()
        mx = upload_stack(vq, synth, synth.FMT_MXFP4, 0, args.threads)
        mbytes = mx.nbytes
        x0_16 = torch.from_numpy(synth.activations(0, 16, H)).to(dev)
        logits16 = torch.empty((16, V), dtype=torch.float32, device=dev)
        ws16 = torch.empty(mx.workspace_bytes(16), dtype=torch.uint8, device=dev)
        ms16 = time_graph(torch, lambda: vq.decode_pass(mx, x0_16, logits16, ws=ws16), args.steps,
                          args.warmup)[0]
        assert mx.barrier_error(16, ws16) == 0
        pps = 1000 / ms16
        sweep["K16"] = {"workload": synth.C5["name"], "weight_bytes": mbytes, "path": "f16 mfma",
                        "ms_per_step": round(ms16, 4), "gbps": round(mbytes / ms16 / 1e6, 2),
                        "passes_per_s": round(pps, 2),
                        "frac_of_hbm_peak": round(mbytes / ms16 / 1e6 / HBM_PEAK_GBPS, 4),
                        "implied_tok_s": {f"alpha_{a}": round(pps * tau(a, 15), 2) for a in ALPHAS}}
        del mx, ws16
        torch.cuda.empty_cache()
        # the scaled MXFP4 instruction (E4M3 activations, an approximation) against the exact
        # f16 path, matrix by matrix: each distinct shape of the stack timed once through
        # vq_verify_linear_mx and vq_verify_linear, summed over the 449 matrices of a pass
        def t_event(f, n):
            for _ in range(2):
                f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                f()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n
        per_shape, t_mx, t_ex = {}, 0.0, 0.0
        counts = {synth.MAT_Q: 64, synth.MAT_K: 128, synth.MAT_O: 64, synth.MAT_GATE: 128, synth.MAT_DOWN: 64,
                  synth.MAT_LM_HEAD: 1}
        for mid, cnt in counts.items():
            r, c = shape.mat_shape(mid)
            mat = vq.DeviceMatrix.from_host(synth.weight_matrix(synth.FMT_MXFP4, 0, 0, mid, r, c, threads=args.threads))
            xk = torch.from_numpy(synth.activations(0, 16, c)).to(dev)
            yk = torch.empty((16, r), dtype=torch.float32, device=dev)
            wsm = torch.empty(vq.workspace_bytes(vq.OP_LINEAR_MX, mat.desc, 16), dtype=torch.uint8, device=dev)
            a = t_event(lambda: vq.verify_linear_mx(mat, xk, y=yk, ws=wsm), 10)
            til = mat.tiled
            wse = torch.empty(vq.workspace_bytes(vq.OP_LINEAR, til.desc, 16), dtype=torch.uint8, device=dev)
            b = t_event(lambda: vq.verify_linear(til, xk, y=yk, ws=wse), 10)
            per_shape[f"{r}x{c}"] = {"scaled_us": round(a * 1e3, 1), "exact_us": round(b * 1e3, 1),
                                     "scaled_gbps": round(mat.nbytes / a / 1e6, 1),
                                     "exact_gbps": round(mat.nbytes / b / 1e6, 1)}
            t_mx += cnt * a
            t_ex += cnt * b
            del mat, til, wsm, wse, xk, yk
            torch.cuda.empty_cache()
        sweep["K16"]["matrix_by_matrix"] = {
            "note": "449 separate linear launches per pass, no stage glue; the scaled path rounds the "
                    "activations to E4M3 with E8M0 block scales (an approximation)",
            "scaled_mxfp4_mfma_ms": round(t_mx, 3), "exact_f16_mfma_ms": round(t_ex, 3),
            "scaled_gbps": round(mbytes / t_mx / 1e6, 1), "exact_gbps": round(mbytes / t_ex / 1e6, 1),
            "per_shape": per_shape}
        log("K=16", sweep["K16"])
    out["sweep"] = sweep
    if not args.no_q4k:
        if 16 not in Ks:
            del model
            torch.cuda.empty_cache()
        out["q4_k"] = bench_q4k(torch, vq, synth, dev, args)
        log("Q4_K", out["q4_k"])

    # ---------------------------------------------------------- attention (next row)
    if not args.no_attn:
        out["attention"] = bench_attention(torch, vq, synth, dev, args)
        log("attention", out["attention"])

    if not args.no_cpu:
        import oracle as oracle_mod
        log("CPU baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(synth, oracle_mod, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
