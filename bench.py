#!/usr/bin/env python3
"""Verify-pass benchmark on one MI355X.

One step = one pass of the whole hot path over one batch: vq_decode_pass streams every
weight of the 27B-class stack (64 layers of hidden 5120, kv 1024, ffn 17408, plus a
151936-row lm_head; 4-bit block-32 codes with fp16 scale and fp16 min, 13,698,252,800
bytes) once for a K-wide window, then vq_verify_accept turns the logits into tokens.
The headline line is K = 1 (plain decode, sampled with temperature 0.6, top-p 0.95,
min-p 0.05); K = 4 (greedy, drafts agreeing with the target argmax at alpha 0.7),
K = 8 (the sampling path over 1,000 synthetic windows) and K = 16 (MXFP4 stack) are
reported in the same JSON line under "sweep".

Inputs are synthetic and seeded (synth): weights are generated on the host and copied
to HBM before timing.  Timed steps replay a captured HIP graph of the step; the weight
stream is HBM-bound, so "value" is weight bytes per pass / seconds per step.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--sweep 4,8,16] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E peak
METRIC = "verify-pass weight GB/s (% of ~8 TB/s HBM) and passes/s at K=1,4,8,16"
SAMPLER = dict(T=0.6, top_p=0.95, min_p=0.05)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def tau(alpha: float, k: int) -> float:
    """Expected tokens per pass with k drafts accepted independently with prob. alpha."""
    return (1 - alpha ** (k + 1)) / (1 - alpha)


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
        if l % 16 == 15:
            log(f"uploaded {l + 1}/{shape.n_layers} layers ({time.time() - t0:.1f} s)")
    r, c = shape.mat_shape(synth.MAT_LM_HEAD)
    lm = vq.DeviceMatrix.from_host(synth.weight_matrix(fmt, seed, shape.n_layers, synth.MAT_LM_HEAD, r, c,
                                                       threads=threads))
    model = vq.DeviceModel(layers, lm)
    log(f"stack fmt {fmt}: {model.nbytes} bytes on the device in {time.time() - t0:.1f} s")
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


def time_eager(torch, step, steps):
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


PROFILE = os.path.join(ROOT, "profiles", "k_stage_valu_q4min_k1_27b_decode.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "speculative_decoding_verification_bit_amd", "csrc", f)
                  for f in ("linear.hip", "vq_device.h", "vq_internal.h")]


def profiled_traffic(kernel_key):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a 1 GiB copy), or None when the summary
    covers another kernel or the kernel sources have changed since the counters were taken."""
    import hashlib
    try:
        fields = dict(line.split(": ", 1) for line in open(PROFILE).read().splitlines()
                      if line.startswith(("traffic_bytes_per_launch: ", "source_sha256: ", "kernel_key: ")))
    except OSError:
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    if fields.get("source_sha256") != h.hexdigest() or fields.get("kernel_key") != kernel_key:
        return None
    return int(fields["traffic_bytes_per_launch"])


def stage_weight_bytes(shape, synth, fmt):
    """Weight bytes of each stage of a pass: q|k|v, o, gate|up, down per layer, lm_head."""
    H, KV, FF, V = shape.hidden, shape.kv_dim, shape.ffn, shape.vocab
    per = [(H + 2 * KV) * H, H * H, 2 * FF * H, H * FF]
    w = [per[i % 4] for i in range(4 * shape.n_layers)] + [V * H]
    return [n * synth.bytes_per_weight(fmt) for n in w]


def time_stream_kernel(torch, vq, model, x0, logits, ws, passes, path, stage_bytes):
    """Per-launch durations of the weight-streaming kernels, from HIP events that the
    library records around each launch on the stream it launches on, grouped by kernel
    instantiation (single- or multi-chunk items).  The event brackets themselves
    serialise the launches (about 2 us each), so every group's time is scaled by the
    ratio of an unbracketed pass (two events on the same stream around decode_pass) to
    the sum of the bracketed launch times.  Returns {name: (launches per pass, ms per pass,
    weight bytes per pass, raw bracketed ms per pass)} and the launches per pass."""
    n_st = 4 * len(model.layers) + 1
    events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_st)]
    for ev in events:
        ev.record()                     # creates the HIP event handles
    torch.cuda.synchronize()
    groups = {}
    n = 0
    bracketed = 0.0
    for _ in range(passes):
        runs = vq.decode_pass_timed(model, x0, events, logits, ws, path=path)
        torch.cuda.synchronize()
        n = len(runs)
        for i, r in enumerate(runs):
            key = "persistent" if r == 0 else "stream" if r == -1 else "rows" if r < 0 else "multi" if r > 1 else "single"
            ms = events[2 * i].elapsed_time(events[2 * i + 1])
            bracketed += ms
            b = stage_bytes[i] if r > 0 or r < -1 else sum(stage_bytes) / n
            c, t, bb = groups.get(key, (0, 0.0, 0.0))
            groups[key] = (c + 1, t + ms, bb + b)
    # the same passes without per-launch events
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    plain = 0.0
    for _ in range(passes):
        e0.record()
        vq.decode_pass(model, x0, logits, path=path, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        plain += e0.elapsed_time(e1)
    scale = min(1.0, plain / bracketed) if bracketed > 0 else 1.0
    return {k: (c / passes, t * scale / passes, b / passes, t / passes) for k, (c, t, b) in groups.items()}, n


def cpu_baseline(synth, oracle_mod, budget_s: float):
    """The fp64 oracle on host cores: whole layers of the stack at K = 1 until `budget_s`
    of oracle time, scaled to the full pass; plus acceptance of C4 windows."""
    threads = min(16, len(os.sched_getaffinity(0)))
    shape = synth.SHAPE_27B
    x = {c: synth.activations(0, 1, c) for c in (shape.hidden, shape.ffn)}
    weights, spent, layers = 0, 0.0, 0
    for l in range(shape.n_layers):
        for mid in range(7):
            r, c = shape.mat_shape(mid)
            m = synth.weight_matrix(synth.FMT_Q4_MIN, 0, l, mid, r, c, threads=threads)
            t0 = time.time()
            oracle_mod.linear(m, x[c], threads=threads)
            spent += time.time() - t0
            weights += r * c
        layers += 1
        if spent >= budget_s:
            break
    w_per_s = weights / spent
    total_w = shape.n_weights()
    gbps = w_per_s * synth.bytes_per_weight(synth.FMT_Q4_MIN) / 1e9
    c4 = synth.C4
    nwin = 2
    t, d = synth.logits_batch(c4["logits"], 0, nwin, threads=threads)
    f32 = lambda v: float(np.float32(v))
    t0 = time.time()
    oracle_mod.accept(oracle_mod.MODE_SAMPLE, t, d, None, oracle_mod.DRAFT_Q_SAMPLE, f32(c4["T"]),
                      f32(c4["top_p"]), f32(c4["min_p"]), 0.0, c4["philox_seed"], 0, threads=threads)
    acc_s = time.time() - t0
    return {
        "value": round(gbps, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "passes_per_s": w_per_s / total_w,
        "sample": (f"{layers} of 64 layers (7 matrices each, {weights} weights) of the 27B stack at "
                   f"K=1, {spent:.1f} s of fp64 oracle time on {threads} threads, scaled to the "
                   f"{total_w}-weight pass; plus {nwin} C4 acceptance windows (K 8, V 151936)"),
        "accept_windows_per_s": nwin / acc_s,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--sweep", default="4,8,16", help="other K values to time ('' for none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle time to sample")
    ap.add_argument("--threads", type=int, default=16, help="host threads for input generation")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip timing the other launch mode (e.g. under a profiler)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 1 GiB device copy (reference for HBM counter scaling)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the verify pass on one GPU; runs on more than one GPU are not "
              "part of this benchmark (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import speculative_decoding_verification_bit_amd as vq
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    shape = synth.SHAPE_27B
    H, V = shape.hidden, shape.vocab

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
    eager1 = time_eager(torch, step1, max(3, args.steps // 4))
    sbytes = stage_weight_bytes(shape, synth, synth.FMT_Q4_MIN)
    groups, n_launch = time_stream_kernel(torch, vq, model, x0_1, logits1, ws1, args.steps, vq.PATH_AUTO, sbytes)
    # the dominant kernel: the instantiation with the most time per pass
    dom = max(groups, key=lambda k: groups[k][1])
    n_dom, ms_dom, b_dom, raw_dom = groups[dom]
    avg_launch_ms = ms_dom / n_dom
    bytes_per_launch = b_dom / n_dom
    achieved = bytes_per_launch / (avg_launch_ms * 1e-3) / 1e9
    kname = {"single": "k_stage_valu<1, 1, false, false> (Q4_MIN, K 1, one chunk per item)",
             "multi": "k_stage_valu<1, 1, true, false> (Q4_MIN, K 1, chunk runs per item)",
             "rows": "k_rows_s<1, 1, NSG> (Q4_MIN, K 1, row strips)",
             "stream": "k_stream<1, 1> (Q4_MIN, K 1, stream-ahead)",
             "persistent": "k_pass<1, 1, false> (Q4_MIN, K 1, persistent)"}[dom]
    value = wbytes / (ms1 * 1e-3) / 1e9
    log(f"K=1 step {ms1:.3f} ms ({value:.0f} GB/s), eager {eager1:.3f} ms; launches per pass {n_launch}; "
        + "; ".join(f"{k}: {c:.0f} launches {t:.3f} ms ({r:.3f} ms bracketed) {b / t / 1e6:.0f} GB/s"
                    for k, (c, t, b, r) in groups.items()))
    del g1
    other1 = None
    if not args.no_compare:
        other = vq.LAUNCH_PERSISTENT if n_launch > 16 else vq.LAUNCH_STAGED
        other1 = time_graph(torch, lambda: vq.decode_pass(model, x0_1, logits1, path=other, ws=ws1),
                            args.steps, args.warmup)[0]
        log(f"K=1 pass with the other launch mode ({'persistent' if n_launch > 16 else 'staged'}): {other1:.3f} ms")
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms1, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16xf16->f32 (4-bit codes widened exactly to f16)",
        "data": "synthetic",
        "config": {"workload": synth.C2["name"], "layers": shape.n_layers, "hidden": H,
                   "kv": shape.kv_dim, "ffn": shape.ffn, "vocab": V, "K": 1,
                   "format": "q4 block-32 + fp16 scale + fp16 min", "weight_bytes": wbytes,
                   "accept": "sample T 0.6 top-p 0.95 min-p 0.05"},
        "passes_per_s": round(1000.0 / ms1, 2),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "implied_tok_s": round(1000.0 / ms1, 2),
        "eager_ms_per_step": round(eager1, 4),
        ("persistent_pass_ms" if n_launch > 16 else "staged_pass_ms"): other1 and round(other1, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": profiled_traffic(dom),
                     "kernel": kname, "launches_per_pass": round(n_dom),
                     "avg_launch_us": round(avg_launch_ms * 1e3, 3),
                     "event_bracketed_avg_launch_us": round(raw_dom / n_dom * 1e3, 3),
                     "bytes_per_launch": round(bytes_per_launch)},
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
            acc.probe = probe
            return acc

        step4, x0_4, logits4, ws4 = make_step(model, 4, agree)
        ms4, g4 = time_graph(torch, step4, args.steps, args.warmup)
        del g4
        # measured acceptance on the pass's own logits, fresh Philox windows
        t = logits4.view(1, 4, V).expand(2000, 4, V).contiguous()
        r = vq.verify_accept(vq.MODE_GREEDY, t, draft_mode=vq.DRAFT_AGREE, alpha=alpha, seed=0)
        am = torch.argmax(logits4, dim=1)[:3]
        agree_rate = float((r["draft_tokens"] == am.view(1, 3)).float().mean())
        tau_meas = float((r["n_accepted"] + 1).float().mean())
        del t, r
        ms4v = time_graph(torch, lambda: vq.decode_pass(model, x0_4, logits4, path=vq.PATH_VALU, ws=ws4),
                          args.steps, args.warmup)[0]
        ms4m = time_graph(torch, lambda: vq.decode_pass(model, x0_4, logits4, path=vq.PATH_MFMA, ws=ws4),
                          args.steps, args.warmup)[0]
        sweep["K4"] = {"workload": synth.C3["name"], "ms_per_step": round(ms4, 4),
                       "gbps": round(wbytes / ms4 / 1e6, 2), "passes_per_s": round(1000 / ms4, 2),
                       "frac_of_hbm_peak": round(wbytes / ms4 / 1e6 / HBM_PEAK_GBPS, 4),
                       "pass_ms_valu": round(ms4v, 4), "pass_ms_mfma": round(ms4m, 4),
                       "accept": "greedy, drafts agree with the target argmax at alpha 0.7",
                       "measured_alpha": round(agree_rate, 4), "measured_tau": round(tau_meas, 4),
                       "tau_at_alpha": round(tau(alpha, 3), 4),
                       "implied_tok_s": round(1000 / ms4 * tau_meas, 2)}
        log("K=4", sweep["K4"])
        del ws4
    if 8 in Ks:
        x0_8 = torch.from_numpy(synth.activations(0, 8, H)).to(dev)
        logits8 = torch.empty((8, V), dtype=torch.float32, device=dev)
        ws8 = torch.empty(model.workspace_bytes(8), dtype=torch.uint8, device=dev)
        ms8 = {}
        for name, path in (("auto", vq.PATH_AUTO), ("valu", vq.PATH_VALU), ("mfma", vq.PATH_MFMA)):
            ms8[name] = time_graph(torch, lambda: vq.decode_pass(model, x0_8, logits8, path=path, ws=ws8),
                                   args.steps, args.warmup)[0]
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
        acc_ms = time_eager(torch, lambda: vq.verify_accept(vq.MODE_SAMPLE, td, dd, out=r, **kw), 3)
        n_acc = r["n_accepted"].cpu().numpy()
        beta = [float((n_acc >= i).mean()) for i in range(1, 8)]
        tau8 = float((n_acc + 1).mean())
        del td, dd, r
        torch.cuda.empty_cache()
        best = min(ms8.values())
        sweep["K8"] = {"workload": synth.C4["name"], "ms_per_step": round(ms8["auto"], 4),
                       "gbps": round(wbytes / ms8["auto"] / 1e6, 2),
                       "passes_per_s": round(1000 / ms8["auto"], 2),
                       "frac_of_hbm_peak": round(wbytes / ms8["auto"] / 1e6 / HBM_PEAK_GBPS, 4),
                       "pass_ms_valu": round(ms8["valu"], 4), "pass_ms_mfma": round(ms8["mfma"], 4),
                       "ratio_to_K1_pass": round(best / ms1, 4),
                       "accept_ms_1000_windows": round(acc_ms, 4),
                       "accept_us_per_window": round(acc_ms * 1000 / W, 3),
                       "measured_tau": round(tau8, 4),
                       "reach_position": [round(b, 4) for b in beta],
                       "implied_tok_s": round(1000 / best * tau8, 2)}
        log("K=8", sweep["K8"])
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
        x0_1m = torch.from_numpy(synth.activations(0, 1, H)).to(dev)
        logits1m = torch.empty((1, V), dtype=torch.float32, device=dev)
        ws1m = torch.empty(mx.workspace_bytes(1), dtype=torch.uint8, device=dev)
        ms1m = time_graph(torch, lambda: vq.decode_pass(mx, x0_1m, logits1m, ws=ws1m), args.steps,
                          args.warmup)[0]
        sweep["K16"] = {"workload": synth.C5["name"], "weight_bytes": mbytes, "path": "mfma",
                        "ms_per_step": round(ms16, 4), "gbps": round(mbytes / ms16 / 1e6, 2),
                        "passes_per_s": round(1000 / ms16, 2),
                        "frac_of_hbm_peak": round(mbytes / ms16 / 1e6 / HBM_PEAK_GBPS, 4),
                        "mxfp4_K1_pass_ms": round(ms1m, 4)}
        log("K=16", sweep["K16"])
        del mx, ws16, ws1m
        torch.cuda.empty_cache()
    out["sweep"] = sweep

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = 1 << 30

    if not args.no_cpu:
        import oracle as oracle_mod
        log("CPU baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(synth, oracle_mod, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
