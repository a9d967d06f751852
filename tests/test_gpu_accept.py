"""GPU parity of vq_verify_accept against the fp64 oracle.

Greedy decisions compare identical fp32 logits and must agree on every window.  Sampling
must agree on every window whose oracle decisions are not within 1e-6 of a threshold
(ratio test, inverse-CDF draw, top-p or min-p cut); such windows are counted and printed.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import f32, need_gpu, report, say

pytestmark = pytest.mark.gpu


def _gpu(mode, t, d=None, dtok=None, draft_mode=0, T=1.0, top_p=1.0, min_p=0.0, alpha=0.0, seed=0,
         window_base=0, top_k=0):
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    td = torch.from_numpy(np.ascontiguousarray(t)).cuda()
    dd = None if d is None else torch.from_numpy(np.ascontiguousarray(d)).cuda()
    dt = None if dtok is None else torch.from_numpy(np.ascontiguousarray(dtok)).cuda()
    out = vq.verify_accept(mode, td, dd, dt, draft_mode, T, top_p, min_p, alpha, seed, window_base,
                           top_k=top_k)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}


def _oracle(mode, t, d=None, dtok=None, draft_mode=0, T=1.0, top_p=1.0, min_p=0.0, alpha=0.0, seed=0,
            window_base=0, top_k=0):
    return oracle.accept(mode, t, d, dtok, draft_mode, f32(T), f32(top_p), f32(min_p), f32(alpha), seed,
                         window_base, threads=8, top_k=top_k)


def _compare(g, o, exact: bool, what: str, max_near_frac=0.05):
    """Exact: every window agrees.  Otherwise every window agrees except those with an
    oracle decision within 1e-6 of its threshold (flagged), of which at most max_near_frac
    may exist; flagged windows are counted and reported whether or not they agree."""
    W = len(o["n_accepted"])
    same = ((g["n_accepted"] == o["n_accepted"]) & (g["status"] == o["status"])
            & np.all(g["tokens"] == o["tokens"], axis=1))
    if g.get("draft_tokens") is not None and o["draft_tokens"].size:
        same &= np.all(g["draft_tokens"] == o["draft_tokens"], axis=1)
    near = o["near"] != 0
    n_near, n_bad = int(near.sum()), int((~same).sum())
    n_bad_far = int((~same & ~near).sum())
    line = (f"{what}: {W} windows, flagged (within 1e-6 of a threshold) {n_near}, mismatches {n_bad} "
            f"(flagged {n_bad - n_bad_far}, unflagged {n_bad_far})")
    report(line)
    if exact:
        assert same.all(), f"{line}; windows {np.nonzero(~same)[0][:10]} differ"
    else:
        assert n_bad_far == 0, f"{line}; unflagged windows {np.nonzero(~same & ~near)[0][:10]} differ"
        assert n_near <= max_near_frac * W, f"{line}; more than {max_near_frac:.0%} of the windows flagged"
    return n_near


def test_c1_greedy_and_sampling():
    """10,000 windows, K = 4, V = 256, target ~N(0,2), drafter = target + N(0,0.5), T = 1."""
    c = synth.C1
    t, d = synth.logits_batch(c["logits"], 0, c["windows"], threads=16)
    o = _oracle(oracle.MODE_GREEDY, t, d, draft_mode=oracle.DRAFT_Q_ARGMAX)
    g = _gpu(0, t, d, draft_mode=1)
    _compare(g, o, True, "C1 greedy (drafter argmax)")
    kw = dict(draft_mode=oracle.DRAFT_Q_SAMPLE, T=c["T"], seed=c["philox_seed"])
    o = _oracle(oracle.MODE_SAMPLE, t, d, **kw)
    g = _gpu(1, t, d, **kw)
    _compare(g, o, False, "C1 sampling (x ~ q)")
    # mean tokens per pass near the product-of-overlaps expectation is an oracle pin;
    # here only the two sides' agreement is checked


def test_c4_sampler_settings_reduced_windows():
    """K = 8, V = 151936, target ~N(0,3), drafter + N(0,1), T 0.6, top-p 0.95, min-p 0.05."""
    c = synth.C4
    t, d = synth.logits_batch(c["logits"], 0, 48, threads=16)
    kw = dict(draft_mode=oracle.DRAFT_Q_SAMPLE, T=c["T"], top_p=c["top_p"], min_p=c["min_p"],
              seed=c["philox_seed"])
    o = _oracle(oracle.MODE_SAMPLE, t, d, **kw)
    g = _gpu(1, t, d, **kw)
    _compare(g, o, False, "C4 first 48 windows", max_near_frac=0.05)


@pytest.mark.parametrize("T,top_p,min_p", [(0.6, 0.9, 0.0), (0.6, 0.5, 0.0), (0.8, 0.9, 0.0),
                                            (1.0, 1.0, 0.1), (0.6, 0.95, 0.05)])
def test_top_p_radix_select_and_min_p(T, top_p, min_p):
    """Top-p without min-p needs the exact cut over the whole vocabulary (V = 151936).  The
    settings keep the cut's cumulative mass away from top_p on at least 95% of the windows
    (target logits ~N(0, 3)), so that the radix select is checked window by window."""
    spec = synth.LogitSpec(seed=7, K=3, vocab=151936, target_sigma=3.0, noise_sigma=1.0)
    t, d = synth.logits_batch(spec, 0, 40, threads=12)
    kw = dict(draft_mode=oracle.DRAFT_Q_SAMPLE, T=T, top_p=top_p, min_p=min_p, seed=5)
    o = _oracle(oracle.MODE_SAMPLE, t, d, **kw)
    g = _gpu(1, t, d, **kw)
    _compare(g, o, False, f"V 151936 T {T} top-p {top_p} min-p {min_p}", max_near_frac=0.05)


def test_single_window_k1_sampled_full_vocab():
    """One window, K = 1, V = 151936 (a sampled plain-decode step: the bonus token only);
    the row statistics run split over many workgroups.  Eight independent windows."""
    spec = synth.LogitSpec(seed=11, K=1, vocab=151936, target_sigma=3.0, noise_sigma=1.0)
    t, _ = synth.logits_batch(spec, 0, 8, threads=8)
    kw = dict(T=0.6, top_p=0.95, min_p=0.05, seed=3)
    gs, os_ = {}, {}
    for w in range(8):
        g = _gpu(1, t[w:w + 1], np.zeros((1, 0, spec.vocab), np.float32), window_base=w, **kw)
        o = _oracle(oracle.MODE_SAMPLE, t[w:w + 1], np.zeros((1, 0, spec.vocab), np.float32), window_base=w, **kw)
        for k in o:
            if g.get(k) is not None:
                gs.setdefault(k, []).append(g[k])
            os_.setdefault(k, []).append(o[k])
    gs = {k: np.concatenate(v) for k, v in gs.items()}
    os_ = {k: np.concatenate(v) for k, v in os_.items()}
    _compare(gs, os_, False, "K=1 single windows, T 0.6 top-p 0.95 min-p 0.05", max_near_frac=0.05)
    for w in range(8):
        g = _gpu(0, t[w:w + 1])
        assert g["tokens"][0, 0] == int(np.argmax(t[w, 0]))


def test_top_p_ties_resolved_by_index():
    """Equal logits at the top-p cut: the lower indices are kept first."""
    V, K, W = 64, 2, 400
    rng = np.random.default_rng(3)
    base = np.round(rng.standard_normal((W, K, V)) * 2).astype(np.float32)   # many exact ties
    d = (base[:, :1] + np.round(rng.standard_normal((W, 1, V)))).astype(np.float32)
    kw = dict(draft_mode=oracle.DRAFT_Q_SAMPLE, T=1.0, top_p=0.6, seed=2)
    o = _oracle(oracle.MODE_SAMPLE, base, d, **kw)
    g = _gpu(1, base, d, **kw)
    _compare(g, o, False, "integer logits (ties) top-p 0.6", max_near_frac=0.05)


def test_agree_drafter_greedy_full_vocab():
    """C3-style windows: drafts agree with the target argmax with alpha = 0.7 (exact)."""
    spec = synth.LogitSpec(seed=3, K=4, vocab=151936, target_sigma=3.0, noise_sigma=1.0)
    t, _ = synth.logits_batch(spec, 0, 64, threads=16)
    kw = dict(draft_mode=oracle.DRAFT_AGREE, alpha=0.7, seed=0)
    o = _oracle(oracle.MODE_GREEDY, t, **kw)
    g = _gpu(0, t, **kw)
    _compare(g, o, True, "agree alpha 0.7 greedy")
    kw = dict(draft_mode=oracle.DRAFT_Q_SAMPLE, T=0.6, top_p=0.95, min_p=0.05, seed=4)
    t2, d2 = synth.logits_batch(synth.LogitSpec(3, 4, 151936, 3.0, 1.0), 100, 116, threads=16)
    o = _oracle(oracle.MODE_GREEDY, t2, d2, **kw)
    g = _gpu(0, t2, d2, **kw)
    _compare(g, o, False, "greedy verify of sampled drafts", max_near_frac=0.05)


def test_edge_cases():
    rng = np.random.default_rng(9)
    # K = 1: plain decode
    t = rng.standard_normal((50, 1, 300)).astype(np.float32)
    for mode, kw in ((0, {}), (1, dict(T=0.7, top_p=0.9, min_p=0.02, seed=3))):
        o = _oracle(mode, t, np.zeros((50, 0, 300), np.float32), **kw)
        g = _gpu(mode, t, np.zeros((50, 0, 300), np.float32) if mode else None, **kw)
        _compare(g, o, mode == 0, f"K=1 mode {mode}")
    # V = 1
    t1 = rng.standard_normal((5, 3, 1)).astype(np.float32)
    dt = np.zeros((5, 2), np.int32)
    o = _oracle(0, t1, dtok=dt)
    g = _gpu(0, t1, dtok=dt)
    _compare(g, o, True, "V=1")
    # status: a NaN logit in window 1, an out-of-range draft in window 2
    t = rng.standard_normal((4, 3, 100)).astype(np.float32)
    d = (t[:, :2] + 0.3).astype(np.float32)
    t[1, 2, 50] = np.nan
    dt = rng.integers(0, 100, (4, 2)).astype(np.int32)
    dt[2, 1] = 100
    for mode in (0, 1):
        kw = dict(T=1.0) if mode else {}
        o = _oracle(mode, t, d if mode else None, dtok=dt, **kw)
        g = _gpu(mode, t, d if mode else None, dtok=dt, **kw)
        assert list(g["status"]) == [0, 1, 2, 0] == list(o["status"])
        _compare(g, o, mode == 0, f"status codes mode {mode}")
    # window_base: window w with base b == window w + b with base 0
    spec = synth.LogitSpec(seed=1, K=4, vocab=500, target_sigma=2.0, noise_sigma=0.5)
    t, d = synth.logits_batch(spec, 0, 40, threads=8)
    kw = dict(draft_mode=2, T=1.0, seed=11)
    a = _gpu(1, t[10:], d[10:], window_base=10, **kw)
    b = _gpu(1, t, d, **kw)
    assert np.array_equal(a["tokens"], b["tokens"][10:])
    assert np.array_equal(a["n_accepted"], b["n_accepted"][10:])
    # W = 0 is a no-op
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    out = vq.verify_accept(0, torch.zeros((0, 3, 10), device="cuda"))
    assert out["tokens"].shape == (0, 3)


def test_c4_full_size_all_windows():
    """All 1,000 C4 windows (K 8, V 151936, 9.1 GB of logits) on the GPU in one call, every
    window against the oracle (which consumes the same counter-based uniforms)."""
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    c = synth.C4
    spec = c["logits"]
    W = c["windows"]
    td = torch.empty((W, spec.K, spec.vocab), dtype=torch.float32, device="cuda")
    dd = torch.empty((W, spec.K - 1, spec.vocab), dtype=torch.float32, device="cuda")
    okw = dict(draft_mode=oracle.DRAFT_Q_SAMPLE, T=c["T"], top_p=c["top_p"], min_p=c["min_p"],
               seed=c["philox_seed"])
    o = {}
    for w0 in range(0, W, 100):
        t, d = synth.logits_batch(spec, w0, w0 + 100, threads=16)
        td[w0:w0 + 100].copy_(torch.from_numpy(t))
        dd[w0:w0 + 100].copy_(torch.from_numpy(d))
        r = oracle.accept(oracle.MODE_SAMPLE, t, d, None, window_base=w0, threads=16,
                          **{k: (f32(v) if k in ("T", "top_p", "min_p") else v) for k, v in okw.items()})
        for k, v in r.items():
            o.setdefault(k, []).append(v)
        say(f"C4 windows {w0}..{w0 + 99}: uploaded, oracle done")
    o = {k: np.concatenate(v) for k, v in o.items()}
    out = vq.verify_accept(1, td, dd, **okw)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    del td, dd
    torch.cuda.empty_cache()
    assert np.all(g["status"] == 0)
    _compare(g, o, False, "C4 all 1000 windows (K 8, V 151936, T 0.6, top-p 0.95, min-p 0.05)",
             max_near_frac=0.05)
    emitted = g["n_accepted"] + 1
    report(f"C4 mean tokens per pass {emitted.mean():.3f} (oracle {(o['n_accepted'] + 1).mean():.3f})")


# (top-p cuts deep in the tail, where each token adds ~1e-6 of mass, flag most windows as
# near the threshold; the top-p settings here keep the cut in the head)
@pytest.mark.parametrize("top_k,top_p,min_p", [(40, 1.0, 0.0), (40, 0.95, 0.05), (2000, 0.6, 0.0),
                                              (1, 1.0, 0.0), (151936, 0.9, 0.0), (7, 0.5, 0.0)])
def test_top_k_cut_full_vocab(top_k, top_p, min_p):
    """The top-k cut (a count radix select) alone and with top-p / min-p, over V = 151936
    (80 windows): the kept set is the shortest of the prefixes; k = 1 is the argmax; k >= V
    no cut."""
    spec = synth.LogitSpec(seed=13, K=3, vocab=151936, target_sigma=3.0, noise_sigma=1.0)
    t, d = synth.logits_batch(spec, 0, 80, threads=16)
    kw = dict(draft_mode=oracle.DRAFT_Q_SAMPLE, T=0.7, top_p=top_p, min_p=min_p, seed=6, top_k=top_k)
    o = _oracle(oracle.MODE_SAMPLE, t, d, **kw)
    g = _gpu(1, t, d, **kw)
    _compare(g, o, False, f"V 151936 top-k {top_k} top-p {top_p} min-p {min_p}", max_near_frac=0.05)


def test_top_k_ties_at_the_cut():
    """Integer logits (runs of equal values straddle the k-th entry): lower indices first."""
    V, K, W = 300, 3, 300
    rng = np.random.default_rng(8)
    t = np.round(rng.standard_normal((W, K, V)) * 1.5).astype(np.float32)
    d = (t[:, :K - 1] + np.round(rng.standard_normal((W, K - 1, V)))).astype(np.float32)
    for top_k in (3, 17, 150):
        kw = dict(draft_mode=oracle.DRAFT_Q_SAMPLE, T=1.0, top_k=top_k, seed=9)
        o = _oracle(oracle.MODE_SAMPLE, t, d, **kw)
        g = _gpu(1, t, d, **kw)
        _compare(g, o, False, f"integer logits (ties) top-k {top_k}", max_near_frac=0.05)


def test_top_k_single_window_split_stats():
    """K = 1 single windows over V = 151936 (the row statistics run split over many
    workgroups) with top-k 50 and the production sampler."""
    spec = synth.LogitSpec(seed=17, K=1, vocab=151936, target_sigma=3.0, noise_sigma=1.0)
    t, _ = synth.logits_batch(spec, 0, 6, threads=8)
    kw = dict(T=0.6, top_p=0.95, min_p=0.05, seed=4, top_k=50)
    for w in range(6):
        e = np.zeros((1, 0, spec.vocab), np.float32)
        g = _gpu(1, t[w:w + 1], e, window_base=w, **kw)
        o = _oracle(oracle.MODE_SAMPLE, t[w:w + 1], e, window_base=w, **kw)
        _compare(g, o, False, f"K=1 window {w} top-k 50", max_near_frac=1.0)


def test_negative_zero_logits_tie_with_positive_zero():
    """-0.0 and +0.0 logits are equal: at a cut inside a run of zeros, the lower indices are
    kept first whichever sign the zeros carry (top-k and top-p)."""
    V, K, W = 64, 2, 200
    rng = np.random.default_rng(12)
    t = np.round(rng.standard_normal((W, K, V))).astype(np.float32)
    t[np.abs(t) == 0] = np.where(rng.random(int((t == 0).sum())) < 0.5, np.float32(-0.0), np.float32(0.0))
    d = (t[:, :1] + np.round(rng.standard_normal((W, 1, V)))).astype(np.float32)
    assert np.signbit(t[t == 0]).any() and (~np.signbit(t[t == 0])).any()
    for kw in (dict(top_k=30), dict(top_p=0.7)):
        kw.update(draft_mode=oracle.DRAFT_Q_SAMPLE, T=1.0, seed=3)
        o = _oracle(oracle.MODE_SAMPLE, t, d, **kw)
        g = _gpu(1, t, d, **kw)
        _compare(g, o, False, f"signed zeros {kw}", max_near_frac=0.05)
