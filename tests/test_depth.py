"""Adaptive draft depth (host arithmetic in libvq: vq_depth_observe, vq_depth_choose) against
the oracle: the running statistics equal the oracle's fold (to the last bit: the same fp64
operations in the same order), and the chosen depth equals the oracle's argmax on synthetic
acceptance traces and random pass-time curves (where two rates tie within 1e-12 either
depth is valid).  No GPU: these entry points do only host arithmetic."""
import ctypes

import numpy as np
import pytest

import oracle
import speculative_decoding_verification_bit_amd as vq


def _windows(rng, alpha, k, W):
    """W windows of k drafts, each accepted with probability alpha until the first reject."""
    u = rng.random((W, k)) if k > 0 else np.zeros((W, 0))
    rej = u >= alpha
    n = np.where(rej.any(axis=1), rej.argmax(axis=1), k) if k > 0 else np.zeros(W, np.int64)
    return n.astype(np.int32), np.full(W, k, np.int32)


@pytest.mark.parametrize("decay", [1.0, 0.99, 0.5])
def test_observe_matches_oracle(decay):
    rng = np.random.default_rng(1)
    st = vq.VqDepthStats(0.0, 0.0)
    ref = (0.0, 0.0)
    for alpha, k in [(0.9, 7), (0.3, 3), (0.6, 15), (1.0, 4), (0.0, 2), (0.5, 0)]:
        n, d = _windows(rng, alpha, k, 500)
        vq.depth_observe(st, n, d, decay)
        ref = oracle.depth_observe(ref, n, d, decay)
        assert (st.accepted, st.rejected) == ref


def _close_choice(k, ref_k, rates):
    return k == ref_k or abs(rates[k] - rates[ref_k]) <= 1e-12 * rates[ref_k]


def test_choose_matches_oracle_on_random_curves():
    rng = np.random.default_rng(2)
    for _ in range(2000):
        kmax = int(rng.integers(0, 16))
        base = rng.uniform(1.0, 10.0)
        t = base * (1.0 + np.cumsum(rng.uniform(0.0, 0.2, kmax + 1)) - rng.uniform(0.0, 0.2))
        t = np.maximum(t, 1e-3)
        td = float(rng.choice([0.0, rng.uniform(0.0, 0.3) * base]))
        st = vq.VqDepthStats(float(rng.uniform(0, 100)), float(rng.uniform(0, 100)))
        prior, w = float(rng.uniform()), float(rng.choice([0.0, rng.uniform(0, 10)]))
        if st.accepted + st.rejected + w == 0:
            continue
        k, a, r = vq.depth_choose(st, t, td, prior, w)
        rk, ra, rates = oracle.depth_choose((st.accepted, st.rejected), prior, w, t, td)
        assert abs(a - ra) <= 1e-15 * max(1.0, ra)
        assert _close_choice(k, rk, rates), (k, rk)
        assert abs(r - rates[k]) <= 1e-12 * rates[k]


def test_adaptive_trace_matches_oracle():
    """A synthetic acceptance trace (alpha 0.85, then 0.3, then 0.65, 2000 windows each):
    observe each window, choose the next depth; library and oracle make the same choices."""
    rng = np.random.default_rng(3)
    t = 4.2 + 0.14 * np.arange(9)        # pass time with k drafts (ms), a linear stand-in
    st, ref = vq.VqDepthStats(0.0, 0.0), (0.0, 0.0)
    k = rk = 3
    ks = []
    for alpha in (0.85, 0.3, 0.65):
        for _ in range(2000):
            n, d = _windows(rng, alpha, k, 1)
            vq.depth_observe(st, n, d, 0.98)
            ref = oracle.depth_observe(ref, n, d, 0.98)
            k, _, _ = vq.depth_choose(st, t, 0.2, 0.5, 2.0)
            rk, _, rates = oracle.depth_choose(ref, 0.5, 2.0, t, 0.2)
            assert _close_choice(k, rk, rates)
            ks.append(k)
    ks = np.array(ks)
    # the depth follows the acceptance: deep while it is high, shallow while it is low
    assert ks[1500:2000].mean() > ks[3500:4000].mean() + 2
    assert ks[5500:6000].mean() > ks[3500:4000].mean()


@pytest.mark.parametrize("kw,code", [
    (dict(k_max=-1), vq.ERR_ARG), (dict(k_max=16), vq.ERR_ARG), (dict(alpha_prior=1.5), vq.ERR_ARG),
    (dict(prior_weight=-1.0), vq.ERR_ARG), (dict(t_draft=-0.1), vq.ERR_ARG), (dict(t_bad=0.0), vq.ERR_ARG),
    (dict(t_bad=float("nan")), vq.ERR_ARG), (dict(empty=True), vq.ERR_ARG),
])
def test_choose_argument_errors(kw, code):
    st = vq.VqDepthStats(0.0, 0.0) if kw.get("empty") else vq.VqDepthStats(3.0, 1.0)
    t = np.ones(8)
    if "t_bad" in kw:
        t[3] = kw["t_bad"]
    k = ctypes.c_int32(-7)
    rc = vq.lib.vq_depth_choose(ctypes.byref(st), kw.get("alpha_prior", 0.5), kw.get("prior_weight", 0.0),
                                t.ctypes.data, kw.get("k_max", 7), kw.get("t_draft", 0.1), ctypes.byref(k),
                                None, None)
    assert rc == code and k.value == -7
    assert vq.lib.vq_last_error()


def test_observe_argument_errors_leave_stats():
    st = vq.VqDepthStats(2.0, 1.0)
    n = np.array([1, 4], np.int32)
    d = np.array([3, 3], np.int32)
    assert vq.lib.vq_depth_observe(ctypes.byref(st), n.ctypes.data, d.ctypes.data, 2, 1.0) == vq.ERR_ARG
    assert (st.accepted, st.rejected) == (2.0, 1.0)
    assert vq.lib.vq_depth_observe(ctypes.byref(st), None, None, 0, 1.0) == vq.OK
    assert vq.lib.vq_depth_observe(ctypes.byref(st), n.ctypes.data, d.ctypes.data, 1, 0.0) == vq.ERR_ARG
    assert vq.lib.vq_depth_observe(None, n.ctypes.data, d.ctypes.data, 1, 1.0) == vq.ERR_ARG
