"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test ties an oracle function to something outside the oracle: a value the pages
print, a closed form, an independent library routine (numpy, scipy), an invariant, or
a brute-force count on a tiny input.
"""
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


# ----------------------------------------------------------------- formats

def test_half_matches_numpy_all_bit_patterns():
    """fp16 decode vs numpy's float16 -> float64 conversion, all 65536 encodings."""
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.half_array(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_e2m1_table_ocp_mx():
    """The 16 E2M1 code points of the OCP Microscaling Formats spec v1.0 (FP4 table)."""
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        assert oracle.e2m1(c) == mags[c]
        assert oracle.e2m1(c + 8) == -mags[c]
        assert np.signbit(oracle.e2m1(c + 8))


def test_e8m0_scale():
    """E8M0: 2^(E-127), E = 255 is NaN (OCP MX v1.0)."""
    assert oracle.e8m0(127) == 1.0
    assert oracle.e8m0(119) == 2.0 ** -8
    assert oracle.e8m0(123) == 2.0 ** -4
    assert oracle.e8m0(254) == 2.0 ** 127
    assert oracle.e8m0(0) == 2.0 ** -127
    assert np.isnan(oracle.e8m0(255))


def _pack_q4(q):
    """Encode signed codes q in [-8, 7] ([rows][cols]) as bytes: low nibble = even column."""
    n = (np.asarray(q) + 8).astype(np.uint8)
    return (n[:, 0::2] | (n[:, 1::2] << 4)).astype(np.uint8)


def test_q4_roundtrip_from_encoding():
    """Codes written by the inverse map (n = q + 8, even column low nibble) decode to d*q + m."""
    rng = np.random.default_rng(3)
    rows, cols = 5, 96
    q = rng.integers(-8, 8, size=(rows, cols))
    # scales and mins that are exact in fp16 (k / 1024), so d*q + m is exact in double
    d = (rng.integers(1, 64, size=(rows, cols // 32)) / 1024.0).astype(np.float16)
    m = (rng.integers(-16, 17, size=(rows, cols // 32)) / 1024.0).astype(np.float16)
    for fmt, mins in ((synth.FMT_Q4, None), (synth.FMT_Q4_MIN, m)):
        W = synth.Q4Matrix(fmt, rows, cols, _pack_q4(q), d, mins)
        got = oracle.dequant(W)
        dd = np.repeat(d.astype(np.float64), 32, axis=1)
        mm = 0.0 if mins is None else np.repeat(m.astype(np.float64), 32, axis=1)
        assert np.array_equal(got, dd * q + mm)


def test_q4_nibble_order_single_byte():
    """Byte 0x8F: column 0 has code 15 (q = 7), column 1 has code 8 (q = 0)."""
    qs = np.zeros((1, 16), np.uint8)
    qs[0, 0] = 0x8F
    qs[0, 1:] = 0x88
    W = synth.Q4Matrix(synth.FMT_Q4, 1, 32, qs, np.array([[1.0]], np.float16), None)
    w = oracle.dequant(W)[0]
    assert w[0] == 7.0 and w[1] == 0.0 and np.all(w[2:] == 0.0)


def test_mxfp4_roundtrip():
    """MXFP4 codes decode to e2m1(code) * 2^(E-127); low nibble = even column."""
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 16, size=(3, 64)).astype(np.uint8)
    qs = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    E = rng.integers(119, 124, size=(3, 2)).astype(np.uint8)
    W = synth.Q4Matrix(synth.FMT_MXFP4, 3, 64, qs, E, None)
    got = oracle.dequant(W)
    mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6] * 2) * np.repeat([1.0, -1.0], 8)
    ref = mags[codes] * np.repeat(2.0 ** (E.astype(np.float64) - 127), 32, axis=1)
    assert np.array_equal(got, ref)


def test_mxfp4_values_exact_in_fp16():
    """Every C5 weight (|code| <= 6, scale 2^-8..2^-4) is exactly representable in fp16."""
    mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    for e in range(119, 124):
        v = mags * 2.0 ** (e - 127)
        assert np.array_equal(v.astype(np.float16).astype(np.float64), v)


def _q4k(rows, cols, codes, s, m, d, dmin):
    """A Q4_K matrix from unsigned codes [rows][cols], sub-block s and m [rows][cols/32]
    and super-block d, dmin [rows][cols/256]."""
    n = np.asarray(codes, np.uint8)
    qs = (n[:, 0::2] | (n[:, 1::2] << 4)).astype(np.uint8)
    sup = np.stack([np.asarray(d, np.float64), np.asarray(dmin, np.float64)], axis=-1).astype(np.float16)
    return synth.Q4Matrix(synth.FMT_Q4_K, rows, cols, qs, np.asarray(s, np.uint8), np.asarray(m, np.uint8), sup)


def test_q4k_worked_example():
    """The hand-computed worked example in tests/golden/q4k_worked_example.txt."""
    codes = (np.arange(256) % 16)[None, :]
    W = _q4k(1, 256, codes, [[1, 2, 3, 4, 5, 6, 7, 63]], [[0, 1, 2, 3, 4, 5, 6, 63]], [[0.5]], [[0.125]])
    w = oracle.dequant(W)[0]
    seen = 0
    for line in _golden_rows("q4k_worked_example.txt"):
        kind, idx, val = line.split()
        idx, val = int(idx), float(val)
        got = w[32 * idx:32 * idx + 32].sum() if kind == "sum" else w[idx]
        assert got == val, (kind, idx, got, val)
        seen += 1
    assert seen == 13


def test_q4k_super_block_index_and_roles():
    """Two rows of two super-blocks, all codes 15, s = m = 1: where d = 1, dmin = 0 every
    weight is 15, where d = 0, dmin = 1 it is -1; the roles swap between the rows."""
    codes = np.full((2, 512), 15)
    ones = np.ones((2, 16))
    W = _q4k(2, 512, codes, ones, ones, [[1, 0], [0, 1]], [[0, 1], [1, 0]])
    w = oracle.dequant(W)
    assert np.all(w[0, :256] == 15) and np.all(w[0, 256:] == -1)
    assert np.all(w[1, :256] == -1) and np.all(w[1, 256:] == 15)


def test_q4k_reduces_to_q4_min():
    """d*s*n - dmin*m = (d*s)*(n - 8) + (8*d*s - dmin*m): a Q4_K matrix equals the Q4_MIN
    matrix with block scale d*s and block min 8*d*s - dmin*m, same codes.  With d, dmin in
    {1..4}/1024 and s, m < 64 both are exact in fp16, so the two decodings agree exactly."""
    rng = np.random.default_rng(11)
    rows, cols = 7, 768
    nb, ns = cols // 32, cols // 256
    codes = rng.integers(0, 16, size=(rows, cols))
    s = rng.integers(0, 64, size=(rows, nb))
    m = rng.integers(0, 64, size=(rows, nb))
    d = rng.integers(1, 5, size=(rows, ns)) / 1024.0
    dmin = rng.integers(1, 5, size=(rows, ns)) / 1024.0
    K = _q4k(rows, cols, codes, s, m, d, dmin)
    ds = np.repeat(d, 8, axis=1) * s
    mm = 8 * ds - np.repeat(dmin, 8, axis=1) * m
    assert np.array_equal(ds.astype(np.float16).astype(np.float64), ds)
    assert np.array_equal(mm.astype(np.float16).astype(np.float64), mm)
    M = synth.Q4Matrix(synth.FMT_Q4_MIN, rows, cols, K.qs, ds.astype(np.float16), mm.astype(np.float16))
    assert np.array_equal(oracle.dequant(K), oracle.dequant(M))


def test_q4k_synthetic_weights_are_centred():
    """The generator's Q4_K weights: s in 16..63, m in 0..63, mean weight small beside the spread."""
    W = synth.weight_matrix(synth.FMT_Q4_K, 3, 0, 0, 64, 1024)
    assert W.scales.min() >= 16 and W.scales.max() <= 63 and W.mins.max() <= 63
    w = oracle.dequant(W)
    assert abs(w.mean()) < 0.1 * w.std()


def test_q4k_rejects_cols_not_multiple_of_256():
    W = synth.Q4Matrix(synth.FMT_Q4_K, 1, 32, np.zeros((1, 16), np.uint8), np.zeros((1, 1), np.uint8),
                       np.zeros((1, 1), np.uint8), np.zeros((1, 1, 2), np.float16))
    with pytest.raises(ValueError):
        oracle.linear(W, np.zeros((1, 32), np.float16))


# ------------------------------------------------------------------ linear

def _small_matrix(fmt=synth.FMT_Q4_MIN, rows=40, cols=128, seed=7):
    if fmt == synth.FMT_Q4_K:
        cols = 512
    return synth.weight_matrix(fmt, seed, 0, 0, rows, cols)


@pytest.mark.parametrize("fmt", [synth.FMT_Q4, synth.FMT_Q4_MIN, synth.FMT_MXFP4, synth.FMT_Q4_K])
def test_linear_vs_numpy_matmul(fmt):
    """W x agrees with numpy's float64 matmul of the dequantised matrix (library routine)."""
    W = _small_matrix(fmt)
    x = synth.activations(1, 3, W.cols)
    y, a = oracle.linear(W, x)
    ref = x.astype(np.float64) @ oracle.dequant(W).T
    assert np.all(np.abs(y - ref) <= 1e-12 * a + 1e-300)
    assert np.all(a >= np.abs(y))


def test_linear_unit_vectors_recover_columns():
    """x = e_j returns column j of W exactly."""
    W = _small_matrix(rows=17, cols=64)
    Wd = oracle.dequant(W)
    x = np.zeros((64, 64), np.float16)
    x[np.arange(64), np.arange(64)] = 1.0
    y, _ = oracle.linear(W, x)
    assert np.array_equal(y, Wd.T)


def test_linear_hand_cases():
    """One block: q = 7, d = 0.5, m = 0 gives 3.5 * sum(x); q = 0 gives m * sum(x)."""
    x = synth.activations(2, 2, 32)
    xs = x.astype(np.float64).sum(axis=1)
    W7 = synth.Q4Matrix(synth.FMT_Q4, 1, 32, np.full((1, 16), 0xFF, np.uint8),
                        np.array([[0.5]], np.float16), None)
    y, _ = oracle.linear(W7, x)
    assert np.allclose(y[:, 0], 3.5 * xs, rtol=1e-15, atol=1e-15)
    m = np.float16(0.0078125)
    W0 = synth.Q4Matrix(synth.FMT_Q4_MIN, 1, 32, np.full((1, 16), 0x88, np.uint8),
                        np.array([[0.5]], np.float16), np.array([[m]], np.float16))
    y, _ = oracle.linear(W0, x)
    assert np.allclose(y[:, 0], float(m) * xs, rtol=1e-15, atol=1e-15)


def test_linear_linearity_and_zero_row():
    """y(x1 + x2) = y(x1) + y(x2) (inputs chosen so the fp16 sum is exact); zero rows give 0."""
    W = _small_matrix(rows=9, cols=96)
    qs = W.qs.copy()
    qs[4] = 0x88                                # row 4: every code q = 0
    mins = W.mins.copy()
    mins[4] = 0
    W = synth.Q4Matrix(W.fmt, W.rows, W.cols, qs, W.scales, mins)
    rng = np.random.default_rng(5)
    x1 = (rng.integers(-64, 64, size=(2, 96)) / 64).astype(np.float16)
    x2 = (rng.integers(-64, 64, size=(2, 96)) / 64).astype(np.float16)
    y1, _ = oracle.linear(W, x1)
    y2, _ = oracle.linear(W, x2)
    y12, a12 = oracle.linear(W, (x1.astype(np.float32) + x2).astype(np.float16))
    assert np.allclose(y12, y1 + y2, rtol=0, atol=1e-12)
    assert np.all(y12[:, 4] == 0.0) and np.all(a12[:, 4] == 0.0)


# -------------------------------------------------------------------- glue

def test_rho_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((3, 1000)).astype(np.float32) * np.float32(7.5)
    r = oracle.rho(v)
    assert np.allclose(np.sqrt((r ** 2).mean(axis=1)), 1.0, rtol=1e-14)
    r2 = oracle.rho(v * np.float32(4.0))      # power-of-two scaling is exact in fp32
    assert np.allclose(r, r2, rtol=1e-14)


def test_silu_mul_vs_scipy():
    rng = np.random.default_rng(7)
    g = rng.standard_normal(1000).astype(np.float32) * 4
    u = rng.standard_normal(1000).astype(np.float32)
    ref = g.astype(np.float64) * scipy.special.expit(g.astype(np.float64)) * u
    assert np.allclose(oracle.silu_mul(g, u), ref, rtol=1e-13, atol=1e-300)


# ------------------------------------------------------------------ Philox

def test_philox_matches_numpy_philox():
    """Philox4x64-10 vs numpy.random.Philox, an independent implementation of Salmon et al.

    numpy increments the 256-bit counter before each block, so starting it at c - 1
    yields the block for counter c.
    """
    rng = np.random.default_rng(8)
    for _ in range(200):
        key = rng.integers(0, 2 ** 63, size=2, dtype=np.uint64) * np.uint64(2) + \
            rng.integers(0, 2, size=2, dtype=np.uint64)
        ctr = rng.integers(1, 2 ** 63, size=4, dtype=np.uint64)
        prev = ctr.copy()
        prev[0] -= np.uint64(1)
        bg = np.random.Philox(key=key, counter=prev)
        assert np.array_equal(bg.random_raw(4).astype(np.uint64), oracle.philox4x64(ctr, key))
    for w in (0, 1, 9999, 2 ** 40 + 3):
        for i in (1, 2, 8, 16):
            prev = np.array([w - 1 if w else 2 ** 64 - 1, i if w else i - 1, 0, 0], np.uint64)
            bg = np.random.Philox(key=np.array([5, 0], np.uint64), counter=prev)
            ref = bg.random_raw(4).astype(np.uint64)
            assert np.array_equal(ref, oracle.philox4x64([w, i, 0, 0], [5, 0]))


def test_uniforms_definition_and_chi_square():
    """u = top 24 bits * 2^-24 in [0, 1); 2^16 draws pass a 64-bin chi-square at 1e-3."""
    r = oracle.philox4x64([17, 3, 0, 0], [11, 0])
    u = oracle.uniforms(11, 17, 3)
    assert np.array_equal(u, (r >> np.uint64(40)).astype(np.float64) / 2.0 ** 24)
    draws = np.concatenate([oracle.uniforms(2, w, 1) for w in range(16384)])
    assert draws.min() >= 0.0 and draws.max() < 1.0
    counts = np.histogram(draws, bins=64, range=(0, 1))[0]
    assert scipy.stats.chisquare(counts).pvalue > 1e-3
    assert len(set(map(tuple, [oracle.philox4x64([w, 1, 0, 0], [2, 0]) for w in range(64)]))) == 64


# -------------------------------------------------------------------- warp

def test_warp_no_filters_is_softmax():
    rng = np.random.default_rng(9)
    l = rng.standard_normal(300).astype(np.float32) * 3
    for T in (1.0, 0.6, 2.5):
        p, info = oracle.warp(l, T)
        ref = scipy.special.softmax(l.astype(np.float64) / T)
        assert np.allclose(p, ref, rtol=1e-12, atol=1e-300)
        assert info.n_keep == 300


def test_warp_hand_case():
    """pi = (.5, .3, .15, .05), top_p .75, min_p .2: top-p keeps 2, min-p keeps 3 -> keep 2."""
    pi = np.array([0.5, 0.3, 0.15, 0.05])
    l = np.log(pi).astype(np.float32)
    p, info = oracle.warp(l, 1.0, top_p=0.75, min_p=0.2)
    assert info.m_p == 2 and info.m_m == 3 and info.n_keep == 2
    assert np.allclose(p, [0.625, 0.375, 0, 0], rtol=1e-6)
    # min-p alone at 0.35 keeps pi >= .175: 2 tokens; top-p alone at 0.9 keeps 3
    assert oracle.warp(l, 1.0, min_p=0.35)[1].n_keep == 2
    assert oracle.warp(l, 1.0, top_p=0.9)[1].n_keep == 3


def test_warp_invariants_and_monotone_subsets():
    rng = np.random.default_rng(10)
    for _ in range(20):
        l = rng.standard_normal(500).astype(np.float32) * 3
        prev = None
        for top_p, min_p in ((1.0, 0.0), (0.99, 0.0), (0.95, 0.01), (0.9, 0.05), (0.5, 0.2)):
            p, info = oracle.warp(l, 0.6, top_p, min_p)
            keep = p > 0
            assert abs(p.sum() - 1) < 1e-12
            assert keep[np.argmax(l)]
            if prev is not None:
                assert np.all(prev | ~keep)           # subset of the looser setting
            prev = keep
            # the kept set is a prefix of the (logit desc, index asc) order
            order = np.lexsort((np.arange(500), -l.astype(np.float64)))
            assert np.all(keep[order][:info.n_keep]) and not np.any(keep[order][info.n_keep:])


def test_warp_zero_temperature_and_ties():
    l = np.array([1.0, 3.0, 3.0, -2.0], np.float32)
    p, info = oracle.warp(l, 0.0)
    assert np.array_equal(p, [0, 1, 0, 0]) and info.argmax == 1
    assert oracle.argmax(l) == 1
    p, _ = oracle.warp(l, 1e-3, top_p=0.4)            # the tie breaks to the lower index
    assert p[1] == 1.0


def test_warp_top_p_matches_brute_force():
    """Shortest prefix of the sorted order with mass >= top_p, by exhaustive count."""
    rng = np.random.default_rng(11)
    for _ in range(50):
        l = rng.standard_normal(40).astype(np.float32) * 2
        top_p = float(rng.uniform(0.05, 0.99))
        p, info = oracle.warp(l, 1.0, top_p=top_p)
        pi = scipy.special.softmax(l.astype(np.float64))
        order = np.lexsort((np.arange(40), -pi))
        m = next(m for m in range(1, 41) if pi[order[:m]].sum() >= top_p)
        assert info.n_keep == m


# --------------------------------------------------------------- categorical

def test_cat_inverse_cdf_brute_force():
    w = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    assert oracle.cat(w, 0.0)[0] == 1
    assert oracle.cat(w, 0.2499)[0] == 1
    assert oracle.cat(w, 0.25)[0] == 3            # C_j > u*S is strict
    assert oracle.cat(w, 0.7499)[0] == 3
    assert oracle.cat(w, 0.9999)[0] == 4
    rng = np.random.default_rng(12)
    draws = np.array([oracle.cat(w, u)[0] for u in rng.random(20000)])
    counts = np.bincount(draws, minlength=5)
    assert counts[0] == 0 and counts[2] == 0
    assert scipy.stats.chisquare(counts[[1, 3, 4]], 20000 * w[[1, 3, 4]]).pvalue > 1e-3


# ------------------------------------------------------------------ greedy

def test_greedy_worked_example():
    """The "D E F" example (Hacker News thread 49596054), tokens A..H = 0..7, V = 8."""
    tok = {c: i for i, c in enumerate("ABCDEFGH")}
    for line in _golden_rows("greedy_worked_example.txt"):
        drafts, target, emitted = (s.split() for s in line.split("|"))
        K = len(drafts) + 1
        logits = np.zeros((1, K, 8), np.float32)
        for i, c in enumerate(target + ["A"]):       # bonus position: unrelated token
            logits[0, i, tok[c]] = 5.0
        out = oracle.accept(oracle.MODE_GREEDY, logits,
                            draft_tokens=np.array([[tok[c] for c in drafts]], np.int32))
        n = int(out["n_accepted"][0])
        got = [ "ABCDEFGH"[t] for t in out["tokens"][0, : n + 1]]
        assert got == emitted
        assert np.all(out["tokens"][0, n + 1:] == -1)


def test_greedy_invariants():
    """1 <= emitted <= K; emitted tokens are the target argmaxes; full accept emits K."""
    rng = np.random.default_rng(13)
    W, K, V = 500, 5, 16
    t = rng.standard_normal((W, K, V)).astype(np.float32)
    am = t.argmax(axis=2)
    drafts = np.where(rng.random((W, K - 1)) < 0.6, am[:, : K - 1],
                      rng.integers(0, V, size=(W, K - 1))).astype(np.int32)
    out = oracle.accept(oracle.MODE_GREEDY, t, draft_tokens=drafts)
    for w in range(W):
        n = out["n_accepted"][w]
        assert 0 <= n <= K - 1
        assert np.array_equal(out["tokens"][w, : n + 1], am[w, : n + 1])
        match = drafts[w] == am[w, : K - 1]
        expect_n = K - 1 if match.all() else int(np.argmin(match))
        assert n == expect_n


def _tau(alpha, k):
    return (1 - alpha ** (k + 1)) / (1 - alpha)


def test_tau_formula_matches_printed_table():
    """The closed form reproduces the printed 18-cell table to its 2 decimals."""
    for line in _golden_rows("tau_table.txt"):
        a, *vals = map(float, line.split())
        for k, v in zip((1, 3, 5), vals):
            assert abs(_tau(a, k) - v) <= 0.005 + 1e-12


def test_ceilings_and_inverse_checks_printed_on_the_pages():
    """Ceiling = bandwidth / bytes per pass; 82 tok/s over a 59 passes/s ceiling is >= 1.4
    tokens/pass; 1.8-2 tokens at k = 3 puts acceptance at about 0.47-0.54."""
    for line in _golden_rows("ceilings.txt"):
        bw, gb, printed = map(float, line.split())
        assert abs(bw / gb - printed) < 1.0
    assert abs(82 / 59 - 1.4) < 0.05
    from scipy.optimize import brentq
    a18 = brentq(lambda a: _tau(a, 3) - 1.8, 0.01, 0.99)
    a20 = brentq(lambda a: _tau(a, 3) - 2.0, 0.01, 0.99)
    assert abs(a18 - 0.47) < 0.01 and abs(a20 - 0.54) < 0.01


@pytest.mark.parametrize("alpha,k", [(0.9, 5), (0.7, 3), (0.5, 1), (0.35, 5), (0.8, 3)])
def test_greedy_monte_carlo_tokens_per_pass(alpha, k):
    """Drafts agreeing independently with prob alpha give mean (1 - alpha^(k+1))/(1 - alpha)
    tokens per pass (4.69 at alpha 0.9, k 5)."""
    K, V, W = k + 1, 32, 40000
    rng = np.random.default_rng(14)
    t = rng.standard_normal((W, K, V)).astype(np.float32)
    out = oracle.accept(oracle.MODE_GREEDY, t, draft_mode=oracle.DRAFT_AGREE,
                        alpha=alpha, seed=3, threads=8)
    emitted = out["n_accepted"] + 1
    se = emitted.std() / np.sqrt(W)
    assert abs(emitted.mean() - _tau(alpha, k)) < 4.5 * se
    # every pass emits at least one token
    assert emitted.min() >= 1
    # the per-position agreement rate is alpha
    am = t.argmax(axis=2)[:, :k]
    agree = (out["draft_tokens"] == am).mean()
    assert abs(agree - alpha) < 4.5 * np.sqrt(alpha * (1 - alpha) / (W * k))


# ---------------------------------------------------------------- sampling

def _fixed_rows(V, K, rng, sigma=1.5, noise=0.8):
    t = (rng.standard_normal((K, V)) * sigma).astype(np.float32)
    d = (t[: K - 1] + rng.standard_normal((K - 1, V)) * noise).astype(np.float32)
    return t, d


def _tile(a, W):
    return np.ascontiguousarray(np.broadcast_to(a, (W,) + a.shape))


def test_sampling_acceptance_rate_is_overlap():
    """P(accept x_1) = sum_x min(p(x), q(x)), x_1 ~ q (99.9% binomial interval)."""
    rng = np.random.default_rng(15)
    V, K, W = 8, 2, 200000
    t, d = _fixed_rows(V, K, rng)
    for T, top_p, min_p in ((1.0, 1.0, 0.0), (0.6, 0.95, 0.05)):
        out = oracle.accept(oracle.MODE_SAMPLE, _tile(t, W), _tile(d, W),
                            draft_mode=oracle.DRAFT_Q_SAMPLE, T=T, top_p=top_p, min_p=min_p,
                            seed=21, threads=8)
        p, _ = oracle.warp(t[0], T, top_p, min_p)
        q, _ = oracle.warp(d[0], T, top_p, min_p)
        beta = np.minimum(p, q).sum()
        rate = (out["n_accepted"] >= 1).mean()
        assert abs(rate - beta) < 3.3 * np.sqrt(beta * (1 - beta) / W)


def test_sampling_one_hot_drafter_accepts_with_p():
    """A greedy (one-hot) drafter at x is accepted with probability p(x)."""
    rng = np.random.default_rng(16)
    V, W = 8, 200000
    t, _ = _fixed_rows(V, 2, rng)
    d = np.zeros((1, V), np.float32)
    x = 3
    d[0, x] = 200.0                                  # q is one-hot at x in double
    out = oracle.accept(oracle.MODE_SAMPLE, _tile(t, W), _tile(d, W),
                        draft_mode=oracle.DRAFT_Q_SAMPLE, seed=5, threads=8)
    assert np.all(out["draft_tokens"] == x)
    p, _ = oracle.warp(t[0], 1.0)
    rate = (out["n_accepted"] >= 1).mean()
    assert abs(rate - p[x]) < 3.3 * np.sqrt(p[x] * (1 - p[x]) / W)


def test_sampling_lossless_chi_square():
    """The token at output index j is distributed as p_{j+1} (target-only sampling):
    V = 8, K = 4, fixed p and q, 10^6 windows, chi-square per index, Bonferroni 1e-3."""
    rng = np.random.default_rng(17)
    V, K, W = 8, 4, 1_000_000
    t, d = _fixed_rows(V, K, rng)
    out = oracle.accept(oracle.MODE_SAMPLE, _tile(t, W), _tile(d, W),
                        draft_mode=oracle.DRAFT_Q_SAMPLE, seed=9, threads=8)
    n = out["n_accepted"]
    assert n.min() >= 0 and n.max() <= K - 1
    for j in range(K):
        sel = n >= j
        toks = out["tokens"][sel, j]
        counts = np.bincount(toks, minlength=V)
        p, _ = oracle.warp(t[j], 1.0)
        assert scipy.stats.chisquare(counts, counts.sum() * p).pvalue > 1e-3 / K


def test_sampling_lossless_pit_on_fresh_windows():
    """C1-like windows (fresh p per window): the randomized probability-integral transform
    of the first emitted token under p_1 is U(0,1) (chi-square over 20 bins)."""
    spec = synth.LogitSpec(seed=0, K=4, vocab=256, target_sigma=2.0, noise_sigma=0.5)
    t, d = synth.logits_batch(spec, 0, 20000, threads=8)
    out = oracle.accept(oracle.MODE_SAMPLE, t, d, draft_mode=oracle.DRAFT_Q_SAMPLE,
                        seed=0, threads=8)
    rng = np.random.default_rng(18)
    v = np.empty(len(t))
    for w in range(len(t)):
        p, _ = oracle.warp(t[w, 0], 1.0)
        tok = out["tokens"][w, 0]
        F = np.cumsum(p)
        lo = F[tok - 1] if tok else 0.0
        v[w] = lo + rng.random() * (F[tok] - lo)
    counts = np.histogram(v, bins=20, range=(0, 1))[0]
    assert scipy.stats.chisquare(counts).pvalue > 1e-3


def test_sampling_q_equals_p_accepts_all_and_disjoint_accepts_none():
    rng = np.random.default_rng(19)
    V, K, W = 8, 4, 20000
    t, _ = _fixed_rows(V, K, rng)
    out = oracle.accept(oracle.MODE_SAMPLE, _tile(t, W), _tile(t[: K - 1], W),
                        draft_mode=oracle.DRAFT_Q_SAMPLE, seed=4, threads=8)
    assert np.all(out["n_accepted"] == K - 1)
    # disjoint supports: p lives on tokens 0..3, q on 4..7
    tp = np.full((K, V), -1e4, np.float32)
    tp[:, :4] = rng.standard_normal((K, 4))
    dq = np.full((K - 1, V), -1e4, np.float32)
    dq[:, 4:] = rng.standard_normal((K - 1, 4))
    out = oracle.accept(oracle.MODE_SAMPLE, _tile(tp, W), _tile(dq, W),
                        draft_mode=oracle.DRAFT_Q_SAMPLE, seed=4, threads=8)
    assert np.all(out["n_accepted"] == 0)
    p, _ = oracle.warp(tp[0], 1.0)
    counts = np.bincount(out["tokens"][:, 0], minlength=V)
    assert counts[4:].sum() == 0
    assert scipy.stats.chisquare(counts[:4], W * p[:4]).pvalue > 1e-3


def test_sampling_mean_tokens_is_product_of_overlaps():
    """Mean tokens per pass = sum_{j<K} prod_{i<=j} beta_i with beta_i = sum min(p_i, q_i)."""
    rng = np.random.default_rng(20)
    V, K, W = 8, 5, 300000
    t, d = _fixed_rows(V, K, rng, noise=0.5)
    out = oracle.accept(oracle.MODE_SAMPLE, _tile(t, W), _tile(d, W),
                        draft_mode=oracle.DRAFT_Q_SAMPLE, seed=6, threads=8)
    beta = [np.minimum(oracle.warp(t[i], 1.0)[0], oracle.warp(d[i], 1.0)[0]).sum()
            for i in range(K - 1)]
    expect = sum(np.prod(beta[:j]) for j in range(K))
    emitted = out["n_accepted"] + 1
    assert abs(emitted.mean() - expect) < 4.5 * emitted.std() / np.sqrt(W)


def test_accept_status_codes():
    rng = np.random.default_rng(21)
    t = rng.standard_normal((3, 3, 8)).astype(np.float32)
    t[1, 2, 5] = np.nan
    drafts = np.array([[1, 2], [1, 2], [1, 9]], np.int32)
    out = oracle.accept(oracle.MODE_GREEDY, t, draft_tokens=drafts)
    assert list(out["status"]) == [0, 1, 2]
    assert np.all(out["tokens"][1:] == -1) and np.all(out["n_accepted"][1:] == 0)


def test_k1_is_plain_decode():
    """K = 1: no drafts; greedy emits the argmax, sampling one draw from p_1."""
    rng = np.random.default_rng(22)
    V, W = 8, 100000
    t = (rng.standard_normal((1, V)) * 1.5).astype(np.float32)
    g = oracle.accept(oracle.MODE_GREEDY, _tile(t, 3))
    assert np.all(g["tokens"][:, 0] == t[0].argmax()) and np.all(g["n_accepted"] == 0)
    s = oracle.accept(oracle.MODE_SAMPLE, _tile(t, W), np.zeros((W, 0, V), np.float32),
                      seed=2, threads=8)
    p, _ = oracle.warp(t[0], 1.0)
    counts = np.bincount(s["tokens"][:, 0], minlength=V)
    assert scipy.stats.chisquare(counts, W * p).pvalue > 1e-3


# ------------------------------------------------ tolerance base and near-threshold flags

@pytest.mark.parametrize("fmt", [synth.FMT_Q4, synth.FMT_Q4_MIN, synth.FMT_MXFP4, synth.FMT_Q4_K])
def test_tolerance_base_is_sum_of_abs_products(fmt):
    """a[k][r] = sum_j |w_rj x_kj| exactly (numpy on the dequantised matrix), so that the
    parity bound 1e-3 * a is neither loosened (e.g. sum|w| * sum|x|) nor tightened."""
    W = _small_matrix(fmt, rows=23, cols=160)
    x = synth.activations(3, 4, W.cols)
    x[0, :7] = -x[0, :7]                       # mixed signs inside a block
    _, a = oracle.linear(W, x)
    Wd = oracle.dequant(W)
    for k in range(x.shape[0]):
        ref = np.abs(Wd * x[k].astype(np.float64)[None, :]).sum(axis=1)
        assert np.allclose(a[k], ref, rtol=1e-13, atol=0), f"column {k}"
    # a strict bound: a row with cancelling terms has |y| < a
    y, _ = oracle.linear(W, x)
    assert np.any(np.abs(y) < 0.5 * a)


def _softmax64(l):
    z = l.astype(np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


# six distinct logits: masses in decreasing order, cumulative sums C_1..C_6
_L6 = np.array([2.0, 1.5, 1.0, 0.5, 0.0, -0.5], np.float32)
_P6 = _softmax64(_L6)
_C6 = np.cumsum(_P6)


@pytest.mark.parametrize("delta,near,m_p", [(5e-7, 1, 3), (2e-6, 0, 3), (-5e-7, 1, 2), (-2e-6, 0, 2)])
def test_near_top_p_flag_straddles_1e6(delta, near, m_p):
    """The top-p flag: cumulative mass at the cut (C_m) or before it (C_{m-1}) within 1e-6
    of top_p.  top_p = C_2 + delta: the cut is token 3 and C_2 is the mass before it
    (delta > 0), or token 2 with C_2 the mass at it (delta < 0)."""
    _, info = oracle.warp(_L6, 1.0, top_p=float(_C6[1] + delta))
    assert info.m_p == m_p and info.n_keep == m_p
    assert info.near_top_p == near, (delta, info.near_top_p)
    assert info.near_min_p == 0


@pytest.mark.parametrize("delta,near,m_m", [(5e-7, 1, 3), (2e-6, 0, 3), (-5e-7, 1, 4), (-2e-6, 0, 4)])
def test_near_min_p_flag_straddles_1e6(delta, near, m_m):
    """The min-p flag: the last kept or the first dropped token within 1e-6 * pi_max of
    min_p * pi_max.  min_p = pi_4 / pi_max + delta drops token 4 just below the cut
    (delta > 0) or keeps it just above (delta < 0); the margin scales with pi_max."""
    _, info = oracle.warp(_L6, 1.0, min_p=float(_P6[3] / _P6[0] + delta))
    assert info.m_m == m_m and info.n_keep == m_m
    assert info.near_min_p == near, (delta, info.near_min_p)
    assert info.near_top_p == 0


def test_near_flags_only_where_the_cut_binds():
    """A near top-p cut is not flagged when min-p keeps fewer tokens, and a near min-p cut
    is not flagged when top-p keeps fewer."""
    _, info = oracle.warp(_L6, 1.0, top_p=float(_C6[1] + 5e-7), min_p=0.99)
    assert info.m_p == 3 and info.m_m == 1 and info.n_keep == 1
    assert info.near_top_p == 0 and info.near_min_p == 0
    _, info = oracle.warp(_L6, 1.0, top_p=float(_C6[1] + 5e-7), min_p=0.01)
    assert info.n_keep == 3 and info.near_top_p == 1
    _, info = oracle.warp(_L6, 1.0, top_p=float(_C6[0] - 0.01), min_p=float(_P6[3] / _P6[0] + 5e-7))
    assert info.m_p == 1 and info.m_m == 3 and info.n_keep == 1
    assert info.near_min_p == 0 and info.near_top_p == 0
    _, info = oracle.warp(_L6, 1.0, top_p=0.999, min_p=float(_P6[3] / _P6[0] + 5e-7))
    assert info.n_keep == 3 and info.near_min_p == 1


@pytest.mark.parametrize("scale", [1.0, 4.0])
def test_near_cat_flag_straddles_1e6_of_the_total(scale):
    """The draw's flag: u * S within 1e-6 * S of C_j (the mass up to the drawn token) or of
    C_{j-1} (the mass before it).  Weights summing to 4 check that the margin scales with S."""
    w = scale * np.array([0.25, 0.25, 0.5])
    assert oracle.cat(w, 0.25 + 5e-7) == (1, True)      # just past C_0
    assert oracle.cat(w, 0.25 + 2e-6) == (1, False)
    assert oracle.cat(w, 0.5 - 5e-7) == (1, True)       # just short of C_1
    assert oracle.cat(w, 0.5 - 2e-6) == (1, False)
    assert oracle.cat(w, 0.75) == (2, False)


@pytest.mark.parametrize("delta", [5e-7, -5e-7, 2e-6, -2e-6])
def test_near_ratio_flag_straddles_1e6(delta):
    """The ratio test's flag: |u_A - p(x)/q(x)| < 1e-6.  One draft (token 0) over two
    tokens; the target logits are set so that p(x)/q(x) = u_A + delta, with u_A the
    window's first uniform at position 1."""
    seed, win = 21, 0
    uA = float(oracle.uniforms(seed, win, 1)[0])
    dl = np.array([0.0, np.log(0.25)], np.float32)
    q0 = float(_softmax64(dl)[0])
    target_p0 = q0 * (uA + delta)
    assert 0.0 < target_p0 < 1.0
    d = np.float32(np.log(1.0 / target_p0 - 1.0))
    tl = np.array([0.0, d], np.float32)
    r = float(_softmax64(tl)[0]) / q0                  # what the oracle computes, in double
    assert abs((r - uA) - delta) < 1e-7
    out = oracle.accept(oracle.MODE_SAMPLE, np.stack([tl, tl])[None], dl[None, None],
                        np.zeros((1, 1), np.int32), oracle.DRAFT_GIVEN, T=1.0, seed=seed)
    near = int(out["near"][0])
    assert bool(near & oracle.NEAR_RATIO) == (abs(delta) < 1e-6), (delta, near)
    assert out["n_accepted"][0] == (1 if uA < r else 0)


# -------------------------------------------- MX-quantised activations (scaled MFMA path)

def test_e4m3_table_ocp_mx():
    """OCP MX v1.0 E4M3: subnormals m/8 * 2^-6, 1.0 = 0x38, largest 448 = 0x7E, NaN at
    S.1111.111, sign symmetric; magnitudes strictly increasing over codes 0..0x7E."""
    v = np.array([oracle.e4m3(c) for c in range(256)])
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert v[0x38] == 1.0 and v[0x39] == 1.125 and v[0x7E] == 448.0 and v[0x77] == 240.0 and v[0x78] == 256.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.all(np.diff(v[:0x7F]) > 0)
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F]) and np.signbit(v[0x80])


def test_e4m3_rounding_ties_even_and_saturation():
    """Nearest value, ties to the even mantissa, saturation at 448, the sign of -0."""
    assert oracle.e4m3_code(1.0625) == 0x38          # halfway 1.0 / 1.125 -> even (1.0)
    assert oracle.e4m3_code(1.1875) == 0x3A          # halfway 1.125 / 1.25 -> even (1.25)
    assert oracle.e4m3_code(1.07) == 0x39
    assert oracle.e4m3_code(3 * 2.0 ** -10) == 0x02  # halfway 1/512 and 2/512 -> even (2)
    assert oracle.e4m3_code(480.0) == 0x7E and oracle.e4m3_code(1e6) == 0x7E
    assert oracle.e4m3_code(-0.0) == 0x80 and oracle.e4m3_code(-1.0) == 0xB8
    rng = np.random.default_rng(4)
    for x in rng.uniform(-440, 440, 2000):
        c = oracle.e4m3_code(x)
        vals = np.array([oracle.e4m3(k) for k in range(0x7F)])
        assert abs(abs(oracle.e4m3(c)) - abs(x)) == np.min(np.abs(vals - abs(x)))


def test_mx_quant_block_rules():
    """Shared exponent: the block's largest magnitude lands in [256, 512) before rounding;
    representable blocks are recovered exactly; every element within half a step of
    its E4M3 neighbourhood; an all-zero block has scale byte 0."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((3, 256)) * np.exp(rng.uniform(-6, 6, (3, 256)))).astype(np.float16)
    x[2, 32:64] = 0
    codes, scales = oracle.mx_quant(x)
    xh = oracle.mx_dequant(codes, scales)
    xd = x.astype(np.float64)
    for k in range(3):
        for b in range(8):
            blk = xd[k, 32 * b:32 * b + 32]
            E = int(scales[k, b]) - 127
            amax = np.abs(blk).max()
            if amax == 0:
                assert scales[k, b] == 0 and np.all(codes[k, 32 * b:32 * b + 32] & 0x7F == 0)
                continue
            assert 256 <= amax / 2.0 ** E < 512
            v = blk / 2.0 ** E
            err = np.abs(xh[k, 32 * b:32 * b + 32] / 2.0 ** E - v)
            # half the spacing of the E4M3 values around |v| (1/16 of the binade, 2^-10
            # below 2^-6), or the saturation above 448
            step = np.where(np.abs(v) < 2.0 ** -6, 2.0 ** -9,
                            2.0 ** np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6))) / 8)
            ok = (err <= step / 2) | ((np.abs(v) > 448) & (np.abs(xh[k, 32 * b:32 * b + 32] / 2.0 ** E) == 448))
            assert ok.all(), (k, b)
    # a block made of E4M3 values times 2^-3 whose largest is 448 * 2^-3 is recovered exactly
    vals = np.array([oracle.e4m3(c) for c in rng.integers(0, 0x7E, 32)])
    vals[7] = 448.0
    xb = (vals * 2.0 ** -3).astype(np.float16)[None]
    assert np.array_equal(xb.astype(np.float64), (vals * 2.0 ** -3)[None])
    c2, s2 = oracle.mx_quant(xb)
    assert s2[0, 0] == 127 - 3
    assert np.array_equal(oracle.mx_dequant(c2, s2), xb.astype(np.float64))


@pytest.mark.parametrize("fmt", [synth.FMT_MXFP4, synth.FMT_Q4_MIN])
def test_linear_x64_vs_numpy(fmt):
    """W x with double activations agrees with numpy's fp64 matmul of the dequantised matrix."""
    W = _small_matrix(fmt)
    codes, scales = oracle.mx_quant(synth.activations(8, 5, W.cols))
    xh = oracle.mx_dequant(codes, scales)
    y, a = oracle.linear_x64(W, xh)
    ref = xh @ oracle.dequant(W).T
    assert np.all(np.abs(y - ref) <= 1e-12 * a + 1e-300)
    assert np.allclose(a, np.abs(xh[:, None, :] * oracle.dequant(W)[None]).sum(axis=2), rtol=1e-13)


# ------------------------------------------------------ attention over a KV cache

def _kv(kf, vf, Hkv=2, L=200, D=64, seed=3):
    kc, ks = synth.kv_cache(kf, seed, 0, 0, Hkv, L, D)
    vc, vs = synth.kv_cache(vf, seed, 0, 1, Hkv, L, D)
    return kc, ks, vc, vs


def _dequant_by_hand(fmt, codes, scales):
    D = scales.shape[-1] * 32
    out = np.empty(scales.shape[:-1] + (D,))
    for idx in np.ndindex(scales.shape[:-1]):
        for d in range(D):
            sc = float(scales[idx + (d // 32,)])
            if fmt == synth.KV_Q8_0:
                c = int(np.int8(codes[idx + (d,)].view(np.int8)))
            else:
                b = int(codes[idx + (d // 2,)])
                c = ((b >> 4) if d & 1 else (b & 15)) - 8
            out[idx + (d,)] = sc * c
    return out


@pytest.mark.parametrize("kf,vf", [(synth.KV_Q8_0, synth.KV_Q4_0), (synth.KV_Q4_0, synth.KV_Q8_0)])
def test_attention_vs_scipy_softmax(kf, vf):
    """Causal GQA attention over the dequantised cache, against scipy's softmax and numpy
    matmuls (library routines): 4 query rows, 6 query heads on 2 kv heads."""
    kc, ks, vc, vs = _kv(kf, vf, Hkv=2, L=70, D=64)
    q = synth.queries(1, 4, 6, 64)
    out, a = oracle.attention(kf, kc, ks, vf, vc, vs, q)
    Kd, Vd = _dequant_by_hand(kf, kc, ks), _dequant_by_hand(vf, vc, vs)
    assert np.array_equal(Kd, oracle.kv_dequant(kf, kc, ks)) and np.array_equal(Vd, oracle.kv_dequant(vf, vc, vs))
    for i in range(4):
        for h in range(6):
            g = h // 3
            n = 70 - 4 + i + 1
            s = Kd[g, :n] @ q[i, h].astype(np.float64) / np.sqrt(64)
            p = scipy.special.softmax(s)
            ref = p @ Vd[g, :n]
            assert np.allclose(out[i, h], ref, rtol=1e-12, atol=1e-14)
            assert np.allclose(a[i, h], p @ np.abs(Vd[g, :n]), rtol=1e-12)


def test_attention_uniform_keys_average_values_and_causality():
    """Equal keys give equal weights: the output is the mean of the visible values.  A
    query's output does not depend on the positions after its own."""
    kc, ks, vc, vs = _kv(synth.KV_Q8_0, synth.KV_Q4_0, Hkv=1, L=50, D=32)
    kc[:] = kc[0, 0]
    ks[:] = ks[0, 0]
    q = synth.queries(2, 3, 2, 32)
    out, _ = oracle.attention(synth.KV_Q8_0, kc, ks, synth.KV_Q4_0, vc, vs, q)
    Vd = oracle.kv_dequant(synth.KV_Q4_0, vc, vs)
    for i in range(3):
        assert np.allclose(out[i, 0], Vd[0, :50 - 3 + i + 1].mean(axis=0), rtol=1e-12, atol=1e-15)
    kc2, vc2 = _kv(synth.KV_Q8_0, synth.KV_Q4_0, Hkv=1, L=50, D=32, seed=9)[0], vc.copy()
    kc3 = kc.copy()
    kc3[0, 48:] = kc2[0, 48:]            # change positions 48, 49: visible only to queries 1 and 2
    vc2[0, 48:] = vc2[0, 48:] ^ 0x11
    out3, _ = oracle.attention(synth.KV_Q8_0, kc3, ks, synth.KV_Q4_0, vc2, vs, q)
    assert np.array_equal(out3[0], out[0])
    assert not np.allclose(out3[2], out[2])


def test_attention_dominant_key_and_shared_group():
    """One key far above the rest takes all the weight; query heads of one group with the
    same query read the same kv head and give the same output."""
    kc, ks, vc, vs = _kv(synth.KV_Q8_0, synth.KV_Q8_0, Hkv=2, L=40, D=32)
    q = np.zeros((1, 4, 32), np.float16)
    q[0, :, :] = 1.0
    kc[:, 17] = np.int8(127).view(np.uint8)
    ks[:, 17] = 1.0                      # key 17 scores 127 * 32 / sqrt(32), the others < 3
    out, _ = oracle.attention(synth.KV_Q8_0, kc, ks, synth.KV_Q8_0, vc, vs, q)
    Vd = oracle.kv_dequant(synth.KV_Q8_0, vc, vs)
    assert np.allclose(out[0, 0], Vd[0, 17], rtol=1e-12) and np.allclose(out[0, 3], Vd[1, 17], rtol=1e-12)
    assert np.array_equal(out[0, 0], out[0, 1])


# ------------------------------------------------------------ adaptive draft depth
def test_depth_tau_matches_printed_table():
    """oracle.tau against the acceptance-by-depth table the page prints (2 d.p.)."""
    n = 0
    for line in _golden_rows("tau_table.txt"):
        f = line.split()
        a = float(f[0])
        for k, v in zip((1, 3, 5), f[1:]):
            assert abs(oracle.tau(a, k) - float(v)) <= 0.005 + 1e-12, (a, k)
            n += 1
    assert n == 18
    assert oracle.tau(1.0, 4) == 5.0 and oracle.tau(0.0, 7) == 1.0


def test_depth_observe_hand_case_and_decay():
    # windows (accepted, drafted): all 3 kept (no failure), none kept, 2 kept then a reject
    assert oracle.depth_observe((0.0, 0.0), [3, 0, 2], [3, 3, 3], 1.0) == (5.0, 2.0)
    # decay 0.5 in window order: acc 0.5*(0.5*(0.5*0+3)+0)+2 = 2.75; rej 0.5*(0.5*0+1)+1 = 1.5
    acc, rej = oracle.depth_observe((0.0, 0.0), [3, 0, 2], [3, 3, 3], 0.5)
    assert acc == 2.75 and rej == 1.5
    with pytest.raises(ValueError):
        oracle.depth_observe((0.0, 0.0), [4], [3], 1.0)


@pytest.mark.parametrize("alpha,k", [(0.3, 3), (0.6, 5), (0.9, 7), (0.75, 1)])
def test_depth_estimate_is_consistent(alpha, k):
    """Windows simulated with independent per-draft acceptance: accepted / (accepted +
    rejected) converges to alpha (counting windows instead of rejections, or treating an
    all-accepted window as a failure, would be biased and fail this)."""
    rng = np.random.default_rng(7)
    W = 40000
    u = rng.random((W, k))
    n = np.where((u >= alpha).any(axis=1), (u >= alpha).argmax(axis=1), k)
    acc, rej = oracle.depth_observe((0.0, 0.0), n, np.full(W, k), 1.0)
    est = acc / (acc + rej)
    se = np.sqrt(alpha * (1 - alpha) / (acc + rej))
    assert abs(est - alpha) < 5 * se, (est, alpha)


def test_depth_choose_against_exact_rationals():
    """The chosen depth equals a brute-force argmax over exact rationals (fractions), for
    random costs and acceptance counts."""
    from fractions import Fraction
    rng = np.random.default_rng(3)
    for _ in range(300):
        kmax = int(rng.integers(0, 16))
        t = [Fraction(int(rng.integers(900, 1100)) + 40 * k, 1000) for k in range(kmax + 1)]
        td = Fraction(int(rng.integers(0, 200)), 1000)
        acc, rej = int(rng.integers(0, 50)), int(rng.integers(1, 50))
        a = Fraction(acc, acc + rej)
        def rate(k):
            tau = sum(a ** i for i in range(k + 1))
            return tau / (t[k] + k * td)
        best = max(range(kmax + 1), key=lambda k: (rate(k), -k))
        k, ah, _ = oracle.depth_choose((acc, rej), 0.5, 0.0, [float(x) for x in t], float(td))
        assert abs(ah - float(a)) < 1e-15
        # ties within rounding may go either way; otherwise the argmax must agree
        if k != best:
            assert abs(float(rate(k) - rate(best))) <= 1e-12 * float(rate(best))


def test_depth_choose_special_cases():
    flat = [1.0] * 8
    # no acceptance at all: no drafts
    assert oracle.depth_choose((0.0, 10.0), 0.5, 0.0, flat, 0.0)[0] == 0
    # free drafts and a flat pass time: the deepest window
    assert oracle.depth_choose((9.0, 1.0), 0.5, 0.0, flat, 0.0)[0] == 7
    # every draft accepted so far (no rejection): alpha 1, deepest
    assert oracle.depth_choose((12.0, 0.0), 0.5, 0.0, flat, 0.0)[0] == 7
    # no statistics: the prior decides
    assert oracle.depth_choose((0.0, 0.0), 0.0, 1.0, flat, 0.1)[0] == 0
    # the page's reading of its table: at 0.35 going from three to five drafts buys 0.02
    # tokens per pass, so any draft cost above 0.01 of a pass prefers three over five
    r = oracle.depth_choose((35.0, 65.0), 0.5, 0.0, flat[:6], 0.011)[2]
    assert r[3] > r[5]
    # the page's speedup formula with a drafter cost c (pass time 1): at 0.9 and c = 0.1,
    # five drafts beat three (4.69 / 1.5 > 3.44 / 1.3)
    r = oracle.depth_choose((90.0, 10.0), 0.5, 0.0, flat[:6], 0.1)[2]
    assert r[5] > r[3] and abs(r[5] - 4.68559 / 1.5) < 1e-12


# --------------------------------------------------------------- n-gram map drafter
def test_ngram_hand_cases():
    m = oracle.NgramMap(2)
    m.append([1, 2, 3, 4, 1, 2])
    assert m.propose(3) == [3, 4, 1]
    assert m.propose(10) == [3, 4, 1, 2]            # clamped at the sequence's end
    assert m.propose(0) == []
    m = oracle.NgramMap(2)
    m.append([5, 6, 7, 5, 6, 8, 5, 6])              # the latest occurrence of (5, 6) wins
    assert m.propose(3) == [8, 5, 6]
    m = oracle.NgramMap(2)
    m.append([1, 2, 3])                             # (2, 3) never seen before: a miss
    assert m.propose(4) == []
    m = oracle.NgramMap(1)
    m.append([7, 7])                                # (7) was followed by 7
    assert m.propose(2) == [7]
    m = oracle.NgramMap(3)
    m.append([1, 2])                                # shorter than the key
    assert m.propose(2) == []


def _scan_propose(seq, k, d):
    """Brute force: the last earlier occurrence of the final k tokens whose next token
    exists; its continuation, clamped at the end."""
    n = len(seq)
    if d <= 0 or n < k:
        return []
    key = seq[n - k:]
    for s in range(n - 1 - k, -1, -1):
        if seq[s:s + k] == key:
            return seq[s + k:min(s + k + d, n)]
    return []


@pytest.mark.parametrize("k", [1, 2, 3, 6])
def test_ngram_against_brute_force(k):
    rng = np.random.default_rng(k)
    for trial in range(40):
        seq = [int(x) for x in rng.integers(0, 4 if trial % 2 else 9, int(rng.integers(1, 120)))]
        m = oracle.NgramMap(k)
        for i, t in enumerate(seq):
            m.append([t])
            d = int(rng.integers(0, 9))
            assert m.propose(d) == _scan_propose(seq[:i + 1], k, d)


def test_ngram_exact_repeat_is_always_right():
    """A stream that repeats one block of 50 distinct tokens: once the first period has been
    seen, every proposal is exactly the true next tokens."""
    block = list(range(1000, 1050))
    seq = block * 5
    m = oracle.NgramMap(6)
    m.append(seq[:60])
    for i in range(60, len(seq) - 8):
        assert m.propose(8) == seq[i:i + 8]
        m.append([seq[i]])


# ------------------------------------------------------------------------ top-k cut
def test_topk_hand_cases():
    l = np.array([0, 3, 1, 3, 2], np.float32)
    p, info = oracle.warp(l, 1.0, top_k=2)                 # the two 3s
    assert info.n_keep == 2 and abs(p[1] - 0.5) < 1e-15 and abs(p[3] - 0.5) < 1e-15
    p, _ = oracle.warp(l, 1.0, top_k=3)                    # and the 2
    e = np.exp(np.array([3.0, 3.0, 2.0]))
    assert np.allclose([p[1], p[3], p[4]], e / e.sum(), rtol=1e-15) and p[0] == p[2] == 0
    p, _ = oracle.warp(np.array([5, 1, 1, 1, 0], np.float32), 1.0, top_k=2)
    assert p[0] > 0 and p[1] > 0 and p[2] == p[3] == p[4] == 0   # ties: lowest index first
    p, _ = oracle.warp(l, 0.7, top_k=1)                    # one-hot on the first maximum
    assert p[1] == 1.0 and p.sum() == 1.0


def test_topk_no_cut_and_composition():
    rng = np.random.default_rng(4)
    l = rng.standard_normal(300).astype(np.float32) * 2
    base, _ = oracle.warp(l, 0.8, top_p=0.9, min_p=0.02)
    for k in (0, 300, 10**6):
        p, _ = oracle.warp(l, 0.8, top_p=0.9, min_p=0.02, top_k=k)
        assert np.array_equal(p, base)
    _, ip = oracle.warp(l, 0.8, top_p=0.9)
    m_p = ip.n_keep
    _, i1 = oracle.warp(l, 0.8, top_p=0.9, top_k=m_p - 3)   # top-k shorter: it decides
    _, i2 = oracle.warp(l, 0.8, top_p=0.9, top_k=m_p + 3)   # top-p shorter: it decides
    assert i1.n_keep == m_p - 3 and i2.n_keep == m_p


def test_topk_kept_set_against_numpy_ranking():
    """The kept set is exactly the top_k entries by (logit descending, index ascending),
    ranked with numpy's lexsort on integer-valued logits full of ties."""
    rng = np.random.default_rng(9)
    for _ in range(50):
        V = int(rng.integers(1, 400))
        l = rng.integers(-4, 5, V).astype(np.float32)
        k = int(rng.integers(1, V + 2))
        p, info = oracle.warp(l, 1.3, top_k=k)
        order = np.lexsort((np.arange(V), -l.astype(np.float64)))
        keep = set(order[:min(k, V)].tolist())
        assert set(np.nonzero(p)[0].tolist()) == keep
        assert info.n_keep == min(k, V)
