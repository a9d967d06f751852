"""The n-gram map drafter in libvq (vq_ngram_*: host arithmetic) against the oracle: the
proposals are identical at every step of synthetic code-like streams and of exact
repeats, for key lengths 1 .. 12 and window sizes 0 .. 15, across the table's growth.
No GPU."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
import speculative_decoding_verification_bit_amd as vq


@pytest.mark.parametrize("k", [1, 2, 4, 6, 12])
def test_proposals_match_oracle_on_code_like_stream(k):
    s = synth.token_stream(k, 6000, vocab=5000 if k <= 2 else 151936)
    a, b = vq.NgramMap(k), oracle.NgramMap(k)
    rng = np.random.default_rng(k)
    i, hits = 0, 0
    while i < s.size:
        step = int(rng.integers(1, 9))          # a window's emitted tokens, or a prompt chunk
        a.append(s[i:i + step])
        b.append(s[i:i + step])
        i += step
        d = int(rng.integers(0, 16))
        pa, pb = a.propose(d), b.propose(d)
        assert pa == pb, (i, d)
        hits += len(pa) > 0
    assert hits > 0


def test_prompt_in_one_call_and_repeats():
    block = list(range(10, 90))
    seq = block * 40 + [3, 1, 4, 1, 5] + block[:30]
    a, b = vq.NgramMap(6), oracle.NgramMap(6)
    a.append(seq[:2000])
    b.append(seq[:2000])
    for t in seq[2000:]:
        assert a.propose(8) == b.propose(8)
        a.append([t])
        b.append([t])
    assert a.propose(15) == b.propose(15)


def test_small_alphabet_collisions_and_growth():
    """Two symbols: every key recurs constantly (overwrites), and 20,000 tokens at k = 12
    grow the table well past its first size."""
    rng = np.random.default_rng(5)
    s = rng.integers(0, 2, 20000).astype(np.int32)
    for k in (3, 12):
        a, b = vq.NgramMap(k), oracle.NgramMap(k)
        for i in range(0, s.size, 7):
            a.append(s[i:i + 7])
            b.append(s[i:i + 7])
            assert a.propose(9) == b.propose(9)


def test_argument_errors():
    h = ctypes.c_void_p()
    assert vq.lib.vq_ngram_create(0, ctypes.byref(h)) == vq.ERR_ARG
    assert vq.lib.vq_ngram_create(65, ctypes.byref(h)) == vq.ERR_ARG
    assert vq.lib.vq_ngram_create(6, None) == vq.ERR_ARG
    assert vq.lib.vq_ngram_create(6, ctypes.byref(h)) == vq.OK and h.value
    bad = np.array([1, -1, 2], np.int32)
    assert vq.lib.vq_ngram_append(h, bad.ctypes.data, 3) == vq.ERR_ARG
    assert vq.lib.vq_ngram_append(h, None, 2) == vq.ERR_ARG
    assert vq.lib.vq_ngram_append(h, None, 0) == vq.OK
    assert vq.lib.vq_ngram_append(h, bad.ctypes.data, -1) == vq.ERR_ARG
    n = ctypes.c_int32(-9)
    assert vq.lib.vq_ngram_propose(h, -1, None, ctypes.byref(n)) == vq.ERR_ARG
    assert vq.lib.vq_ngram_propose(h, 3, None, ctypes.byref(n)) == vq.ERR_ARG
    assert vq.lib.vq_ngram_propose(h, 0, None, ctypes.byref(n)) == vq.OK and n.value == 0
    # nothing was appended by the failed calls: the sequence is empty, nothing to propose
    out = np.empty(4, np.int32)
    assert vq.lib.vq_ngram_propose(h, 4, out.ctypes.data, ctypes.byref(n)) == vq.OK and n.value == 0
    vq.lib.vq_ngram_destroy(h)
    vq.lib.vq_ngram_destroy(None)
    assert vq.lib.vq_status_string(vq.ERR_HOST) == b"host allocation failed"
