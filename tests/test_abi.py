"""The C-ABI library loads, exports what include/vq.h declares, and rejects bad arguments
on the host before anything is enqueued.  No GPU: every call here either fails
validation or has nothing to launch, so no device pointer is ever dereferenced."""
import ctypes
import os
import re

import pytest

import speculative_decoding_verification_bit_amd as vq

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "vq.h")
FAKE = 0x10000          # a 256-byte aligned non-NULL address that is never dereferenced


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vq_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_exports():
    assert set(_declared()) == set(vq.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(vq.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_abi_version_matches_header():
    m = re.search(r"#define VQ_ABI_VERSION (\d+)", open(HEADER).read())
    assert vq.lib.vq_abi_version() == int(m.group(1))


def test_status_strings():
    for code in (vq.OK, vq.ERR_ARG, vq.ERR_UNSUPPORTED, vq.ERR_WORKSPACE, vq.ERR_HIP):
        assert vq.lib.vq_status_string(code)
    assert vq.lib.vq_status_string(-99) == b"unknown status"


def _mat(fmt=vq.FMT_Q4_MIN, rows=64, cols=256, qs=FAKE, scales=FAKE, mins=FAKE, supers=FAKE):
    return vq.VqMatrix(fmt, rows, cols, 0, qs, scales, mins if fmt in (vq.FMT_Q4_MIN, vq.FMT_Q4_K) else None,
                       supers if fmt == vq.FMT_Q4_K else None)


def _til(fmt=vq.FMT_Q4_MIN, rows=64, cols=256, order=vq.ROWS_PLAIN, data=FAKE):
    return vq.VqTiled(fmt, rows, cols, order, data)


def _lin(W, K=4, x=FAKE, y=FAKE, dtype=vq.DTYPE_F32, ws=FAKE, nbytes=None):
    if nbytes is None:
        nbytes = 1 << 40
    return vq.lib.vq_verify_linear(ctypes.byref(W), x, K, y, dtype, ws, nbytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(K=0), vq.ERR_ARG),
    (dict(K=17), vq.ERR_ARG),
    (dict(dtype=5), vq.ERR_ARG),
    (dict(x=None), vq.ERR_ARG),
    (dict(y=None), vq.ERR_ARG),
    (dict(x=FAKE + 8), vq.ERR_ARG),
    (dict(y=FAKE + 2), vq.ERR_ARG),
    (dict(y=FAKE + 1, dtype=vq.DTYPE_F16), vq.ERR_ARG),
    (dict(ws=None), vq.ERR_WORKSPACE),
    (dict(ws=FAKE + 64), vq.ERR_WORKSPACE),
    (dict(nbytes=0), vq.ERR_WORKSPACE),
])
def test_linear_argument_errors(kw, code):
    assert _lin(_til(), **kw) == code
    assert vq.lib.vq_last_error()


@pytest.mark.parametrize("W", [
    _til(cols=48), _til(cols=0), _til(rows=-1), _til(fmt=4), _til(fmt=-1), _til(data=None), _til(data=FAKE + 16),
    _til(order=2), _til(order=vq.ROWS_PAIR8), _til(fmt=vq.FMT_Q4_K, cols=384),
])
def test_linear_bad_matrix(W):
    assert _lin(W) == vq.ERR_ARG


def test_linear_zero_rows_is_a_no_op():
    W = _til(rows=0, data=None)
    assert _lin(W, x=None, y=None, ws=None, nbytes=0) == vq.OK


def test_linear_workspace_is_small_and_exact():
    for rows, cols in ((5120, 5120), (5120, 17408), (151936, 5120), (64, 1056), (77, 32)):
        W = _til(rows=rows, cols=cols)
        for K in (1, 4, 16):
            n = vq.lib.vq_workspace_bytes(vq.OP_LINEAR, ctypes.byref(W), K)
            assert 0 < n
            if K == 1:
                assert n < 1 << 20, (rows, cols, n)     # one window: two partials per workgroup
            assert _lin(W, K=K, nbytes=n - 1) == vq.ERR_WORKSPACE
    assert vq.lib.vq_workspace_bytes(9, ctypes.byref(_til()), 4) == 0
    assert vq.lib.vq_workspace_bytes(vq.OP_LINEAR, ctypes.byref(_til()), 0) == 0


def test_tiled_bytes():
    # Q4_K: per row of a 128-column group 8 bytes of 6-bit scales and mins, and one fp16
    # of its super-block (D in the even group, Dmin in the odd): 1024 + 16 * 10 bytes
    per = 1184
    assert vq.lib.vq_tiled_bytes(vq.FMT_Q4_K, 16, 256) == 2 * per
    assert vq.lib.vq_tiled_bytes(vq.FMT_Q4_K, 77, 1024) == 5 * 8 * per
    assert vq.lib.vq_tiled_bytes(vq.FMT_Q4_K, 5120, 17408) == 320 * 136 * per
    assert vq.lib.vq_tiled_bytes(vq.FMT_Q4_K, 5120, 5120) == 5120 * 5120 * 37 // 64   # 4.625 bits
    for cols in (128, 288, 1056):
        assert vq.lib.vq_tiled_bytes(vq.FMT_Q4_K, 16, cols) == 0
    for fmt, per in ((vq.FMT_Q4, 1152), (vq.FMT_Q4_MIN, 1280), (vq.FMT_MXFP4, 1088)):
        # groups of 128 columns come in pairs (one step of the streaming kernel)
        assert vq.lib.vq_tiled_bytes(fmt, 16, 128) == 2 * per
        assert vq.lib.vq_tiled_bytes(fmt, 16, 256) == 2 * per
        # partial tiles and groups are padded to whole chunks
        assert vq.lib.vq_tiled_bytes(fmt, 77, 1056) == 5 * 10 * per
        assert vq.lib.vq_tiled_bytes(fmt, 5120, 17408) == 320 * 136 * per
        # every weight's 4 bits and its block's scale (and min) are stored once, no more
        if fmt == vq.FMT_Q4_MIN:
            assert vq.lib.vq_tiled_bytes(fmt, 5120, 5120) == 5120 * 5120 * 5 // 8
    assert vq.lib.vq_tiled_bytes(4, 16, 128) == 0
    assert vq.lib.vq_tiled_bytes(vq.FMT_Q4, 16, 100) == 0
    assert vq.lib.vq_tiled_bytes(vq.FMT_Q4, -1, 128) == 0


def _tile(src, dst, row0=0):
    return vq.lib.vq_tile(ctypes.byref(src), ctypes.byref(dst), row0, None)


def test_tile_argument_errors():
    assert _tile(_mat(rows=0, qs=None, scales=None, mins=None), _til()) == vq.OK     # nothing to write
    assert _tile(_mat(fmt=vq.FMT_Q4), _til()) == vq.ERR_ARG                          # format differs
    assert _tile(_mat(cols=512), _til()) == vq.ERR_ARG                                # cols differ
    assert _tile(_mat(rows=64), _til(rows=64), 16) == vq.ERR_ARG                     # past dst
    assert _tile(_mat(rows=16), _til(rows=64), 8) == vq.ERR_ARG                      # row0 % 16
    assert _tile(_mat(rows=16), _til(rows=64), -16) == vq.ERR_ARG
    assert _tile(_mat(rows=16), _til(rows=64, order=vq.ROWS_PAIR8), 16) == vq.ERR_ARG  # pair8: halves only
    assert _tile(_mat(rows=32), _til(rows=64, order=vq.ROWS_PAIR8), 16) == vq.ERR_ARG
    assert _tile(_mat(rows=16), _til(rows=64, data=None)) == vq.ERR_ARG
    assert _tile(_mat(rows=16, qs=None), _til(rows=64)) == vq.ERR_ARG


def test_tile_q4k_planes():
    """Q4_K takes exactly qs, scales, mins and supers, with cols a multiple of 256."""
    K = vq.FMT_Q4_K
    dst = _til(fmt=K, rows=64)
    assert _tile(_mat(fmt=K, rows=16, supers=None), dst) == vq.ERR_ARG
    assert _tile(_mat(fmt=K, rows=16, mins=None), dst) == vq.ERR_ARG
    assert _tile(_mat(fmt=K, rows=16, supers=FAKE + 8), dst) == vq.ERR_ARG
    assert _tile(_mat(fmt=K, rows=16, cols=384), _til(fmt=K, rows=64, cols=384)) == vq.ERR_ARG
    bad = vq.VqMatrix(vq.FMT_Q4_MIN, 16, 256, 0, FAKE, FAKE, FAKE, FAKE)   # supers on another format
    assert _tile(bad, _til(rows=64)) == vq.ERR_ARG
    assert _tile(_mat(fmt=K, rows=0, qs=None, scales=None, mins=None, supers=None), dst) == vq.OK


def _acc(**kw):
    base = dict(mode=vq.MODE_SAMPLE, draft_mode=vq.DRAFT_GIVEN, W=4, K=4, V=256, top_k=0,
                target_logits=FAKE, draft_logits=FAKE, draft_tokens=FAKE, temperature=1.0, top_p=1.0,
                min_p=0.0, alpha=0.0, seed=0, window_base=0, n_accepted=FAKE, tokens=FAKE, status=FAKE)
    base.update(kw)
    return vq.VqAcceptDesc(**base)


@pytest.mark.parametrize("kw", [
    dict(mode=2), dict(draft_mode=4), dict(W=-1), dict(K=0), dict(K=17), dict(V=0),
    dict(V=(1 << 19) + 1), dict(temperature=0.0), dict(temperature=-1.0), dict(top_p=0.0),
    dict(top_p=1.5), dict(min_p=1.0), dict(min_p=-0.1), dict(target_logits=None),
    dict(draft_logits=None), dict(draft_tokens=None), dict(tokens=None), dict(status=None),
    dict(n_accepted=None), dict(top_k=-1), dict(draft_mode=vq.DRAFT_AGREE, mode=vq.MODE_GREEDY, V=1),
    dict(draft_mode=vq.DRAFT_AGREE, mode=vq.MODE_GREEDY, alpha=1.5),
    dict(temperature=float("nan")),
])
def test_accept_argument_errors(kw):
    d = _acc(**kw)
    assert vq.lib.vq_verify_accept(ctypes.byref(d), FAKE, 1 << 30, None) == vq.ERR_ARG


def test_accept_workspace_errors_and_empty():
    d = _acc()
    assert vq.lib.vq_verify_accept(ctypes.byref(d), None, 0, None) == vq.ERR_WORKSPACE
    need = vq.lib.vq_workspace_bytes(vq.OP_ACCEPT, ctypes.byref(d), 4)
    assert need > 0
    assert vq.lib.vq_verify_accept(ctypes.byref(d), FAKE, need - 1, None) == vq.ERR_WORKSPACE
    e = _acc(W=0, target_logits=None, n_accepted=None, tokens=None, status=None)
    assert vq.lib.vq_verify_accept(ctypes.byref(e), None, 0, None) == vq.OK
    # greedy with given drafts ignores the sampler settings and needs no drafter logits
    g = _acc(mode=vq.MODE_GREEDY, temperature=0.0, top_p=0.0, draft_logits=None)
    assert vq.lib.vq_verify_accept(ctypes.byref(g), None, 0, None) == vq.ERR_WORKSPACE


def _model(L=2, H=256, KV=64, FF=512, V=1000, fmt=vq.FMT_Q4_MIN, bad=None):
    shapes = dict(qkv=(H + 2 * KV, H, vq.ROWS_PLAIN), o=(H, H, vq.ROWS_PLAIN), gu=(2 * FF, H, vq.ROWS_PAIR8),
                  down=(H, FF, vq.ROWS_PLAIN))
    arr = (vq.VqLayer * L)()
    for i in range(L):
        for n, (r, c, order) in shapes.items():
            if bad == (i, n):
                r += 64
            setattr(arr[i], n, _til(fmt, r, c, order))
    return vq.VqModel(L, 0, ctypes.cast(arr, ctypes.POINTER(vq.VqLayer)), _til(fmt, V, H)), arr


def _dec(M, K=4, x=FAKE, logits=FAKE, ws=FAKE, nbytes=0):
    return vq.lib.vq_decode_pass(ctypes.byref(M), x, K, logits, ws, nbytes, None)


def test_decode_validation_and_layout():
    M, keep = _model()
    n1 = vq.lib.vq_workspace_bytes(vq.OP_DECODE, ctypes.byref(M), 1)
    n4 = vq.lib.vq_workspace_bytes(vq.OP_DECODE, ctypes.byref(M), 4)
    assert 0 < n1 < n4
    assert _dec(M, ws=None, nbytes=0) == vq.ERR_WORKSPACE
    assert _dec(M, nbytes=n4 - 1) == vq.ERR_WORKSPACE
    assert _dec(M, ws=FAKE + 64, nbytes=n4) == vq.ERR_WORKSPACE          # not 256-byte aligned
    assert _dec(M, K=0, nbytes=n4) == vq.ERR_ARG
    assert _dec(M, K=17, nbytes=n4) == vq.ERR_ARG
    assert _dec(M, x=None, nbytes=n4) == vq.ERR_ARG
    assert _dec(M, x=FAKE + 8, nbytes=n4) == vq.ERR_ARG
    assert _dec(M, logits=None, nbytes=n4) == vq.ERR_ARG
    Mb, kb = _model(bad=(1, "down"))
    assert _dec(Mb, nbytes=n4) == vq.ERR_ARG
    assert vq.lib.vq_workspace_bytes(vq.OP_DECODE, ctypes.byref(Mb), 4) == 0
    Mu, ku = _model(H=96 * 4 + 32)   # hidden not a multiple of 64
    assert _dec(Mu, nbytes=n4) == vq.ERR_UNSUPPORTED
    Mf, kf = _model(fmt=vq.FMT_Q4_MIN)
    Mf.lm_head.format = vq.FMT_Q4
    assert _dec(Mf, nbytes=n4) == vq.ERR_ARG                               # one format per stack
    Mo, ko = _model()
    ko[1].gu.order = vq.ROWS_PLAIN
    assert _dec(Mo, nbytes=n4) == vq.ERR_ARG                               # gate|up must be paired
    # stage pointers: distinct, ordered, inside the workspace
    seen = []
    for s in range(9):
        a, b = ctypes.c_void_p(), ctypes.c_void_p()
        assert vq.lib.vq_decode_stage_ptr(ctypes.byref(M), 4, FAKE, s, ctypes.byref(a), ctypes.byref(b)) == vq.OK
        assert FAKE <= a.value < FAKE + n4
        seen.append(a.value)
        if s < 8:
            assert a.value < b.value < FAKE + n4
        else:
            assert b.value is None
    assert seen == sorted(seen) and len(set(seen)) == 9
    a, b = ctypes.c_void_p(), ctypes.c_void_p()
    assert vq.lib.vq_decode_stage_ptr(ctypes.byref(M), 4, FAKE, 9, ctypes.byref(a), ctypes.byref(b)) == vq.ERR_ARG


def test_decode_error_word_lies_in_the_workspace():
    M, keep = _model()
    for K in (1, 4, 16):
        n = vq.lib.vq_workspace_bytes(vq.OP_DECODE, ctypes.byref(M), K)
        w = ctypes.c_void_p()
        assert vq.lib.vq_decode_error_word(ctypes.byref(M), K, FAKE, ctypes.byref(w)) == vq.OK
        assert FAKE <= w.value and w.value + 4 <= FAKE + n and w.value % 4 == 0
        a, b = ctypes.c_void_p(), ctypes.c_void_p()
        vq.lib.vq_decode_stage_ptr(ctypes.byref(M), K, FAKE, 8, ctypes.byref(a), ctypes.byref(b))
        assert w.value > a.value                    # after the stage tensors, not inside them
    assert vq.lib.vq_decode_error_word(ctypes.byref(M), 0, FAKE, ctypes.byref(w)) == vq.ERR_ARG
    assert vq.lib.vq_decode_error_word(ctypes.byref(M), 4, None, ctypes.byref(w)) == vq.ERR_ARG
    assert vq.lib.vq_decode_error_word(ctypes.byref(M), 4, FAKE, None) == vq.ERR_ARG


def test_decode_timed_argument_errors():
    M, keep = _model()
    n4 = vq.lib.vq_workspace_bytes(vq.OP_DECODE, ctypes.byref(M), 4)
    nl = ctypes.c_int32(-1)
    ev = (ctypes.c_void_p * 2)(FAKE, FAKE)
    for launch in (1, 12, 16, -4):
        assert vq.lib.vq_decode_pass_timed(ctypes.byref(M), FAKE, 4, FAKE, launch, FAKE, n4, None, ev, 2,
                                           ctypes.byref(nl)) == vq.ERR_ARG
    assert vq.lib.vq_decode_pass_timed(ctypes.byref(M), FAKE, 4, FAKE, 0, FAKE, n4, None, ev, 1,
                                       ctypes.byref(nl)) == vq.ERR_ARG      # a pair is needed
    ev2 = (ctypes.c_void_p * 2)(FAKE, None)
    assert vq.lib.vq_decode_pass_timed(ctypes.byref(M), FAKE, 4, FAKE, 0, FAKE, n4, None, ev2, 2,
                                       ctypes.byref(nl)) == vq.ERR_ARG      # a NULL event
    assert vq.lib.vq_decode_pass_timed(ctypes.byref(M), FAKE, 4, FAKE, 0, FAKE, n4, None, None, 0,
                                       ctypes.byref(nl)) == vq.ERR_ARG
    assert nl.value == -1


def _att(kf=vq.KV_Q8_0, vf=vq.KV_Q4_0, Hq=40, Hkv=8, D=128, L=1000, kc=FAKE, ks=FAKE, vc=FAKE, vs=FAKE):
    return vq.VqAttention(kf, vf, Hq, Hkv, D, L, kc, ks, vc, vs)


def _attn(C, K=4, q=FAKE, out=FAKE, ws=FAKE, nbytes=1 << 40):
    return vq.lib.vq_verify_attention(ctypes.byref(C), q, K, out, ws, nbytes, None)


@pytest.mark.parametrize("C,K,kw,code", [
    (_att(kf=2), 4, {}, vq.ERR_ARG),
    (_att(vf=-1), 4, {}, vq.ERR_ARG),
    (_att(D=64), 4, {}, vq.ERR_ARG),
    (_att(Hkv=0), 4, {}, vq.ERR_ARG),
    (_att(Hq=12), 4, {}, vq.ERR_ARG),            # not a multiple of Hkv
    (_att(L=0), 1, {}, vq.ERR_ARG),
    (_att(L=3), 4, {}, vq.ERR_ARG),              # K > L
    (_att(), 0, {}, vq.ERR_ARG),
    (_att(), 17, {}, vq.ERR_ARG),
    (_att(Hq=72, Hkv=2), 4, {}, vq.ERR_ARG),     # 36 q heads per kv head x 4 rows > 128
    (_att(kc=None), 4, {}, vq.ERR_ARG),
    (_att(vs=None), 4, {}, vq.ERR_ARG),
    (_att(kc=FAKE + 8), 4, {}, vq.ERR_ARG),
    (_att(ks=FAKE + 8), 4, {}, vq.ERR_ARG),
    (_att(), 4, dict(q=None), vq.ERR_ARG),
    (_att(), 4, dict(out=FAKE + 2), vq.ERR_ARG),
    (_att(), 4, dict(ws=None), vq.ERR_WORKSPACE),
    (_att(), 4, dict(ws=FAKE + 64), vq.ERR_WORKSPACE),
    (_att(), 4, dict(nbytes=0), vq.ERR_WORKSPACE),
])
def test_attention_argument_errors(C, K, kw, code):
    assert _attn(C, K, **kw) == code
    assert vq.lib.vq_last_error()


def test_attention_workspace():
    for Hq, Hkv, L, K in ((40, 8, 32768, 16), (40, 8, 1, 1), (32, 1, 300, 4), (8, 8, 65, 16)):
        C = _att(Hq=Hq, Hkv=Hkv, L=L)
        n = vq.lib.vq_workspace_bytes(vq.OP_ATTENTION, ctypes.byref(C), K)
        # per-span partials: Hq / Hkv * K rows of D + 2 floats per span and kv head
        spans = -(-L // 64)
        assert 0 < n <= Hkv * min(spans, 4 * 256) * (Hq // Hkv) * K * (128 + 2) * 4 + 512, (Hq, Hkv, L, K, n)
        assert _attn(C, K, nbytes=n - 1) == vq.ERR_WORKSPACE
    assert vq.lib.vq_workspace_bytes(vq.OP_ATTENTION, ctypes.byref(_att(D=96)), 4) == 0
