"""CPU oracle for the verify pass -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  It wraps ``oracle.c`` (plain C, double precision, no fast-math),
which shares no code with the HIP library.  What each function computes, and which
passage of the pages it follows, is stated in ``oracle.c``.

The stage-composition glue of a full decode pass (a stage's input is the previous
stage's output rounded to fp16 -- the q rows of q|k|v, o, silu(gate) * up, down -- and
the stage scales its dot products by rho = 1 / sqrt(mean(v^2)) of that output) is
written here in terms of the C primitives.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FMT_Q4, FMT_Q4_MIN, FMT_MXFP4, FMT_Q4_K = 0, 1, 2, 3
MODE_GREEDY, MODE_SAMPLE = 0, 1
DRAFT_GIVEN, DRAFT_Q_ARGMAX, DRAFT_Q_SAMPLE, DRAFT_AGREE = 0, 1, 2, 3
NEAR_RATIO, NEAR_CAT, NEAR_TOP_P, NEAR_MIN_P, NEAR_DRAFT_CAT = 1, 2, 4, 8, 16


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, IEEE semantics, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                        "-ffp-contract=off", "-Wall", "-o", tmp, _SRC, "-lm", "-lpthread"],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.or_half.restype = D
        L.or_half.argtypes = [ctypes.c_uint16]
        L.or_half_array.argtypes = [P, P, I64]
        L.or_e2m1.restype = D
        L.or_e2m1.argtypes = [I32]
        L.or_e8m0.restype = D
        L.or_e8m0.argtypes = [ctypes.c_uint8]
        L.or_dequant.argtypes = [I32, P, P, P, P, I64, I64, P]
        L.or_attention.restype = I32
        L.or_attention.argtypes = [I32, P, P, I32, P, P, I64, I64, I64, P, I64, I64, P, P]
        L.or_linear_x64.restype = I32
        L.or_linear_x64.argtypes = [I32, P, P, P, P, I64, I64, P, I32, P, P, I32]
        L.or_e4m3.restype = D
        L.or_e4m3.argtypes = [I32]
        L.or_e4m3_code.restype = I32
        L.or_e4m3_code.argtypes = [D]
        L.or_mx_quant.restype = I32
        L.or_mx_quant.argtypes = [P, I64, I64, P, P]
        L.or_linear.restype = I32
        L.or_linear.argtypes = [I32, P, P, P, P, I64, I64, P, I32, P, P, I32]
        L.or_rho.argtypes = [P, I32, I64, P]
        L.or_rms_scale.argtypes = [P, I32, I64, P]
        L.or_silu_mul.argtypes = [P, P, I64, P]
        L.or_philox4x64.argtypes = [P, P, P]
        L.or_uniforms.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, P]
        L.or_warp.restype = I32
        L.or_warp.argtypes = [P, I64, D, D, D, I64, P, P]
        L.or_argmax.restype = I64
        L.or_argmax.argtypes = [P, I64]
        L.or_cat.restype = I64
        L.or_cat.argtypes = [P, I64, D, P]
        L.or_accept.restype = I32
        L.or_accept.argtypes = [P, I32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def half(h: int) -> float:
    return lib().or_half(h)


def half_array(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h).view(np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().or_half_array(_p(h), _p(out), h.size)
    return out


def e2m1(code: int) -> float:
    return lib().or_e2m1(code)


def e8m0(e: int) -> float:
    return lib().or_e8m0(e)


def _mins_supers(m):
    """The mins plane (or None) and, for Q4_K, the super-block (d, dmin) plane."""
    mn = None if m.mins is None else np.ascontiguousarray(m.mins)
    sp = None
    if m.fmt == FMT_Q4_K:
        if m.cols % 256 or m.supers is None:
            raise ValueError("Q4_K needs cols % 256 == 0 and the super-block plane")
        sp = np.ascontiguousarray(m.supers).view(np.uint16)
    return mn, sp


def dequant(m) -> np.ndarray:
    """Dequantised weights [rows][cols] in double for a synth.Q4Matrix."""
    out = np.empty((m.rows, m.cols), np.float64)
    qs = np.ascontiguousarray(m.qs)
    sc = np.ascontiguousarray(m.scales)
    mn, sp = _mins_supers(m)
    lib().or_dequant(m.fmt, _p(qs), _p(sc), _p(mn), _p(sp), m.rows, m.cols, _p(out))
    return out


def linear(m, x: np.ndarray, threads: int = 1):
    """y[K][rows] = W x (double) and the row tolerance base A[K][rows] = sum |w x|."""
    x = np.ascontiguousarray(x, dtype=np.float16)
    K = x.shape[0]
    assert x.shape[1] == m.cols
    y = np.empty((K, m.rows), np.float64)
    a = np.empty((K, m.rows), np.float64)
    qs = np.ascontiguousarray(m.qs)
    sc = np.ascontiguousarray(m.scales)
    mn, sp = _mins_supers(m)
    rc = lib().or_linear(m.fmt, _p(qs), _p(sc), _p(mn), _p(sp), m.rows, m.cols, _p(x), K,
                         _p(y), _p(a), threads)
    if rc:
        raise RuntimeError(f"or_linear failed ({rc})")
    return y, a


def linear_x64(m, x: np.ndarray, threads: int = 1):
    """linear() with double activations x [K][cols] (e.g. MX-dequantised ones)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    K = x.shape[0]
    assert x.shape[1] == m.cols
    y = np.empty((K, m.rows), np.float64)
    a = np.empty((K, m.rows), np.float64)
    qs = np.ascontiguousarray(m.qs)
    sc = np.ascontiguousarray(m.scales)
    mn, sp = _mins_supers(m)
    rc = lib().or_linear_x64(m.fmt, _p(qs), _p(sc), _p(mn), _p(sp), m.rows, m.cols, _p(x), K, _p(y), _p(a),
                             threads)
    if rc:
        raise RuntimeError(f"or_linear_x64 failed ({rc})")
    return y, a


KV_Q8_0, KV_Q4_0 = 0, 1


def attention(kfmt, kcodes, kscales, vfmt, vcodes, vscales, q: np.ndarray, threads: int = 1):
    """The window's attention over a quantised KV cache (double).  kcodes/vcodes: uint8
    [Hkv][L][D] (q8_0, int8 bit patterns) or [Hkv][L][D/2] (q4_0); scales fp16
    [Hkv][L][D/32]; q fp16 [K][Hq][D].  Returns out [K][Hq][D] and a = sum_j p_j |v_j|."""
    q = np.ascontiguousarray(q, dtype=np.float16)
    K, Hq, D = q.shape
    Hkv, L = kscales.shape[0], kscales.shape[1]
    out = np.empty((K, Hq, D), np.float64)
    a = np.empty((K, Hq, D), np.float64)
    kc, vc = np.ascontiguousarray(kcodes), np.ascontiguousarray(vcodes)
    ks = np.ascontiguousarray(kscales).view(np.uint16)
    vs = np.ascontiguousarray(vscales).view(np.uint16)
    rc = lib().or_attention(kfmt, _p(kc), _p(ks), vfmt, _p(vc), _p(vs), Hkv, L, D, _p(q.view(np.uint16)), K, Hq,
                            _p(out), _p(a))
    if rc:
        raise RuntimeError(f"or_attention failed ({rc})")
    return out, a


def kv_dequant(fmt, codes, scales) -> np.ndarray:
    """Cache values [Hkv][L][D] in double (q8_0: d * int8; q4_0: d * (n - 8), low nibble first)."""
    sc = np.repeat(np.ascontiguousarray(scales).astype(np.float64), 32, axis=-1)
    if fmt == KV_Q8_0:
        return sc * codes.view(np.int8).astype(np.float64)
    lo = (codes & 15).astype(np.int64) - 8
    hi = (codes >> 4).astype(np.int64) - 8
    v = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
    return sc * v


def e4m3(code: int) -> float:
    """Value of an OCP E4M3 code."""
    return float(lib().or_e4m3(int(code)))


def e4m3_code(v: float) -> int:
    return int(lib().or_e4m3_code(float(v)))


def mx_quant(x: np.ndarray):
    """fp16 activations [K][cols] -> (E4M3 codes [K][cols] u8, E8M0 scales [K][cols/32] u8)."""
    x = np.ascontiguousarray(x, dtype=np.float16)
    K, cols = x.shape
    codes = np.empty((K, cols), np.uint8)
    scales = np.empty((K, cols // 32), np.uint8)
    rc = lib().or_mx_quant(_p(x.view(np.uint16)), K, cols, _p(codes), _p(scales))
    if rc:
        raise RuntimeError(f"or_mx_quant failed ({rc})")
    return codes, scales


def mx_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The activations an MX-quantised block stands for, in double: e4m3(code) * 2^(s - 127)."""
    table = np.array([e4m3(c) for c in range(256)], np.float64)
    sc = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return table[codes] * np.repeat(sc, 32, axis=1)


def rho(v: np.ndarray) -> np.ndarray:
    """Per activation column (row of v [K][n]): v / sqrt(mean(v^2)), in double.
    float32 input (a stage output) converts to double exactly."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.float64)
    lib().or_rho(_p(v), v.shape[0], v.shape[1], _p(out))
    return out


def rms_scale(v: np.ndarray) -> np.ndarray:
    """Per activation column k (row of v [K][n]): 1 / sqrt(mean(v^2)), in double."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape[0], np.float64)
    lib().or_rms_scale(_p(v), v.shape[0], v.shape[1], _p(out))
    return out


STAGE_QKV, STAGE_O, STAGE_GU, STAGE_DOWN = 0, 1, 2, 3


def stage_glue(prev_out: np.ndarray, prev_kind: int, hidden: int, ffn: int):
    """What the next stage of a decode pass gets from a stage's fp32 output prev_out
    [K][rows]: the value v [K][n] (double) whose fp16 rounding is the next input, and the
    scale rho [K] of the next stage's dot products.  prev_kind is the producing stage:
    q|k|v feeds its q rows, o and down feed themselves, gate|up feeds silu(gate) * up."""
    prev_out = np.asarray(prev_out, dtype=np.float32)
    if prev_kind == STAGE_QKV:
        v = prev_out[:, :hidden].astype(np.float64)
    elif prev_kind == STAGE_GU:
        v = np.stack([silu_mul(prev_out[k, :ffn], prev_out[k, ffn:2 * ffn]) for k in range(prev_out.shape[0])])
    else:
        v = prev_out.astype(np.float64)
    return v, rms_scale(v)


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    out = np.empty(g.shape, np.float64)
    lib().or_silu_mul(_p(g), _p(u), g.size, _p(out))
    return out


def philox4x64(counter, key) -> np.ndarray:
    c = np.asarray(counter, dtype=np.uint64).copy()
    k = np.asarray(key, dtype=np.uint64).copy()
    out = np.empty(4, np.uint64)
    lib().or_philox4x64(_p(c), _p(k), _p(out))
    return out


def uniforms(seed: int, window: int, position: int) -> np.ndarray:
    out = np.empty(4, np.float64)
    lib().or_uniforms(seed, window, position, _p(out))
    return out


class WarpInfo(ctypes.Structure):
    _fields_ = [("n_keep", ctypes.c_int64), ("m_p", ctypes.c_int64), ("m_m", ctypes.c_int64),
                ("m_k", ctypes.c_int64),
                ("near_top_p", ctypes.c_int), ("near_min_p", ctypes.c_int),
                ("nonfinite", ctypes.c_int), ("argmax", ctypes.c_int64)]


def warp(logits: np.ndarray, T: float, top_p: float = 1.0, min_p: float = 0.0, top_k: int = 0):
    """Warped distribution p[V] (double) and the WarpInfo of one logits row."""
    l = np.ascontiguousarray(logits, dtype=np.float32)
    p = np.empty(l.shape[0], np.float64)
    info = WarpInfo()
    lib().or_warp(_p(l), l.shape[0], T, top_p, min_p, top_k, _p(p), ctypes.byref(info))
    return p, info


def argmax(logits: np.ndarray) -> int:
    l = np.ascontiguousarray(logits, dtype=np.float32)
    return int(lib().or_argmax(_p(l), l.shape[0]))


def cat(w: np.ndarray, u: float):
    w = np.ascontiguousarray(w, dtype=np.float64)
    near = ctypes.c_int(0)
    j = lib().or_cat(_p(w), w.shape[0], u, ctypes.byref(near))
    return int(j), bool(near.value)


class _AcceptArgs(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("draft_mode", ctypes.c_int),
                ("W", ctypes.c_int64), ("K", ctypes.c_int64), ("V", ctypes.c_int64),
                ("target", ctypes.c_void_p), ("draft", ctypes.c_void_p),
                ("draft_tokens", ctypes.c_void_p),
                ("T", ctypes.c_double), ("top_p", ctypes.c_double),
                ("min_p", ctypes.c_double), ("alpha", ctypes.c_double),
                ("seed", ctypes.c_uint64), ("window_base", ctypes.c_uint64),
                ("n_accepted", ctypes.c_void_p), ("tokens", ctypes.c_void_p),
                ("status", ctypes.c_void_p), ("near", ctypes.c_void_p),
                ("top_k", ctypes.c_int64)]


def accept(mode: int, target: np.ndarray, draft: np.ndarray | None = None,
           draft_tokens: np.ndarray | None = None, draft_mode: int = DRAFT_GIVEN,
           T: float = 1.0, top_p: float = 1.0, min_p: float = 0.0, alpha: float = 0.0,
           seed: int = 0, window_base: int = 0, threads: int = 1, top_k: int = 0) -> dict:
    """Acceptance of W windows.  target [W][K][V] f32, draft [W][K-1][V] f32.

    Returns n_accepted [W], tokens [W][K] (-1 padded), status [W], near [W] (bits of
    decisions within 1e-6 of a threshold) and draft_tokens [W][K-1] (drafted or given).
    """
    target = np.ascontiguousarray(target, dtype=np.float32)
    W, K, V = target.shape
    if draft is not None:
        draft = np.ascontiguousarray(draft, dtype=np.float32)
        assert draft.shape == (W, K - 1, V)
    if draft_tokens is None:
        draft_tokens = np.full((W, max(K - 1, 0)), -1, np.int32)
    else:
        draft_tokens = np.ascontiguousarray(draft_tokens, dtype=np.int32).copy()
    n_acc = np.zeros(W, np.int32)
    tokens = np.full((W, K), -1, np.int32)
    status = np.zeros(W, np.int32)
    near = np.zeros(W, np.int32)
    args = _AcceptArgs(mode, draft_mode, W, K, V, _p(target).value if W else None,
                       None if draft is None else _p(draft).value,
                       _p(draft_tokens).value if draft_tokens.size else None,
                       T, top_p, min_p, alpha, seed, window_base,
                       _p(n_acc).value, _p(tokens).value, _p(status).value, _p(near).value, top_k)
    rc = lib().or_accept(ctypes.byref(args), threads)
    if rc:
        raise RuntimeError(f"or_accept failed ({rc})")
    return dict(n_accepted=n_acc, tokens=tokens, status=status, near=near,
                draft_tokens=draft_tokens)



# ------------------------------------------------------------ adaptive draft depth
def tau(alpha: float, k: int) -> float:
    """Expected tokens per verify pass with k drafts, each accepted with probability alpha
    independently ("Decode is memory-bound ...", section "Speculative decoding"):
    (1 - alpha^(k+1)) / (1 - alpha), and k + 1 at alpha = 1."""
    if alpha == 1.0:
        return float(k + 1)
    return (1.0 - alpha ** (k + 1)) / (1.0 - alpha)


def depth_observe(stats, n_accepted, n_drafted, decay: float):
    """Fold windows into (accepted, rejected) in window order: accepted = decay * accepted +
    n; rejected = decay * rejected + (1 if the window ended on a rejected draft, n < drafted).
    A window with every draft accepted adds no failure (the next draft was never tried);
    accepted / (accepted + rejected) is then the maximum-likelihood per-draft acceptance."""
    acc, rej = float(stats[0]), float(stats[1])
    for n, d in zip(n_accepted, n_drafted):
        n, d = int(n), int(d)
        if d < 0 or n < 0 or n > d:
            raise ValueError("n_accepted outside [0, n_drafted]")
        acc = decay * acc + n
        rej = decay * rej + (1.0 if n < d else 0.0)
    return acc, rej


def depth_choose(stats, alpha_prior: float, prior_weight: float, t_pass, t_draft: float):
    """The depth k in 0 .. len(t_pass) - 1 maximising tau(a, k) / (t_pass[k] + k t_draft),
    a = (accepted + prior_weight alpha_prior) / (accepted + rejected + prior_weight) ("Decode
    is memory-bound ...", sections "Speculative decoding" and "Two things the math says to
    do": pick the depth from measured acceptance).  Ties go to the smaller k.  Returns
    (k, a, rates)."""
    acc, rej = float(stats[0]), float(stats[1])
    a = (acc + prior_weight * alpha_prior) / (acc + rej + prior_weight)
    rates = [tau(a, k) / (float(t_pass[k]) + k * t_draft) for k in range(len(t_pass))]
    best = 0
    for k in range(1, len(rates)):
        if rates[k] > rates[best]:
            best = k
    return best, a, rates


# --------------------------------------------------------------- n-gram map drafter
class NgramMap:
    """Prompt lookup generalised ("100 tokens per second ...", section "Lever 3: an n-gram
    overlay for repetition"): an incremental map from the k-token keys of the sequence so
    far to the position that followed their latest occurrence; the most recent k tokens
    look up their continuation, proposed as drafts.  A key enters the map once the token
    after it exists, so the current last k tokens find an earlier occurrence only."""

    def __init__(self, key_len: int):
        if key_len < 1:
            raise ValueError("key_len >= 1")
        self.k = key_len
        self.seq: list[int] = []
        self.map: dict[tuple, int] = {}

    def append(self, tokens):
        for t in tokens:
            self.seq.append(int(t))
            n = len(self.seq)
            # the key ending just before the new token now has a continuation (position n - 1)
            if n - 1 >= self.k:
                key = tuple(self.seq[n - 1 - self.k:n - 1])
                self.map[key] = n - 1

    def propose(self, max_drafts: int) -> list[int]:
        n = len(self.seq)
        if max_drafts <= 0 or n < self.k:
            return []
        p = self.map.get(tuple(self.seq[n - self.k:]))
        if p is None:
            return []
        return self.seq[p:min(p + max_drafts, n)]
