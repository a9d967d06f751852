"""Python binding of libvq, the speculative-decoding verify pass for MI355X (gfx950).

Argument marshalling only: every step of the pass runs in the HIP kernels of libvq.so;
PyTorch supplies device memory and the stream.  Importing this package loads the
library and fails loudly if it has not been built (``python
speculative_decoding_verification_bit_amd/build.py``); there is no CPU fallback.

Entry points (same names as the C ABI, without the ``vq_`` prefix):
  tile(W, dst, row0)         plain planes -> the tiled layout the kernels read
  verify_linear(W, x, ...)   y[K][rows] = W x, every weight byte read once
  verify_accept(...)         greedy / sampling acceptance over W windows
  decode_pass(model, x0)     the whole weight stack for a K-wide window -> logits
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
# torch first: its HIP runtime (soname libamdhip64.so.7) is then the one libvq.so binds
# to, so device memory, streams and kernels share a single runtime in the process.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvq.so")

OK, ERR_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_HOST = 0, -1, -2, -3, -4, -5
FMT_Q4, FMT_Q4_MIN, FMT_MXFP4, FMT_Q4_K = 0, 1, 2, 3
ABI_VERSION = 5            # the structs below mirror include/vq.h at this version
DTYPE_F32, DTYPE_F16 = 0, 1
LAUNCH_AUTO, LAUNCH_STAGED, LAUNCH_PERSISTENT = 0, 4, 8
ROWS_PLAIN, ROWS_PAIR8 = 0, 1
MODE_GREEDY, MODE_SAMPLE = 0, 1
DRAFT_GIVEN, DRAFT_Q_ARGMAX, DRAFT_Q_SAMPLE, DRAFT_AGREE = 0, 1, 2, 3
OP_LINEAR, OP_ACCEPT, OP_DECODE, OP_LINEAR_MX, OP_ATTENTION = 0, 1, 2, 3, 4
KV_Q8_0, KV_Q4_0 = 0, 1
MAX_K = 16

_P = ctypes.c_void_p


class VqMatrix(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("qs", _P), ("scales", _P), ("mins", _P), ("supers", _P)]


class VqTiled(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("order", ctypes.c_int32), ("data", _P)]


class VqLayer(ctypes.Structure):
    _fields_ = [(n, VqTiled) for n in ("qkv", "o", "gu", "down")]


class VqModel(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("layers", ctypes.POINTER(VqLayer)), ("lm_head", VqTiled)]


class VqAttention(ctypes.Structure):
    _fields_ = [("k_format", ctypes.c_int32), ("v_format", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("length", ctypes.c_int32),
                ("k_codes", _P), ("k_scales", _P), ("v_codes", _P), ("v_scales", _P)]


class VqDepthStats(ctypes.Structure):
    _fields_ = [("accepted", ctypes.c_double), ("rejected", ctypes.c_double)]


class VqAcceptDesc(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("draft_mode", ctypes.c_int32), ("W", ctypes.c_int32),
                ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("target_logits", _P), ("draft_logits", _P), ("draft_tokens", _P),
                ("temperature", ctypes.c_float), ("top_p", ctypes.c_float),
                ("min_p", ctypes.c_float), ("alpha", ctypes.c_float),
                ("seed", ctypes.c_uint64), ("window_base", ctypes.c_uint64),
                ("n_accepted", _P), ("tokens", _P), ("status", _P)]


EXPORTS = ("vq_tiled_bytes", "vq_tile", "vq_verify_linear", "vq_verify_linear_noalloc", "vq_verify_linear_mx",
           "vq_verify_attention", "vq_verify_accept", "vq_depth_observe", "vq_depth_choose",
           "vq_ngram_create", "vq_ngram_destroy", "vq_ngram_append", "vq_ngram_propose", "vq_decode_pass", "vq_decode_pass_timed",
           "vq_decode_stage_ptr", "vq_decode_error_word",
           "vq_workspace_bytes", "vq_status_string", "vq_last_error", "vq_abi_version")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"libvq.so not built at {path}; run "
                          "`python speculative_decoding_verification_bit_amd/build.py`")
    L = ctypes.CDLL(path)
    I32, SZ = ctypes.c_int32, ctypes.c_size_t
    L.vq_tiled_bytes.restype = SZ
    L.vq_tiled_bytes.argtypes = [I32, I32, I32]
    L.vq_tile.restype = I32
    L.vq_tile.argtypes = [ctypes.POINTER(VqMatrix), ctypes.POINTER(VqTiled), I32, _P]
    L.vq_verify_linear.restype = I32
    L.vq_verify_linear.argtypes = [ctypes.POINTER(VqTiled), _P, I32, _P, I32, _P, SZ, _P]
    L.vq_verify_linear_noalloc.restype = I32
    L.vq_verify_linear_noalloc.argtypes = [ctypes.POINTER(VqTiled), _P, I32, _P, I32, _P]
    L.vq_verify_linear_mx.restype = I32
    L.vq_verify_linear_mx.argtypes = [ctypes.POINTER(VqMatrix), _P, I32, _P, _P, SZ, _P]
    L.vq_verify_attention.restype = I32
    L.vq_verify_attention.argtypes = [ctypes.POINTER(VqAttention), _P, I32, _P, _P, SZ, _P]
    L.vq_depth_observe.restype = I32
    L.vq_depth_observe.argtypes = [ctypes.POINTER(VqDepthStats), _P, _P, I32, ctypes.c_double]
    L.vq_depth_choose.restype = I32
    L.vq_depth_choose.argtypes = [ctypes.POINTER(VqDepthStats), ctypes.c_double, ctypes.c_double, _P, I32,
                                  ctypes.c_double, ctypes.POINTER(I32), ctypes.POINTER(ctypes.c_double),
                                  ctypes.POINTER(ctypes.c_double)]
    L.vq_ngram_create.restype = I32
    L.vq_ngram_create.argtypes = [I32, ctypes.POINTER(_P)]
    L.vq_ngram_destroy.restype = None
    L.vq_ngram_destroy.argtypes = [_P]
    L.vq_ngram_append.restype = I32
    L.vq_ngram_append.argtypes = [_P, _P, I32]
    L.vq_ngram_propose.restype = I32
    L.vq_ngram_propose.argtypes = [_P, I32, _P, ctypes.POINTER(I32)]
    L.vq_verify_accept.restype = I32
    L.vq_verify_accept.argtypes = [ctypes.POINTER(VqAcceptDesc), _P, SZ, _P]
    L.vq_decode_pass.restype = I32
    L.vq_decode_pass.argtypes = [ctypes.POINTER(VqModel), _P, I32, _P, _P, SZ, _P]
    L.vq_decode_pass_timed.restype = I32
    L.vq_decode_pass_timed.argtypes = [ctypes.POINTER(VqModel), _P, I32, _P, I32, _P, SZ, _P,
                                       ctypes.POINTER(_P), I32, ctypes.POINTER(I32)]
    L.vq_decode_stage_ptr.restype = I32
    L.vq_decode_stage_ptr.argtypes = [ctypes.POINTER(VqModel), I32, _P, I32,
                                      ctypes.POINTER(_P), ctypes.POINTER(_P)]
    L.vq_decode_error_word.restype = I32
    L.vq_decode_error_word.argtypes = [ctypes.POINTER(VqModel), I32, _P, ctypes.POINTER(_P)]
    L.vq_workspace_bytes.restype = SZ
    L.vq_workspace_bytes.argtypes = [I32, _P, I32]
    L.vq_status_string.restype = ctypes.c_char_p
    L.vq_status_string.argtypes = [I32]
    L.vq_last_error.restype = ctypes.c_char_p
    L.vq_last_error.argtypes = []
    L.vq_abi_version.restype = I32
    L.vq_abi_version.argtypes = []
    if L.vq_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} has ABI version {L.vq_abi_version()}, this binding needs "
                          f"{ABI_VERSION}; rebuild it")
    return L


lib = load_library()


class VqError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = lib.vq_last_error().decode() or lib.vq_status_string(code).decode()
        super().__init__(f"{where}: {lib.vq_status_string(code).decode()} ({code}): {msg}")


def _check(rc: int, where: str):
    if rc != OK:
        raise VqError(rc, where)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _empty(nbytes: int, device):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


class DeviceMatrix:
    """A block-quantised matrix in device memory in the plain planes (torch tensors)."""

    def __init__(self, fmt: int, rows: int, cols: int, qs, scales, mins=None, supers=None):
        self.fmt, self.rows, self.cols = fmt, rows, cols
        self.qs, self.scales, self.mins, self.supers = qs, scales, mins, supers
        self.desc = VqMatrix(fmt, rows, cols, 0, _ptr(qs), _ptr(scales), _ptr(mins), _ptr(supers))
        self._tiled = None

    @classmethod
    def from_host(cls, m, device="cuda"):
        """Upload a synth.Q4Matrix (numpy arrays)."""
        import torch

        def up(a):
            if a is None:
                return None
            a = np.ascontiguousarray(a)
            return torch.from_numpy(a.view(np.uint16) if a.dtype == np.float16 else a).to(device)
        return cls(m.fmt, m.rows, m.cols, up(m.qs), up(m.scales), up(m.mins), up(getattr(m, "supers", None)))

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.qs, self.scales, self.mins, self.supers)
                   if t is not None)

    @property
    def tiled(self) -> "DeviceTiled":
        """The matrix in the tiled layout (made on first use, then kept)."""
        if self._tiled is None:
            self._tiled = DeviceTiled.empty(self.fmt, self.rows, self.cols, ROWS_PLAIN, self.qs.device)
            tile(self, self._tiled, 0)
        return self._tiled

    def drop_planes(self):
        self.qs = self.scales = self.mins = self.supers = None


class DeviceTiled:
    """A matrix in the library's tiled layout (one uint8 tensor) and its descriptor."""

    def __init__(self, fmt: int, rows: int, cols: int, order: int, data):
        self.fmt, self.rows, self.cols, self.order, self.data = fmt, rows, cols, order, data
        self.desc = VqTiled(fmt, rows, cols, order, _ptr(data))

    @classmethod
    def empty(cls, fmt: int, rows: int, cols: int, order: int = ROWS_PLAIN, device="cuda"):
        n = int(lib.vq_tiled_bytes(fmt, rows, cols))
        if n == 0 and rows > 0:
            raise ValueError(f"invalid tiled matrix fmt {fmt} {rows}x{cols}")
        return cls(fmt, rows, cols, order, _empty(n, device))

    @property
    def nbytes(self) -> int:
        return int(lib.vq_tiled_bytes(self.fmt, self.rows, self.cols))


def tile(src: DeviceMatrix, dst: DeviceTiled, row0: int = 0, stream=None):
    """Write src's rows into rows [row0, row0 + src.rows) of the tiled matrix dst."""
    _check(lib.vq_tile(ctypes.byref(src.desc), ctypes.byref(dst.desc), row0, _stream(stream)), "vq_tile")


def workspace_bytes(op: int, desc, K: int) -> int:
    return int(lib.vq_workspace_bytes(op, ctypes.cast(ctypes.pointer(desc), _P), K))


def verify_linear(W, x, y=None, y_dtype: int = DTYPE_F32, ws=None, stream=None):
    """y[K][rows] = W x for fp16 x [K][cols] on the device (W: DeviceTiled or DeviceMatrix)."""
    import torch
    if isinstance(W, DeviceMatrix):
        W = W.tiled
    K = x.shape[0]
    if y is None:
        y = torch.empty((K, W.rows), dtype=torch.float32 if y_dtype == DTYPE_F32 else torch.float16,
                        device=x.device)
    if ws is None:
        ws = _empty(workspace_bytes(OP_LINEAR, W.desc, K), x.device)
    _check(lib.vq_verify_linear(ctypes.byref(W.desc), _ptr(x), K, _ptr(y), y_dtype, _ptr(ws), ws.numel(),
                                _stream(stream)), "vq_verify_linear")
    return y


def verify_linear_noalloc(W, x, y=None, y_dtype: int = DTYPE_F32, stream=None):
    """verify_linear through the entry point that allocates nothing (library scratch)."""
    import torch
    if isinstance(W, DeviceMatrix):
        W = W.tiled
    K = x.shape[0]
    if y is None:
        y = torch.empty((K, W.rows), dtype=torch.float32 if y_dtype == DTYPE_F32 else torch.float16,
                        device=x.device)
    _check(lib.vq_verify_linear_noalloc(ctypes.byref(W.desc), _ptr(x), K, _ptr(y), y_dtype, _stream(stream)),
           "vq_verify_linear_noalloc")
    return y


def verify_linear_mx(W, x, y=None, ws=None, stream=None):
    """y ~= W x on the scaled MXFP4 matrix instruction with E4M3 activations (an
    approximation; W: DeviceMatrix with its plain MXFP4 planes)."""
    import torch
    K = x.shape[0]
    if y is None:
        y = torch.empty((K, W.rows), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = _empty(workspace_bytes(OP_LINEAR_MX, W.desc, K), x.device)
    _check(lib.vq_verify_linear_mx(ctypes.byref(W.desc), _ptr(x), K, _ptr(y), _ptr(ws), ws.numel(),
                                   _stream(stream)), "vq_verify_linear_mx")
    return y


class DeviceKV:
    """One layer's quantised KV cache on the device (torch tensors: codes uint8
    [Hkv][L][D or D/2], scales fp16 [Hkv][L][D/32]) and the query heads that read it."""

    def __init__(self, k_format: int, kcodes, kscales, v_format: int, vcodes, vscales, n_q_heads: int):
        self.k_codes, self.k_scales, self.v_codes, self.v_scales = kcodes, kscales, vcodes, vscales
        Hkv, L = kscales.shape[0], kscales.shape[1]
        self.desc = VqAttention(k_format, v_format, n_q_heads, Hkv, kscales.shape[2] * 32, L,
                                _ptr(kcodes), _ptr(kscales), _ptr(vcodes), _ptr(vscales))

    @classmethod
    def from_host(cls, k_format, kcodes, kscales, v_format, vcodes, vscales, n_q_heads, device="cuda"):
        import torch
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
        return cls(k_format, t(kcodes), t(kscales), v_format, t(vcodes), t(vscales), n_q_heads)

    def workspace_bytes(self, K: int) -> int:
        return int(lib.vq_workspace_bytes(OP_ATTENTION, ctypes.byref(self.desc), K))


def verify_attention(C: DeviceKV, q, out=None, ws=None, stream=None):
    """The window's attention over the cache: q fp16 [K][Hq][D] -> out f32 [K][Hq][D]."""
    import torch
    K = q.shape[0]
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = _empty(C.workspace_bytes(K), q.device)
    _check(lib.vq_verify_attention(ctypes.byref(C.desc), _ptr(q), K, _ptr(out), _ptr(ws), ws.numel(),
                                   _stream(stream)), "vq_verify_attention")
    return out


def depth_observe(stats: VqDepthStats, n_accepted, n_drafted, decay: float = 1.0) -> VqDepthStats:
    """Fold windows (host int arrays) into the running acceptance statistics (in place)."""
    a = np.ascontiguousarray(n_accepted, dtype=np.int32)
    d = np.ascontiguousarray(n_drafted, dtype=np.int32)
    _check(lib.vq_depth_observe(ctypes.byref(stats), a.ctypes.data, d.ctypes.data, a.size, decay),
           "vq_depth_observe")
    return stats


def depth_choose(stats: VqDepthStats, t_pass, t_draft: float, alpha_prior: float = 0.5,
                 prior_weight: float = 0.0):
    """The draft depth maximising expected tokens per unit time at the measured pass times
    t_pass[k] (k drafts): returns (k, alpha estimate, rate)."""
    t = np.ascontiguousarray(t_pass, dtype=np.float64)
    k = ctypes.c_int32(-1)
    a, r = ctypes.c_double(), ctypes.c_double()
    _check(lib.vq_depth_choose(ctypes.byref(stats), alpha_prior, prior_weight, t.ctypes.data, t.size - 1,
                               t_draft, ctypes.byref(k), ctypes.byref(a), ctypes.byref(r)), "vq_depth_choose")
    return k.value, a.value, r.value


class NgramMap:
    """The library's n-gram map drafter over one token sequence (host memory)."""

    def __init__(self, key_len: int):
        h = _P()
        _check(lib.vq_ngram_create(key_len, ctypes.byref(h)), "vq_ngram_create")
        self._h = h
        self._lib = lib
        self._buf = np.empty(16, dtype=np.int32)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.vq_ngram_destroy(h)
            self._h = None

    def append(self, tokens):
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        _check(lib.vq_ngram_append(self._h, t.ctypes.data, t.size), "vq_ngram_append")

    def propose(self, max_drafts: int) -> list:
        if self._buf.size < max_drafts:
            self._buf = np.empty(max_drafts, dtype=np.int32)
        n = ctypes.c_int32(-1)
        _check(lib.vq_ngram_propose(self._h, max_drafts, self._buf.ctypes.data, ctypes.byref(n)),
               "vq_ngram_propose")
        return self._buf[:n.value].tolist()


def accept_desc(mode, target, draft=None, draft_tokens=None, draft_mode=DRAFT_GIVEN, T=1.0,
                top_p=1.0, min_p=0.0, alpha=0.0, seed=0, window_base=0, n_accepted=None,
                tokens=None, status=None, top_k=0) -> VqAcceptDesc:
    W, K, V = target.shape
    return VqAcceptDesc(mode, draft_mode, W, K, V, top_k, _ptr(target), _ptr(draft), _ptr(draft_tokens),
                        T, top_p, min_p, alpha, seed, window_base, _ptr(n_accepted), _ptr(tokens),
                        _ptr(status))


def verify_accept(mode: int, target, draft=None, draft_tokens=None, draft_mode: int = DRAFT_GIVEN,
                  T: float = 1.0, top_p: float = 1.0, min_p: float = 0.0, alpha: float = 0.0,
                  seed: int = 0, window_base: int = 0, ws=None, out=None, stream=None,
                  top_k: int = 0) -> dict:
    """Acceptance over W windows of fp32 target [W][K][V] / drafter [W][K-1][V] logits."""
    import torch
    W, K, V = target.shape
    dev = target.device
    if out is None:
        out = dict(n_accepted=torch.empty(W, dtype=torch.int32, device=dev),
                   tokens=torch.empty((W, K), dtype=torch.int32, device=dev),
                   status=torch.empty(W, dtype=torch.int32, device=dev))
    if draft_tokens is None and K > 1:
        draft_tokens = torch.full((W, K - 1), -1, dtype=torch.int32, device=dev)
    d = accept_desc(mode, target, draft, draft_tokens, draft_mode, T, top_p, min_p, alpha, seed,
                    window_base, out["n_accepted"], out["tokens"], out["status"], top_k)
    need = int(lib.vq_workspace_bytes(OP_ACCEPT, ctypes.byref(d), K))
    if ws is None:
        ws = _empty(need, dev)
    _check(lib.vq_verify_accept(ctypes.byref(d), _ptr(ws), ws.numel(), _stream(stream)),
           "vq_verify_accept")
    out["draft_tokens"] = draft_tokens
    return out


class DeviceModel:
    """A dense decoder's weight stack on the device, in the tiled stage matrices the pass
    reads: per layer q|k|v stacked, o, gate|up paired by 8 rows, down; and the lm_head.

    layers: dicts of DeviceMatrix (q, k, v, o, gate, up, down); lm_head: DeviceMatrix.
    With drop_planes the plain planes are released once tiled."""

    def __init__(self, layers: list[dict], lm_head, drop_planes: bool = True):
        arr = (VqLayer * len(layers))()
        self.tiled = []
        self.shapes = []
        for i, L in enumerate(layers):
            q, k, v, o, g, u, d = (L[n] for n in ("q", "k", "v", "o", "gate", "up", "down"))
            dev = q.qs.device
            H, KV, FF = q.cols, k.rows, g.rows
            qkv = DeviceTiled.empty(q.fmt, H + 2 * KV, H, ROWS_PLAIN, dev)
            tile(q, qkv, 0)
            tile(k, qkv, H)
            tile(v, qkv, H + KV)
            gu = DeviceTiled.empty(q.fmt, 2 * FF, H, ROWS_PAIR8, dev)
            tile(g, gu, 0)
            tile(u, gu, FF)
            to = DeviceTiled.empty(q.fmt, o.rows, o.cols, ROWS_PLAIN, dev)
            tile(o, to, 0)
            td = DeviceTiled.empty(q.fmt, d.rows, d.cols, ROWS_PLAIN, dev)
            tile(d, td, 0)
            t = {"qkv": qkv, "o": to, "gu": gu, "down": td}
            self.tiled.append(t)
            self.shapes.append(dict(H=H, KV=KV, FF=FF))
            for n in ("qkv", "o", "gu", "down"):
                setattr(arr[i], n, t[n].desc)
            if drop_planes:
                for m in (q, k, v, o, g, u, d):
                    m.drop_planes()
        if isinstance(lm_head, DeviceMatrix):
            self.lm_head = lm_head.tiled
            if drop_planes:
                lm_head.drop_planes()
        else:
            self.lm_head = lm_head
        self.n_layers = len(layers)
        self._arr = arr
        self.desc = VqModel(len(layers), 0, ctypes.cast(arr, ctypes.POINTER(VqLayer)), self.lm_head.desc)

    @property
    def hidden(self) -> int:
        return self.shapes[0]["H"]

    @property
    def vocab(self) -> int:
        return self.lm_head.rows

    @property
    def nbytes(self) -> int:
        """Bytes of the tiled weights a pass streams."""
        n = self.lm_head.nbytes
        for L in self.tiled:
            n += sum(m.nbytes for m in L.values())
        return n

    def workspace_bytes(self, K: int) -> int:
        return int(lib.vq_workspace_bytes(OP_DECODE, ctypes.byref(self.desc), K))

    def stage_ptrs(self, K: int, ws, stage: int):
        a, b = _P(), _P()
        _check(lib.vq_decode_stage_ptr(ctypes.byref(self.desc), K, _ptr(ws), stage,
                                       ctypes.byref(a), ctypes.byref(b)), "vq_decode_stage_ptr")
        return a.value, b.value

    def barrier_error(self, K: int, ws) -> int:
        """The grid-barrier error word of the last pass in ws (0: every barrier completed)."""
        import torch
        a = _P()
        _check(lib.vq_decode_error_word(ctypes.byref(self.desc), K, _ptr(ws), ctypes.byref(a)),
               "vq_decode_error_word")
        return int(stage_tensor(ws, a.value, (1,), torch.int32).item())


def decode_pass(model: DeviceModel, x0, logits=None, ws=None, stream=None):
    """logits[K][V] of one verify pass over the whole stack; ws keeps every stage's tensors."""
    import torch
    K = x0.shape[0]
    if logits is None:
        logits = torch.empty((K, model.vocab), dtype=torch.float32, device=x0.device)
    if ws is None:
        ws = _empty(model.workspace_bytes(K), x0.device)
    _check(lib.vq_decode_pass(ctypes.byref(model.desc), _ptr(x0), K, _ptr(logits), _ptr(ws), ws.numel(),
                              _stream(stream)), "vq_decode_pass")
    return logits, ws


def decode_pass_launch(model: DeviceModel, x0, logits=None, ws=None, launch: int = LAUNCH_AUTO, events=None,
                       stream=None):
    """decode_pass with a chosen launch mode (LAUNCH_STAGED: one launch per stage), and
    optionally HIP events around each launch.  Returns (logits, ws, number of launches).

    events: a list of torch.cuda.Event(enable_timing=True), already recorded once (so that
    their HIP handles exist); events[2 i] / events[2 i + 1] bracket launch i."""
    import torch
    K = x0.shape[0]
    if logits is None:
        logits = torch.empty((K, model.vocab), dtype=torch.float32, device=x0.device)
    if ws is None:
        ws = _empty(model.workspace_bytes(K), x0.device)
    if not events:
        sink = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for ev in sink:
            ev.record()
        events = sink
    arr = (_P * len(events))(*[ev.cuda_event for ev in events])
    n = ctypes.c_int32(0)
    _check(lib.vq_decode_pass_timed(ctypes.byref(model.desc), _ptr(x0), K, _ptr(logits), launch, _ptr(ws),
                                    ws.numel(), _stream(stream), arr, len(events), ctypes.byref(n)),
           "vq_decode_pass_timed")
    return logits, ws, n.value


def stage_tensor(ws, addr: int, shape, dtype):
    """A view of a tensor inside the decode workspace at device address addr."""
    import torch
    off = addr - ws.data_ptr()
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    return ws[off:off + n].view(dtype).view(*shape)
