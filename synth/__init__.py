"""Seeded synthetic inputs for the speculative-decoding verify pass.

Both the HIP path and the CPU oracle consume the bytes this module produces.  It holds
only random draws and their packing into the byte layouts the library reads; none of
the method's arithmetic (no dequantisation, no dot products, no softmax, no sampling)
lives here.

Every array is a pure function of (seed, what it is, where it is), drawn from numpy's
``default_rng`` seeded by a ``SeedSequence`` built from those integers, so any matrix,
any 256-row chunk of a matrix and any acceptance window can be regenerated on its own.

Layouts (all row-major, C order):
  * 4-bit weights ``qs``: uint8 ``[rows][cols/2]``; byte ``j//2`` of a row holds column
    ``j`` in its low nibble when ``j`` is even and in its high nibble when ``j`` is odd.
  * Q4 block scales / mins: float16 ``[rows][cols/32]`` (one per 32 consecutive columns).
  * MXFP4 block scales: uint8 E8M0 ``[rows][cols/32]``.
  * Activations: float16 ``[K][cols]`` (column k of the verify window is row k here).
  * Logits: float32, target ``[W][K][V]`` and drafter ``[W][K-1][V]``.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

FMT_Q4 = 0          # 4-bit code + fp16 block scale
FMT_Q4_MIN = 1      # 4-bit code + fp16 block scale + fp16 block min
FMT_MXFP4 = 2       # E2M1 code + E8M0 block scale
FMT_Q4_K = 3        # unsigned 4-bit code, 6-bit sub-block scale and min, fp16 super-block d, dmin

BLOCK = 32
SUPER = 256         # weights per Q4_K super-block (eight blocks)
ROW_CHUNK = 256     # rows per independently seeded chunk of a weight matrix

_TAG_WEIGHT = 1
_TAG_ACT = 2
_TAG_LOGITS = 3

# Matrix ids inside one decoder layer, in stage order.
MAT_Q, MAT_K, MAT_V, MAT_O, MAT_GATE, MAT_UP, MAT_DOWN, MAT_LM_HEAD = range(8)
LAYER_MATS = ("q", "k", "v", "o", "gate", "up", "down")


def _rng(*keys: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in keys]))


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Shapes of a dense decoder's weight stack (no attention/norm weights)."""
    n_layers: int
    hidden: int
    kv_dim: int
    ffn: int
    vocab: int

    def mat_shape(self, mat: int) -> tuple[int, int]:
        h, kv, ff = self.hidden, self.kv_dim, self.ffn
        return {MAT_Q: (h, h), MAT_K: (kv, h), MAT_V: (kv, h), MAT_O: (h, h),
                MAT_GATE: (ff, h), MAT_UP: (ff, h), MAT_DOWN: (h, ff),
                MAT_LM_HEAD: (self.vocab, h)}[mat]

    def n_weights(self) -> int:
        per_layer = sum(r * c for r, c in (self.mat_shape(m) for m in range(7)))
        r, c = self.mat_shape(MAT_LM_HEAD)
        return self.n_layers * per_layer + r * c


# The 27B-class stack: 64 layers of hidden 5120, kv 1024, ffn 17408, vocab 151936.
SHAPE_27B = ModelShape(n_layers=64, hidden=5120, kv_dim=1024, ffn=17408, vocab=151936)
# A small stack with the same structure, for full (every row, every stage) parity.
SHAPE_MINI = ModelShape(n_layers=2, hidden=256, kv_dim=64, ffn=512, vocab=1000)


def bytes_per_weight(fmt: int) -> float:
    return {FMT_Q4: 0.5 + 2 / 32, FMT_Q4_MIN: 0.5 + 4 / 32, FMT_MXFP4: 0.5 + 1 / 32,
            FMT_Q4_K: 0.5 + 2 / 32 + 4 / 256}[fmt]


@dataclasses.dataclass
class Q4Matrix:
    fmt: int
    rows: int
    cols: int
    qs: np.ndarray                 # uint8 [rows][cols/2]
    scales: np.ndarray             # [rows][cols/32]: float16 (Q4, Q4_MIN), uint8 E8M0 (MXFP4),
                                   # uint8 6-bit sub-block scale s (Q4_K)
    mins: np.ndarray | None        # [rows][cols/32]: float16 (Q4_MIN), uint8 6-bit m (Q4_K), else None
    supers: np.ndarray | None = None   # Q4_K: float16 [rows][cols/256][2] = (d, dmin)

    @property
    def nbytes(self) -> int:
        n = self.qs.nbytes + self.scales.nbytes
        n += self.mins.nbytes if self.mins is not None else 0
        return n + (self.supers.nbytes if self.supers is not None else 0)

    def take(self, pick) -> "Q4Matrix":
        """The listed rows, as a matrix of their own."""
        pick = np.asarray(pick, dtype=np.int64)
        return Q4Matrix(self.fmt, len(pick), self.cols, self.qs[pick], self.scales[pick],
                        None if self.mins is None else self.mins[pick],
                        None if self.supers is None else self.supers[pick])


def _chunk_arrays(fmt: int, seed: int, layer: int, mat: int, chunk: int,
                  nrows: int, cols: int, scale_lo: float, scale_hi: float):
    rng = _rng(seed, _TAG_WEIGHT, layer, mat, chunk)
    nb = cols // BLOCK
    qs = rng.integers(0, 256, size=(nrows, cols // 2), dtype=np.uint8)
    if fmt == FMT_MXFP4:
        scales = rng.integers(119, 124, size=(nrows, nb), dtype=np.uint8)
        mins = None
    elif fmt == FMT_Q4_K:
        ns = cols // SUPER
        d = rng.uniform(scale_lo, scale_hi, size=(nrows, ns)) / 32
        dmin = d * rng.uniform(6.0, 12.0, size=(nrows, ns))
        supers = np.stack([d, dmin], axis=-1).astype(np.float16)
        scales = rng.integers(16, 64, size=(nrows, nb), dtype=np.uint8)
        mins = rng.integers(0, 64, size=(nrows, nb), dtype=np.uint8)
        return qs, scales, mins, supers
    else:
        scales = rng.uniform(scale_lo, scale_hi, size=(nrows, nb)).astype(np.float16)
        mins = (rng.uniform(-0.01, 0.01, size=(nrows, nb)).astype(np.float16)
                if fmt == FMT_Q4_MIN else None)
    return qs, scales, mins, None


def weight_matrix(fmt: int, seed: int, layer: int, mat: int, rows: int, cols: int,
                  row_begin: int = 0, row_end: int | None = None,
                  scale_lo: float = 0.005, scale_hi: float = 0.02,
                  threads: int = 1) -> Q4Matrix:
    """Rows [row_begin, row_end) of weight matrix (layer, mat), in chunks of ROW_CHUNK rows.

    Q4 / Q4_MIN: nibble bytes uniform over 0..255 (both nibbles uniform on 16 codes),
    fp16 scales ~U(scale_lo, scale_hi), fp16 mins ~U(-0.01, 0.01).
    MXFP4: nibble bytes uniform (E2M1 codes uniform on 16 codes), E8M0 bytes uniform on
    {119..123}, i.e. block scales 2^-8 .. 2^-4.
    Q4_K: nibble bytes uniform, super-block d ~ U(scale_lo, scale_hi) / 32 and
    dmin = d * U(6, 12) (fp16), sub-block s uniform on 16..63 and m on 0..63: the
    sub-block scale d*s spans the Q4 range and dmin*m sits near the middle of the
    code range, so the weights are roughly centred.
    """
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 32")
    if fmt == FMT_Q4_K and cols % SUPER:
        raise ValueError("Q4_K cols must be a multiple of 256")
    row_end = rows if row_end is None else row_end
    c0, c1 = row_begin // ROW_CHUNK, (row_end + ROW_CHUNK - 1) // ROW_CHUNK
    nb = cols // BLOCK
    n = row_end - row_begin
    qs = np.empty((n, cols // 2), np.uint8)
    scales = np.empty((n, nb), np.uint8 if fmt in (FMT_MXFP4, FMT_Q4_K) else np.float16)
    mins = (np.empty((n, nb), np.float16) if fmt == FMT_Q4_MIN else
            np.empty((n, nb), np.uint8) if fmt == FMT_Q4_K else None)
    supers = np.empty((n, cols // SUPER, 2), np.float16) if fmt == FMT_Q4_K else None

    def work(ci: int):
        r0 = ci * ROW_CHUNK
        nr = min(ROW_CHUNK, rows - r0)
        q, s, m, sp = _chunk_arrays(fmt, seed, layer, mat, ci, nr, cols, scale_lo, scale_hi)
        a, b = max(r0, row_begin), min(r0 + nr, row_end)
        qs[a - row_begin:b - row_begin] = q[a - r0:b - r0]
        scales[a - row_begin:b - row_begin] = s[a - r0:b - r0]
        if mins is not None:
            mins[a - row_begin:b - row_begin] = m[a - r0:b - r0]
        if supers is not None:
            supers[a - row_begin:b - row_begin] = sp[a - r0:b - r0]

    if threads > 1 and c1 - c0 > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(c0, c1)))
    else:
        for ci in range(c0, c1):
            work(ci)
    return Q4Matrix(fmt, n, cols, qs, scales, mins, supers)


def weight_rows(fmt: int, seed: int, layer: int, mat: int, rows: int, cols: int,
                row_ids) -> Q4Matrix:
    """Only the listed rows of a matrix (regenerating just their chunks)."""
    row_ids = np.asarray(row_ids, dtype=np.int64)
    parts = [weight_matrix(fmt, seed, layer, mat, rows, cols, int(r), int(r) + 1) for r in row_ids]
    return Q4Matrix(fmt, len(row_ids), cols,
                    np.concatenate([p.qs for p in parts]),
                    np.concatenate([p.scales for p in parts]),
                    None if parts[0].mins is None else np.concatenate([p.mins for p in parts]),
                    None if parts[0].supers is None else np.concatenate([p.supers for p in parts]))


def activations(seed: int, K: int, cols: int, tag: int = 0) -> np.ndarray:
    """K activation columns ~N(0,1), rounded to fp16: array [K][cols]."""
    rng = _rng(seed, _TAG_ACT, tag, K, cols)
    return rng.standard_normal((K, cols), dtype=np.float32).astype(np.float16)


_TAG_KV = 4
KV_Q8_0, KV_Q4_0 = 0, 1


def kv_cache(fmt: int, seed: int, layer: int, which: int, n_kv_heads: int, length: int, head_dim: int = 128,
             threads: int = 1):
    """One layer's key (which = 0) or value (which = 1) cache: codes and fp16 block scales
    (blocks of 32 along the head dimension), generated in chunks of 1024 positions.
    q8_0: int8 codes uniform in -127..127, scales ~U(0.01, 0.03);
    q4_0: nibble bytes uniform over 0..255, scales ~U(0.1, 0.3).
    Returns codes uint8 [Hkv][L][D] (q8_0, int8 bit patterns) or [Hkv][L][D/2] (q4_0) and
    scales float16 [Hkv][L][D/32]."""
    cb = head_dim if fmt == KV_Q8_0 else head_dim // 2
    codes = np.empty((n_kv_heads, length, cb), np.uint8)
    scales = np.empty((n_kv_heads, length, head_dim // 32), np.float16)
    jobs = [(g, c0) for g in range(n_kv_heads) for c0 in range(0, length, 1024)]

    def work(job):
        g, c0 = job
        n = min(1024, length - c0)
        rng = _rng(seed, _TAG_KV, layer, which, fmt, g, c0)
        if fmt == KV_Q8_0:
            codes[g, c0:c0 + n] = rng.integers(-127, 128, size=(n, cb)).astype(np.int8).view(np.uint8)
            scales[g, c0:c0 + n] = rng.uniform(0.01, 0.03, size=(n, head_dim // 32)).astype(np.float16)
        else:
            codes[g, c0:c0 + n] = rng.integers(0, 256, size=(n, cb), dtype=np.uint8)
            scales[g, c0:c0 + n] = rng.uniform(0.1, 0.3, size=(n, head_dim // 32)).astype(np.float16)

    if threads > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, jobs))
    else:
        for j in jobs:
            work(j)
    return codes, scales


def queries(seed: int, K: int, n_q_heads: int, head_dim: int = 128) -> np.ndarray:
    """K query rows per head ~N(0,1), fp16: [K][Hq][D]."""
    rng = _rng(seed, _TAG_KV, 1 << 20, K, n_q_heads, head_dim)
    return rng.standard_normal((K, n_q_heads, head_dim), dtype=np.float32).astype(np.float16)


@dataclasses.dataclass(frozen=True)
class LogitSpec:
    seed: int
    K: int
    vocab: int
    target_sigma: float
    noise_sigma: float


def window_logits(spec: LogitSpec, window: int):
    """Target [K][V] ~N(0, target_sigma) and drafter [K-1][V] = target rows 0..K-2 + N(0, noise_sigma).

    Drafter row i (0-based) scores the same position as target row i; target row K-1 is
    the bonus position, which no draft covers.
    """
    rng = _rng(spec.seed, _TAG_LOGITS, window)
    t = rng.standard_normal((spec.K, spec.vocab), dtype=np.float32) * np.float32(spec.target_sigma)
    n = rng.standard_normal((spec.K - 1, spec.vocab), dtype=np.float32) * np.float32(spec.noise_sigma)
    return t, (t[: spec.K - 1] + n).astype(np.float32)


def logits_batch(spec: LogitSpec, w0: int, w1: int, threads: int = 1):
    """Windows [w0, w1): target [W][K][V] and drafter [W][K-1][V] float32."""
    W = w1 - w0
    tgt = np.empty((W, spec.K, spec.vocab), np.float32)
    drf = np.empty((W, max(spec.K - 1, 0), spec.vocab), np.float32)

    def work(i):
        t, d = window_logits(spec, w0 + i)
        tgt[i] = t
        drf[i] = d

    if threads > 1 and W > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(W)))
    else:
        for i in range(W):
            work(i)
    return tgt, drf


# The five workloads: sizes, formats, seeds and sampler settings.
C1 = dict(name="tiny-1024x1024-q4-K4-V256", seed=0, rows=1024, cols=1024, fmt=FMT_Q4, K=4,
          logits=LogitSpec(seed=0, K=4, vocab=256, target_sigma=2.0, noise_sigma=0.5),
          windows=10_000, T=1.0, top_p=1.0, min_p=0.0, philox_seed=0)
C2 = dict(name="27b-q4min-K1-decode", seed=0, shape=SHAPE_27B, fmt=FMT_Q4_MIN, K=1)
C3 = dict(name="27b-q4min-K4-greedy", seed=0, shape=SHAPE_27B, fmt=FMT_Q4_MIN, K=4,
          alpha=0.7, philox_seed=0)
C4 = dict(name="27b-q4min-K8-sample", seed=0, shape=SHAPE_27B, fmt=FMT_Q4_MIN, K=8,
          logits=LogitSpec(seed=1, K=8, vocab=151936, target_sigma=3.0, noise_sigma=1.0),
          windows=1000, T=0.6, top_p=0.95, min_p=0.05, philox_seed=1)
C5 = dict(name="27b-mxfp4-K16", seed=0, shape=SHAPE_27B, fmt=FMT_MXFP4, K=16)
# The window's attention in one layer of the 27B-class stack over a 32K-position cache with
# keys at q8_0 and values at q4_0 (40 query heads, 8 kv heads, head dimension 128).
ATTN = dict(name="27b-attn-32k-k8v4", seed=0, n_q_heads=40, n_kv_heads=8, head_dim=128, length=32768,
            kfmt=KV_Q8_0, vfmt=KV_Q4_0)


_TAG_TOKENS = 5


def token_stream(seed: int, n: int, vocab: int = 151936, n_snippets: int = 400, p_novel: float = 0.3,
                 p_edit: float = 0.05) -> np.ndarray:
    """A token stream with the repetition of code (identifiers, imports, call signatures and
    re-emitted spans recur): a library of n_snippets random snippets (lengths 4..40 tokens,
    uniform over the vocabulary) drawn with Zipf-like weights (rank r at 1/(r+1)), each
    occurrence with every token replaced with probability p_edit, and runs of 1..20 novel
    uniform tokens between snippets with probability p_novel.  int32 [n]."""
    rng = _rng(seed, _TAG_TOKENS, n, vocab, n_snippets)
    lens = rng.integers(4, 41, n_snippets)
    lib = [rng.integers(0, vocab, L).astype(np.int32) for L in lens]
    w = 1.0 / (np.arange(n_snippets) + 1.0)
    w /= w.sum()
    out, m = [], 0
    while m < n:
        if rng.random() < p_novel:
            piece = rng.integers(0, vocab, int(rng.integers(1, 21))).astype(np.int32)
        else:
            piece = lib[int(rng.choice(n_snippets, p=w))].copy()
            edit = rng.random(piece.size) < p_edit
            piece[edit] = rng.integers(0, vocab, int(edit.sum()))
        out.append(piece)
        m += piece.size
    return np.concatenate(out)[:n].astype(np.int32)
