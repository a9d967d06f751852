/*
 * vq.h -- C ABI of libvq, the speculative-decoding verify pass on AMD Instinct MI355X
 * (gfx950).
 *
 * The pass has two parts, both described on the page "100 tokens per second from a
 * 27B model on a 24 GB AMD card" (section "How speculative decoding gets past a
 * per-token wall") and on the Hacker News thread 49596054:
 *   1. every block-quantised weight matrix of a dense decoder is read from HBM once and
 *      multiplied into the K drafted-token activation columns, layer by layer
 *      (vq_verify_linear for one matrix, vq_decode_pass for the whole stack);
 *   2. a lossless acceptance rule turns the [K][vocab] logits into emitted tokens
 *      (vq_verify_accept).
 *
 * Conventions for every entry point:
 *   - Buffers are caller-owned DEVICE pointers unless stated otherwise; descriptors are
 *     HOST structs, read only during the call.  Per-call scratch space is a caller-provided
 *     workspace sized by vq_workspace_bytes().
 *   - Work lists: the weight-streaming kernel follows, per compute wave, a list of steps
 *     that depends only on the shapes, K and the device's compute-unit count.  The first
 *     vq_verify_linear or vq_decode_pass call with a new (device, shapes, K, launch mode)
 *     builds that list on the host, allocates device memory for it, copies it and waits
 *     for `stream`; the library keeps it until the process ends (about 44 MB for a
 *     27B-class pass at one K) and reuses it in every later call with the same key.  Such
 *     a first call cannot be captured into a graph (it returns VQ_ERR_UNSUPPORTED under
 *     capture): call once before capturing.  vq_verify_linear_noalloc keeps its lists in
 *     static device memory instead.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).  Apart from
 *     the first call with a new key above, no call synchronises the host, copies to the
 *     host or allocates.  Buffers must stay alive until the stream has executed the work.
 *   - Return value: VQ_OK (0) or a negative VQ_ERR_* code.  Arguments are validated on
 *     the host before anything is launched; on an argument error nothing is enqueued.
 *     vq_last_error() returns a thread-local text for the last failure.
 *   - No C++ exception crosses this interface.  Global state: the work lists above (behind
 *     a mutex) and that thread-local text.
 *   - Calls that share a workspace must not overlap on the device.
 */
#ifndef VQ_H
#define VQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VQ_ABI_VERSION 5

/* ------------------------------------------------------------------ status */
#define VQ_OK 0
#define VQ_ERR_ARG (-1)          /* invalid argument (NULL, size, range, alignment)     */
#define VQ_ERR_UNSUPPORTED (-2)  /* valid but not instantiated (format / K / path)      */
#define VQ_ERR_WORKSPACE (-3)    /* workspace NULL or smaller than vq_workspace_bytes() */
#define VQ_ERR_HIP (-4)          /* a HIP launch or runtime call failed                 */
#define VQ_ERR_HOST (-5)         /* a host allocation failed                            */

/* ------------------------------------------------------------ weight format */
/* Block-quantised weights, row-major, blocks of 32 consecutive input columns.
 *   qs     : uint8 [rows][cols/2]; byte j/2 of a row holds column j in its low nibble
 *            when j is even, in its high nibble when j is odd.
 *   VQ_FMT_Q4      : code n in 0..15, q = n - 8, w = d * q          (d: fp16 scale)
 *   VQ_FMT_Q4_MIN  : w = d * q + m                                   (m: fp16 block min)
 *   VQ_FMT_MXFP4   : w = e2m1(n) * 2^(E - 127)  (OCP Microscaling v1.0: E2M1 code, E8M0 E)
 *   VQ_FMT_Q4_K    : K-quant super-blocks of 256 columns (8 blocks): unsigned code n,
 *                    w = D * s * n - Dmin * m  (s, m: the block's 6-bit scale and min,
 *                    D, Dmin: the super-block's fp16 scale and min scale); cols % 256 == 0
 *   scales : fp16 [rows][cols/32] (Q4, Q4_MIN), uint8 E8M0 [rows][cols/32] (MXFP4),
 *            uint8 s [rows][cols/32] (Q4_K; K-quant encoders use 0..63, any byte decodes)
 *   mins   : fp16 [rows][cols/32] for Q4_MIN, uint8 m [rows][cols/32] for Q4_K, NULL
 *            otherwise
 *   supers : fp16 pairs (D, Dmin) [rows][cols/256][2] for Q4_K, NULL otherwise
 * Alignment: qs, scales, mins and supers 16-byte aligned.
 * The pages name 4-bit block formats (Q4_K_M, UD-Q4_K_XL, q4_0) and MXFP4 without
 * defining them; these are the layouts the library implements (Q4_K: the public GGML
 * K-quant arithmetic, with one byte per 6-bit value instead of its packed 12 bytes). */
#define VQ_FMT_Q4 0
#define VQ_FMT_Q4_MIN 1
#define VQ_FMT_MXFP4 2
#define VQ_FMT_Q4_K 3

typedef struct vq_matrix {
    int32_t format;       /* VQ_FMT_*                                   */
    int32_t rows;         /* output features, >= 0                      */
    int32_t cols;         /* input features, > 0, multiple of 32        */
    int32_t reserved;     /* must be 0                                  */
    const void* qs;       /* device */
    const void* scales;   /* device */
    const void* mins;     /* device or NULL */
    const void* supers;   /* device (Q4_K) or NULL */
} vq_matrix;

/* --------------------------------------------------------------- tiled layout */
/* The streaming kernels read weights in a tiled layout made once, at load time, from the
 * plain planes above by vq_tile.  It keeps every 16-row x 128-column piece (a chunk) of
 * a matrix contiguous, with its codes in the order the matrix cores take them and its
 * rows' block scales (and mins) beside them, so that a chunk is two 16-byte loads per
 * lane; the layout is private to the library and may change with VQ_ABI_VERSION.
 * Rows past the matrix and columns past a multiple of 128 are stored as zero weights.
 *   order VQ_ROWS_PLAIN : tile t holds rows 16t .. 16t+15
 *   order VQ_ROWS_PAIR8 : rows [0, R/2) and [R/2, R) are two matrices of equal shape
 *                         (gate and up); tile t holds rows 8t..8t+7 of each, so that a
 *                         tile's outputs give silu(gate) * up directly.  R % 16 == 0. */
#define VQ_ROWS_PLAIN 0
#define VQ_ROWS_PAIR8 1

typedef struct vq_tiled {
    int32_t format;       /* VQ_FMT_*                                              */
    int32_t rows;         /* output features, >= 0                                 */
    int32_t cols;         /* input features, > 0, multiple of 32                   */
    int32_t order;        /* VQ_ROWS_*                                             */
    const void* data;     /* device, vq_tiled_bytes() bytes, 256-byte aligned      */
} vq_tiled;

/* Bytes of a tiled matrix (0 for invalid arguments). */
size_t vq_tiled_bytes(int32_t format, int32_t rows, int32_t cols);

/*
 * vq_tile -- write the plain matrix `src` into rows [row0, row0 + src->rows) of the tiled
 * matrix `dst` (same format and cols).  One call fills a whole matrix (row0 = 0); a
 * stacked matrix such as q|k|v is filled by one call per part (row0 = 0, H, H + KV;
 * every part but the last a multiple of 16 rows), a VQ_ROWS_PAIR8 one by a call for each
 * half (row0 = 0 and rows / 2).  Rows of dst outside the range are left as they are,
 * except the zero rows past dst->rows in the last tile, which every call writes.
 * Errors: VQ_ERR_ARG for bad descriptors, mismatched format or cols, a range outside
 * dst, a misaligned row0 or a NULL pointer; VQ_ERR_HIP.
 */
int vq_tile(const vq_matrix* src, const vq_tiled* dst, int32_t row0, void* stream);

/* Output element type of vq_verify_linear. */
#define VQ_DTYPE_F32 0
#define VQ_DTYPE_F16 1

#define VQ_MAX_K 16

/*
 * vq_verify_linear -- y = W x for K activation columns, each weight byte read once.
 *
 * The target model scores all K drafted tokens in one forward pass: each weight matrix
 * is fetched from memory a single time and multiplied into the K activation columns
 * together, not into one column per pass (page "100 tokens per second ...", section
 * "How speculative decoding gets past a per-token wall"); streaming the weights is what
 * bounds the pass (same page, section "The wall").
 *
 *   W       : host descriptor of a tiled device matrix (order VQ_ROWS_PLAIN)
 *   x_f16   : device fp16 [K][cols]  (row k = activation column k of the window)
 *   K       : 1..16
 *   y       : device [K][rows], fp32 or fp16 (y_dtype); y[k][r] = sum_j w[r][j] x[k][j]
 *   ws      : device workspace >= vq_workspace_bytes(VQ_OP_LINEAR, W, K), 256-byte
 *             aligned: partial sums of tiles that several workgroups share
 * Arithmetic: codes widen exactly to fp16 (q = n - 8, or the E2M1 value), products with
 * the fp16 activations are exact, sums are fp32; the block scale multiplies the fp32 sum
 * of its block and the min the fp32 sum of the block's activations, so no weight is
 * rounded.  Summation orders depend only on the shapes and the device's compute-unit
 * count, so results are reproducible bit for bit.
 * Errors: VQ_ERR_ARG for NULL pointers, K outside 1..16, cols not a positive multiple of
 * 32, rows < 0, misaligned pointers (x 16-byte, y its element size), an unknown
 * format/dtype/order; VQ_ERR_UNSUPPORTED for a shape the split cannot handle;
 * VQ_ERR_WORKSPACE; VQ_ERR_HIP.  rows == 0 is valid and enqueues nothing.
 */
int vq_verify_linear(const vq_tiled* W, const void* x_f16, int32_t K, void* y, int32_t y_dtype,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * vq_verify_linear_noalloc -- vq_verify_linear for callers that cannot allocate memory
 * (code under stream capture, tight serving loops, hosts that forbid allocation): no
 * workspace argument, and the call allocates nothing, on the device or the host.
 *
 * The partial sums, counters and work lists live in a fixed array of the library's own
 * device data (4.5 MiB + 16 KiB; each device the library runs on holds one copy until
 * the process ends).  Limits: the shape must need no column windows (K * cols small
 * enough for the activations to stay in LDS, e.g. cols <= 8704 at K = 8), at most 512 KiB
 * of split-tile partial sums and 4 MiB of work lists (a 151936 x 5120 matrix fits); other
 * shapes return VQ_ERR_UNSUPPORTED.  The first call with a shape on a device copies that
 * shape's work lists into the array (and waits for the stream), so it cannot be captured;
 * later calls with the same shape enqueue two kernels only.  Every call on a device uses
 * the same array: calls that overlap on one device (several streams or threads) race.
 * Results are bit-identical to vq_verify_linear's.
 * Errors: as vq_verify_linear, without VQ_ERR_WORKSPACE; VQ_ERR_UNSUPPORTED for the limits.
 */
int vq_verify_linear_noalloc(const vq_tiled* W, const void* x_f16, int32_t K, void* y,
                             int32_t y_dtype, void* stream);

/*
 * vq_verify_linear_mx -- y ~= W x for MXFP4 weights on CDNA4's scaled matrix instruction,
 * an APPROXIMATION offered beside vq_verify_linear (which is exact).
 *
 * The activations are first converted to the 8-bit MX format E4M3 with one E8M0 scale per
 * 32 values (OCP Microscaling Formats v1.0: shared exponent floor(log2 max|x|) - 8, each
 * value to nearest E4M3, ties to even, saturating at 448); the E2M1 weight codes and their
 * E8M0 scales go into v_mfma_scale_f32_16x16x128_f8f6f4 as they are, with fp32 sums.  This
 * is the K = 16 MXFP4 window's case for the CDNA4 MXFP4 instructions (Hacker News thread
 * 49596054 names MXFP4-native checkpoints); the result is W applied to the E4M3-rounded
 * activations, not to x.
 *
 *   W     : host descriptor of PLAIN device planes (vq_matrix), format VQ_FMT_MXFP4,
 *           cols a positive multiple of 128
 *   x_f16 : device fp16 [K][cols], K 1..16
 *   y     : device f32 [K][rows]
 *   ws    : device workspace >= vq_workspace_bytes(VQ_OP_LINEAR_MX, W, K), 256-byte aligned:
 *           the converted activations and per-split partial sums
 * Summation orders depend only on the shapes and the compute-unit count.
 * Errors: VQ_ERR_ARG for NULL pointers, K outside 1..16, a format other than MXFP4, cols not
 * a positive multiple of 128, misaligned pointers; VQ_ERR_WORKSPACE; VQ_ERR_HIP.  rows == 0
 * is valid and enqueues nothing.
 */
int vq_verify_linear_mx(const vq_matrix* W, const void* x_f16, int32_t K, float* y, void* ws,
                        size_t ws_bytes, void* stream);

/* ------------------------------------------------------ attention over the cache */
/* KV-cache formats: blocks of 32 along the head dimension, one fp16 scale d per block.
 *   VQ_KV_Q8_0 : int8 code c, value d * c;          codes [L][D] per kv head
 *   VQ_KV_Q4_0 : nibble n (low nibble first), value d * (n - 8); codes [L][D/2] per kv head
 * The pages name q8_0 (keys) and q4_0 (values) as the target's cache formats without
 * defining them; this is the block-32 layout the library implements. */
#define VQ_KV_Q8_0 0
#define VQ_KV_Q4_0 1

/* One layer's KV cache and the heads that read it (host struct, device planes). */
typedef struct vq_attention {
    int32_t k_format, v_format;   /* VQ_KV_*                                             */
    int32_t n_q_heads;            /* Hq, a multiple of n_kv_heads                        */
    int32_t n_kv_heads;           /* Hkv; query head h reads kv head h / (Hq / Hkv)      */
    int32_t head_dim;             /* D, must be 128                                      */
    int32_t length;               /* L: cached positions, the window's K included       */
    const void* k_codes;          /* uint8 [Hkv][L][D or D/2], 16-byte aligned           */
    const void* k_scales;         /* fp16 [Hkv][L][D/32], 16-byte aligned               */
    const void* v_codes;          /* as k_codes for v_format                             */
    const void* v_scales;         /* as k_scales                                         */
} vq_attention;

/*
 * vq_verify_attention -- the verify window's attention in one layer over a quantised KV
 * cache.  At long context the cache is read on every pass beside the weights ("Decode is
 * memory-bound ...", section "The ceiling"); the target's cache is kept at q8_0 keys and
 * q4_0 values ("100 tokens per second from a 27B model ...", section "The wall").  The K
 * window tokens are the cache's last K positions (already appended); window row i attends
 * causally to positions 0 .. L - K + i:
 *     s_j = q . k_j / sqrt(D),  p = softmax(s) over the visible j,  out = sum_j p_j v_j
 * with k_j, v_j the dequantised cache rows of the query head's kv head.
 *   q_f16 : device fp16 [K][Hq][D], 2-byte aligned
 *   K     : 1..16, K <= L, and (Hq / Hkv) * K <= 128
 *   out   : device f32 [K][Hq][D], 4-byte aligned
 *   ws    : device workspace >= vq_workspace_bytes(VQ_OP_ATTENTION, desc, K), 256-byte
 *           aligned: per-span partial results
 * Dequantisation is exact in fp32; products, the softmax and the sums are fp32 (the
 * cache is cut into spans of positions, each reduced in position order, then the spans
 * are combined in order); the summation order depends only on the shapes and the
 * compute-unit count.
 * Errors: VQ_ERR_ARG for NULL pointers, unknown formats, head_dim != 128, heads or K out of
 * range, misaligned pointers; VQ_ERR_WORKSPACE; VQ_ERR_HIP.
 */
int vq_verify_attention(const vq_attention* desc, const void* q_f16, int32_t K, float* out, void* ws,
                        size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ adaptive draft depth */
/* Running acceptance statistics (a HOST struct owned by the caller; zero it to start). */
typedef struct vq_depth_stats {
    double accepted;   /* decayed sum of accepted drafts                                 */
    double rejected;   /* decayed count of windows that ended on a rejected draft        */
} vq_depth_stats;

/*
 * vq_depth_observe -- fold W windows' outcomes, in window order, into the statistics:
 *     accepted = decay * accepted + n_accepted[w]
 *     rejected = decay * rejected + (n_accepted[w] < n_drafted[w] ? 1 : 0)
 * A window that ends on a rejected draft is n successes and one failure; a window whose
 * drafts were all accepted is n successes and no failure (the next draft was never tried),
 * so accepted / (accepted + rejected) is the maximum-likelihood per-draft acceptance under
 * independent acceptance (page "Decode is memory-bound ...", section "Speculative
 * decoding"), older windows weighted down by `decay` per window.
 *   n_accepted : HOST int32 [W], e.g. vq_verify_accept's n_accepted copied back (windows
 *                with status != 0 left out by the caller)
 *   n_drafted  : HOST int32 [W], the drafts of each window (K - 1)
 *   decay      : (0, 1]
 * Host arithmetic only (no GPU call).  Errors: VQ_ERR_ARG for NULL pointers (unless W == 0),
 * W < 0, decay outside (0, 1], n_drafted < 0 or n_accepted outside [0, n_drafted]; on an
 * error the statistics are left unchanged.
 */
int vq_depth_observe(vq_depth_stats* st, const int32_t* n_accepted, const int32_t* n_drafted,
                     int32_t W, double decay);

/*
 * vq_depth_choose -- the draft depth k (drafts per window, K = k + 1 columns) for the next
 * windows: the k in 0 .. k_max that maximises the expected tokens per unit time
 *     rate(k) = tau(a, k) / (t_pass[k] + k * t_draft),  tau(a, k) = (1 - a^(k+1)) / (1 - a)
 * (tau = k + 1 at a = 1), with a the statistics' estimate shrunk toward a prior,
 *     a = (accepted + prior_weight * alpha_prior) / (accepted + rejected + prior_weight)
 * (page "Decode is memory-bound ...", sections "Speculative decoding": tau and the speedup
 * with a drafter cost; "Two things the math says to do": adapt the depth to the measured
 * acceptance, which falls on hard text).  Ties go to the smaller k.
 *   t_pass  : HOST double [k_max + 1], the measured verify-pass time with k drafts
 *   t_draft : the time of one draft step (same unit), >= 0
 *   k_out   : HOST out, the chosen depth; alpha_out, rate_out: HOST out or NULL
 * Host arithmetic only.  Errors: VQ_ERR_ARG for NULL st / t_pass / k_out, k_max outside
 * 0 .. VQ_MAX_K - 1, a time that is not finite and > 0 (t_draft: >= 0), alpha_prior outside
 * [0, 1], prior_weight < 0, or no evidence at all (accepted + rejected + prior_weight == 0).
 */
int vq_depth_choose(const vq_depth_stats* st, double alpha_prior, double prior_weight,
                    const double* t_pass, int32_t k_max, double t_draft, int32_t* k_out,
                    double* alpha_out, double* rate_out);

/* ------------------------------------------------------------- n-gram map drafter */
/* An incremental map over one token sequence (an opaque HOST object). */
typedef struct vq_ngram vq_ngram;

/*
 * vq_ngram_create -- an empty map with keys of key_len tokens.  Prompt lookup generalised
 * (page "100 tokens per second ...", section "Lever 3: an n-gram overlay for repetition"):
 * the map takes every key_len-token key of the sequence so far to the position that
 * followed its latest occurrence; the most recent key_len tokens look up their
 * continuation, which is proposed as drafts.  The page found 6 better than 12 (12 matching
 * tokens almost never occur).  Host memory only; grows with the sequence (4 bytes per token
 * plus a table of at most 16 bytes per distinct key).
 * Errors: VQ_ERR_ARG for NULL out or key_len outside 1..64; VQ_ERR_HOST.
 */
int vq_ngram_create(int32_t key_len, vq_ngram** out);

/* vq_ngram_destroy -- free the map (NULL is ignored). */
void vq_ngram_destroy(vq_ngram* m);

/*
 * vq_ngram_append -- append n tokens (the prompt, or each window's emitted tokens) to the
 * sequence.  The key that ends just before each new token maps to that token's position
 * (replacing its earlier occurrence), so a key enters the map only once its continuation
 * exists.
 *   tokens : HOST int32 [n], token ids >= 0 (the -1 padding of vq_verify_accept's tokens
 *            must not be passed)
 * Errors: VQ_ERR_ARG for NULL m, n < 0, NULL tokens with n > 0, a negative token id or a
 * sequence past 2^31 - 1 tokens (nothing is appended then); VQ_ERR_HOST.
 */
int vq_ngram_append(vq_ngram* m, const int32_t* tokens, int32_t n);

/*
 * vq_ngram_propose -- the drafts for the next window: if the sequence's last key_len tokens
 * occurred before with a continuation, the tokens that followed their latest such
 * occurrence, at most max_drafts of them and none past the end of the sequence; otherwise
 * none.
 *   drafts   : HOST int32 [max_drafts] out;  n_drafts : HOST out, 0 .. max_drafts
 * Errors: VQ_ERR_ARG for NULL m / n_drafts, max_drafts < 0, NULL drafts with max_drafts > 0.
 * Calls on one map must not overlap; separate maps are independent.
 */
int vq_ngram_propose(const vq_ngram* m, int32_t max_drafts, int32_t* drafts, int32_t* n_drafts);

/* ---------------------------------------------------------------- acceptance */
#define VQ_MODE_GREEDY 0      /* accept x_i while it equals the target argmax            */
#define VQ_MODE_SAMPLE 1      /* accept x_i with prob. min(1, p(x_i)/q(x_i)), else resample */

/* Where the drafted tokens come from.  GIVEN reads draft_tokens; the others are
 * synthetic drafters that write the tokens they draw into draft_tokens. */
#define VQ_DRAFT_GIVEN 0      /* draft_tokens is an input                                */
#define VQ_DRAFT_Q_ARGMAX 1   /* x_i = argmax of drafter row i                           */
#define VQ_DRAFT_Q_SAMPLE 2   /* x_i ~ q_i (warped drafter row i) with uniform u_D       */
#define VQ_DRAFT_AGREE 3      /* x_i = target argmax if u_D < alpha, else another token
                                 uniform over the other V-1 via u_X                      */

typedef struct vq_accept_desc {
    int32_t mode;              /* VQ_MODE_*                                              */
    int32_t draft_mode;        /* VQ_DRAFT_*                                             */
    int32_t W;                 /* windows, >= 0                                          */
    int32_t K;                 /* positions per window (K-1 drafts + 1 bonus), 1..16     */
    int32_t V;                 /* vocabulary size, 1 .. 2^19 (fixed-point mass sums)     */
    int32_t top_k;             /* top-k cut, >= 0; 0 (or >= V) disables it               */
    const float* target_logits;/* device f32 [W][K][V]: row i scores position i+1        */
    const float* draft_logits; /* device f32 [W][K-1][V], or NULL when not needed        */
    int32_t* draft_tokens;     /* device i32 [W][K-1]: input (GIVEN) or output           */
    float temperature;         /* > 0; 0 with VQ_MODE_SAMPLE is rejected                 */
    float top_p;               /* (0, 1]; 1 disables the top-p cut                        */
    float min_p;               /* [0, 1); 0 disables the min-p cut                        */
    float alpha;               /* [0, 1]: agreement rate of VQ_DRAFT_AGREE                */
    uint64_t seed;             /* Philox key                                              */
    uint64_t window_base;      /* counter offset: window w uses counter window_base + w   */
    int32_t* n_accepted;       /* device i32 [W]: accepted drafts n (tokens emitted n+1)  */
    int32_t* tokens;           /* device i32 [W][K]: emitted tokens, -1 padded            */
    int32_t* status;           /* device i32 [W]: 0 ok, 1 non-finite logit, 2 draft token
                                  outside [0, V); on status != 0 nothing is emitted       */
} vq_accept_desc;

/*
 * vq_verify_accept -- the lossless acceptance rule over W independent windows.
 *
 * GREEDY: draft x_i is kept as long as it matches the target's most likely token at its
 * position, and the first mismatch ends the run (page "100 tokens per second ...",
 * section "How speculative decoding gets past a per-token wall"); argmax ties go
 * to the lowest index; the target's own token at the first disagreement (or at the
 * bonus position K when every draft is accepted) caps the window (page "Decode is
 * memory-bound ...", section "Speculative decoding").
 * SAMPLE: p_i and q_i are the target and drafter rows after the sampler warp
 * (temperature, softmax, top-p and min-p cuts over the order probability-descending /
 * index-ascending, renormalised; page "Decode is memory-bound ...", section "Two things
 * the math says to do"; the optional top-k cut keeps the first top_k entries of the same
 * order; page "100 tokens per second ...", section "What failed", names top-k sampling;
 * the kept set is the shortest of the three prefixes, each computed on the full
 * distribution).  For i = 1..K-1: accept x_i iff u_A < p_i(x_i)/q_i(x_i); on the
 * first rejection draw from the normalised positive part of p_i - q_i (p_i itself if
 * that part is zero) and stop; if all are accepted draw the bonus from p_K.  Draws are
 * inverse-CDF over vocabulary order.
 * Uniforms: Philox4x64-10 (Salmon et al., SC'11), key (seed, 0), counter
 * (window_base + w, position, 0, 0); u = (r >> 40) * 2^-24 of output lanes
 * 0 (u_A), 1 (u_R: residual / bonus), 2 (u_D: drafting), 3 (u_X: "other token").
 * Errors: VQ_ERR_ARG for NULL pointers, sizes or sampler settings out of range;
 * VQ_ERR_WORKSPACE; VQ_ERR_HIP.  Data errors never abort: they go to status[w].
 */
int vq_verify_accept(const vq_accept_desc* d, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------- decode pass */
typedef struct vq_layer {
    vq_tiled qkv;              /* [H + 2 KV][H]: q, k, v stacked (VQ_ROWS_PLAIN)        */
    vq_tiled o;                /* [H][H]                                                */
    vq_tiled gu;               /* [2 FF][H]: gate, up (VQ_ROWS_PAIR8)                    */
    vq_tiled down;             /* [H][FF]                                               */
} vq_layer;

typedef struct vq_model {
    int32_t n_layers;          /* >= 1                                                  */
    int32_t reserved;          /* must be 0                                             */
    const vq_layer* layers;    /* HOST array [n_layers] of device-matrix descriptors    */
    vq_tiled lm_head;          /* [vocab][hidden]                                       */
} vq_model;

/*
 * vq_decode_pass -- one verify pass of the whole weight stack for K columns.
 *
 * The window goes through layer 1, then layer 2, and so on, reading each layer's weights
 * once (Hacker News thread 49596054); the output is a [K][vocab] logits tensor.  Per
 * layer four dependent stages run: S1 q|k|v = W_qkv x_attn, S2 o = W_o x_o,
 * S3 gate|up = W_gu x_mlp, S4 down = W_down x_down, then logits = W_lm x_final.
 * The stack has no attention, norm weights or residuals.  Stage glue: a stage's input is
 * the previous stage's fp32 output v rounded to fp16 (x_o = q rows of q|k|v,
 * x_mlp = o, x_down = silu(gate) * up, the next x_attn and x_final = down), and the
 * stage multiplies its fp32 sums by rho = 1 / sqrt(mean(v^2)) of that v per column, so
 * that every output is what a unit-RMS input would give.  The first x_attn is x0 and
 * stage 0 is not scaled.
 *
 *   M      : host model descriptor; H = qkv.cols, FF = down.cols, every layer the same
 *            shapes (qkv: [H + 2 KV][H], o: [H][H], gu: [2 FF][H] in VQ_ROWS_PAIR8 order,
 *            down: [H][FF], lm_head: [V][H]); all matrices of one format; H, KV, FF
 *            multiples of 64
 *   x0_f16 : device fp16 [K][H]
 *   logits : device f32 [K][V]
 *   ws     : device workspace >= vq_workspace_bytes(VQ_OP_DECODE, M, K); after the call
 *            it holds every stage's fp16 input and fp32 output (vq_decode_stage_ptr)
 * The pass runs as one persistent launch per 16 layers (the last one also runs the
 * lm_head): one workgroup per compute unit, every workgroup resident (a cooperative
 * launch; the runtime refuses it otherwise and the call returns VQ_ERR_HIP).  Inside a
 * launch a stage waits for the previous one on device-scope completion counters; a wait
 * gives up after about a second and raises the error word (vq_decode_error_word), after
 * which the logits are not meaningful -- callers that cannot rule out such a stall read
 * that word after the pass before trusting the logits.
 * Errors: as vq_verify_linear, plus VQ_ERR_ARG for inconsistent layer shapes,
 * VQ_ERR_UNSUPPORTED for sizes that are not multiples of 64, VQ_ERR_WORKSPACE.
 */
int vq_decode_pass(const vq_model* M, const void* x0_f16, int32_t K, float* logits,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * vq_decode_error_word -- where a decode pass in `ws` keeps its wait-timeout word.
 *   *word : DEVICE address of an int32 that is 0 after a pass whose waits all completed
 *           and 1 if one timed out (read it after the pass has finished)
 * Pure host arithmetic: no GPU call.  Errors: VQ_ERR_ARG for a bad model, K or NULL.
 */
int vq_decode_error_word(const vq_model* M, int32_t K, void* ws, int32_t** word);

/* Launch modes of vq_decode_pass_timed. */
#define VQ_LAUNCH_AUTO 0        /* what vq_decode_pass does: persistent                  */
#define VQ_LAUNCH_STAGED 4      /* one ordinary launch per stage (257 for 64 layers); the
                                   same per-tile arithmetic, so the same bits            */
#define VQ_LAUNCH_PERSISTENT 8  /* one cooperative launch per 16 layers                  */

/*
 * vq_decode_pass_timed -- measurement hook: the work of vq_decode_pass with a chosen
 * launch mode, plus hipEventRecord(events[2i]) before and hipEventRecord(events[2i+1])
 * after the i-th launch (for i < n_events / 2), on `stream`.
 *   launch     : VQ_LAUNCH_*
 *   events     : HOST array of n_events caller-created hipEvent_t handles
 *   n_launches : HOST out, the number of launches of the pass (may be NULL)
 * Errors: as vq_decode_pass, plus VQ_ERR_ARG for an unknown launch mode or a short or
 * NULL-holding events array.
 */
int vq_decode_pass_timed(const vq_model* M, const void* x0_f16, int32_t K, float* logits,
                         int32_t launch, void* ws, size_t ws_bytes, void* stream,
                         void* const* events, int32_t n_events, int32_t* n_launches);

/*
 * vq_decode_stage_ptr -- where a decode pass left stage s's tensors inside ws.
 * Stage s = 4*layer + j (j: 0 qkv, 1 o, 2 gate|up, 3 down), s = 4*n_layers is the
 * lm_head.  *in_f16 receives the device address of the fp16 input [K][cols] (natural
 * column order) and *out_f32 of the fp32 output [K][rows] (rows of the fused stage:
 * qkv = H + 2 KV, gate|up = 2 FF with gate first; NULL for the lm_head, whose output is
 * the logits).  Host-only arithmetic; no device access.
 */
int vq_decode_stage_ptr(const vq_model* M, int32_t K, void* ws, int32_t stage,
                        void** in_f16, void** out_f32);

/* ---------------------------------------------------------------- queries */
#define VQ_OP_LINEAR 0         /* desc = const vq_tiled*        */
#define VQ_OP_ACCEPT 1         /* desc = const vq_accept_desc*  */
#define VQ_OP_DECODE 2         /* desc = const vq_model*        */
#define VQ_OP_LINEAR_MX 3      /* desc = const vq_matrix* (plain MXFP4 planes) */
#define VQ_OP_ATTENTION 4      /* desc = const vq_attention*    */

/* Workspace bytes needed by an op for the given descriptor and K (0 on bad input). */
size_t vq_workspace_bytes(int32_t op, const void* desc, int32_t K);

/* Static text for a status code. */
const char* vq_status_string(int32_t status);

/* Thread-local text of the last error raised on this thread ("" if none). */
const char* vq_last_error(void);

/* VQ_ABI_VERSION of the built library. */
int32_t vq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* VQ_H */
