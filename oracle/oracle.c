/*
 * CPU oracle for the speculative-decoding verify pass.  TEST INFRASTRUCTURE ONLY:
 * the tests, the package's smoke check and the benchmark's CPU-baseline leg call it;
 * the library never does.  It shares no code, header or table with the HIP path.
 *
 * Plain, slow, obviously correct: every floating-point result is computed in double
 * precision (IEEE binary64), in the order the definitions state, with no fast-math.
 *
 * Sources, by page title and section:
 *  - "100 tokens per second from a 27B model on a 24 GB AMD card", sections "The wall"
 *    (decode streams every weight once and multiplies it against the activation
 *    vector) and "How speculative decoding gets past a per-token wall" (K drafted
 *    tokens are scored in one pass over the weights; greedy keeps a draft while it
 *    equals the target argmax; sampling accepts x with probability
 *    min(1, p_target(x)/p_draft(x)) and on rejection resamples from the normalised
 *    positive part of p_target - p_draft; the target's own token caps the window).
 *  - "Decode is memory-bound: the ~59 tok/s ceiling on an RTX 4090 ...", sections
 *    "Speculative decoding" (at the first disagreement the target's own token is
 *    taken, so no pass ends with zero new tokens) and "Two things the math says to do"
 *    (the production sampler: temperature 0.6, top-p 0.95, min-p 0.05).
 *  - Hacker News thread 49596054: the target runs the whole window through each layer
 *    once, and outputs a [n_tokens, vocab] logits tensor; the "D E F" worked example.
 *  - Weight formats: 4-bit codes in blocks of 32 with an fp16 scale (and optional fp16
 *    min); MXFP4 = E2M1 codes with an E8M0 scale per 32 (OCP Microscaling Formats v1.0).
 *    The K-quant 4-bit format the pages name (Q4_K_M, UD-Q4_K_XL) in its public GGML
 *    definition: super-blocks of 256 weights, each of eight 32-weight sub-blocks with a
 *    6-bit scale s and a 6-bit min m, under the super-block's fp16 d and dmin; an
 *    unsigned code n in 0..15 gives w = d*s*n - dmin*m.
 *  - Philox4x64-10: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 *    1, 2, 3", SC'11 (round function, multipliers, Weyl key schedule).
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *  - code n -> q = n - 8; even column = low nibble; w = d*q + m (m = 0 without mins).
 *  - Q4_K planes: one byte per 6-bit s and m (uint8 [rows][cols/32] each), d and dmin as
 *    an fp16 pair per super-block (uint16 [rows][cols/256][2]); nibbles as above, but
 *    the code is taken unsigned.
 *  - warp order: temperature, softmax, then the top-p and min-p cuts over the order
 *    (probability descending, index ascending); top-p keeps the shortest prefix whose
 *    mass reaches top_p; min-p keeps pi >= min_p * pi_max; keep the shorter prefix;
 *    renormalise over the kept set.  top_p >= 1 or min_p == 0 disables that cut.
 *    A top-k cut (the first top_k tokens of the same order; 0 or >= V disables it) is a
 *    third prefix: the kept set is the shortest of the three.
 *  - greedy argmax ties go to the lowest index; greedy ignores T, top-p and min-p.
 *  - the ratio test accepts iff u_A < p/q with IEEE division (q = 0 < p gives +inf and
 *    accepts; p = q = 0 gives NaN and rejects).
 *  - a categorical draw over weights w picks the smallest index j (in vocabulary order)
 *    whose running sum exceeds u * sum(w); when rounding leaves no such j, the last j
 *    with w_j > 0.  An all-zero residual falls back to p itself.
 *  - the decode pass's stage glue (the pages give the layer order, not the layer
 *    internals): a stage's input is the previous stage's output rounded to fp16 (the q
 *    rows of q|k|v for the o stage, silu(gate) * up for the down stage) and the stage
 *    multiplies its dot products by rho = 1 / sqrt(mean(v^2)) of that previous output v.
 *  - uniforms: u = (r >> 40) * 2^-24 from the 64-bit Philox outputs; counter
 *    (window_base + w, position, 0, 0), key (seed, 0); lanes 0..3 are u_A (ratio
 *    test), u_R (residual / bonus draw), u_D (harness draft draw), u_X (harness
 *    "other token" pick).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_FMT_Q4 0
#define OR_FMT_Q4_MIN 1
#define OR_FMT_MXFP4 2
#define OR_FMT_Q4_K 3

/* ---------------------------------------------------------------- fp16 -> double */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double or_half(uint16_t h) {
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1.0 + (double)f / 1024.0, e - 15);
    return s ? -v : v;
}

void or_half_array(const uint16_t* h, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_half(h[i]);
}

/* ------------------------------------------------------------- weight decoding */

/* E2M1 (OCP MX v1.0): bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * exponent 0 is subnormal: 0.5 * mantissa. */
double or_e2m1(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E8M0 (OCP MX v1.0): 2^(E - 127); E = 255 is NaN. */
double or_e8m0(uint8_t e) {
    return e == 255 ? NAN : ldexp(1.0, (int)e - 127);
}

/* Weight (r, j) of a row-major block-quantised matrix with cols columns.  supers is
 * used by Q4_K only (NULL otherwise). */
double or_weight(int fmt, const uint8_t* qs, const void* scales, const void* mins,
                 const uint16_t* supers, int64_t cols, int64_t r, int64_t j) {
    int64_t nb = cols / 32, b = j / 32;
    uint8_t byte = qs[r * (cols / 2) + j / 2];
    int n = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
    if (fmt == OR_FMT_MXFP4) {
        uint8_t e = ((const uint8_t*)scales)[r * nb + b];
        return or_e2m1(n) * or_e8m0(e);
    }
    if (fmt == OR_FMT_Q4_K) {
        const uint16_t* sup = supers + (r * (cols / 256) + j / 256) * 2;
        double d = or_half(sup[0]), dmin = or_half(sup[1]);
        double s = (double)((const uint8_t*)scales)[r * nb + b];
        double m = (double)((const uint8_t*)mins)[r * nb + b];
        return d * s * (double)n - dmin * m;
    }
    double d = or_half(((const uint16_t*)scales)[r * nb + b]);
    double m = (fmt == OR_FMT_Q4_MIN) ? or_half(((const uint16_t*)mins)[r * nb + b]) : 0.0;
    return d * (double)(n - 8) + m;
}

void or_dequant(int fmt, const uint8_t* qs, const void* scales, const void* mins,
                const uint16_t* supers, int64_t rows, int64_t cols, double* out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < cols; ++j)
            out[r * cols + j] = or_weight(fmt, qs, scales, mins, supers, cols, r, j);
}

/* --------------------------------------------------------------------- linear */

/* y[k][r] = sum_j w[r][j] * x[k][j]  and  a[k][r] = sum_j |w[r][j] * x[k][j]|,
 * a scalar loop over j in order, in double.  x is fp16 [K][cols]. */
typedef struct {
    int fmt;
    const uint8_t* qs;
    const void* scales;
    const void* mins;
    const uint16_t* supers;
    int64_t rows, cols;
    const double* x;     /* decoded activations [K][cols] */
    int K;
    double* y;
    double* a;
    int64_t r0, r1;
} lin_job;

static void* lin_worker(void* p) {
    lin_job* J = (lin_job*)p;
    for (int64_t r = J->r0; r < J->r1; ++r) {
        for (int k = 0; k < J->K; ++k) {
            double acc = 0.0, aacc = 0.0;
            const double* xk = J->x + (int64_t)k * J->cols;
            for (int64_t j = 0; j < J->cols; ++j) {
                double t = or_weight(J->fmt, J->qs, J->scales, J->mins, J->supers, J->cols, r, j) * xk[j];
                acc += t;
                aacc += fabs(t);
            }
            J->y[(int64_t)k * J->rows + r] = acc;
            J->a[(int64_t)k * J->rows + r] = aacc;
        }
    }
    return NULL;
}

int or_linear(int fmt, const uint8_t* qs, const void* scales, const void* mins,
              const uint16_t* supers, int64_t rows, int64_t cols, const uint16_t* x_f16, int K,
              double* y, double* a, int nthreads) {
    if (cols % 32 || K < 1 || rows < 0 || (fmt == OR_FMT_Q4_K && cols % 256)) return -1;
    double* x = (double*)malloc(sizeof(double) * (size_t)K * (size_t)cols);
    if (!x) return -2;
    or_half_array(x_f16, x, (int64_t)K * cols);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > rows) nthreads = rows > 0 ? (int)rows : 1;
    pthread_t th[256];
    lin_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        lin_job J = {fmt, qs, scales, mins, supers, rows, cols, x, K, y, a,
                     rows * t / nthreads, rows * (t + 1) / nthreads};
        jobs[t] = J;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, lin_worker, &jobs[t]);
    lin_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(x);
    return 0;
}

/* Same, with the activations given in double ([K][cols]), for inputs that are not fp16
 * values (the MX-quantised activations below). */
int or_linear_x64(int fmt, const uint8_t* qs, const void* scales, const void* mins,
                  const uint16_t* supers, int64_t rows, int64_t cols, const double* x, int K,
                  double* y, double* a, int nthreads) {
    if (cols % 32 || K < 1 || rows < 0 || (fmt == OR_FMT_Q4_K && cols % 256)) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > rows) nthreads = rows > 0 ? (int)rows : 1;
    pthread_t th[256];
    lin_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        lin_job J = {fmt, qs, scales, mins, supers, rows, cols, x, K, y, a,
                     rows * t / nthreads, rows * (t + 1) / nthreads};
        jobs[t] = J;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, lin_worker, &jobs[t]);
    lin_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    return 0;
}

/* ------------------------------------------------------- MX-quantised activations */

/* The CDNA4 scaled matrix instructions multiply MXFP4 weights with activations in an
 * 8-bit MX format; this is the activation side of that (approximate) path, following
 * the OCP Microscaling Formats v1.0 specification.
 *
 * E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is subnormal
 * (m/8 * 2^-6); S.1111.111 is NaN; there are no infinities; the largest finite value is
 * 448. */
double or_e4m3(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + (double)m, e - 10);
    return s ? -mag : mag;
}

/* The E4M3 code of v: the finite value nearest to |v|, ties to the code with an even
 * mantissa, saturating at 448 (a search over the 127 non-negative finite codes); the
 * sign bit is v's. */
static int e4m3_code(double v) {
    double a = fabs(v);
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double d = fabs(or_e4m3(c) - a);
        if (d < bd || (d == bd && (c & 1) == 0)) {
            bd = d;
            best = c;
        }
    }
    return signbit(v) ? (best | 0x80) : best;
}

int or_e4m3_code(double v) { return e4m3_code(v); }

/* One block of 32 activations -> a shared E8M0 scale and 32 E4M3 codes, as the OCP MX
 * specification converts a block: the shared exponent is floor(log2(max |x|)) minus the
 * largest exponent of the element type (8 for E4M3), and each element is x / 2^shared
 * converted to E4M3 (to nearest, ties to even, saturating).  An all-zero block gets
 * shared exponent -127 (scale byte 0).  x fp16 [K][cols]; codes [K][cols], scales
 * [K][cols / 32]. */
int or_mx_quant(const uint16_t* x, int64_t K, int64_t cols, uint8_t* codes, uint8_t* scales) {
    if (cols % 32 || K < 1) return -1;
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t b = 0; b < cols / 32; ++b) {
            const uint16_t* xb = x + k * cols + 32 * b;
            double amax = 0.0;
            for (int j = 0; j < 32; ++j) {
                double v = or_half(xb[j]);
                if (!isfinite(v)) return -2;
                if (fabs(v) > amax) amax = fabs(v);
            }
            int E = -127;
            if (amax > 0.0) {
                int ex;
                frexp(amax, &ex);           /* amax = f * 2^ex, 0.5 <= f < 1 */
                E = (ex - 1) - 8;
                if (E < -127) E = -127;
                if (E > 127) E = 127;
            }
            scales[k * (cols / 32) + b] = (uint8_t)(E + 127);
            for (int j = 0; j < 32; ++j)
                codes[k * cols + 32 * b + j] = (uint8_t)e4m3_code(ldexp(or_half(xb[j]), -E));
        }
    }
    return 0;
}

/* ----------------------------------------------------- attention over a KV cache */

/* The window's attention in one layer, over a block-quantised KV cache ("Decode is
 * memory-bound ...", section "The ceiling": at long context the cache joins the weights
 * on every pass; "100 tokens per second ...", section "The wall": the measured
 * configuration keeps the target's cache at q8_0 / q4_0).
 *
 * Cache formats, blocks of 32 along the head dimension, one fp16 scale d per block:
 *   q8_0: an int8 code c per value, value = d * c
 *   q4_0: a 4-bit code n per value (low nibble = even index), value = d * (n - 8)
 * Layout: codes [Hkv][L][D] (q8_0: bytes; q4_0: D/2 bytes per row), scales [Hkv][L][D/32].
 *
 * Queries q fp16 [K][Hq][D]; query head h reads kv head h / (Hq / Hkv).  The window's own
 * K positions are the last K of the cache; query i sees positions 0 .. L - K + i.
 *   s_j = (q . k_j) / sqrt(D),  p_j = exp(s_j - max s) / sum exp(s - max s),  o = sum p_j v_j
 * in double, with a[k][h][d] = sum_j p_j |v_j[d]| as the tolerance base. */
static double kv_value(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t D, int64_t row, int64_t d) {
    double sc = or_half(scales[row * (D / 32) + d / 32]);
    if (fmt == 0) return sc * (double)(int8_t)codes[row * D + d];
    uint8_t b = codes[row * (D / 2) + d / 2];
    int n = (d & 1) ? (b >> 4) : (b & 15);
    return sc * (double)(n - 8);
}

int or_attention(int kfmt, const uint8_t* kc, const uint16_t* ks, int vfmt, const uint8_t* vc, const uint16_t* vs,
                 int64_t Hkv, int64_t L, int64_t D, const uint16_t* q, int64_t K, int64_t Hq,
                 double* out, double* a) {
    if (D % 32 || Hkv < 1 || Hq % Hkv || K < 1 || K > L) return -1;
    double* sc = (double*)malloc(sizeof(double) * (size_t)L);
    if (!sc) return -2;
    const double inv = 1.0 / sqrt((double)D);
    for (int64_t i = 0; i < K; ++i) {
        const int64_t n = L - K + i + 1;               /* visible positions */
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t g = h / (Hq / Hkv);
            const uint16_t* qh = q + (i * Hq + h) * D;
            double mx = -INFINITY;
            for (int64_t j = 0; j < n; ++j) {
                double t = 0.0;
                for (int64_t d = 0; d < D; ++d) t += or_half(qh[d]) * kv_value(kfmt, kc, ks, D, g * L + j, d);
                sc[j] = t * inv;
                if (sc[j] > mx) mx = sc[j];
            }
            double Z = 0.0;
            for (int64_t j = 0; j < n; ++j) Z += exp(sc[j] - mx);
            for (int64_t d = 0; d < D; ++d) {
                double o = 0.0, ab = 0.0;
                for (int64_t j = 0; j < n; ++j) {
                    double pj = exp(sc[j] - mx) / Z;
                    double v = kv_value(vfmt, vc, vs, D, g * L + j, d);
                    o += pj * v;
                    ab += pj * fabs(v);
                }
                out[(i * Hq + h) * D + d] = o;
                a[(i * Hq + h) * D + d] = ab;
            }
        }
    }
    free(sc);
    return 0;
}

/* ------------------------------------------------------------------ stage glue */

/* rho: out[k][j] = v[k][j] / sqrt(mean_j v[k][j]^2), per activation column k. */
void or_rho(const double* v, int K, int64_t n, double* out) {
    for (int k = 0; k < K; ++k) {
        const double* vk = v + (int64_t)k * n;
        double ss = 0.0;
        for (int64_t j = 0; j < n; ++j) ss += vk[j] * vk[j];
        double rms = sqrt(ss / (double)n);
        for (int64_t j = 0; j < n; ++j) out[(int64_t)k * n + j] = vk[j] / rms;
    }
}

/* The scale a decode-pass stage applies to its dot products: rho_k = 1 / sqrt(mean_j
 * v[k][j]^2) of the previous stage's output v, per activation column k (the stage's
 * input is v itself rounded to fp16, so its outputs are what the unit-RMS input v * rho
 * would give).  n > 0. */
void or_rms_scale(const double* v, int K, int64_t n, double* rho) {
    for (int k = 0; k < K; ++k) {
        const double* vk = v + (int64_t)k * n;
        double ss = 0.0;
        for (int64_t j = 0; j < n; ++j) ss += vk[j] * vk[j];
        rho[k] = 1.0 / sqrt(ss / (double)n);
    }
}

/* silu(g) * u = g / (1 + exp(-g)) * u, elementwise. */
void or_silu_mul(const float* g, const float* u, int64_t n, double* out) {
    for (int64_t j = 0; j < n; ++j) {
        double gj = g[j];
        out[j] = gj / (1.0 + exp(-gj)) * (double)u[j];
    }
}

/* ---------------------------------------------------------------- Philox4x64-10 */

static void mulhilo64(uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo) {
    unsigned __int128 p = (unsigned __int128)a * (unsigned __int128)b;
    *hi = (uint64_t)(p >> 64);
    *lo = (uint64_t)p;
}

void or_philox4x64(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
    const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
    uint64_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t hi0, lo0, hi1, lo1;
        mulhilo64(M0, c[0], &hi0, &lo0);
        mulhilo64(M1, c[2], &hi1, &lo1);
        uint64_t n0 = hi1 ^ c[1] ^ k0, n1 = lo1, n2 = hi0 ^ c[3] ^ k1, n3 = lo0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
        k0 += W0;
        k1 += W1;
    }
    memcpy(out, c, sizeof(c));
}

/* The four uniforms of (window, position): u = top 24 bits * 2^-24. */
void or_uniforms(uint64_t seed, uint64_t window, uint64_t position, double u[4]) {
    uint64_t ctr[4] = {window, position, 0, 0}, key[2] = {seed, 0}, r[4];
    or_philox4x64(ctr, key, r);
    for (int i = 0; i < 4; ++i) u[i] = ldexp((double)(r[i] >> 40), -24);
}

/* ------------------------------------------------------------------------ warp */

typedef struct {
    int64_t n_keep;   /* tokens in the kept set */
    int64_t m_p;      /* top-p prefix length (V when disabled) */
    int64_t m_m;      /* min-p prefix length (V when disabled) */
    int64_t m_k;      /* top-k prefix length (V when disabled) */
    int near_top_p;   /* cumulative mass within 1e-6 of top_p at m_p or m_p - 1 */
    int near_min_p;   /* a token at the min-p cut within 1e-6*pi_max of min_p*pi_max */
    int nonfinite;    /* a logit was NaN or infinite */
    int64_t argmax;   /* first maximum of the raw logits */
} or_warp_info;

typedef struct { double pi; int64_t idx; } pi_idx;

static int cmp_pi_desc_idx_asc(const void* pa, const void* pb) {
    const pi_idx* a = (const pi_idx*)pa;
    const pi_idx* b = (const pi_idx*)pb;
    if (a->pi > b->pi) return -1;
    if (a->pi < b->pi) return 1;
    return (a->idx < b->idx) ? -1 : (a->idx > b->idx);
}

int64_t or_argmax(const float* l, int64_t V) {
    int64_t best = 0;
    for (int64_t j = 1; j < V; ++j)
        if (l[j] > l[best]) best = j;
    return best;
}

/* p[V] = warp(l; T, top_p, min_p, top_k).  T == 0 gives the one-hot argmax. */
int or_warp(const float* l, int64_t V, double T, double top_p, double min_p, int64_t top_k,
            double* p, or_warp_info* info) {
    memset(info, 0, sizeof(*info));
    for (int64_t j = 0; j < V; ++j)
        if (!isfinite(l[j])) info->nonfinite = 1;
    info->argmax = or_argmax(l, V);
    if (info->nonfinite) {
        for (int64_t j = 0; j < V; ++j) p[j] = 0.0;
        return 1;
    }
    if (T == 0.0) {
        for (int64_t j = 0; j < V; ++j) p[j] = 0.0;
        p[info->argmax] = 1.0;
        info->n_keep = 1;
        info->m_p = info->m_m = info->m_k = V;
        return 0;
    }
    /* (1) tempered softmax */
    double M = -INFINITY;
    for (int64_t j = 0; j < V; ++j) {
        double z = (double)l[j] / T;
        if (z > M) M = z;
    }
    double Z = 0.0;
    for (int64_t j = 0; j < V; ++j) Z += exp((double)l[j] / T - M);
    pi_idx* ord = (pi_idx*)malloc(sizeof(pi_idx) * (size_t)V);
    if (!ord) return -2;
    for (int64_t j = 0; j < V; ++j) {
        ord[j].pi = exp((double)l[j] / T - M) / Z;
        ord[j].idx = j;
    }
    /* (2) order: probability descending, index ascending */
    qsort(ord, (size_t)V, sizeof(pi_idx), cmp_pi_desc_idx_asc);
    double pi_max = ord[0].pi;
    /* (3a) top-p: shortest prefix whose mass reaches top_p */
    int64_t m_p = V;
    if (top_p < 1.0) {
        double cum = 0.0;
        for (int64_t m = 1; m <= V; ++m) {
            double prev = cum;
            cum += ord[m - 1].pi;
            if (cum >= top_p) {
                m_p = m;
                if (fabs(cum - top_p) < 1e-6 || fabs(prev - top_p) < 1e-6) info->near_top_p = 1;
                break;
            }
        }
    }
    /* (3b) min-p: tokens with pi >= min_p * pi_max */
    int64_t m_m = V;
    if (min_p > 0.0) {
        double thr = min_p * pi_max;
        m_m = 0;
        for (int64_t j = 0; j < V; ++j)
            if (ord[j].pi >= thr) ++m_m;
        /* tokens at the cut: the last kept and the first dropped */
        if (m_m >= 1 && fabs(ord[m_m - 1].pi - thr) < 1e-6 * pi_max) info->near_min_p = 1;
        if (m_m < V && fabs(ord[m_m].pi - thr) < 1e-6 * pi_max) info->near_min_p = 1;
    }
    /* (3c) top-k: the first top_k tokens of the order */
    const int64_t m_k = (top_k > 0 && top_k < V) ? top_k : V;
    int64_t n_keep = m_p < m_m ? m_p : m_m;
    if (m_k < n_keep) n_keep = m_k;
    /* A near-threshold cut matters only where it decides the kept set: moving the
     * top-p cut by one token changes the shortest prefix only when m_p is (one of) the
     * shortest, and likewise the min-p cut. */
    const int64_t other_p = m_m < m_k ? m_m : m_k, other_m = m_p < m_k ? m_p : m_k;
    if (m_p > other_p) info->near_top_p = 0;
    if (m_m > other_m) info->near_min_p = 0;
    /* (4) renormalise over the kept set */
    double S = 0.0;
    for (int64_t m = 0; m < n_keep; ++m) S += ord[m].pi;
    for (int64_t j = 0; j < V; ++j) p[j] = 0.0;
    for (int64_t m = 0; m < n_keep; ++m) p[ord[m].idx] = ord[m].pi / S;
    info->n_keep = n_keep;
    info->m_p = m_p;
    info->m_m = m_m;
    info->m_k = m_k;
    free(ord);
    return 0;
}

/* ----------------------------------------------------------- categorical draw */

/* Smallest j (vocabulary order) with running sum C_j > u * sum(w); if rounding
 * leaves none, the last j with w_j > 0.  *near: u*S within 1e-6*S of C_j or C_{j-1}. */
int64_t or_cat(const double* w, int64_t V, double u, int* near) {
    double S = 0.0;
    for (int64_t j = 0; j < V; ++j) S += w[j];
    double t = u * S, C = 0.0;
    for (int64_t j = 0; j < V; ++j) {
        double prev = C;
        C += w[j];
        if (C > t) {
            if (fabs(t - C) < 1e-6 * S || fabs(t - prev) < 1e-6 * S) *near = 1;
            return j;
        }
    }
    *near = 1;
    for (int64_t j = V - 1; j >= 0; --j)
        if (w[j] > 0.0) return j;
    return -1;
}

/* ------------------------------------------------------------------ acceptance */

#define OR_MODE_GREEDY 0
#define OR_MODE_SAMPLE 1

#define OR_DRAFT_GIVEN 0          /* drafts are an input */
#define OR_DRAFT_Q_ARGMAX 1       /* x_i = argmax of drafter row i */
#define OR_DRAFT_Q_SAMPLE 2       /* x_i = Cat(q_i, u_D) */
#define OR_DRAFT_AGREE 3          /* x_i = target argmax if u_D < alpha, else another token via u_X */

#define OR_NEAR_RATIO 1
#define OR_NEAR_CAT 2
#define OR_NEAR_TOP_P 4
#define OR_NEAR_MIN_P 8
#define OR_NEAR_DRAFT_CAT 16

typedef struct {
    int mode, draft_mode;
    int64_t W, K, V;
    const float* target;     /* [W][K][V] */
    const float* draft;      /* [W][K-1][V] or NULL */
    int32_t* draft_tokens;   /* [W][K-1]: input (GIVEN) or output */
    double T, top_p, min_p, alpha;
    uint64_t seed, window_base;
    int32_t* n_accepted;     /* [W] */
    int32_t* tokens;         /* [W][K], -1 padded */
    int32_t* status;         /* [W]: 0 ok, 1 non-finite logit, 2 draft token out of range */
    int32_t* near;           /* [W]: OR_NEAR_* bits */
    int64_t top_k;           /* top-k cut (0 = none) */
} or_accept_args;

typedef struct {
    const or_accept_args* A;
    int64_t w0, w1;
    int err;
} acc_job;

static int row_finite(const float* l, int64_t V) {
    for (int64_t j = 0; j < V; ++j)
        if (!isfinite(l[j])) return 0;
    return 1;
}

static void accept_window(const or_accept_args* A, int64_t w, double* p, double* q, double* res) {
    const int64_t K = A->K, V = A->V;
    const float* tgt = A->target + w * K * V;
    const float* drf = A->draft ? A->draft + w * (K - 1) * V : NULL;
    int32_t* dtok = A->draft_tokens ? A->draft_tokens + w * (K - 1) : NULL;
    int32_t* out = A->tokens + w * K;
    uint64_t win = A->window_base + (uint64_t)w;
    int near = 0, status = 0;
    for (int64_t i = 0; i < K; ++i) out[i] = -1;
    A->n_accepted[w] = 0;

    int uses_drafter = (A->mode == OR_MODE_SAMPLE) || A->draft_mode == OR_DRAFT_Q_ARGMAX ||
                       A->draft_mode == OR_DRAFT_Q_SAMPLE;
    for (int64_t i = 0; i < K; ++i)
        if (!row_finite(tgt + i * V, V)) status = 1;
    if (uses_drafter)
        for (int64_t i = 0; i + 1 < K; ++i)
            if (!row_finite(drf + i * V, V)) status = 1;

    /* Drafts x_1..x_{K-1} (position i = 1..K-1 is row i-1). */
    int32_t x[64];
    for (int64_t i = 1; i < K && !status; ++i) {
        double u[4];
        or_uniforms(A->seed, win, (uint64_t)i, u);
        int64_t xi = -1;
        if (A->draft_mode == OR_DRAFT_GIVEN) {
            xi = dtok[i - 1];
            if (xi < 0 || xi >= V) status = 2;
        } else if (A->draft_mode == OR_DRAFT_Q_ARGMAX) {
            xi = or_argmax(drf + (i - 1) * V, V);
        } else if (A->draft_mode == OR_DRAFT_Q_SAMPLE) {
            or_warp_info qi;
            or_warp(drf + (i - 1) * V, V, A->T, A->top_p, A->min_p, A->top_k, q, &qi);
            if (qi.near_top_p) near |= OR_NEAR_TOP_P;
            if (qi.near_min_p) near |= OR_NEAR_MIN_P;
            int nc = 0;
            xi = or_cat(q, V, u[2], &nc);
            if (nc) near |= OR_NEAR_DRAFT_CAT;
        } else { /* OR_DRAFT_AGREE */
            int64_t a = or_argmax(tgt + (i - 1) * V, V);
            if (u[2] < A->alpha) {
                xi = a;
            } else {
                uint64_t r[4], ctr[4] = {win, (uint64_t)i, 0, 0}, key[2] = {A->seed, 0};
                or_philox4x64(ctr, key, r);
                /* floor(u_X * (V - 1)), computed exactly in integers */
                int64_t o = (int64_t)(((r[3] >> 40) * (uint64_t)(V - 1)) >> 24);
                xi = o < a ? o : o + 1;
            }
        }
        x[i] = (int32_t)xi;
    }
    if (status) {
        A->status[w] = status;
        A->near[w] = 0;
        if (dtok && A->draft_mode != OR_DRAFT_GIVEN)
            for (int64_t i = 0; i + 1 < K; ++i) dtok[i] = -1;
        return;
    }
    if (dtok && A->draft_mode != OR_DRAFT_GIVEN)
        for (int64_t i = 1; i < K; ++i) dtok[i - 1] = x[i];

    if (A->mode == OR_MODE_GREEDY) {
        int64_t n = 0;
        while (n < K - 1 && x[n + 1] == or_argmax(tgt + n * V, V)) {
            out[n] = x[n + 1];
            ++n;
        }
        out[n] = (int32_t)or_argmax(tgt + n * V, V);
        A->n_accepted[w] = (int32_t)n;
        A->status[w] = 0;
        A->near[w] = near;
        return;
    }

    /* Sampling: ratio test at positions 1..K-1, then the bonus at position K. */
    for (int64_t i = 1; i <= K; ++i) {
        double u[4];
        or_uniforms(A->seed, win, (uint64_t)i, u);
        or_warp_info pi;
        or_warp(tgt + (i - 1) * V, V, A->T, A->top_p, A->min_p, A->top_k, p, &pi);
        if (pi.near_top_p) near |= OR_NEAR_TOP_P;
        if (pi.near_min_p) near |= OR_NEAR_MIN_P;
        if (i == K) {             /* every draft accepted: bonus token from p_K */
            int nc = 0;
            out[K - 1] = (int32_t)or_cat(p, V, u[1], &nc);
            if (nc) near |= OR_NEAR_CAT;
            A->n_accepted[w] = (int32_t)(K - 1);
            break;
        }
        or_warp_info qi;
        or_warp(drf + (i - 1) * V, V, A->T, A->top_p, A->min_p, A->top_k, q, &qi);
        if (qi.near_top_p) near |= OR_NEAR_TOP_P;
        if (qi.near_min_p) near |= OR_NEAR_MIN_P;
        double r = p[x[i]] / q[x[i]];
        if (isfinite(r) && fabs(u[0] - r) < 1e-6) near |= OR_NEAR_RATIO;
        if (u[0] < r) {           /* accept x_i */
            out[i - 1] = x[i];
            continue;
        }
        /* reject: resample from norm(max(0, p - q)), or from p if that is all zero */
        double S = 0.0;
        for (int64_t j = 0; j < V; ++j) {
            res[j] = p[j] > q[j] ? p[j] - q[j] : 0.0;
            S += res[j];
        }
        int nc = 0;
        out[i - 1] = (int32_t)or_cat(S > 0.0 ? res : p, V, u[1], &nc);
        if (nc) near |= OR_NEAR_CAT;
        A->n_accepted[w] = (int32_t)(i - 1);
        break;
    }
    A->status[w] = 0;
    A->near[w] = near;
}

static void* acc_worker(void* arg) {
    acc_job* J = (acc_job*)arg;
    const int64_t V = J->A->V;
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    double* q = (double*)malloc(sizeof(double) * (size_t)V);
    double* r = (double*)malloc(sizeof(double) * (size_t)V);
    if (!p || !q || !r) {
        J->err = -2;
    } else {
        for (int64_t w = J->w0; w < J->w1; ++w) accept_window(J->A, w, p, q, r);
    }
    free(p); free(q); free(r);
    return NULL;
}

int or_accept(const or_accept_args* A, int nthreads) {
    if (A->K < 1 || A->K > 64 || A->V < 1 || A->W < 0) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > A->W) nthreads = A->W > 0 ? (int)A->W : 1;
    pthread_t th[256];
    acc_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        acc_job J = {A, A->W * t / nthreads, A->W * (t + 1) / nthreads, 0};
        jobs[t] = J;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, acc_worker, &jobs[t]);
    acc_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].err) return jobs[t].err;
    return 0;
}
