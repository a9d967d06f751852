// Lossless acceptance of drafted tokens against the target's [K][vocab] logits.
//
// Greedy: a draft is kept while it equals the target argmax; sampling: draft x
// survives with probability min(1, p(x)/q(x)) and on rejection a token is drawn from
// the normalised positive part of p - q (page "100 tokens per second from a 27B model
// on a 24 GB AMD card", section "How speculative decoding gets past a per-token wall";
// page "Decode is memory-bound ...", section "Speculative decoding").  p and q are the
// rows after the sampler warp: temperature, softmax, then the top-p and min-p cuts
// (page "Decode is memory-bound ...", section "Two things the math says to do") and an
// optional top-k cut (the first top_k entries; page "100 tokens per second ...", section
// "What failed", names top-k sampling): each cut is a prefix of one order, the kept set
// the shortest.
//
// Kernels:
//  * k_row_stats: one 512-thread workgroup per logits row.  Pass 1 finds the maximum,
//    the first argmax and non-finite entries.  For sampling rows, pass 2 sums
//    e_j = exp((l_j - l_max) / T) in 2^-44 fixed point (integer sums are exact and
//    order-independent, so every run is bitwise identical), pass 3 locates the top-p
//    cut exactly by a three-level radix select on the order-preserving bit pattern of
//    the logit (12 + 12 + 8 bits, histograms of probability mass in LDS) and then
//    resolves equal logits by index; the top-k cut is the same select over counts; pass 4
//    sums the kept mass.  The kept set is then "min-p test passes and (key, index) ranks
//    at or before the earlier cut".
//  * k_accept: one 512-thread workgroup per window.  Thread 0 runs the sequential
//    rule; inverse-CDF draws are block-wide: each thread owns a contiguous slice of
//    the vocabulary, slice masses are scanned, and the slice holding the crossing is
//    walked in index order.
// Uniforms come from Philox4x64-10 (Salmon et al., SC'11) keyed by the seed, with the
// counter (window, position, 0, 0); u = top 24 bits * 2^-24, exact in fp32 and fp64.
#include <hip/hip_runtime.h>

#include "vq_internal.h"

namespace vq {
namespace {

constexpr int NT = 512;                        // threads per workgroup
constexpr double FX = 17592186044416.0;        // 2^44, fixed-point unit of mass
constexpr float FXF = 17592186044416.0f;

struct RowStat {
    int32_t argmax;
    int32_t nonfinite;
    float lmax;
    uint32_t thr_key;    // the cut: keys above are kept, equal keys up to thr_idx
    int32_t thr_idx;
    int32_t n_keep;
    uint64_t z_fx;       // sum of e over the row
    uint64_t keep_fx;    // sum of e over the kept set
};

// Order-preserving map of a finite float to uint32 (larger float -> larger key; -0 and +0
// compare equal, so both take the key of +0).
__device__ __forceinline__ uint32_t fkey(float v) {
    const uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float e_of(float l, float lmax, float T) {
    return expf(__fdiv_rn(l - lmax, T));
}

__device__ __forceinline__ uint64_t to_fx(float e) { return (uint64_t)(e * FXF); }

__device__ __forceinline__ bool kept(const RowStat& s, float l, float e, int j, float min_p) {
    if (min_p > 0.f && !(e >= min_p)) return false;
    const uint32_t k = fkey(l);
    return k > s.thr_key || (k == s.thr_key && j <= s.thr_idx);
}

// ---------------------------------------------------------------- block helpers

// f(v, j) for the entries j = t, t + NT, t + 2 NT, ... of a row, in increasing j per
// thread; RU consecutive strides are loaded together so that many loads are in flight.
constexpr int RU = 16;
template <class F>
__device__ __forceinline__ void row_for(const float* l, int V, F&& f) {
    int j = threadIdx.x;
    for (; j + (RU - 1) * NT < V; j += RU * NT) {
        float v[RU];
#pragma unroll
        for (int u = 0; u < RU; ++u) v[u] = l[j + u * NT];
#pragma unroll
        for (int u = 0; u < RU; ++u) f(v[u], j + u * NT);
    }
    for (; j < V; j += NT) f(l[j], j);
}

__device__ uint64_t block_sum_u64(uint64_t v, uint64_t* sh) {
    sh[threadIdx.x] = v;
    __syncthreads();
    for (int s = NT / 2; s > 0; s >>= 1) {
        if (threadIdx.x < (unsigned)s) sh[threadIdx.x] += sh[threadIdx.x + s];
        __syncthreads();
    }
    const uint64_t r = sh[0];
    __syncthreads();
    return r;
}

// Exclusive prefix sum over threads 0..NT-1 in thread order; *total gets the sum.
__device__ uint64_t block_excl_scan_u64(uint64_t v, uint64_t* sh, uint64_t* total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    uint64_t x = v;
    for (int o = 1; o < 64; o <<= 1) {
        const uint64_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[wv] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t run = 0;
        for (int w = 0; w < NT / 64; ++w) {
            const uint64_t t = sh[w];
            sh[w] = run;
            run += t;
        }
        sh[NT / 64] = run;
    }
    __syncthreads();
    const uint64_t r = sh[wv] + x - v;
    *total = sh[NT / 64];
    __syncthreads();
    return r;
}

// Highest bin b of hist[0..n) (n = 256 or 4096) with sum_{b' >= b} hist >= tgt; also the
// mass strictly above b.  Requires sum(hist) >= tgt.
__device__ void find_bin(const uint64_t* hist, int n, uint64_t tgt, uint64_t* sh, int* bin,
                         uint64_t* above, int* sbin, uint64_t* sabove) {
    const int bpt = n >= NT ? n / NT : 1;
    const int active = n / bpt;
    const int t = threadIdx.x;
    uint64_t local = 0;
    if (t < active)
        for (int i = 0; i < bpt; ++i) local += hist[n - 1 - (t * bpt + i)];
    uint64_t tot;
    const uint64_t before = block_excl_scan_u64(local, sh, &tot);
    if (t < active && before < tgt && tgt <= before + local) {
        uint64_t c = before;
        for (int i = 0; i < bpt; ++i) {
            const int b = n - 1 - (t * bpt + i);
            if (c + hist[b] >= tgt) {
                *sbin = b;
                *sabove = c;
                break;
            }
            c += hist[b];
        }
    }
    __syncthreads();
    *bin = *sbin;
    *above = *sabove;
    __syncthreads();
}

// ------------------------------------------------------------------ row stats

struct StatArgs {
    const float* logits;   // rows of length V
    int nrows;
    int V;
    int full;              // 0: argmax and non-finite only
    float T, top_p, min_p;
    int top_k;             // 0: no top-k cut
    RowStat* out;
    // With few rows, the first two passes run split over SPLIT_S workgroups per row
    // (k_row_part1, k_row_part2) and k_row_stats starts from their partials; NULL: not split.
    const struct Part1* p1;
    const struct Part2* p2;
};

// Split row statistics: a row is cut into SPLIT_S slices, one workgroup each.  Their
// partials combine exactly (the maximum with its first index, the or of non-finite
// flags, integer fixed-point sums), so the statistics are the same bits as one
// workgroup's passes.
constexpr int SPLIT_S = 64;
constexpr int SPLIT_MAX_ROWS = 64;
constexpr int SPLIT_MIN_V = 16384;
struct Part1 {
    float m;
    int i, nf, pad;
};
struct Part2 {
    uint64_t z, zm, nm, pad;
};

__device__ __forceinline__ void slice_of(int V, int sl, int& j0, int& j1) {
    const int chunk = (V + SPLIT_S - 1) / SPLIT_S;
    j0 = min(V, sl * chunk);
    j1 = min(V, j0 + chunk);
}

// Largest value with its first index over the workgroup (the pass-1 tree order).
__device__ void block_max_first(float& best, int& bi, float* shf, int* shi) {
    const int t = threadIdx.x;
    shf[t] = best;
    shi[t] = bi;
    __syncthreads();
    for (int s = NT / 2; s > 0; s >>= 1) {
        if (t < s) {
            const float ob = shf[t + s];
            const int oi = shi[t + s];
            if (ob > shf[t] || (ob == shf[t] && oi < shi[t])) { shf[t] = ob; shi[t] = oi; }
        }
        __syncthreads();
    }
    best = shf[0];
    bi = shi[0];
    __syncthreads();
}

// Pass 1 of one slice: maximum, first argmax, non-finite entries.
__global__ __launch_bounds__(NT) void k_row_part1(const float* logits, int V, Part1* out) {
    __shared__ float shf[NT];
    __shared__ int shi[NT];
    const int row = blockIdx.x / SPLIT_S, sl = blockIdx.x % SPLIT_S;
    const float* l = logits + (size_t)row * V;
    int j0, j1;
    slice_of(V, sl, j0, j1);
    float best = -INFINITY;
    int bi = 0x7fffffff;
    int nf = 0;
    for (int j = j0 + (int)threadIdx.x; j < j1; j += NT) {
        const float v = l[j];
        if (!isfinite(v)) nf = 1;
        else if (v > best) { best = v; bi = j; }
    }
    block_max_first(best, bi, shf, shi);
    const int anynf = __syncthreads_or(nf);
    if (threadIdx.x == 0) out[blockIdx.x] = Part1{best, bi, anynf ? 1 : 0, 0};
}

// The row's maximum, first argmax and non-finite flag from its slices (slice order).
__device__ __forceinline__ void combine_part1(const Part1* p, float& lmax, int& amax, int& nf) {
    lmax = -INFINITY;
    amax = 0x7fffffff;
    nf = 0;
    for (int i = 0; i < SPLIT_S; ++i) {
        const Part1 q = p[i];
        nf |= q.nf;
        if (q.m > lmax || (q.m == lmax && q.i < amax)) { lmax = q.m; amax = q.i; }
    }
}


// Pass 2 of one slice: the mass and the min-p set's mass and size.
__global__ __launch_bounds__(NT) void k_row_part2(StatArgs A, Part2* out) {
    __shared__ uint64_t sh[NT + 1];
    __shared__ float s_lmax;
    __shared__ int s_skip;
    const int row = blockIdx.x / SPLIT_S, sl = blockIdx.x % SPLIT_S;
    if (threadIdx.x == 0) {
        float lmax;
        int amax, nf;
        combine_part1(A.p1 + (size_t)row * SPLIT_S, lmax, amax, nf);
        s_lmax = lmax;
        s_skip = nf || !A.full;
    }
    __syncthreads();
    if (s_skip) return;
    const float lmax = s_lmax, T = A.T, min_p = A.min_p;
    const float* l = A.logits + (size_t)row * A.V;
    int j0, j1;
    slice_of(A.V, sl, j0, j1);
    uint64_t z = 0, zm = 0, nm = 0;
    for (int j = j0 + (int)threadIdx.x; j < j1; j += NT) {
        const float e = e_of(l[j], lmax, T);
        const uint64_t f = to_fx(e);
        z += f;
        if (e >= min_p) { zm += f; ++nm; }
    }
    z = block_sum_u64(z, sh);
    zm = block_sum_u64(zm, sh);
    nm = block_sum_u64(nm, sh);
    if (threadIdx.x == 0) out[blockIdx.x] = Part2{z, zm, nm, 0};
}

__global__ __launch_bounds__(NT) void k_row_stats(StatArgs A) {
    __shared__ uint64_t hist[4096];
    __shared__ uint64_t sh[NT + 1];
    __shared__ float shf[NT];
    __shared__ int shi[NT];
    __shared__ int s_bin;
    __shared__ uint64_t s_above;
    const int row = blockIdx.x;
    const int V = A.V;
    const float* l = A.logits + (size_t)row * V;
    const int t = threadIdx.x;

    // pass 1: maximum, first argmax, non-finite entries (or their split partials)
    float best = -INFINITY;
    int bi = 0x7fffffff;
    int nf = 0;
    if (A.p1) {
        if (t == 0) combine_part1(A.p1 + (size_t)row * SPLIT_S, best, bi, nf);
    } else {
        row_for(l, V, [&](float v, int j) {
            if (!isfinite(v)) nf = 1;
            else if (v > best) { best = v; bi = j; }
        });
    }
    block_max_first(best, bi, shf, shi);
    const float lmax = best;
    const int amax = bi;
    const int anynf = __syncthreads_or(nf);
    RowStat st;
    st.argmax = amax == 0x7fffffff ? 0 : amax;
    st.nonfinite = anynf ? 1 : 0;
    st.lmax = lmax;
    st.thr_key = 0u;
    st.thr_idx = 0x7fffffff;
    st.n_keep = 0;
    st.z_fx = 0;
    st.keep_fx = 0;
    if (anynf || !A.full) {
        if (t == 0) A.out[row] = st;
        return;
    }
    const float T = A.T;

    // pass 2: total mass, and the mass and size of the min-p set (e >= min_p).  The
    // min-p set is a prefix of the (logit descending, index ascending) order, like every
    // top-p prefix, and the kept set is the shorter of the two.
    uint64_t z = 0, zm = 0, nm = 0;
    const float min_p = A.min_p;
    if (A.p2) {
        if (t < SPLIT_S) {
            const Part2 q = A.p2[(size_t)row * SPLIT_S + t];
            z = q.z;
            zm = q.zm;
            nm = q.nm;
        }
    } else {
        row_for(l, V, [&](float v, int) {
            const float e = e_of(v, lmax, T);
            const uint64_t f = to_fx(e);
            z += f;
            if (e >= min_p) { zm += f; ++nm; }
        });
    }
    st.z_fx = block_sum_u64(z, sh);

    // pass 3: the cuts, each the entry of the order (key descending, index ascending) at
    // which a running measure first reaches a target: top-p over probability mass,
    // top-k over counts.  The kept set ends at the earlier one.
    auto cut_at = [&](bool by_count, uint64_t tgt, uint32_t& kout, int& iout) {
        uint32_t prefix = 0;
        int shift_hi = 32;      // bits already fixed: key >> shift_hi == prefix
        uint64_t above = 0;
        const int levels[3] = {12, 12, 8};
        for (int lv = 0; lv < 3; ++lv) {
            const int nbits = levels[lv];
            const int nbins = 1 << nbits;
            const int shift = shift_hi - nbits;
            for (int i = t; i < nbins; i += NT) hist[i] = 0;
            __syncthreads();
            row_for(l, V, [&](float v, int) {
                const uint32_t k = fkey(v);
                if (shift_hi == 32 || (k >> shift_hi) == prefix)
                    atomicAdd((unsigned long long*)&hist[(k >> shift) & (nbins - 1)],
                              by_count ? 1ull : (unsigned long long)to_fx(e_of(v, lmax, T)));
            });
            __syncthreads();
            int b;
            uint64_t ab;
            find_bin(hist, nbins, tgt - above, sh, &b, &ab, &s_bin, &s_above);
            above += ab;
            prefix = (shift_hi == 32 ? 0u : (prefix << nbits)) | (uint32_t)b;
            shift_hi = shift;
        }
        const uint32_t kstar = prefix;
        // equal keys: the c-th smallest index among them crosses the target
        const uint64_t need = tgt - above;
        uint64_t c = need;
        if (!by_count) {
            const float lstar = __uint_as_float((kstar & 0x80000000u) ? (kstar & 0x7fffffffu) : ~kstar);
            const uint64_t estar = to_fx(e_of(lstar, lmax, T));
            c = estar ? (need + estar - 1) / estar : 1;
        }
        // The entries with key kstar: usually a handful.  Up to NT of them are listed in
        // LDS and the cc-th smallest index is found by ranking; more than that (long runs
        // of equal logits) take an ordered scan over contiguous slices.
        if (t == 0) s_bin = 0;
        __syncthreads();
        uint64_t cnt = 0;
        row_for(l, V, [&](float v, int j) {
            if (fkey(v) == kstar) {
                ++cnt;
                const int at = atomicAdd(&s_bin, 1);
                if (at < NT) shi[at] = j;
            }
        });
        const uint64_t tot = block_sum_u64(cnt, sh);
        const uint64_t cc = c > tot ? tot : c;
        if (tot <= (uint64_t)NT) {
            __syncthreads();
            int pick = -1;
            if ((uint64_t)t < tot) {
                const int mine = shi[t];
                uint64_t rank = 0;
                for (int i = 0; i < (int)tot; ++i) rank += shi[i] < mine;
                if (rank + 1 == cc) pick = mine;
            }
            __syncthreads();
            if (pick >= 0) s_bin = pick;
        } else {
            const int chunk = (V + NT - 1) / NT;
            const int j0 = t * chunk, j1 = min(V, j0 + chunk);
            uint64_t cs = 0;
            for (int j = j0; j < j1; ++j) cs += fkey(l[j]) == kstar;
            uint64_t tot2;
            const uint64_t before = block_excl_scan_u64(cs, sh, &tot2);
            if (before < cc && cc <= before + cs) {
                uint64_t seen = before;
                for (int j = j0; j < j1; ++j)
                    if (fkey(l[j]) == kstar && ++seen == cc) { s_bin = j; break; }
            }
        }
        __syncthreads();
        kout = kstar;
        iout = s_bin;
        __syncthreads();
    };
    bool cut = false;
    uint32_t ck = 0u;
    int ci = 0x7fffffff;
    if (A.top_k > 0 && A.top_k < V) {
        cut_at(true, (uint64_t)A.top_k, ck, ci);
        cut = true;
    }
    if (A.top_p < 1.f) {
        uint64_t tgt = (uint64_t)ceil((double)A.top_p * (double)st.z_fx);
        if (tgt < 1) tgt = 1;
        // a min-p set holding less than the top-p mass lies inside every top-p prefix:
        // then the top-p cut cannot be the shorter one
        const bool minp_inside = min_p > 0.f && block_sum_u64(zm, sh) < tgt;
        if (!minp_inside) {
            uint32_t pk;
            int pi;
            cut_at(false, tgt, pk, pi);
            if (!cut || pk > ck || (pk == ck && pi < ci)) {
                ck = pk;
                ci = pi;
            }
            cut = true;
        }
    }
    st.thr_key = ck;
    st.thr_idx = ci;

    // pass 4: kept mass and size
    uint64_t kf = 0, kn = 0;
    row_for(l, V, [&](float v, int j) {
        const float e = e_of(v, lmax, T);
        if (kept(st, v, e, j, A.min_p)) { kf += to_fx(e); ++kn; }
    });
    st.keep_fx = block_sum_u64(kf, sh);
    st.n_keep = (int)block_sum_u64(kn, sh);
    if (t == 0) A.out[row] = st;
}

// ------------------------------------------------------------------ Philox

__device__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
        const uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
        const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
        k0 += W0;
        k1 += W1;
    }
}

// Top 24 bits of the four Philox lanes of (window, position).
__device__ void uniforms24(uint64_t seed, uint64_t window, uint64_t pos, uint32_t (&u)[4]) {
    uint64_t c[4] = {window, pos, 0, 0};
    philox4x64_10(c, seed, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = (uint32_t)(c[i] >> 40);
}

// ------------------------------------------------------------------ accept

struct AcceptArgs {
    int mode, draft_mode, W, K, V;
    const float* tgt;          // [W][K][V]
    const float* drf;          // [W][K-1][V]
    int32_t* draft_tokens;
    float T, top_p, min_p;
    uint32_t alpha24;          // ceil(alpha * 2^24)
    uint64_t seed, window_base;
    const RowStat* st_t;       // [W*K]
    const RowStat* st_d;       // [W*(K-1)]
    int32_t *n_acc, *tokens, *status;
    // Split draw (few windows): k_accept stops before the final draw and leaves it in
    // rec[w]; k_draw_part sums SPLIT_S slices' weights, k_draw_final picks the token.
    struct DrawRec* rec;
    struct DrawPart* part;
};

// A window's final draw: at position stop (K: the bonus token from p; else the residual
// norm(max(0, p - q)), falling back to p when it is all zero) with the 24-bit uniform u24;
// need = 0 when the window needs no draw (greedy, or a data error).
struct DrawRec {
    int need, stop, n;
    uint32_t u24;
};
struct DrawPart {
    uint64_t sr, sp;           // residual and p weight sums of a slice
};

// The draw's weights in 2^-44 fixed point: p (the warped target row) and the residual.
struct DrawRows {
    RowStat sp, sq;
    const float *lp, *lq;
    double Sp, Sq;
    float T, min_p;
};

__device__ __forceinline__ uint64_t w_p(const DrawRows& R, int j) {
    const float v = R.lp[j];
    const float e = e_of(v, R.sp.lmax, R.T);
    return kept(R.sp, v, e, j, R.min_p) ? to_fx(e) : 0ull;
}

__device__ __forceinline__ uint64_t w_r(const DrawRows& R, int j) {
    const float v = R.lp[j];
    const float e = e_of(v, R.sp.lmax, R.T);
    if (!kept(R.sp, v, e, j, R.min_p)) return 0ull;
    const double pj = (double)e / R.Sp;
    const float vq = R.lq[j];
    const float eq = e_of(vq, R.sq.lmax, R.T);
    const double qj = kept(R.sq, vq, eq, j, R.min_p) ? (double)eq / R.Sq : 0.0;
    const double d = pj - qj;
    return d > 0.0 ? (uint64_t)(d * FX) : 0ull;
}

__device__ __forceinline__ DrawRows draw_rows(const AcceptArgs& A, int w, int stop) {
    DrawRows R;
    const int K = A.K, V = A.V;
    R.sp = A.st_t[(size_t)w * K + stop - 1];
    R.lp = A.tgt + ((size_t)w * K + stop - 1) * V;
    R.Sp = (double)R.sp.keep_fx / FX;
    R.T = A.T;
    R.min_p = A.min_p;
    if (stop < K) {
        R.sq = A.st_d[(size_t)w * (K - 1) + stop - 1];
        R.lq = A.drf + ((size_t)w * (K - 1) + stop - 1) * V;
        R.Sq = (double)R.sq.keep_fx / FX;
    } else {
        R.sq = R.sp;
        R.lq = R.lp;
        R.Sq = R.Sp;
    }
    return R;
}

// C * 2^24 > u24 * S with 128-bit integers.
__device__ __forceinline__ bool cross(uint64_t C, uint32_t u24, uint64_t S) {
    const uint64_t ahi = C >> 40, alo = C << 24;
    const uint64_t bhi = __umul64hi((uint64_t)u24, S), blo = (uint64_t)u24 * S;
    return ahi > bhi || (ahi == bhi && alo > blo);
}

// Smallest j with prefix_j(w) * 2^24 > u24 * sum(w) (vocabulary order); -1 if sum is 0.
// The row is read in tiles of NT * CU entries, thread t taking entries t * CU .. t * CU +
// CU - 1 of a tile (so a wave reads contiguous memory) and TU tiles' loads in flight at
// once; each wave's sum per tile goes to LDS.  One thread then walks the (tile, wave)
// sums in vocabulary order to the one holding the crossing, and that wave alone re-reads
// its 64 * CU entries of that tile: a wave prefix sum finds the crossing thread, which
// walks its CU entries.  Sums are in fixed point, so any order gives the same totals.
// Rows longer than MAX_TILES tiles use the slice walk of block_cat_slices.
constexpr int CAT_CU = 8, CAT_TU = 4, CAT_MAX_TILES = 64;

template <class WF>
__device__ int block_cat_slices(WF wf, int V, uint32_t u24, uint64_t* sh, int* sres) {
    const int chunk = (V + NT - 1) / NT;
    const int j0 = threadIdx.x * chunk, j1 = min(V, j0 + chunk);
    uint64_t local = 0;
    for (int j = j0; j < j1; ++j) local += wf(j);
    uint64_t S;
    const uint64_t before = block_excl_scan_u64(local, sh, &S);
    if (threadIdx.x == 0) *sres = -1;
    __syncthreads();
    if (S > 0 && local > 0 && !cross(before, u24, S) && cross(before + local, u24, S)) {
        uint64_t C = before;
        for (int j = j0; j < j1; ++j) {
            C += wf(j);
            if (cross(C, u24, S)) { *sres = j; break; }
        }
    }
    __syncthreads();
    const int r = *sres;
    __syncthreads();
    return r;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <class WF>
__device__ int block_cat(WF wf, int V, uint32_t u24, uint64_t* sh, int* sres) {
    constexpr int CU = CAT_CU, TILE = NT * CU, NW = NT / 64;
    const int ntile = (V + TILE - 1) / TILE;
    if (ntile > CAT_MAX_TILES) return block_cat_slices(wf, V, u24, sh, sres);
    __shared__ uint64_t tw[CAT_MAX_TILES][NW];
    __shared__ int s_tile, s_wave;
    __shared__ uint64_t s_before, s_total;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    for (int tb = 0; tb < ntile; tb += CAT_TU) {
        uint64_t w[CAT_TU][CU];
#pragma unroll
        for (int u = 0; u < CAT_TU; ++u)
#pragma unroll
            for (int e = 0; e < CU; ++e) {
                const int j = (tb + u) * TILE + t * CU + e;
                w[u][e] = j < V ? wf(j) : 0ull;
            }
#pragma unroll
        for (int u = 0; u < CAT_TU; ++u) {
            uint64_t l = 0;
#pragma unroll
            for (int e = 0; e < CU; ++e) l += w[u][e];
            l = wave_sum_u64(l);
            if (lane == 0 && tb + u < ntile) tw[tb + u][wave] = l;
        }
    }
    __syncthreads();
    if (t == 0) {
        uint64_t S = 0;
        for (int i = 0; i < ntile; ++i)
            for (int v = 0; v < NW; ++v) S += tw[i][v];
        int ft = -1, fw = 0;
        uint64_t C = 0;
        if (S > 0)
            for (int i = 0; i < ntile && ft < 0; ++i)
                for (int v = 0; v < NW; ++v) {
                    if (cross(C + tw[i][v], u24, S)) { ft = i; fw = v; break; }
                    C += tw[i][v];
                }
        s_tile = ft;
        s_wave = fw;
        s_before = C;
        s_total = S;
        *sres = -1;
    }
    __syncthreads();
    if (s_tile >= 0 && wave == s_wave) {
        const uint64_t S = s_total;
        const int base = s_tile * TILE + t * CU;
        uint64_t w[CU], l = 0;
#pragma unroll
        for (int e = 0; e < CU; ++e) {
            w[e] = base + e < V ? wf(base + e) : 0ull;
            l += w[e];
        }
        // inclusive prefix over the wave's lanes, then the lane whose range crosses
        uint64_t x = l;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint64_t y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        const uint64_t before = s_before + x - l;
        if (l > 0 && !cross(before, u24, S) && cross(before + l, u24, S)) {
            uint64_t C = before;
            for (int e = 0; e < CU; ++e) {
                C += w[e];
                if (cross(C, u24, S)) { *sres = base + e; break; }
            }
        }
    }
    __syncthreads();
    const int r = *sres;
    __syncthreads();
    return r;
}

__device__ __forceinline__ double prob_of(const RowStat& s, const float* l, int x, float T, float min_p) {
    const float v = l[x];
    const float e = e_of(v, s.lmax, T);
    if (!kept(s, v, e, x, min_p)) return 0.0;
    return (double)e / ((double)s.keep_fx / FX);
}

__global__ __launch_bounds__(NT) void k_accept(AcceptArgs A) {
    __shared__ uint64_t sh[NT + 1];
    __shared__ int sres;
    __shared__ int x[VQ_MAX_K + 1];
    __shared__ int s_status, s_n, s_stop;
    __shared__ uint32_t s_u[4];
    const int w = blockIdx.x;
    const int K = A.K, V = A.V;
    const float T = A.T, min_p = A.min_p;
    const uint64_t win = A.window_base + (uint64_t)w;
    const RowStat* stt = A.st_t + (size_t)w * K;
    const RowStat* std_ = A.st_d ? A.st_d + (size_t)w * (K - 1) : nullptr;
    const float* tl = A.tgt + (size_t)w * K * V;
    const float* dl = A.drf ? A.drf + (size_t)w * (K - 1) * V : nullptr;
    int32_t* out = A.tokens + (size_t)w * K;
    int32_t* dtok = A.draft_tokens ? A.draft_tokens + (size_t)w * (K - 1) : nullptr;
    const bool uses_drafter = A.mode == VQ_MODE_SAMPLE || A.draft_mode == VQ_DRAFT_Q_ARGMAX ||
                              A.draft_mode == VQ_DRAFT_Q_SAMPLE;

    if (threadIdx.x == 0) {
        int st = 0;
        for (int i = 0; i < K; ++i) st |= stt[i].nonfinite;
        if (uses_drafter)
            for (int i = 0; i + 1 < K; ++i) st |= std_[i].nonfinite;
        s_status = st ? 1 : 0;
    }
    __syncthreads();

    // drafts x_1..x_{K-1}
    for (int i = 1; i < K && s_status == 0; ++i) {
        if (threadIdx.x == 0) {
            uint32_t u[4];
            uniforms24(A.seed, win, (uint64_t)i, u);
            for (int q = 0; q < 4; ++q) s_u[q] = u[q];
        }
        __syncthreads();
        if (A.draft_mode == VQ_DRAFT_Q_SAMPLE) {
            const RowStat sq = std_[i - 1];
            const float* lq = dl + (size_t)(i - 1) * V;
            auto wf = [&](int j) -> uint64_t {
                const float v = lq[j];
                const float e = e_of(v, sq.lmax, T);
                return kept(sq, v, e, j, min_p) ? to_fx(e) : 0ull;
            };
            const int r = block_cat(wf, V, s_u[2], sh, &sres);
            if (threadIdx.x == 0) x[i] = r >= 0 ? r : sq.argmax;   // the argmax always has mass
        } else if (threadIdx.x == 0) {
            int xi;
            if (A.draft_mode == VQ_DRAFT_GIVEN) {
                xi = dtok[i - 1];
                if (xi < 0 || xi >= V) s_status = 2;
            } else if (A.draft_mode == VQ_DRAFT_Q_ARGMAX) {
                xi = std_[i - 1].argmax;
            } else {
                const int a = stt[i - 1].argmax;
                if (s_u[2] < A.alpha24) {
                    xi = a;
                } else {
                    const int o = (int)(((uint64_t)s_u[3] * (uint64_t)(V - 1)) >> 24);
                    xi = o < a ? o : o + 1;
                }
            }
            x[i] = xi;
        }
        __syncthreads();
    }

    if (A.rec && threadIdx.x == 0 && (s_status != 0 || A.mode == VQ_MODE_GREEDY)) A.rec[w] = DrawRec{0, 0, 0, 0u};
    if (s_status != 0) {
        for (int i = threadIdx.x; i < K; i += NT) out[i] = -1;
        if (dtok && A.draft_mode != VQ_DRAFT_GIVEN)
            for (int i = threadIdx.x; i + 1 < K; i += NT) dtok[i] = -1;
        if (threadIdx.x == 0) {
            A.n_acc[w] = 0;
            A.status[w] = s_status;
        }
        return;
    }
    if (dtok && A.draft_mode != VQ_DRAFT_GIVEN)
        for (int i = threadIdx.x + 1; i < K; i += NT) dtok[i - 1] = x[i];
    for (int i = threadIdx.x; i < K; i += NT) out[i] = -1;
    __syncthreads();

    if (A.mode == VQ_MODE_GREEDY) {
        if (threadIdx.x == 0) {
            int n = 0;
            while (n < K - 1 && x[n + 1] == stt[n].argmax) {
                out[n] = x[n + 1];
                ++n;
            }
            out[n] = stt[n].argmax;
            A.n_acc[w] = n;
            A.status[w] = 0;
        }
        return;
    }

    // sampling: ratio tests at positions 1..K-1 (thread 0), then one draw
    if (threadIdx.x == 0) {
        int n = 0, stop = K;          // stop: position of the draw (K = bonus)
        for (int i = 1; i < K; ++i) {
            uint32_t u[4];
            uniforms24(A.seed, win, (uint64_t)i, u);
            const double p = prob_of(stt[i - 1], tl + (size_t)(i - 1) * V, x[i], T, min_p);
            const double q = prob_of(std_[i - 1], dl + (size_t)(i - 1) * V, x[i], T, min_p);
            const double r = p / q;
            const double uA = (double)u[0] * (1.0 / 16777216.0);
            if (uA < r) {
                out[i - 1] = x[i];
                n = i;
            } else {
                stop = i;
                break;
            }
        }
        uint32_t u[4];
        uniforms24(A.seed, win, (uint64_t)stop, u);
        s_u[1] = u[1];
        s_n = n;
        s_stop = stop;
    }
    __syncthreads();
    const int stop = s_stop;
    if (A.rec) {
        // the draw is left to k_draw_part / k_draw_final
        if (threadIdx.x == 0) A.rec[w] = DrawRec{1, stop, s_n, s_u[1]};
        return;
    }
    const RowStat sp = stt[stop - 1];
    const float* lp = tl + (size_t)(stop - 1) * V;
    auto wp = [&](int j) -> uint64_t {
        const float v = lp[j];
        const float e = e_of(v, sp.lmax, T);
        return kept(sp, v, e, j, min_p) ? to_fx(e) : 0ull;
    };
    int tok;
    if (stop == K) {
        tok = block_cat(wp, V, s_u[1], sh, &sres);
    } else {
        const RowStat sq = std_[stop - 1];
        const float* lq = dl + (size_t)(stop - 1) * V;
        const double Sp = (double)sp.keep_fx / FX, Sq = (double)sq.keep_fx / FX;
        auto wr = [&](int j) -> uint64_t {
            const float v = lp[j];
            const float e = e_of(v, sp.lmax, T);
            if (!kept(sp, v, e, j, min_p)) return 0ull;
            const double pj = (double)e / Sp;
            const float vq = lq[j];
            const float eq = e_of(vq, sq.lmax, T);
            const double qj = kept(sq, vq, eq, j, min_p) ? (double)eq / Sq : 0.0;
            const double d = pj - qj;
            return d > 0.0 ? (uint64_t)(d * FX) : 0ull;
        };
        tok = block_cat(wr, V, s_u[1], sh, &sres);
        if (tok < 0) tok = block_cat(wp, V, s_u[1], sh, &sres);
    }
    if (threadIdx.x == 0) {
        out[stop - 1] = tok;
        A.n_acc[w] = s_n;
        A.status[w] = 0;
    }
}

// Split draw, part 1: the residual and p weight sums of slice sl of window w's draw row.
__global__ __launch_bounds__(NT) void k_draw_part(AcceptArgs A) {
    __shared__ uint64_t sh[NT + 1];
    const int w = blockIdx.x / SPLIT_S, sl = blockIdx.x % SPLIT_S;
    const DrawRec rc = A.rec[w];
    if (!rc.need) return;
    const DrawRows R = draw_rows(A, w, rc.stop);
    const bool resid = rc.stop < A.K;
    int j0, j1;
    slice_of(A.V, sl, j0, j1);
    uint64_t sr = 0, sp = 0;
    for (int j = j0 + (int)threadIdx.x; j < j1; j += NT) {
        sp += w_p(R, j);
        if (resid) sr += w_r(R, j);
    }
    sp = block_sum_u64(sp, sh);
    sr = block_sum_u64(sr, sh);
    if (threadIdx.x == 0) A.part[blockIdx.x] = DrawPart{sr, sp};
}

// Split draw, part 2: the slice holding the crossing (slice order), then the smallest
// index in it whose running sum crosses, found as block_cat finds it within one tile.
__global__ __launch_bounds__(NT) void k_draw_final(AcceptArgs A) {
    __shared__ uint64_t sh[NT + 1];
    __shared__ int s_sl, s_res, s_useq;
    __shared__ uint64_t s_C, s_S;
    const int w = blockIdx.x;
    const DrawRec rc = A.rec[w];
    if (!rc.need) return;
    const DrawRows R = draw_rows(A, w, rc.stop);
    const DrawPart* P = A.part + (size_t)w * SPLIT_S;
    if (threadIdx.x == 0) {
        uint64_t Sr = 0, Sp = 0;
        for (int i = 0; i < SPLIT_S; ++i) {
            Sr += P[i].sr;
            Sp += P[i].sp;
        }
        const bool resid = rc.stop < A.K && Sr > 0;     // an all-zero residual falls back to p
        const uint64_t S = resid ? Sr : Sp;
        uint64_t C = 0;
        int sl = -1;
        for (int i = 0; i < SPLIT_S && S > 0; ++i) {
            const uint64_t x = resid ? P[i].sr : P[i].sp;
            if (cross(C + x, rc.u24, S)) { sl = i; break; }
            C += x;
        }
        s_sl = sl;
        s_C = C;
        s_S = S;
        s_useq = resid ? 1 : 0;
        s_res = -1;
    }
    __syncthreads();
    const int sl = s_sl;
    if (sl >= 0) {
        int j0, j1;
        slice_of(A.V, sl, j0, j1);
        const bool resid = s_useq != 0;
        const uint64_t S = s_S;
        // one pass over the slice: each thread a contiguous run, prefix over the threads
        const int n = j1 - j0, per = (n + NT - 1) / NT;
        const int a = min(j1, j0 + (int)threadIdx.x * per), b = min(j1, a + per);
        uint64_t loc = 0;
        for (int j = a; j < b; ++j) loc += resid ? w_r(R, j) : w_p(R, j);
        uint64_t tot;
        const uint64_t before = s_C + block_excl_scan_u64(loc, sh, &tot);
        if (loc > 0 && !cross(before, rc.u24, S) && cross(before + loc, rc.u24, S)) {
            uint64_t C = before;
            for (int j = a; j < b; ++j) {
                C += resid ? w_r(R, j) : w_p(R, j);
                if (cross(C, rc.u24, S)) { s_res = j; break; }
            }
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        A.tokens[(size_t)w * A.K + rc.stop - 1] = s_res;
        A.n_acc[w] = rc.n;
        A.status[w] = 0;
    }
}

}  // namespace

// Workspace: row statistics of the target rows, then of the drafter rows, then (rows
// split over workgroups) the slices' partials of each.
struct AcceptLayout {
    size_t st_d, p1_t, p2_t, p1_d, p2_d, rec, dpart, total;
    bool split_t, split_d, split_draw;
};

bool split_rows(int nrows, int V) { return nrows > 0 && nrows <= SPLIT_MAX_ROWS && V >= SPLIT_MIN_V; }

AcceptLayout accept_layout(const vq_accept_desc* d) {
    AcceptLayout L{};
    const size_t rt = (size_t)d->W * d->K, rd = (size_t)d->W * (d->K > 1 ? d->K - 1 : 0);
    size_t p = align_up(rt * sizeof(RowStat), 256);
    L.st_d = p;
    p += align_up(rd * sizeof(RowStat), 256);
    L.split_t = split_rows((int)rt, d->V);
    L.split_d = split_rows((int)rd, d->V);
    if (L.split_t) {
        L.p1_t = p;
        p += align_up(rt * SPLIT_S * sizeof(Part1), 256);
        L.p2_t = p;
        p += align_up(rt * SPLIT_S * sizeof(Part2), 256);
    }
    if (L.split_d) {
        L.p1_d = p;
        p += align_up(rd * SPLIT_S * sizeof(Part1), 256);
        L.p2_d = p;
        p += align_up(rd * SPLIT_S * sizeof(Part2), 256);
    }
    // sampling with few windows: the final draws split over workgroups
    L.split_draw = d->mode == VQ_MODE_SAMPLE && split_rows(d->W, d->V);
    if (L.split_draw) {
        L.rec = p;
        p += align_up((size_t)d->W * sizeof(DrawRec), 256);
        L.dpart = p;
        p += align_up((size_t)d->W * SPLIT_S * sizeof(DrawPart), 256);
    }
    L.total = p;
    return L;
}

size_t accept_ws_bytes(const vq_accept_desc* d) { return accept_layout(d).total; }

// Row statistics of one set of rows: split over workgroups when the rows are few.
hipError_t launch_row_stats(StatArgs a, bool split, char* ws, size_t p1_off, size_t p2_off, hipStream_t st) {
    if (a.nrows == 0) return hipSuccess;
    if (split) {
        Part1* p1 = (Part1*)(ws + p1_off);
        Part2* p2 = (Part2*)(ws + p2_off);
        k_row_part1<<<dim3(a.nrows * SPLIT_S), NT, 0, st>>>(a.logits, a.V, p1);
        a.p1 = p1;
        k_row_part2<<<dim3(a.nrows * SPLIT_S), NT, 0, st>>>(a, p2);
        a.p2 = a.full ? p2 : nullptr;
    }
    k_row_stats<<<dim3(a.nrows), NT, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_accept(const vq_accept_desc* d, void* ws, hipStream_t st) {
    if (d->W == 0) return hipSuccess;
    const AcceptLayout L = accept_layout(d);
    char* wsb = (char*)ws;
    RowStat* st_t = (RowStat*)wsb;
    RowStat* st_d = (RowStat*)(wsb + L.st_d);
    const bool sample = d->mode == VQ_MODE_SAMPLE;
    const bool drafter = sample || d->draft_mode == VQ_DRAFT_Q_ARGMAX || d->draft_mode == VQ_DRAFT_Q_SAMPLE;
    const float T = d->temperature;
    StatArgs sa{d->target_logits, d->W * d->K, d->V, sample ? 1 : 0, T, d->top_p, d->min_p, d->top_k, st_t,
                nullptr, nullptr};
    hipError_t e = launch_row_stats(sa, L.split_t, wsb, L.p1_t, L.p2_t, st);
    if (e != hipSuccess) return e;
    if (drafter && d->K > 1) {
        const int full = (sample || d->draft_mode == VQ_DRAFT_Q_SAMPLE) ? 1 : 0;
        StatArgs sd{d->draft_logits, d->W * (d->K - 1), d->V, full, T, d->top_p, d->min_p, d->top_k, st_d,
                    nullptr, nullptr};
        e = launch_row_stats(sd, L.split_d, wsb, L.p1_d, L.p2_d, st);
        if (e != hipSuccess) return e;
    }
    double a24 = ceil((double)d->alpha * 16777216.0);
    if (a24 < 0) a24 = 0;
    if (a24 > 16777216.0) a24 = 16777216.0;
    AcceptArgs aa{d->mode, d->draft_mode, d->W, d->K, d->V, d->target_logits,
                  drafter ? d->draft_logits : nullptr, d->draft_tokens, T, d->top_p, d->min_p,
                  (uint32_t)a24, d->seed, d->window_base, st_t, drafter ? st_d : nullptr,
                  d->n_accepted, d->tokens, d->status, nullptr, nullptr};
    if (L.split_draw) {
        aa.rec = (DrawRec*)(wsb + L.rec);
        aa.part = (DrawPart*)(wsb + L.dpart);
    }
    k_accept<<<dim3(d->W), NT, 0, st>>>(aa);
    if (L.split_draw) {
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        k_draw_part<<<dim3(d->W * SPLIT_S), NT, 0, st>>>(aa);
        k_draw_final<<<dim3(d->W), NT, 0, st>>>(aa);
    }
    return hipGetLastError();
}

}  // namespace vq
