// C ABI of libvq: argument validation, the decode workspace layout, and the launch
// sequence of a pass.  Every check runs on the host before anything is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "steps.h"
#include "vq_internal.h"

namespace vq {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_err[0] = 0; }

namespace {

int hip_fail(hipError_t e, const char* what) {
    return fail(VQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_matrix(const vq_matrix* W, const char* name) {
    if (!W) return fail(VQ_ERR_ARG, "%s: NULL matrix descriptor", name);
    if (W->format < VQ_FMT_Q4 || W->format > VQ_FMT_Q4_K)
        return fail(VQ_ERR_ARG, "%s: unknown format %d", name, W->format);
    if (W->reserved != 0) return fail(VQ_ERR_ARG, "%s: reserved field must be 0", name);
    if (W->rows < 0) return fail(VQ_ERR_ARG, "%s: rows %d < 0", name, W->rows);
    if (W->cols <= 0 || W->cols % 32)
        return fail(VQ_ERR_ARG, "%s: cols %d is not a positive multiple of 32", name, W->cols);
    if (W->format == VQ_FMT_Q4_K && W->cols % 256)
        return fail(VQ_ERR_ARG, "%s: VQ_FMT_Q4_K needs cols %% 256 == 0 (cols %d)", name, W->cols);
    if (W->rows == 0) return VQ_OK;
    if (!W->qs || !W->scales) return fail(VQ_ERR_ARG, "%s: NULL qs or scales", name);
    const bool has_mins = W->format == VQ_FMT_Q4_MIN || W->format == VQ_FMT_Q4_K;
    if (has_mins != (W->mins != nullptr))
        return fail(VQ_ERR_ARG, "%s: mins must be given exactly for VQ_FMT_Q4_MIN and VQ_FMT_Q4_K", name);
    if ((W->format == VQ_FMT_Q4_K) != (W->supers != nullptr))
        return fail(VQ_ERR_ARG, "%s: supers must be given exactly for VQ_FMT_Q4_K", name);
    if (!aligned(W->qs, 16) || !aligned(W->scales, 16) || (W->mins && !aligned(W->mins, 16)) ||
        (W->supers && !aligned(W->supers, 16)))
        return fail(VQ_ERR_ARG, "%s: qs, scales, mins and supers must be 16-byte aligned", name);
    return VQ_OK;
}

int check_tiled(const vq_tiled* W, const char* name) {
    if (!W) return fail(VQ_ERR_ARG, "%s: NULL matrix descriptor", name);
    if (W->format < VQ_FMT_Q4 || W->format > VQ_FMT_Q4_K)
        return fail(VQ_ERR_ARG, "%s: unknown format %d", name, W->format);
    if (W->order != VQ_ROWS_PLAIN && W->order != VQ_ROWS_PAIR8)
        return fail(VQ_ERR_ARG, "%s: unknown row order %d", name, W->order);
    if (W->rows < 0) return fail(VQ_ERR_ARG, "%s: rows %d < 0", name, W->rows);
    if (W->cols <= 0 || W->cols % 32)
        return fail(VQ_ERR_ARG, "%s: cols %d is not a positive multiple of 32", name, W->cols);
    if (W->format == VQ_FMT_Q4_K && W->cols % 256)
        return fail(VQ_ERR_ARG, "%s: VQ_FMT_Q4_K needs cols %% 256 == 0 (cols %d)", name, W->cols);
    if (W->order == VQ_ROWS_PAIR8 && W->rows % 16)
        return fail(VQ_ERR_ARG, "%s: a VQ_ROWS_PAIR8 matrix needs rows %% 16 == 0 (rows %d)", name, W->rows);
    if (tiled_bytes(W->format, W->rows, W->cols) >= ((size_t)1 << 32))
        return fail(VQ_ERR_UNSUPPORTED, "%s: tiled matrix of 4 GiB or more", name);
    if (W->rows == 0) return VQ_OK;
    if (!W->data) return fail(VQ_ERR_ARG, "%s: NULL data", name);
    if (!aligned(W->data, 256)) return fail(VQ_ERR_ARG, "%s: data must be 256-byte aligned", name);
    return VQ_OK;
}

int check_attention(const vq_attention* C, int32_t K) {
    if (!C) return fail(VQ_ERR_ARG, "NULL attention descriptor");
    for (int f : {C->k_format, C->v_format})
        if (f != VQ_KV_Q8_0 && f != VQ_KV_Q4_0) return fail(VQ_ERR_ARG, "unknown KV format %d", f);
    if (C->head_dim != 128) return fail(VQ_ERR_ARG, "head_dim must be 128, got %d", C->head_dim);
    if (C->n_kv_heads < 1 || C->n_kv_heads > 1024) return fail(VQ_ERR_ARG, "n_kv_heads %d outside 1..1024", C->n_kv_heads);
    if (C->n_q_heads < 1 || C->n_q_heads % C->n_kv_heads)
        return fail(VQ_ERR_ARG, "n_q_heads %d is not a positive multiple of n_kv_heads %d", C->n_q_heads, C->n_kv_heads);
    if (C->length < 1 || C->length > (1 << 24)) return fail(VQ_ERR_ARG, "length %d outside 1..2^24", C->length);
    if (K < 1 || K > VQ_MAX_K || K > C->length) return fail(VQ_ERR_ARG, "K %d outside 1..min(%d, length)", K, VQ_MAX_K);
    if ((C->n_q_heads / C->n_kv_heads) * K > 128)
        return fail(VQ_ERR_ARG, "(n_q_heads / n_kv_heads) * K = %d exceeds 128", (C->n_q_heads / C->n_kv_heads) * K);
    if (!C->k_codes || !C->k_scales || !C->v_codes || !C->v_scales) return fail(VQ_ERR_ARG, "NULL cache plane");
    if (!aligned(C->k_codes, 16) || !aligned(C->v_codes, 16) || !aligned(C->k_scales, 16) || !aligned(C->v_scales, 16))
        return fail(VQ_ERR_ARG, "cache codes and scales must be 16-byte aligned");
    return VQ_OK;
}

}  // namespace

// ------------------------------------------------------------------ the split

// The ring holds 4 slots up to K = 4 and 2 above, where the LDS it frees widens the column
// windows (the 17408-column down stage at K = 8: 4 windows instead of 5, 1.2% off the pass).
void lds_plan(int K, int* nsp, int* pbytes, int* ring_off, int* xcap) {
    *pbytes = 256 * ((K + 3) / 4);
    *nsp = K <= 4 ? 4 : 2;
    const int ring = *nsp * FLOW_NCW * *pbytes;
    *ring_off = (FLOW_CTRL_OFF - ring) & ~255;
    *xcap = *ring_off;
}

namespace {
int wg_of_host(const KindPlan& P, long c) {
    const long big = (long)P.r * (P.q + 1);
    return (int)(c < big ? c / (P.q + 1) : P.r + (c - big) / P.q);
}
int window_of(const KindPlan& P, long c) {
    const long span = (long)P.T * P.gw;
    const long w = c / span;
    return (int)(w < P.nwin - 1 ? w : P.nwin - 1);
}
}  // namespace

bool make_plan(KindPlan& P, int fmt, int K, int rows, int cols, int tiles, int nwg, int xcap) {
    P = KindPlan{};
    P.rows = rows;
    P.cols = cols;
    P.T = tiles;
    P.G = (cols + STEP_COLS - 1) / STEP_COLS;
    P.cb = 2 * chunk_bytes(fmt);
    const int xs1 = P.G * 512 + 16;
    if ((long)K * xs1 <= xcap) {
        P.nwin = 1;
        P.gw = P.glast = P.G;
        P.xs = xs1;
    } else {
        const int half = (xcap / 2) & ~15;
        const int gmax = (half / K - 16) / 512;
        if (gmax < 1) return false;
        P.nwin = (P.G + gmax - 1) / gmax;
        P.gw = (P.G + P.nwin - 1) / P.nwin;
        P.glast = P.G - (P.nwin - 1) * P.gw;
        P.xs = P.gw * 512 + 16;
        if (P.glast < 1) return false;
    }
    const long N = (long)P.T * P.G;
    if (N <= 0 || N >= (1L << 31)) return false;
    // every workgroup's range holds at least a whole unit (a tile's chunks in one window),
    // so a unit is shared by two workgroups at most
    P.nwe = (int)std::max(1L, std::min((long)nwg, N / P.gw));
    P.q = (int)(N / P.nwe);
    P.r = (int)(N % P.nwe);
    // Whole tiles per workgroup when that costs little: no tile is then split over two
    // workgroups, which saves the exchange of partial sums at the end of the stage.  Taken
    // when k = ceil(T / nwg) tiles per workgroup divide T and the largest range is within
    // 25% of the balanced one (the 27B stack's q|k|v: 2 tiles against 1.75).  A stage whose
    // chunks are all in flight when it starts (the o projection: 1.25 tiles per workgroup)
    // still ends when its busiest workgroup is done, so it is split evenly too.
    if (P.nwin == 1) {
        const long k = (P.T + nwg - 1) / nwg;
        if (P.T % k == 0 && 4 * k * nwg <= 5L * P.T) {
            P.nwe = (int)(P.T / k);
            P.q = (int)(k * P.G);
            P.r = 0;
        }
    }
    // a range spans at most two windows (two activation buffers)
    if (P.nwin > 1) {
        for (int w = 0; w < P.nwe; ++w) {
            const long lo = (long)w * P.q + std::min(w, P.r);
            const long hi = lo + P.q + (w < P.r ? 1 : 0);
            if (window_of(P, hi - 1) - window_of(P, lo) > 1) return false;
        }
        // split tiles each workgroup finishes: the holder of the last chunk of the tile's
        // unit in window t mod nwin
        std::vector<int> pend(P.nwe, 0);
        for (int t = 0; t < P.T; ++t) {
            const int wf = t % P.nwin;
            const int gl = wf == P.nwin - 1 ? P.glast : P.gw;
            const long lf = (long)wf * P.T * P.gw + (long)(t + 1) * gl - 1;
            if (++pend[wg_of_host(P, lf)] > FLOW_PEND_MAX) return false;
        }
    }
    return true;
}

size_t plan_parts_floats(const KindPlan& P, int pbytes, int nwg, int stages) {
    // one window: two slots per workgroup boundary and stage of a launch; several: two per
    // unit, reused by every stage
    const size_t slots = P.nwin == 1 ? 2 * (size_t)nwg * stages : 2 * (size_t)P.nwin * P.T;
    return slots * (size_t)(pbytes / 4);
}
size_t plan_counters(const KindPlan& P) { return P.nwin == 1 ? (size_t)P.nwe : (size_t)P.T; }

namespace {

// ---------------------------------------------------------------- decode layout

struct Shapes {
    int H, KV, FF, V, L, fmt;
};

int check_model(const vq_model* M, Shapes* s) {
    if (!M) return fail(VQ_ERR_ARG, "NULL model");
    if (M->n_layers < 1 || !M->layers) return fail(VQ_ERR_ARG, "model needs n_layers >= 1 and layers");
    if (M->reserved != 0) return fail(VQ_ERR_ARG, "model reserved field must be 0");
    const vq_layer& l0 = M->layers[0];
    s->H = l0.qkv.cols;
    s->KV = (l0.qkv.rows - s->H) / 2;
    s->FF = l0.down.cols;
    s->V = M->lm_head.rows;
    s->L = M->n_layers;
    s->fmt = l0.qkv.format;
    if (s->H % 64 || s->KV % 64 || s->FF % 64 || s->H <= 0 || s->KV <= 0 || s->FF <= 0 ||
        l0.qkv.rows != s->H + 2 * s->KV)
        return fail(VQ_ERR_UNSUPPORTED, "decode pass needs hidden, kv and ffn sizes that are multiples of 64");
    if (s->V < 1) return fail(VQ_ERR_ARG, "lm_head needs rows >= 1");
    for (int l = 0; l < M->n_layers; ++l) {
        const vq_layer& y = M->layers[l];
        const vq_tiled* ms[4] = {&y.qkv, &y.o, &y.gu, &y.down};
        const int rr[4] = {s->H + 2 * s->KV, s->H, 2 * s->FF, s->H};
        const int cc[4] = {s->H, s->H, s->H, s->FF};
        const int oo[4] = {VQ_ROWS_PLAIN, VQ_ROWS_PLAIN, VQ_ROWS_PAIR8, VQ_ROWS_PLAIN};
        static const char* nm[4] = {"qkv", "o", "gu", "down"};
        for (int i = 0; i < 4; ++i) {
            char buf[48];
            snprintf(buf, sizeof buf, "layer %d %s", l, nm[i]);
            int rc = check_tiled(ms[i], buf);
            if (rc) return rc;
            if (ms[i]->rows != rr[i] || ms[i]->cols != cc[i] || ms[i]->format != s->fmt || ms[i]->order != oo[i])
                return fail(VQ_ERR_ARG, "%s: shape %dx%d fmt %d order %d, expected %dx%d fmt %d order %d", buf,
                            ms[i]->rows, ms[i]->cols, ms[i]->format, ms[i]->order, rr[i], cc[i], s->fmt, oo[i]);
        }
    }
    int rc = check_tiled(&M->lm_head, "lm_head");
    if (rc) return rc;
    if (M->lm_head.cols != s->H || M->lm_head.format != s->fmt || M->lm_head.order != VQ_ROWS_PLAIN)
        return fail(VQ_ERR_ARG, "lm_head: shape, format or order inconsistent with the layers");
    return VQ_OK;
}

// The split of every stage kind of a pass with K columns.
struct PassPlan {
    KindPlan kp[5];
    int nsp, pbytes, ring_off, xcap;
    size_t parts_floats, counters;
};

int pass_plan(const Shapes& s, int K, int nwg, PassPlan* pp) {
    lds_plan(K, &pp->nsp, &pp->pbytes, &pp->ring_off, &pp->xcap);
    const int rows[5] = {s.H + 2 * s.KV, s.H, 2 * s.FF, s.H, s.V};
    const int cols[5] = {s.H, s.H, s.H, s.FF, s.H};
    pp->parts_floats = 0;
    pp->counters = 0;
    for (int k = 0; k < 5; ++k) {
        const int tiles = (rows[k] + TILE_ROWS - 1) / TILE_ROWS;
        if (!make_plan(pp->kp[k], s.fmt, K, rows[k], cols[k], tiles, nwg, pp->xcap))
            return fail(VQ_ERR_UNSUPPORTED, "stage kind %d (%dx%d) cannot be split over %d workgroups at K %d", k,
                        rows[k], cols[k], nwg, K);
        // rho of stage kind k normalises the previous stage's output; the first stage's is set per stage
        pp->kp[k].n_in = k == SK_DOWN ? s.FF : s.H;
        pp->kp[k].stats = k == SK_LM ? 0 : 1;
        pp->parts_floats = std::max(pp->parts_floats, plan_parts_floats(pp->kp[k], pp->pbytes, nwg, 4 * FLOW_MAX_LAYERS + 1));
        pp->counters = std::max(pp->counters, plan_counters(pp->kp[k]));
    }
    return VQ_OK;
}

// Workspace of a decode pass.  Every buffer a later stage reads is written once per pass
// at its own 256-byte aligned place: per layer and stage the fp16 input (x) and the fp32
// output (y); the lm_head's input; per stage the per-workgroup sums of squares; the
// split-tile partial sums; then, zeroed at the start of every pass, the split-tile
// counters, the completion counters and the error word.
struct DecodeLayout {
    size_t off_x[4], off_y[4];
    size_t layer_bytes;
    size_t off_fx;
    size_t off_stats, stats_stride;
    size_t off_parts;
    size_t off_cnt;
    size_t off_sync;
    size_t zero_words;         // from off_cnt: counters, completion counters, error word
    int sync_words;
    size_t total;
};

DecodeLayout decode_layout(const Shapes& s, int K, const PassPlan& pp) {
    DecodeLayout d{};
    size_t p = 0;
    const int rows[4] = {s.H + 2 * s.KV, s.H, 2 * s.FF, s.H};
    const int cols[4] = {s.H, s.H, s.H, s.FF};
    for (int j = 0; j < 4; ++j) {
        d.off_x[j] = p;
        p += align_up((size_t)K * cols[j] * 2, 256);
        d.off_y[j] = p;
        p += align_up((size_t)K * rows[j] * 4, 256);
    }
    d.layer_bytes = p;
    p = d.layer_bytes * s.L;
    d.off_fx = p;
    p += align_up((size_t)K * s.H * 2, 256);
    d.off_stats = p;
    d.stats_stride = align_up((size_t)FLOW_MAX_WG * K, 64);
    p += d.stats_stride * 4 * (size_t)(4 * s.L);
    d.off_parts = p;
    p += align_up(pp.parts_floats * 4, 256);
    d.off_cnt = p;
    p += align_up(pp.counters * 4, 256);
    d.off_sync = p;
    d.sync_words = (4 * s.L + 1) * DONE_WORDS + DONE_STRIDE;
    p += align_up((size_t)d.sync_words * 4, 256);
    d.zero_words = (p - d.off_cnt) / 4;
    d.total = p;
    return d;
}

int* err_word(const DecodeLayout& d, char* ws) {
    return (int*)(ws + d.off_sync) + (d.sync_words - DONE_STRIDE);
}

void fill_common(FlowArgs& A, const Shapes& s, const DecodeLayout& d, const PassPlan& pp, int K, int nwg,
                 const vq_model* M, const void* x0, float* logits, char* ws) {
    A = FlowArgs{};
    A.fmt = s.fmt;
    A.K = K;
    A.H = s.H; A.KV = s.KV; A.FF = s.FF; A.V = s.V; A.L = s.L;
    A.nwg = nwg;
    A.nsp = pp.nsp;
    A.pbytes = pp.pbytes;
    A.ring_off = pp.ring_off;
    A.xoff1 = (pp.xcap / 2) & ~15;
    A.x0 = (const uint16_t*)x0;
    A.out = logits;
    A.ws = ws;
    A.layer_bytes = d.layer_bytes;
    for (int j = 0; j < 4; ++j) {
        A.off_x[j] = d.off_x[j];
        A.off_y[j] = d.off_y[j];
    }
    A.off_fx = d.off_fx;
    A.off_stats = d.off_stats;
    A.stats_stride = d.stats_stride;
    A.parts = (float*)(ws + d.off_parts);
    A.cnt = (unsigned*)(ws + d.off_cnt);
    A.done = (unsigned*)(ws + d.off_sync);
    A.err = err_word(d, ws);
    for (int k = 0; k < 5; ++k) A.kp[k] = pp.kp[k];
    A.lm = (const uint8_t*)M->lm_head.data;
}

void fill_layers(FlowArgs& A, const vq_model* M, int l0) {
    A.l0 = l0;
    for (int i = 0; i < FLOW_MAX_LAYERS && l0 + i < M->n_layers; ++i) {
        const vq_layer& y = M->layers[l0 + i];
        A.w[i][0] = (const uint8_t*)y.qkv.data;
        A.w[i][1] = (const uint8_t*)y.o.data;
        A.w[i][2] = (const uint8_t*)y.gu.data;
        A.w[i][3] = (const uint8_t*)y.down.data;
    }
}

// Workspace of a linear map: split-tile partials, then the counters and an error word
// (zeroed by every call).
struct LinearLayout {
    KindPlan kp;
    int nsp, pbytes, ring_off, xcap;
    size_t off_cnt, zero_words, total;
};

int linear_layout(const vq_tiled* W, int K, int nwg, LinearLayout* L) {
    lds_plan(K, &L->nsp, &L->pbytes, &L->ring_off, &L->xcap);
    if (!make_plan(L->kp, W->format, K, W->rows, W->cols, (W->rows + TILE_ROWS - 1) / TILE_ROWS, nwg, L->xcap))
        return fail(VQ_ERR_UNSUPPORTED, "a %dx%d matrix cannot be split over %d workgroups at K %d", W->rows, W->cols,
                    nwg, K);
    L->kp.n_in = 0;
    L->kp.stats = 0;
    L->off_cnt = align_up(plan_parts_floats(L->kp, L->pbytes, L->kp.nwe, 1) * 4, 256);
    const size_t words = plan_counters(L->kp) + DONE_STRIDE;
    L->zero_words = words;
    L->total = L->off_cnt + align_up(words * 4, 256);
    return VQ_OK;
}

// ---------------------------------------------------------------- work-list cache

// The compute waves' work lists depend only on the shapes, K, the grid and the launch
// split.  They are built on the host at the first call with a shape and kept in device
// memory, one table per device and shape, until the process ends.
struct StepKey {
    int dev, fmt, K, nwg, staged, linear;
    int H, KV, FF, V, L;       // decode shapes (a linear map: rows in V, cols in H)
    bool operator<(const StepKey& o) const { return memcmp(this, &o, sizeof *this) < 0; }
};
struct StepDev {
    uint32_t* buf = nullptr;            // the entries, then every launch's start indices
    std::vector<size_t> launch_start;   // per launch: its start indices, in words from buf
};
std::mutex g_steps_mu;
std::map<StepKey, StepDev>* g_steps = new std::map<StepKey, StepDev>();   // never freed

int get_steps(const StepKey& key, const KindPlan kp[6], const std::vector<std::pair<int, int>>& launches, int L,
              bool linear, int nwg, int xoff1, hipStream_t st, const StepDev** out) {
    std::lock_guard<std::mutex> g(g_steps_mu);
    auto it = g_steps->find(key);
    if (it != g_steps->end()) {
        *out = &it->second;
        return VQ_OK;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
        return fail(VQ_ERR_UNSUPPORTED, "the first call with these shapes builds the work lists (an allocation "
                                        "and a copy) and cannot be captured: call it once before capturing");
    StepTable T;
    std::vector<size_t> hdr;
    for (const auto& l : launches) {
        hdr.push_back(T.start.size());
        if (!build_steps(T, kp, l.first, l.second, L, linear, nwg, xoff1, key.K <= 8))
            return fail(VQ_ERR_UNSUPPORTED, "work lists of stages %d..%d do not fit their encoding", l.first,
                        l.second - 1);
    }
    const size_t ne = T.ent.size(), ns = T.start.size();
    std::vector<uint32_t> h(ne + ns);
    memcpy(h.data(), T.ent.data(), ne * 4);
    memcpy(h.data() + ne, T.start.data(), ns * 4);
    void* d = nullptr;
    hipError_t e = hipMalloc(&d, h.size() * 4);
    if (e != hipSuccess) return hip_fail(e, "work list allocation");
    e = hipMemcpyAsync(d, h.data(), h.size() * 4, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
        (void)hipFree(d);
        return hip_fail(e, "work list upload");
    }
    StepDev sd;
    sd.buf = (uint32_t*)d;
    for (size_t o : hdr) sd.launch_start.push_back(ne + o);
    *out = &g_steps->emplace(key, std::move(sd)).first->second;
    return VQ_OK;
}

int current_device() {
    int dev = 0;
    (void)hipGetDevice(&dev);
    return dev;
}

}  // namespace
}  // namespace vq

using namespace vq;

extern "C" {

int32_t vq_abi_version(void) { return VQ_ABI_VERSION; }

const char* vq_last_error(void) { return vq::g_err; }

const char* vq_status_string(int32_t status) {
    switch (status) {
        case VQ_OK: return "ok";
        case VQ_ERR_ARG: return "invalid argument";
        case VQ_ERR_UNSUPPORTED: return "unsupported configuration";
        case VQ_ERR_WORKSPACE: return "workspace missing or too small";
        case VQ_ERR_HIP: return "HIP runtime error";
        case VQ_ERR_HOST: return "host allocation failed";
        default: return "unknown status";
    }
}

size_t vq_workspace_bytes(int32_t op, const void* desc, int32_t K) {
    if (!desc) return 0;
    if (K < 1 || K > VQ_MAX_K) return 0;
    if (op == VQ_OP_LINEAR) {
        const vq_tiled* W = (const vq_tiled*)desc;
        if (check_tiled(W, "W")) return 0;
        if (W->rows == 0) return 256;
        LinearLayout L;
        if (linear_layout(W, K, flow_grid(), &L)) return 0;
        return L.total;
    }
    if (op == VQ_OP_LINEAR_MX) {
        const vq_matrix* W = (const vq_matrix*)desc;
        if (check_matrix(W, "W") || W->format != VQ_FMT_MXFP4 || W->cols % 128) return 0;
        return mx_workspace_bytes(W->rows, W->cols, K, MX_WG_PER_CU * flow_grid());
    }
    if (op == VQ_OP_ATTENTION) {
        const vq_attention* C = (const vq_attention*)desc;
        if (check_attention(C, K)) return 0;
        return attn_workspace_bytes(C->n_kv_heads, C->n_q_heads, C->length, K, flow_grid());
    }
    if (op == VQ_OP_ACCEPT) {
        const vq_accept_desc* d = (const vq_accept_desc*)desc;
        if (d->W < 0 || d->K < 1 || d->K > VQ_MAX_K) return 0;
        return accept_ws_bytes(d);
    }
    if (op == VQ_OP_DECODE) {
        Shapes s;
        PassPlan pp;
        if (check_model((const vq_model*)desc, &s) || pass_plan(s, K, flow_grid(), &pp)) return 0;
        return decode_layout(s, K, pp).total;
    }
    return 0;
}

size_t vq_tiled_bytes(int32_t format, int32_t rows, int32_t cols) {
    if (format < VQ_FMT_Q4 || format > VQ_FMT_Q4_K || rows < 0 || cols <= 0 || cols % 32) return 0;
    if (format == VQ_FMT_Q4_K && cols % 256) return 0;
    return tiled_bytes(format, rows, cols);
}

int vq_tile(const vq_matrix* src, const vq_tiled* dst, int32_t row0, void* stream) {
    g_err[0] = 0;
    int rc = check_matrix(src, "src");
    if (rc) return rc;
    rc = check_tiled(dst, "dst");
    if (rc) return rc;
    if (src->format != dst->format || src->cols != dst->cols)
        return fail(VQ_ERR_ARG, "src and dst differ in format or cols");
    if (row0 < 0 || (long)row0 + src->rows > dst->rows)
        return fail(VQ_ERR_ARG, "rows [%d, %d) outside dst (%d rows)", row0, row0 + src->rows, dst->rows);
    if (dst->order == VQ_ROWS_PAIR8) {
        const int half = dst->rows / 2;
        if (!((row0 == 0 || row0 == half) && src->rows == half))
            return fail(VQ_ERR_ARG, "a VQ_ROWS_PAIR8 matrix is filled one half (%d rows) at a time", half);
    } else if (row0 % TILE_ROWS) {
        return fail(VQ_ERR_ARG, "row0 %d is not a multiple of %d", row0, TILE_ROWS);
    }
    if (src->rows == 0) return VQ_OK;
    hipError_t e = launch_tile(*src, (uint8_t*)dst->data, dst->rows, dst->order, row0, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "tile launch");
    return VQ_OK;
}

}  // extern "C"

namespace vq {
namespace {

// Argument checks shared by the linear entry points; fills the plan.
int linear_check(const vq_tiled* W, const void* x_f16, int32_t K, void* y, int32_t y_dtype, LinearLayout* L,
                 bool* empty) {
    *empty = false;
    int rc = check_tiled(W, "W");
    if (rc) return rc;
    if (W->order != VQ_ROWS_PLAIN) return fail(VQ_ERR_ARG, "W must be in VQ_ROWS_PLAIN order");
    if (K < 1 || K > VQ_MAX_K) return fail(VQ_ERR_ARG, "K %d outside 1..%d", K, VQ_MAX_K);
    if (y_dtype != VQ_DTYPE_F32 && y_dtype != VQ_DTYPE_F16) return fail(VQ_ERR_ARG, "unknown y_dtype %d", y_dtype);
    if (W->rows == 0) {
        *empty = true;
        return VQ_OK;
    }
    if (!x_f16 || !y) return fail(VQ_ERR_ARG, "NULL x or y");
    if (!aligned(x_f16, 16)) return fail(VQ_ERR_ARG, "x must be 16-byte aligned");
    if (!aligned(y, y_dtype == VQ_DTYPE_F32 ? 4 : 2)) return fail(VQ_ERR_ARG, "y is misaligned");
    return linear_layout(W, K, flow_grid(), L);
}

// The launch of a linear map with its scratch memory: split-tile parts, counters (zeroed
// here, with a kernel), error word, and the work lists.
int linear_launch(const vq_tiled* W, const void* x_f16, int32_t K, void* y, int32_t y_dtype, const LinearLayout& L,
                  float* parts, unsigned* cnt, const uint32_t* steps, const uint32_t* step_start, hipStream_t st) {
    FlowArgs A{};
    A.fmt = W->format;
    A.K = K;
    A.V = W->rows;
    A.H = W->cols;
    A.L = 0;
    A.linear = 1;
    A.y_dtype = y_dtype;
    A.s_begin = 0;
    A.s_end = 1;
    A.nwg = L.kp.nwe;
    A.nsp = L.nsp;
    A.pbytes = L.pbytes;
    A.ring_off = L.ring_off;
    A.xoff1 = (L.xcap / 2) & ~15;
    A.x0 = (const uint16_t*)x_f16;
    A.out = y;
    A.parts = parts;
    A.cnt = cnt;
    A.err = (int*)cnt + (L.zero_words - 1);
    A.kp[SK_LIN] = L.kp;
    A.lm = (const uint8_t*)W->data;
    A.steps = steps;
    A.step_start = step_start;
    hipError_t e = launch_zero_u32(cnt, L.zero_words, st);
    if (e != hipSuccess) return hip_fail(e, "counter reset launch");
    e = launch_flow(A, st);
    if (e != hipSuccess) return hip_fail(e, "linear launch");
    return VQ_OK;
}

// ------------------------------------------------ the entry point that allocates nothing

// Scratch memory of vq_verify_linear_noalloc in the library's own device data: the work
// lists, the split-tile parts, and the counters with the error word.  Each device that
// runs the library holds one copy until the process ends; every call on a device uses
// it, so calls that overlap on one device race.
constexpr size_t NA_TABLE_BYTES = 4u << 20;
constexpr size_t NA_PARTS_BYTES = 512u << 10;
constexpr size_t NA_CNT_WORDS = 4096;
constexpr size_t NA_BYTES = NA_TABLE_BYTES + NA_PARTS_BYTES + 4 * NA_CNT_WORDS;
static __device__ __align__(256) uint8_t scratch[NA_BYTES];

constexpr int NA_MAX_DEV = 64;
struct NoAllocDev {
    uint8_t* ptr = nullptr;       // device address of scratch on this device
    bool has_key = false;
    StepKey key{};                // shape whose work lists scratch holds
};
std::mutex g_na_mu;
NoAllocDev g_na[NA_MAX_DEV];
// host image of the work lists (static: building them allocates nothing either)
uint32_t g_na_host[NA_TABLE_BYTES / 4];

}  // namespace
}  // namespace vq

extern "C" {

int vq_verify_linear(const vq_tiled* W, const void* x_f16, int32_t K, void* y, int32_t y_dtype, void* ws,
                     size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    LinearLayout L;
    bool empty = false;
    int rc = linear_check(W, x_f16, K, y, y_dtype, &L, &empty);
    if (rc || empty) return rc;
    if (!ws || ws_bytes < L.total || !aligned(ws, 256))
        return fail(VQ_ERR_WORKSPACE, "workspace needs %zu bytes (256-byte aligned), got %zu", L.total, ws_bytes);
    char* base = (char*)ws;
    hipStream_t st = (hipStream_t)stream;
    FlowArgs A{};
    A.kp[SK_LIN] = L.kp;
    const StepKey key{current_device(), W->format, K, L.kp.nwe, 0, 1, W->cols, 0, 0, W->rows, 0};
    const StepDev* sd = nullptr;
    rc = get_steps(key, A.kp, {{0, 1}}, 0, true, L.kp.nwe, (L.xcap / 2) & ~15, st, &sd);
    if (rc) return rc;
    return linear_launch(W, x_f16, K, y, y_dtype, L, (float*)base, (unsigned*)(base + L.off_cnt), sd->buf,
                         sd->buf + sd->launch_start[0], st);
}

int vq_verify_linear_noalloc(const vq_tiled* W, const void* x_f16, int32_t K, void* y, int32_t y_dtype,
                             void* stream) {
    g_err[0] = 0;
    LinearLayout L;
    bool empty = false;
    int rc = linear_check(W, x_f16, K, y, y_dtype, &L, &empty);
    if (rc || empty) return rc;
    const size_t parts_bytes = plan_parts_floats(L.kp, L.pbytes, L.kp.nwe, 1) * 4;
    if (L.kp.nwin != 1 || parts_bytes > NA_PARTS_BYTES || L.zero_words > NA_CNT_WORDS)
        return fail(VQ_ERR_UNSUPPORTED,
                    "vq_verify_linear_noalloc: a %dx%d matrix at K %d needs column windows or more than its "
                    "%zu bytes of partial sums; use vq_verify_linear", W->rows, W->cols, K, NA_PARTS_BYTES);
    const int dev = current_device();
    if (dev < 0 || dev >= NA_MAX_DEV) return fail(VQ_ERR_UNSUPPORTED, "device %d beyond %d", dev, NA_MAX_DEV);
    hipStream_t st = (hipStream_t)stream;
    std::lock_guard<std::mutex> g(g_na_mu);
    NoAllocDev& D = g_na[dev];
    if (!D.ptr) {
        // the array's device address on this (current) device; the host-side name of the
        // array is not a device address
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(e, "scratch symbol address");
        D.ptr = (uint8_t*)p;
    }
    uint32_t* const tab = (uint32_t*)D.ptr;
    const StepKey key{dev, W->format, K, L.kp.nwe, 0, 1, W->cols, 0, 0, W->rows, 0};
    const size_t nstart = (size_t)L.kp.nwe * FLOW_NCW;
    const size_t words = NA_TABLE_BYTES / 4;
    if (!D.has_key || memcmp(&D.key, &key, sizeof key) != 0) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
            return fail(VQ_ERR_UNSUPPORTED, "vq_verify_linear_noalloc: the first call with a shape copies its work "
                                            "lists and cannot be captured: call it once before capturing");
        KindPlan kp[6] = {};
        kp[SK_LIN] = L.kp;
        // start indices at the front, entries after them (a multiple of 8 words: entries stay
        // 32-byte aligned)
        const size_t soff = (nstart + 7) / 8 * 8;
        if (soff >= words) return fail(VQ_ERR_UNSUPPORTED, "vq_verify_linear_noalloc: grid too large");
        FixedStepTable T{g_na_host + soff, words - soff, 0, g_na_host, nstart, 0, false};
        if (!build_steps(T, kp, 0, 1, 0, true, L.kp.nwe, (L.xcap / 2) & ~15, K <= 8))
            return fail(VQ_ERR_UNSUPPORTED,
                        "vq_verify_linear_noalloc: the work lists of a %dx%d matrix exceed its %zu bytes; use "
                        "vq_verify_linear", W->rows, W->cols, NA_TABLE_BYTES);
        for (size_t i = 0; i < nstart; ++i) g_na_host[i] += (uint32_t)(soff / 2);   // pairs from tab
        D.has_key = false;
        hipError_t e = hipMemcpyAsync(tab, g_na_host, (soff + T.n_ent()) * 4, hipMemcpyHostToDevice, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) return hip_fail(e, "work list copy");
        D.key = key;
        D.has_key = true;
    }
    uint8_t* const parts = D.ptr + NA_TABLE_BYTES;
    unsigned* const cnt = (unsigned*)(parts + NA_PARTS_BYTES);
    return linear_launch(W, x_f16, K, y, y_dtype, L, (float*)parts, cnt, tab, tab, st);
}

int vq_verify_linear_mx(const vq_matrix* W, const void* x_f16, int32_t K, float* y, void* ws, size_t ws_bytes,
                        void* stream) {
    g_err[0] = 0;
    int rc = check_matrix(W, "W");
    if (rc) return rc;
    if (W->format != VQ_FMT_MXFP4) return fail(VQ_ERR_ARG, "vq_verify_linear_mx takes MXFP4 weights");
    if (W->cols % 128) return fail(VQ_ERR_ARG, "vq_verify_linear_mx needs cols a multiple of 128, got %d", W->cols);
    if (K < 1 || K > VQ_MAX_K) return fail(VQ_ERR_ARG, "K %d outside 1..%d", K, VQ_MAX_K);
    if (W->rows == 0) return VQ_OK;
    if (!x_f16 || !y) return fail(VQ_ERR_ARG, "NULL x or y");
    if (!aligned(x_f16, 16) || !aligned(y, 4)) return fail(VQ_ERR_ARG, "x must be 16-byte and y 4-byte aligned");
    const int nwg = MX_WG_PER_CU * flow_grid();
    const size_t need = mx_workspace_bytes(W->rows, W->cols, K, nwg);
    if (!ws || ws_bytes < need || !aligned(ws, 256))
        return fail(VQ_ERR_WORKSPACE, "workspace needs %zu bytes (256-byte aligned), got %zu", need, ws_bytes);
    hipError_t e = launch_mx_linear(*W, x_f16, K, y, (uint8_t*)ws, nwg, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "mx linear launch");
    return VQ_OK;
}

int vq_verify_attention(const vq_attention* desc, const void* q_f16, int32_t K, float* out, void* ws,
                        size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    int rc = check_attention(desc, K);
    if (rc) return rc;
    if (!q_f16 || !out) return fail(VQ_ERR_ARG, "NULL q or out");
    if (!aligned(q_f16, 2) || !aligned(out, 4)) return fail(VQ_ERR_ARG, "q must be 2-byte and out 4-byte aligned");
    const int nwg = flow_grid();
    const size_t need = attn_workspace_bytes(desc->n_kv_heads, desc->n_q_heads, desc->length, K, nwg);
    if (!ws || ws_bytes < need || !aligned(ws, 256))
        return fail(VQ_ERR_WORKSPACE, "workspace needs %zu bytes (256-byte aligned), got %zu", need, ws_bytes);
    hipError_t e = launch_attention(*desc, q_f16, K, out, (uint8_t*)ws, nwg, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    return VQ_OK;
}

int vq_verify_accept(const vq_accept_desc* d, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    if (!d) return fail(VQ_ERR_ARG, "NULL descriptor");
    if (d->top_k < 0) return fail(VQ_ERR_ARG, "top_k %d < 0", d->top_k);
    if (d->mode != VQ_MODE_GREEDY && d->mode != VQ_MODE_SAMPLE) return fail(VQ_ERR_ARG, "unknown mode %d", d->mode);
    if (d->draft_mode < VQ_DRAFT_GIVEN || d->draft_mode > VQ_DRAFT_AGREE)
        return fail(VQ_ERR_ARG, "unknown draft_mode %d", d->draft_mode);
    if (d->W < 0) return fail(VQ_ERR_ARG, "W %d < 0", d->W);
    if (d->K < 1 || d->K > VQ_MAX_K) return fail(VQ_ERR_ARG, "K %d outside 1..%d", d->K, VQ_MAX_K);
    if (d->V < 1 || d->V > (1 << 19)) return fail(VQ_ERR_ARG, "V %d outside 1..524288", d->V);
    if (d->draft_mode == VQ_DRAFT_AGREE && d->V < 2) return fail(VQ_ERR_ARG, "VQ_DRAFT_AGREE needs V >= 2");
    const bool needs_warp = d->mode == VQ_MODE_SAMPLE || d->draft_mode == VQ_DRAFT_Q_SAMPLE;
    if (needs_warp) {
        if (!(d->temperature > 0.f) || !isfinite(d->temperature))
            return fail(VQ_ERR_ARG, "temperature must be finite and > 0 for sampling (T = 0 means greedy)");
        if (!(d->top_p > 0.f && d->top_p <= 1.f)) return fail(VQ_ERR_ARG, "top_p must be in (0, 1]");
        if (!(d->min_p >= 0.f && d->min_p < 1.f)) return fail(VQ_ERR_ARG, "min_p must be in [0, 1)");
    }
    if (d->draft_mode == VQ_DRAFT_AGREE && !(d->alpha >= 0.f && d->alpha <= 1.f))
        return fail(VQ_ERR_ARG, "alpha must be in [0, 1]");
    if (d->W == 0) return VQ_OK;
    const bool drafter = d->mode == VQ_MODE_SAMPLE || d->draft_mode == VQ_DRAFT_Q_ARGMAX ||
                         d->draft_mode == VQ_DRAFT_Q_SAMPLE;
    if (!d->target_logits || !d->n_accepted || !d->tokens || !d->status)
        return fail(VQ_ERR_ARG, "NULL logits or output pointer");
    if (d->K > 1 && drafter && !d->draft_logits) return fail(VQ_ERR_ARG, "draft_logits required by this mode");
    if (d->K > 1 && !d->draft_tokens) return fail(VQ_ERR_ARG, "draft_tokens required when K > 1");
    if (!aligned(d->target_logits, 4) || (d->draft_logits && !aligned(d->draft_logits, 4)))
        return fail(VQ_ERR_ARG, "logits must be 4-byte aligned");
    const size_t need = accept_ws_bytes(d);
    if (!ws || ws_bytes < need || !aligned(ws, 256))
        return fail(VQ_ERR_WORKSPACE, "workspace needs %zu bytes (256-byte aligned), got %zu", need, ws_bytes);
    hipError_t e = launch_accept(d, ws, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "accept launch");
    return VQ_OK;
}

int vq_decode_stage_ptr(const vq_model* M, int32_t K, void* ws, int32_t stage, void** in_f16,
                        void** out_f32) {
    g_err[0] = 0;
    Shapes s;
    int rc = check_model(M, &s);
    if (rc) return rc;
    if (K < 1 || K > VQ_MAX_K) return fail(VQ_ERR_ARG, "K %d outside 1..%d", K, VQ_MAX_K);
    if (stage < 0 || stage > 4 * s.L) return fail(VQ_ERR_ARG, "stage %d outside 0..%d", stage, 4 * s.L);
    if (!ws || !in_f16 || !out_f32) return fail(VQ_ERR_ARG, "NULL pointer");
    PassPlan pp;
    rc = pass_plan(s, K, flow_grid(), &pp);
    if (rc) return rc;
    const DecodeLayout d = decode_layout(s, K, pp);
    char* base = (char*)ws;
    if (stage == 4 * s.L) {
        *in_f16 = base + d.off_fx;
        *out_f32 = nullptr;
    } else {
        const size_t lb = (size_t)(stage / 4) * d.layer_bytes;
        *in_f16 = base + lb + d.off_x[stage % 4];
        *out_f32 = base + lb + d.off_y[stage % 4];
    }
    return VQ_OK;
}

int vq_decode_error_word(const vq_model* M, int32_t K, void* ws, int32_t** word) {
    g_err[0] = 0;
    Shapes s;
    int rc = check_model(M, &s);
    if (rc) return rc;
    if (K < 1 || K > VQ_MAX_K) return fail(VQ_ERR_ARG, "K %d outside 1..%d", K, VQ_MAX_K);
    if (!ws || !word) return fail(VQ_ERR_ARG, "NULL pointer");
    PassPlan pp;
    rc = pass_plan(s, K, flow_grid(), &pp);
    if (rc) return rc;
    *word = err_word(decode_layout(s, K, pp), (char*)ws);
    return VQ_OK;
}

static int decode_impl(const vq_model* M, const void* x0_f16, int32_t K, float* logits, int32_t launch,
                       void* ws, size_t ws_bytes, void* stream, void* const* events, int32_t n_events,
                       int32_t* n_launches) {
    g_err[0] = 0;
    Shapes s;
    int rc = check_model(M, &s);
    if (rc) return rc;
    if (K < 1 || K > VQ_MAX_K) return fail(VQ_ERR_ARG, "K %d outside 1..%d", K, VQ_MAX_K);
    if (launch != VQ_LAUNCH_AUTO && launch != VQ_LAUNCH_STAGED && launch != VQ_LAUNCH_PERSISTENT)
        return fail(VQ_ERR_ARG, "unknown launch mode %d", launch);
    if (!x0_f16 || !logits) return fail(VQ_ERR_ARG, "NULL x0 or logits");
    if (!aligned(x0_f16, 16) || !aligned(logits, 4)) return fail(VQ_ERR_ARG, "x0 or logits misaligned");
    const int nwg = flow_grid();
    PassPlan pp;
    rc = pass_plan(s, K, nwg, &pp);
    if (rc) return rc;
    const DecodeLayout d = decode_layout(s, K, pp);
    if (!ws || ws_bytes < d.total || !aligned(ws, 256))
        return fail(VQ_ERR_WORKSPACE, "workspace needs %zu bytes (256-byte aligned), got %zu", d.total, ws_bytes);
    hipStream_t st = (hipStream_t)stream;
    char* base = (char*)ws;
    FlowArgs A;
    fill_common(A, s, d, pp, K, nwg, M, x0_f16, logits, base);
    const int S = 4 * s.L + 1;
    const bool staged = launch == VQ_LAUNCH_STAGED;
    std::vector<std::pair<int, int>> launches;
    for (int s0 = 0; s0 < S;) {
        int s1;
        if (staged) {
            s1 = s0 + 1;
        } else {
            // the stages of FLOW_MAX_LAYERS layers (the last launch also runs the lm_head)
            const int l0 = s0 / 4;
            s1 = std::min(S, 4 * (l0 + FLOW_MAX_LAYERS));
            if (s1 == 4 * s.L) s1 = S;
        }
        launches.emplace_back(s0, s1);
        s0 = s1;
    }
    const StepKey key{current_device(), s.fmt, K, nwg, staged ? 1 : 0, 0, s.H, s.KV, s.FF, s.V, s.L};
    const StepDev* sd = nullptr;
    rc = get_steps(key, A.kp, launches, s.L, false, nwg, A.xoff1, st, &sd);
    if (rc) return rc;
    A.steps = sd->buf;
    hipError_t e = launch_zero_u32((unsigned*)(base + d.off_cnt), d.zero_words, st);
    if (e != hipSuccess) return hip_fail(e, "sync reset launch");
    int nl = 0;
    for (const auto& l : launches) {
        const int s0 = l.first, s1 = l.second;
        fill_layers(A, M, std::min(s0 / 4, s.L - 1));
        A.s_begin = s0;
        A.s_end = s1;
        A.step_start = sd->buf + sd->launch_start[nl];
        if (events && 2 * nl + 1 < n_events) {
            e = hipEventRecord((hipEvent_t)events[2 * nl], st);
            if (e != hipSuccess) return hip_fail(e, "event record");
        }
        e = launch_flow(A, st);
        if (e != hipSuccess) return hip_fail(e, "pass launch");
        if (events && 2 * nl + 1 < n_events) {
            e = hipEventRecord((hipEvent_t)events[2 * nl + 1], st);
            if (e != hipSuccess) return hip_fail(e, "event record");
        }
        ++nl;
    }
    if (n_launches) *n_launches = nl;
    return VQ_OK;
}

int vq_decode_pass(const vq_model* M, const void* x0_f16, int32_t K, float* logits, void* ws, size_t ws_bytes,
                   void* stream) {
    return decode_impl(M, x0_f16, K, logits, VQ_LAUNCH_AUTO, ws, ws_bytes, stream, nullptr, 0, nullptr);
}

int vq_decode_pass_timed(const vq_model* M, const void* x0_f16, int32_t K, float* logits, int32_t launch,
                         void* ws, size_t ws_bytes, void* stream, void* const* events, int32_t n_events,
                         int32_t* n_launches) {
    if (!events || n_events < 2) return fail(VQ_ERR_ARG, "events must hold at least one (begin, end) pair");
    for (int i = 0; i < n_events; ++i)
        if (!events[i]) return fail(VQ_ERR_ARG, "event %d is NULL", i);
    return decode_impl(M, x0_f16, K, logits, launch, ws, ws_bytes, stream, events, n_events, n_launches);
}

}  // extern "C"
