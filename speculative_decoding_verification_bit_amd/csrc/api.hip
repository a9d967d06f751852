// C ABI of libvq: argument validation, the decode workspace layout, and the launch
// sequence of a pass.  Every check runs on the host before anything is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "vq_internal.h"

namespace vq {
namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(VQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_matrix(const vq_matrix* W, const char* name) {
    if (!W) return fail(VQ_ERR_ARG, "%s: NULL matrix descriptor", name);
    if (W->format < VQ_FMT_Q4 || W->format > VQ_FMT_MXFP4)
        return fail(VQ_ERR_ARG, "%s: unknown format %d", name, W->format);
    if (W->reserved != 0) return fail(VQ_ERR_ARG, "%s: reserved field must be 0", name);
    if (W->rows < 0) return fail(VQ_ERR_ARG, "%s: rows %d < 0", name, W->rows);
    if (W->cols <= 0 || W->cols % 32)
        return fail(VQ_ERR_ARG, "%s: cols %d is not a positive multiple of 32", name, W->cols);
    if (W->rows == 0) return VQ_OK;
    if (!W->qs || !W->scales) return fail(VQ_ERR_ARG, "%s: NULL qs or scales", name);
    if ((W->format == VQ_FMT_Q4_MIN) != (W->mins != nullptr))
        return fail(VQ_ERR_ARG, "%s: mins must be given exactly for VQ_FMT_Q4_MIN", name);
    if (!aligned(W->qs, 16) || !aligned(W->scales, 16) || (W->mins && !aligned(W->mins, 16)))
        return fail(VQ_ERR_ARG, "%s: qs, scales and mins must be 16-byte aligned", name);
    return VQ_OK;
}

// ---------------------------------------------------------------- decode layout

struct Shapes {
    int H, KV, FF, V, L, fmt;
};

int check_model(const vq_model* M, Shapes* s) {
    if (!M) return fail(VQ_ERR_ARG, "NULL model");
    if (M->n_layers < 1 || !M->layers) return fail(VQ_ERR_ARG, "model needs n_layers >= 1 and layers");
    if (M->reserved != 0) return fail(VQ_ERR_ARG, "model reserved field must be 0");
    const vq_layer& l0 = M->layers[0];
    s->H = l0.q.cols;
    s->KV = l0.k.rows;
    s->FF = l0.gate.rows;
    s->V = M->lm_head.rows;
    s->L = M->n_layers;
    s->fmt = l0.q.format;
    if (s->H % 64 || s->KV % 64 || s->FF % 64 || s->H <= 0 || s->KV <= 0 || s->FF <= 0)
        return fail(VQ_ERR_UNSUPPORTED, "decode pass needs hidden, kv and ffn sizes that are multiples of 64");
    if (s->V < 1) return fail(VQ_ERR_ARG, "lm_head needs rows >= 1");
    for (int l = 0; l < M->n_layers; ++l) {
        const vq_layer& y = M->layers[l];
        const vq_matrix* ms[7] = {&y.q, &y.k, &y.v, &y.o, &y.gate, &y.up, &y.down};
        const int rr[7] = {s->H, s->KV, s->KV, s->H, s->FF, s->FF, s->H};
        const int cc[7] = {s->H, s->H, s->H, s->H, s->H, s->H, s->FF};
        static const char* nm[7] = {"q", "k", "v", "o", "gate", "up", "down"};
        for (int i = 0; i < 7; ++i) {
            char buf[48];
            snprintf(buf, sizeof buf, "layer %d %s", l, nm[i]);
            int rc = check_matrix(ms[i], buf);
            if (rc) return rc;
            if (ms[i]->rows != rr[i] || ms[i]->cols != cc[i] || ms[i]->format != s->fmt)
                return fail(VQ_ERR_ARG, "%s: shape %dx%d fmt %d, expected %dx%d fmt %d", buf, ms[i]->rows,
                            ms[i]->cols, ms[i]->format, rr[i], cc[i], s->fmt);
        }
    }
    int rc = check_matrix(&M->lm_head, "lm_head");
    if (rc) return rc;
    if (M->lm_head.cols != s->H || M->lm_head.format != s->fmt)
        return fail(VQ_ERR_ARG, "lm_head: shape or format inconsistent with the layers");
    return VQ_OK;
}

// Workspace of a decode pass.  Every buffer a later stage reads is written once per pass
// at its own 256-byte aligned place: per layer and stage the fp16 input in natural order
// (xn, kept for inspection), the same input in the MFMA pair order (xp, what the next
// stage reads for the Q4 formats) and the fp32 output (y); the lm_head's input; per stage
// the per-workgroup sums of squares; the completion counters and the error word.
struct DecodeLayout {
    size_t off_xn[4], off_xp[4], off_y[4];
    size_t layer_bytes;
    size_t off_fxn, off_fxp;
    size_t off_stats, stats_stride;
    size_t off_sync;
    int sync_words;            // completion counters, then the error word
    size_t total;
};

DecodeLayout decode_layout(const Shapes& s, int K) {
    DecodeLayout d{};
    size_t p = 0;
    const int rows[4] = {s.H + 2 * s.KV, s.H, 2 * s.FF, s.H};
    const int cols[4] = {s.H, s.H, s.H, s.FF};
    for (int j = 0; j < 4; ++j) {
        d.off_xn[j] = p;
        p += align_up((size_t)K * cols[j] * 2, 256);
        d.off_xp[j] = p;
        p += align_up((size_t)K * cols[j] * 2, 256);
        d.off_y[j] = p;
        p += align_up((size_t)K * rows[j] * 4, 256);
    }
    d.layer_bytes = p;
    p = d.layer_bytes * s.L;
    d.off_fxn = p;
    p += align_up((size_t)K * s.H * 2, 256);
    d.off_fxp = p;
    p += align_up((size_t)K * s.H * 2, 256);
    d.off_stats = p;
    d.stats_stride = align_up((size_t)FLOW_MAX_WG * K, 64);
    p += d.stats_stride * 4 * (size_t)(4 * s.L);
    d.off_sync = p;
    d.sync_words = (4 * s.L + 1) * DONE_WORDS + DONE_STRIDE;
    p += align_up((size_t)d.sync_words * 4, 256);
    d.total = p;
    return d;
}

int* err_word(const DecodeLayout& d, char* ws) {
    return (int*)(ws + d.off_sync) + (d.sync_words - DONE_STRIDE);
}

// Tiles of 16 rows per stage (gate|up: 8 gate + 8 up rows).
int stage_tiles(const Shapes& s, int st) {
    if (st == 4 * s.L) return (s.V + 15) / 16;
    switch (st & 3) {
        case 0: return (s.H + 2 * s.KV) / 16;
        case 1: return s.H / 16;
        case 2: return s.FF / 8;
        default: return s.H / 16;
    }
}

void fill_common(FlowArgs& A, const vq_model* M, const Shapes& s, const DecodeLayout& d, int K,
                 const void* x0, float* logits, char* ws) {
    A = FlowArgs{};
    A.fmt = s.fmt;
    A.K = K;
    A.H = s.H; A.KV = s.KV; A.FF = s.FF; A.V = s.V; A.L = s.L;
    A.nwg = flow_grid();
    A.x0 = (const uint16_t*)x0;
    A.out = logits;
    A.ws = ws;
    A.layer_bytes = d.layer_bytes;
    for (int j = 0; j < 4; ++j) {
        A.off_xn[j] = d.off_xn[j];
        A.off_xp[j] = d.off_xp[j];
        A.off_y[j] = d.off_y[j];
    }
    A.off_fxn = d.off_fxn;
    A.off_fxp = d.off_fxp;
    A.off_stats = d.off_stats;
    A.stats_stride = d.stats_stride;
    A.done = (unsigned*)(ws + d.off_sync);
    A.err = err_word(d, ws);
    A.lm = MatPtr{(const uint8_t*)M->lm_head.qs, M->lm_head.scales, (const uint16_t*)M->lm_head.mins};
}

void fill_layers(FlowArgs& A, const vq_model* M, int l0) {
    A.l0 = l0;
    for (int i = 0; i < FLOW_MAX_LAYERS && l0 + i < M->n_layers; ++i) {
        const vq_layer& y = M->layers[l0 + i];
        const vq_matrix* ms[7] = {&y.q, &y.k, &y.v, &y.o, &y.gate, &y.up, &y.down};
        for (int m = 0; m < 7; ++m)
            A.m[i][m] = MatPtr{(const uint8_t*)ms[m]->qs, ms[m]->scales, (const uint16_t*)ms[m]->mins};
    }
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
        default: return "unknown status";
    }
}

size_t vq_workspace_bytes(int32_t op, const void* desc, int32_t K) {
    if (!desc) return 0;
    if (op == VQ_OP_LINEAR) return 0;            // the linear map needs no workspace
    if (op == VQ_OP_ACCEPT) {
        const vq_accept_desc* d = (const vq_accept_desc*)desc;
        if (d->W < 0 || d->K < 1 || d->K > VQ_MAX_K) return 0;
        return accept_ws_bytes(d);
    }
    if (op == VQ_OP_DECODE) {
        Shapes s;
        if (check_model((const vq_model*)desc, &s) || K < 1 || K > VQ_MAX_K) return 0;
        return decode_layout(s, K).total;
    }
    return 0;
}

int vq_verify_linear(const vq_matrix* W, const void* x_f16, int32_t K, void* y, int32_t y_dtype, void* stream) {
    g_err[0] = 0;
    int rc = check_matrix(W, "W");
    if (rc) return rc;
    if (K < 1 || K > VQ_MAX_K) return fail(VQ_ERR_ARG, "K %d outside 1..%d", K, VQ_MAX_K);
    if (y_dtype != VQ_DTYPE_F32 && y_dtype != VQ_DTYPE_F16) return fail(VQ_ERR_ARG, "unknown y_dtype %d", y_dtype);
    if (W->rows == 0) return VQ_OK;
    if (!x_f16 || !y) return fail(VQ_ERR_ARG, "NULL x or y");
    if (!aligned(x_f16, 16)) return fail(VQ_ERR_ARG, "x must be 16-byte aligned");
    if (!aligned(y, y_dtype == VQ_DTYPE_F32 ? 4 : 2)) return fail(VQ_ERR_ARG, "y is misaligned");
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
    A.nwg = std::min(flow_grid(), (W->rows + 15) / 16);
    A.x0 = (const uint16_t*)x_f16;
    A.out = y;
    A.lm = MatPtr{(const uint8_t*)W->qs, W->scales, (const uint16_t*)W->mins};
    const hipError_t e = launch_flow(A, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "linear launch");
    return VQ_OK;
}

int vq_verify_accept(const vq_accept_desc* d, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    if (!d) return fail(VQ_ERR_ARG, "NULL descriptor");
    if (d->reserved != 0) return fail(VQ_ERR_ARG, "reserved field must be 0");
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
    const DecodeLayout d = decode_layout(s, K);
    char* base = (char*)ws;
    if (stage == 4 * s.L) {
        *in_f16 = base + d.off_fxn;
        *out_f32 = nullptr;
    } else {
        const size_t lb = (size_t)(stage / 4) * d.layer_bytes;
        *in_f16 = base + lb + d.off_xn[stage % 4];
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
    *word = err_word(decode_layout(s, K), (char*)ws);
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
    const DecodeLayout d = decode_layout(s, K);
    if (!ws || ws_bytes < d.total || !aligned(ws, 256))
        return fail(VQ_ERR_WORKSPACE, "workspace needs %zu bytes (256-byte aligned), got %zu", d.total, ws_bytes);
    hipStream_t st = (hipStream_t)stream;
    char* base = (char*)ws;
    hipError_t e = launch_zero_u32((unsigned*)(base + d.off_sync), d.sync_words, st);
    if (e != hipSuccess) return hip_fail(e, "sync reset launch");
    FlowArgs A;
    fill_common(A, M, s, d, K, x0_f16, logits, base);
    const int S = 4 * s.L + 1;
    const bool staged = launch == VQ_LAUNCH_STAGED;
    int nl = 0, base0 = 0, s0 = 0;
    while (s0 < S) {
        int s1;
        if (staged) {
            s1 = s0 + 1;
        } else {
            // the stages of FLOW_MAX_LAYERS layers (the last launch also runs the lm_head)
            const int l0 = s0 / 4;
            s1 = std::min(S, 4 * (l0 + FLOW_MAX_LAYERS));
            if (s1 == 4 * s.L) s1 = S;
        }
        fill_layers(A, M, std::min(s0 / 4, s.L - 1));
        A.s_begin = s0;
        A.s_end = s1;
        for (int t = s0, b = base0; t < s1; ++t) {
            A.base[t - s0] = b;
            b = (b + stage_tiles(s, t)) % A.nwg;
        }
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
        for (int t = s0; t < s1; ++t) base0 = (base0 + stage_tiles(s, t)) % A.nwg;
        ++nl;
        s0 = s1;
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
