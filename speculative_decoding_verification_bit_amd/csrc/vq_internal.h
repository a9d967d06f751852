// Internal declarations of libvq (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stddef.h>
#include <stdint.h>

#include "../../include/vq.h"

namespace vq {

// One weight operand as the kernels see it: up to three row-concatenated matrices of
// the same format and column count (q|k|v, gate|up), each a 64-row multiple except the
// last.  Segment s covers rows [seg_end[s-1], seg_end[s]).
constexpr int MAX_SEG = 3;
struct Mat {
    int fmt;
    int rows, cols;
    int nseg;
    int seg_end[MAX_SEG];
    const uint8_t* qs[MAX_SEG];
    const void* scales[MAX_SEG];
    const uint16_t* mins[MAX_SEG];
};

inline Mat mat_from(const vq_matrix& m) {
    Mat r{};
    r.fmt = m.format;
    r.rows = m.rows;
    r.cols = m.cols;
    r.nseg = 1;
    r.seg_end[0] = m.rows;
    r.qs[0] = (const uint8_t*)m.qs;
    r.scales[0] = m.scales;
    r.mins[0] = (const uint16_t*)m.mins;
    return r;
}

// Geometry of one stage launch: tiles of 64 rows (paired: 32 rows of each of the two
// segments) x chunks of 4 groups of 8 blocks (one group per wave of a workgroup).
struct StageGeom {
    int nb;        // blocks of 32 per row
    int ngroups;   // groups of 8 blocks per row
    int nchunks;   // chunks of 4 groups
    int ntiles;
    int cpw;       // chunks per item (one workgroup's share of a tile)
    int nparts;    // items per tile = split-K partials per output
    // row-strip kernel (rk = 1): items of R whole rows, activations staged per window
    int rk;
    int R;         // rows per item (paired: R / 2 of each half); 4, 8 or 16
    int nitems;    // items of the stage (either kernel)
    int xwb;       // blocks per activation window (a multiple of 64)
    int nphase;    // windows per row
    int nstat;     // sums-of-squares entries the stage writes (row-strip: items; tile: tiles)
};

// Workgroups that convert a stage's input (staged launches): the gate|up, down and lm_head
// stages of the MFMA kernel, and of the VALU kernel from K = PREP_MIN_K_VALU.
constexpr int N_PREP = 16;
constexpr int PREP_MIN_K_VALU = 2;

// Row-strip kernel limits: K <= ROWS_MAX_K, at most ROWS_NLD 16-byte weight loads per
// lane per window (two items' worth are in registers at once), ROWS_X_BYTES of LDS for a
// window's fp16 activations.
constexpr int ROWS_MAX_K = 4;
constexpr int ROWS_NLD = 12;
constexpr int ROWS_X_BYTES = 36864;


inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Glue modes: how a stage builds its input from the previous stage.
enum GlueMode { GLUE_NONE = 0, GLUE_RHO = 1 };

typedef uint32_t u4_t_ __attribute__((ext_vector_type(4)));

// Everything one stage launch reads and writes.
struct StageArgs {
    Mat W;
    int K;
    int paired;                // 1: gate|up pairing (tile t = rows [32t, 32t+32) of both segments)
    // input: GLUE_NONE reads fp16 x16 [K][cols]; GLUE_RHO reads src[k*ld + j] and scales
    // column k by 1/sqrt(sum(stats_in[.][k]) / n_in) before rounding to fp16
    int glue;
    const uint16_t* x16;
    const float* src;
    int ld;
    int n_in;
    const float* stats_in;
    int nstats_in;
    uint16_t* keep;            // fp16 copy of the input [K][cols] (written by tile 0), or NULL
    // scratch
    float* part;               // split-K partials [nparts][K][rows]
    unsigned* counters;        // per-tile arrival counters [ntiles], zero between launches
    // output
    void* y;                   // [K][rows], f32 or f16
    int y_dtype;
    float* stats_out;          // per-tile sums of squares [ntiles][K], or NULL
    int nstat;                 // rows < nstat contribute to stats_out (unpaired)
    float* sbuf;               // paired: silu(gate) * up [K][rows/2]
    int coh;                   // 1: y / stats_out / sbuf are read by other workgroups of the
                               // same launch: stored through to memory (device scope)
    // MFMA kernel, one-stage input conversion: with n_prep > 0 the first n_prep workgroups
    // of the launch (a multiple of 8) convert the whole input into xp (A operands, [block]
    // [lane] 16 bytes) and xpa (block-sum operands, [group][lane] 16 bytes), then count
    // themselves on *xflag; the other workgroups wait for that count before reading them.
    u4_t_* xp;
    u4_t_* xpa;
    unsigned* xflag;
    int* err;                  // raised when the wait for the conversion times out
    int n_prep;
    unsigned* done;            // NULL, or DONE_REPL completion counters DONE_STRIDE words
                               // apart, one per XCD group of workgroups; their sum counts
                               // the tiles (tile kernel) or items (row-strip kernel) whose
                               // outputs are in memory
};

// Completion counters of the persistent pass: one per XCD group of workgroups (blockIdx
// mod 8), each on its own 128-byte line, so that arrivals spread over 8 addresses.
constexpr int DONE_REPL = 8;
constexpr int DONE_STRIDE = 32;
constexpr int DONE_WORDS = DONE_REPL * DONE_STRIDE;     // per stage

// ------------------------------------------------------------- decode pass plan

// The stage sequence of a decode pass, in a form both the host and the device can turn
// into StageArgs.  One launch of the persistent kernel covers up to PASS_LAYERS layers.
constexpr int PASS_LAYERS = 8;

struct MatPtrs {
    const void* qs;
    const void* sc;
    const void* mn;
};

struct PassPlan {
    int fmt, K, H, KV, FF, V, L;   // shapes (every layer alike)
    int layer0, nlayers;           // layers of this plan segment
    int with_lm;                   // 1: the lm_head stage ends this segment
    MatPtrs m[PASS_LAYERS][7];     // q, k, v, o, gate, up, down of layers layer0 + i
    MatPtrs lm;
    StageGeom geo[5];              // geometry of stages q|k|v, o, gate|up, down, lm_head
    const uint16_t* x0;            // pass input fp16 [K][H]
    float* logits;                 // [K][V]
    char* base;                    // workspace
    size_t layer_bytes, in_off[4], out_off[4], final_in_off;
    float* stats;                  // per-tile sums of squares, stats_stride floats per stage
    size_t stats_stride;
    float* sbuf;                   // silu(gate) * up, sbuf_stride floats per layer
    size_t sbuf_stride;
    float* part;
    unsigned* counters;
    unsigned* done;                // DONE_WORDS per stage, 0 at pass start (persistent only)
    int* err;                      // set when a wait for a stage times out
    int coh;
    u4_t_* xp;                     // staged MFMA input conversion buffers of stage 0 (or
    u4_t_* xpa;                    // NULL); stage s's are xp_stride slots further on
    size_t xp_stride;
    unsigned* xflag;               // DONE_WORDS per stage, 0 at pass start
};

__host__ __device__ inline int stage_tiles_of(int rows, int paired, int half) {
    return paired ? (half + 31) / 32 : (rows + 63) / 64;
}

// StageArgs of global stage `stage` (4 per layer + lm_head) of a plan segment.
__host__ __device__ inline void build_stage(const PassPlan& P, int stage, StageArgs& A) {
    const int l = stage / 4, j = stage % 4;
    const bool lm = (l == P.L);
    const int li = l - P.layer0;
    A = StageArgs{};
    A.K = P.K;
    A.coh = P.coh;
    Mat& W = A.W;
    W.fmt = P.fmt;
    auto seg = [&](int i, const MatPtrs& mp, int rows_before) {
        W.qs[i] = (const uint8_t*)mp.qs;
        W.scales[i] = mp.sc;
        W.mins[i] = (const uint16_t*)mp.mn;
        (void)rows_before;
    };
    if (lm) {
        W.rows = P.V; W.cols = P.H; W.nseg = 1; W.seg_end[0] = P.V;
        seg(0, P.lm, 0);
    } else if (j == 0) {
        W.rows = P.H + 2 * P.KV; W.cols = P.H; W.nseg = 3;
        W.seg_end[0] = P.H; W.seg_end[1] = P.H + P.KV; W.seg_end[2] = P.H + 2 * P.KV;
        seg(0, P.m[li][0], 0); seg(1, P.m[li][1], 0); seg(2, P.m[li][2], 0);
    } else if (j == 1) {
        W.rows = P.H; W.cols = P.H; W.nseg = 1; W.seg_end[0] = P.H;
        seg(0, P.m[li][3], 0);
    } else if (j == 2) {
        W.rows = 2 * P.FF; W.cols = P.H; W.nseg = 2; W.seg_end[0] = P.FF; W.seg_end[1] = 2 * P.FF;
        seg(0, P.m[li][4], 0); seg(1, P.m[li][5], 0);
        A.paired = 1;
    } else {
        W.rows = P.H; W.cols = P.FF; W.nseg = 1; W.seg_end[0] = P.H;
        seg(0, P.m[li][6], 0);
    }
    A.keep = (uint16_t*)(lm ? P.base + P.final_in_off : P.base + (size_t)l * P.layer_bytes + P.in_off[j]);
    if (stage == 0) {
        A.glue = GLUE_NONE;
        A.x16 = P.x0;
    } else {
        // the previous stage's raw output: q part of q|k|v, o, silu(gate) * up, down
        const int pl = (stage - 1) / 4, pj = (stage - 1) % 4;
        A.glue = GLUE_RHO;
        A.n_in = W.cols;
        A.stats_in = P.stats + (size_t)(stage - 1) * P.stats_stride;
        A.nstats_in = P.geo[pj].nstat;
        if (pj == 2) {
            A.src = P.sbuf + (size_t)pl * P.sbuf_stride;
            A.ld = P.FF;
        } else {
            A.src = (const float*)(P.base + (size_t)pl * P.layer_bytes + P.out_off[pj]);
            A.ld = pj == 0 ? P.H + 2 * P.KV : P.H;
        }
    }
    A.y_dtype = VQ_DTYPE_F32;
    if (lm) {
        A.y = P.logits;
    } else {
        A.y = P.base + (size_t)l * P.layer_bytes + P.out_off[j];
        A.stats_out = P.stats + (size_t)stage * P.stats_stride;
        A.nstat = j == 0 ? P.H : W.rows;
        A.sbuf = P.sbuf + (size_t)l * P.sbuf_stride;
        A.done = P.done ? P.done + (size_t)stage * DONE_WORDS : nullptr;
    }
    A.part = P.part;
    A.counters = P.counters;
    A.xp = P.xp ? P.xp + (size_t)stage * P.xp_stride : nullptr;
    A.xpa = P.xpa ? P.xpa + (size_t)stage * P.xp_stride : nullptr;
    A.xflag = P.xflag ? P.xflag + (size_t)stage * DONE_WORDS : nullptr;
    A.err = P.err;
}

// Geometry with a given run length (cheap: the kernels call it).
__host__ __device__ inline StageGeom stage_geom_cpw(int rows, int cols, int paired, int half, int cpw) {
    StageGeom g;
    g.nb = cols >> 5;
    g.ngroups = (g.nb + 7) >> 3;
    g.nchunks = (g.ngroups + 3) >> 2;
    g.ntiles = paired ? (half + 31) >> 5 : (rows + 63) >> 6;
    g.cpw = cpw;
    g.nparts = (g.nchunks + cpw - 1) / cpw;
    g.rk = 0;
    g.R = 64;
    g.nitems = g.ntiles * g.nparts;
    g.xwb = 0;
    g.nphase = 0;
    g.nstat = g.ntiles;
    return g;
}

// The most split-K parts a tile geometry of a stage with `cols` columns can have (one
// chunk per item); the partial buffers are sized for it.
__host__ __device__ inline int max_parts(int cols) { return stage_geom_cpw(0, cols, 0, 0, 1).nchunks; }

// Row-strip geometry for K columns: the whole row's activations in one LDS window
// (NSG 64-block segments), R = 4 * rows per wave, with rows per wave 4, 2 or 1 as the
// segments grow (the loads per lane stay at most ROWS_NLD).  rk = 0 when the row does
// not fit one window (the tile kernel runs those stages).
__host__ __device__ constexpr int rows_per_wave(int nsg) { return nsg <= 3 ? 4 : nsg <= 6 ? 2 : 1; }
__host__ __device__ constexpr bool rows_fit(int K, int nsg) {
    return nsg >= 1 && nsg <= 9 && (long)K * nsg * 64 * 64 <= ROWS_X_BYTES;
}

inline StageGeom rows_geom(int rows, int cols, int paired, int half, int K) {
    StageGeom g = stage_geom_cpw(rows, cols, paired, half, 1);
    const int nsg = (g.nb + 63) / 64;
    if (K > ROWS_MAX_K || !rows_fit(K, nsg)) return g;
    g.rk = 1;
    g.xwb = 64 * nsg;
    g.nphase = 1;
    g.R = 4 * rows_per_wave(nsg);
    g.nitems = paired ? (half + g.R / 2 - 1) / (g.R / 2) : (rows + g.R - 1) / g.R;
    g.nstat = g.nitems;
    return g;
}

// Which kernel streams a stage.
enum Kern { KERN_VALU = 0, KERN_MFMA = 1, KERN_ROWS = 2 };

// Geometry of a stage for its kernel: the tile kernels one chunk per item (measured
// fastest for both: a run of chunks is loaded and computed in series by one workgroup;
// at K = 8 runs of several chunks per item cost 10.34 against 9.41 ms per 27B pass), the
// row-strip kernel where the row's activations fit (the VALU tile kernel elsewhere).
inline StageGeom plan_geom(int rows, int cols, int paired, int half, int K, Kern kern) {
    if (kern == KERN_ROWS && K <= ROWS_MAX_K) {
        const StageGeom g = rows_geom(rows, cols, paired, half, K);
        if (g.rk) return g;
    }
    (void)kern;
    return stage_geom_cpw(rows, cols, paired, half, 1);
}
// Stream-ahead pass (LDS-direct weight rings, one 8-wave workgroup per CU): K up to
// STREAM_MAX_K, stage widths up to VQ_STREAM_MAX_COLS columns.
constexpr int STREAM_WAVES = 8;
constexpr int STREAM_MAX_K = 2;
#define VQ_STREAM_MAX_COLS 20480
bool stream_enabled();
size_t stream_lds_bytes(int K, int H, int FF);
int stream_supported(int fmt, int K, int H, int KV, int FF);
hipError_t launch_stream_segment(const PassPlan& P, hipStream_t st);

size_t stage_scratch_bytes(int rows, int cols, int K, int paired, int half);
void stage_scratch_carve(void* base, int rows, int cols, int K, int paired, int half, StageArgs* A);
hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t st);
hipError_t launch_stage(const StageArgs& A, const StageGeom& g, bool mfma, hipStream_t st);
// One persistent (cooperative) launch over the stages of a plan segment.
hipError_t launch_pass_segment(const PassPlan& P, bool mfma, hipStream_t st);

// Acceptance.
size_t accept_ws_bytes(const vq_accept_desc* d);
hipError_t launch_accept(const vq_accept_desc* d, void* ws, hipStream_t st);

}  // namespace vq
