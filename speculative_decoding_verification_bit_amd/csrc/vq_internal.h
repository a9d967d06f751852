// Internal declarations of libvq (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stddef.h>
#include <stdint.h>

#include "../../include/vq.h"

namespace vq {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// One block-quantised matrix as the kernels address it.
struct MatPtr {
    const uint8_t* qs;
    const void* sc;
    const uint16_t* mn;
};

// What a stage computes and where its output goes.
enum StageKind {
    SK_QKV = 0,    // q|k|v = W_qkv x        (rows H + 2 KV; the q rows feed the o stage)
    SK_O = 1,      // o = W_o x              (rows H)
    SK_GU = 2,     // gate|up = W_gu x       (rows 2 FF; tile t = gate rows 8t..8t+7, up rows 8t..8t+7)
    SK_DOWN = 3,   // down = W_down x        (rows H, cols FF)
    SK_LM = 4,     // logits = W_lm x        (rows V)
    SK_LIN = 5     // a single linear map (vq_verify_linear)
};

// Layers whose pointers one launch of the pass kernel carries in its arguments.
constexpr int FLOW_MAX_LAYERS = 16;
// Largest grid the workspace layout provides per-workgroup statistics for.
constexpr int FLOW_MAX_WG = 1024;
// Completion counters of a stage: one per XCD group of workgroups (blockIdx mod 8), each
// on its own 128-byte line.
constexpr int DONE_REPL = 8;
constexpr int DONE_STRIDE = 32;
constexpr int DONE_WORDS = DONE_REPL * DONE_STRIDE;

// Everything one launch of the pass kernel reads.  A launch runs the global stages
// [s_begin, s_end) of a pass (4 per layer + the lm_head), or one linear map.
struct FlowArgs {
    int fmt, K;
    int H, KV, FF, V, L;      // decode shapes; a linear map keeps rows in V and cols in H
    int s_begin, s_end;
    int nwg;                  // grid size
    int base0;                // (unused: see base)
    int linear;               // 1: one plain linear map (stage kind SK_LIN)
    int y_dtype;              // linear: VQ_DTYPE_F32 / VQ_DTYPE_F16
    int l0;                   // layer of m[0]
    int pad_;
    const uint16_t* x0;       // natural-order fp16 input of stage 0 [K][cols]
    void* out;                // logits [K][V] (decode) or y [K][rows] (linear)
    char* ws;                 // decode workspace (NULL for a linear map)
    size_t layer_bytes;       // per layer: [xn, xp, y] of its 4 stages
    size_t off_xn[4], off_xp[4], off_y[4];
    size_t off_fxn, off_fxp;  // lm_head input
    size_t off_stats;         // per stage s < 4L: [FLOW_MAX_WG][K] floats
    size_t stats_stride;      // floats per stage
    unsigned* done;           // [stages][DONE_WORDS] completion counters (NULL: linear)
    int* err;                 // raised when a bounded wait times out (NULL: linear)
    // tile t of stage s_begin + i belongs to workgroup (base[i] + t) mod nwg
    int base[4 * FLOW_MAX_LAYERS + 1];
    MatPtr lm;
    MatPtr m[FLOW_MAX_LAYERS][7];   // q, k, v, o, gate, up, down of layers l0 ..
};

// Geometry of one stage.
struct StageGeo {
    int kind, rows, cols, nb, G, T;
    int n_in;                 // elements of the previous output that rho normalises (0: none)
};

template <class FA>
__host__ __device__ inline StageGeo stage_geo(const FA& A, int s) {
    StageGeo g;
    if (A.linear) {
        g.kind = SK_LIN; g.rows = A.V; g.cols = A.H;
    } else if (s == 4 * A.L) {
        g.kind = SK_LM; g.rows = A.V; g.cols = A.H;
    } else {
        g.kind = s & 3;
        switch (g.kind) {
            case SK_QKV: g.rows = A.H + 2 * A.KV; g.cols = A.H; break;
            case SK_O: g.rows = A.H; g.cols = A.H; break;
            case SK_GU: g.rows = 2 * A.FF; g.cols = A.H; break;
            default: g.rows = A.H; g.cols = A.FF; break;
        }
    }
    g.nb = g.cols >> 5;
    g.G = (g.nb + 3) >> 2;
    g.T = g.kind == SK_GU ? (A.FF >> 3) : (g.rows + 15) >> 4;
    if (A.linear || s == 0) {
        g.n_in = 0;
    } else {
        const int pk = (s - 1) & 3;       // kind of the previous stage
        g.n_in = pk == SK_GU ? A.FF : A.H;
    }
    return g;
}

size_t flow_stage_ws_end(const FlowArgs& A);
hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t st);
// One launch of the pass kernel over A.s_begin .. A.s_end (cooperative when it spans more
// than one stage, so that every workgroup is resident for the grid barriers).
hipError_t launch_flow(const FlowArgs& A, hipStream_t st);
int flow_grid();                 // workgroups of a launch: one per compute unit

// Acceptance.
size_t accept_ws_bytes(const vq_accept_desc* d);
hipError_t launch_accept(const vq_accept_desc* d, void* ws, hipStream_t st);

}  // namespace vq
