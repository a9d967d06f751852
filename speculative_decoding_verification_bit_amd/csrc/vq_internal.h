// Internal declarations of libvq (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stddef.h>
#include <stdint.h>

#include "../../include/vq.h"

namespace vq {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ------------------------------------------------------------------ tiled weights
// A matrix in the tiled layout is a sequence of chunks, tile-major: tile t (16 rows),
// group g (4 blocks = 128 columns) at byte (t * G + g) * chunk_bytes, with G the group
// count rounded up to even (the kernels take two groups of a tile per step).  A chunk is
//   codes  1024 B: lane l = n + 16 q (n = row in the tile, q = quarter of a block)
//                  holds 16 B, dword j = the 8 codes of block 4g + j, columns 8q..8q+7,
//                  of row n, nibble p holding column 8q + kPairSrc[p] (so that the Q4
//                  widening yields natural column order); MXFP4 keeps natural nibbles
//   scales       : per row n, the 4 block scales of the group (fp16: 8 B, E8M0: 4 B),
//                  and for Q4 with mins the 4 fp16 mins after them (16 B per row);
//                  Q4_K: per row n at 8n the 4 blocks' scale bytes s then their 4 min
//                  bytes m, and at 128 + 2n one fp16 of the row's super-block (the
//                  two groups of a step): D in the even group's chunk, Dmin in the odd
// Rows past the matrix and blocks past its columns are zero (codes, scales and mins), so
// they contribute exactly 0.
constexpr int TILE_ROWS = 16;
constexpr int GROUP_COLS = 128;
constexpr int STEP_COLS = 2 * GROUP_COLS;   // columns of one step of the streaming kernel
inline int chunk_bytes(int fmt) {
    return 1024 + (fmt == VQ_FMT_Q4_MIN ? 256 : fmt == VQ_FMT_Q4 ? 128 : fmt == VQ_FMT_Q4_K ? 160 : 64);
}
inline size_t tiled_bytes(int fmt, int rows, int cols) {
    const size_t T = (size_t)(rows + TILE_ROWS - 1) / TILE_ROWS;
    const size_t G = 2 * ((size_t)(cols + STEP_COLS - 1) / STEP_COLS);
    return T * G * (size_t)chunk_bytes(fmt);
}

// Writes rows [row0, row0 + W.rows) of a tiled matrix (rows `dst_rows`, cols W.cols,
// row order `order`) from the plain planes of W.
hipError_t launch_tile(const vq_matrix& W, uint8_t* dst, int dst_rows, int order, int row0, hipStream_t st);

// ------------------------------------------------------------------ the flow kernel

// What a stage computes and where its output goes.
enum StageKind {
    SK_QKV = 0,    // q|k|v = W_qkv x        (rows H + 2 KV; the q rows feed the o stage)
    SK_O = 1,      // o = W_o x              (rows H)
    SK_GU = 2,     // gate|up = W_gu x       (rows 2 FF; tile t = gate rows 8t..8t+7, up rows 8t..8t+7)
    SK_DOWN = 3,   // down = W_down x        (rows H, cols FF)
    SK_LM = 4,     // logits = W_lm x        (rows V)
    SK_LIN = 5     // a single linear map (vq_verify_linear)
};

constexpr int FLOW_MAX_LAYERS = 16;      // layers one launch of the pass kernel carries
constexpr int FLOW_MAX_WG = 1024;        // largest grid the workspace layout provides for
constexpr int FLOW_NCW = 11;             // compute waves per workgroup (plus one conductor)
constexpr int FLOW_LDS = 163840;         // LDS per workgroup (gfx950: 160 KB)
constexpr int FLOW_NSP_MAX = 8;          // slots of the partial-sum ring
constexpr int FLOW_PEND_MAX = 64;        // split tiles one workgroup finishes per stage
constexpr int FLOW_REL_MAX = 256;        // parts whose counters are raised in one batch
// Completion counters of a stage: 64 of them (workgroup w adds to w mod 64), each on its
// own 128-byte line, so that few atomics queue on any one line; a poll reads all 64, one per
// lane.  (With 8, a stage's hand-over waited on 32 atomics per line: the 27B pass took 6%
// longer at K = 1 and 4% at K = 8; 128 or 256 gain nothing more.)
constexpr int DONE_REPL = 64;
constexpr int DONE_STRIDE = 32;
constexpr int DONE_WORDS = DONE_REPL * DONE_STRIDE;

// Control block at the top of the workgroup's LDS.
struct FlowCtrl {
    unsigned pcnt[FLOW_NSP_MAX];     // wave partials written into ring slot i (cumulative)
    unsigned pfree[FLOW_NSP_MAX];    // times ring slot i has been reduced
    unsigned xready;                 // stages (launch-relative, + 1) whose activations are in LDS
    unsigned abort;                  // set by the first wait that times out
    unsigned pad_[2];
    float rho[VQ_MAX_K];
    int pend_t[FLOW_PEND_MAX];
    int rel_t[FLOW_REL_MAX];         // tiles whose part counters the conductor raises next
};
constexpr int FLOW_CTRL_OFF = (FLOW_LDS - (int)sizeof(FlowCtrl)) & ~255;

// How one kind of stage is split over the grid (computed on the host), in steps: a step
// is the two chunks of groups 2g, 2g + 1 of a tile (16 rows x 256 columns); below, a
// "chunk" of a plan is such a step.  The chunks of a stage are ordered window-major: window w (columns of groups [w gw, ...)), then tile,
// then group; workgroup i < nwe takes the contiguous range [i q + min(i, r), ... + q +
// (i < r)), which holds at least one whole unit (a tile's chunks in one window).
struct KindPlan {
    int rows, cols;     // output features (gate|up: 2 FF), input features
    int T, G;           // tiles of 16 rows, steps of 256 columns per tile
    int nwin, gw, glast;// windows: nwin - 1 of gw groups, then one of glast
    int cb;             // bytes of a step (two chunks)
    int nwe, q, r;      // workgroups with work; chunks per workgroup
    int xs;             // LDS row stride of the activation window (bytes)
    int n_in;           // elements rho normalises (0: no rho)
    int stats;          // 1: the stage reports sums of squares of what it feeds on
};

// Everything one launch of the pass kernel reads.  A launch runs the global stages
// [s_begin, s_end) of a pass (4 per layer + the lm_head), or one linear map.
struct FlowArgs {
    int fmt, K;
    int H, KV, FF, V, L;      // decode shapes
    int s_begin, s_end;
    int nwg;                  // grid size
    int linear;               // 1: one plain linear map (stage kind SK_LIN)
    int y_dtype;              // linear: VQ_DTYPE_F32 / VQ_DTYPE_F16
    int l0;                   // layer of w[0]
    int nsp, pbytes;          // ring slots; bytes of one wave's partial
    int xoff1;                // LDS offset of the second activation window
    int ring_off;             // LDS offset of the partial-sum ring
    int pad_;
    const uint16_t* x0;       // fp16 input of stage 0 [K][cols]
    void* out;                // logits [K][V] (decode) or y [K][rows] (linear)
    char* ws;                 // decode workspace (NULL for a linear map)
    size_t layer_bytes;       // per layer: [x, y] of its 4 stages
    size_t off_x[4], off_y[4];
    size_t off_fx;            // lm_head input
    size_t off_stats;         // per stage s < 4L: [K][FLOW_MAX_WG] floats
    size_t stats_stride;      // floats per stage
    float* parts;             // split-tile partial sums
    unsigned* cnt;            // split-tile arrival counters (zero between launches)
    unsigned* done;           // [stages][DONE_WORDS] completion counters (NULL: linear)
    int* err;                 // raised when a bounded wait times out
    KindPlan kp[6];           // by StageKind
    const uint32_t* steps;    // the compute waves' work lists (pairs, see steps.h)
    const uint32_t* step_start;  // per workgroup and compute wave: its first pair in steps
    const uint8_t* lm;        // lm_head, or the linear map
    const uint8_t* w[FLOW_MAX_LAYERS][4];   // q|k|v, o, gate|up, down of layers l0 ..
};

// Host side of the split: fills a KindPlan, or returns false if the shape cannot be split
// (a workgroup's chunks would span more than two windows, or it would finish more than
// FLOW_PEND_MAX split tiles).
bool make_plan(KindPlan& P, int fmt, int K, int rows, int cols, int tiles, int nwg, int xcap);
// LDS bytes left for the activation windows with K columns, and the ring geometry.
void lds_plan(int K, int* nsp, int* pbytes, int* ring_off, int* xcap);
// Floats of split-tile partials and words of counters a plan needs.
size_t plan_parts_floats(const KindPlan& P, int pbytes, int nwg, int stages);
size_t plan_counters(const KindPlan& P);

hipError_t launch_zero_u32(unsigned* p, size_t n, hipStream_t st);
// One launch of the pass kernel over A.s_begin .. A.s_end (cooperative when it spans more
// than one stage, so that every workgroup is resident for the grid barriers).
hipError_t launch_flow(const FlowArgs& A, hipStream_t st);
int flow_grid();                 // workgroups of a launch: one per compute unit

// The scaled MXFP4 path (E4M3 activations): y [K][rows] ~= W x for plain MXFP4 planes.
constexpr int MX_WG_PER_CU = 1;         // workgroups (of 4 waves) per compute unit
void mx_plan(int rows, int cols, int nwg, int* T, int* C, int* S, int* cps);
size_t mx_workspace_bytes(int rows, int cols, int K, int nwg);
hipError_t launch_mx_linear(const vq_matrix& W, const void* x, int K, float* y, uint8_t* ws, int nwg, hipStream_t st);

// Attention over a quantised KV cache: spans of positions per kv head, then their merge.
void attn_plan(int Hkv, int L, int M, int nwg, int* S, int* span);
size_t attn_workspace_bytes(int Hkv, int Hq, int L, int K, int nwg);
hipError_t launch_attention(const vq_attention& C, const void* q, int K, float* out, uint8_t* ws, int nwg,
                            hipStream_t st);

// The thread-local error text of the C ABI: fail() sets it and returns code.
extern thread_local char g_err[512];
int fail(int code, const char* fmt, ...);
void clear_error();

// Acceptance.
size_t accept_ws_bytes(const vq_accept_desc* d);
hipError_t launch_accept(const vq_accept_desc* d, void* ws, hipStream_t st);

}  // namespace vq
