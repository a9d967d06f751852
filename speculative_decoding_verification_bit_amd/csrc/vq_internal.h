// Internal declarations of libvq (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
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

// Geometry of a linear launch: 64-row tiles x chunks of 4 groups of 8 blocks.
struct LinGeom {
    int nb;        // blocks of 32 per row
    int ngroups;   // groups of 8 blocks per row
    int nchunks;   // chunks of 4 groups (one per wave of a 256-thread workgroup)
    int ntiles;    // 64-row tiles
};

inline LinGeom lin_geom(int rows, int cols) {
    LinGeom g;
    g.nb = cols / 32;
    g.ngroups = (g.nb + 7) / 8;
    g.nchunks = (g.ngroups + 3) / 4;
    g.ntiles = (rows + 63) / 64;
    return g;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Scratch of one linear launch: activation layout, block sums, split-K partials.
struct LinScratch {
    void* xlay;      // VALU: packed half2 [K][cols/2]; MFMA: uint4 [nb][64]
    void* aux;       // VALU: float [K][nb] block sums; MFMA: uint4 [ngroups][64] min fragments
    float* part;     // [nchunks][K][rows]
};

size_t lin_scratch_bytes(int fmt, int rows, int cols, int K, bool mfma);
void lin_scratch_carve(void* base, int fmt, int rows, int cols, int K, bool mfma, LinScratch* s);

// Prepare the activation layout from fp16 x [K][cols] (plain input).
hipError_t launch_prep_plain(const Mat& W, const uint16_t* x, int K, bool mfma,
                             const LinScratch& s, uint16_t* x_keep, hipStream_t st);

// Glue input modes for the decode pass.
enum GlueMode { GLUE_NONE = 0, GLUE_RHO = 1, GLUE_RHO_SILU = 2 };

// Prepare the activation layout from a raw fp32 stage output with rho (and silu*up):
//   v[k][j] = src[k*ld + j]              (GLUE_RHO)
//   v[k][j] = silu(src[k*ld + j]) * src[k*ld + up_off + j]   (GLUE_RHO_SILU)
// x[k][j] = fp16(v[k][j] * r_k), r_k = 1/sqrt(sum(stats[.][k]) / n); x is also stored
// to x_keep (fp16 [K][cols]).
hipError_t launch_prep_glue(const Mat& W, const float* src, int ld, int up_off, int mode,
                            const float* stats, int nstats, int K, bool mfma,
                            uint16_t* x_keep, const LinScratch& s, hipStream_t st);

// The main weight-streaming kernel (writes split-K partials).
hipError_t launch_linear_main(const Mat& W, int K, bool mfma, const LinScratch& s, hipStream_t st);

// Sum the partials: y[k][r] (f32 or f16 with leading dim rows).
hipError_t launch_finalize(const Mat& W, int K, const LinScratch& s, void* y, int y_dtype,
                           hipStream_t st);

// Decode-pass finalize: y = sum of partials (f32, leading dim ld_out), plus per-256-row
// partial sums of squares of y over rows < nstat (stats[blk][k]).  SILU: rows [0, half)
// are gate, [half, 2 half) up; the statistic is of silu(gate) * up.
int finalize_stats_blocks(int rows, int silu);
hipError_t launch_finalize_stats(const Mat& W, int K, const LinScratch& s, float* y,
                                 int nstat, int silu, float* stats, hipStream_t st);

// Acceptance.
size_t accept_ws_bytes(const vq_accept_desc* d);
hipError_t launch_accept(const vq_accept_desc* d, void* ws, hipStream_t st);

}  // namespace vq
