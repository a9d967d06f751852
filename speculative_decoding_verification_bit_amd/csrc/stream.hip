// Stream-ahead decode pass for narrow verify windows (K <= 2) on gfx950.
//
// The pass reads every weight of the stack once (page "100 tokens per second from a 27B
// model on a 24 GB AMD card", section "The wall") and applies it to the window's K
// activation columns (same page, section "How speculative decoding gets past a
// per-token wall"), layer after layer (Hacker News thread 49596054).  At K = 1 or 2 the
// arithmetic is light and the pass is bound by how steadily HBM is kept busy, so this
// kernel never lets the weight stream stop at a stage boundary:
//  * one cooperative launch covers up to PASS_LAYERS layers; one 512-thread workgroup
//    per CU, 8 waves, and every wave owns a contiguous range of output rows of every
//    stage (gate|up: rows h of both halves);
//  * a row is cut into 64-block segments.  Each wave streams its segments, in stage
//    order and across stage boundaries, into a private ring of D slots in LDS with
//    LDS-direct loads (global_load_lds: 1 KB of codes + the 64 blocks' scales and mins
//    per slot), D - 1 slots ahead of the slot it computes.  The loads are issued from
//    inline assembly and waited for with explicit vmcnt counts (vector memory operations
//    complete in order, so "at most N outstanding" means everything but the last N
//    issued has landed);
//  * before the first row of a stage, the workgroup waits until every workgroup of the
//    previous stage has counted itself done, then reads that stage's raw output,
//    scales each column to unit RMS, rounds it to fp16 into LDS (the layout the dot
//    products read, quarters swizzled against bank conflicts) and, for Q4 with mins,
//    sums every block's activations.  The ring keeps filling meanwhile;
//  * a lane takes block 64g + lane of segment g: codes widened exactly to fp16 and fed
//    to v_dot2_f32_f16 against the K columns; per block d * sum(q x) (+ m * sum(x)); a
//    row's sum over lanes is a fixed DPP / readlane tree.
// The sums run in a different order from the staged kernels (one lane per block over a
// whole row instead of 1024-column chunks), so the two paths agree to rounding, not bit
// for bit; runs of this path are bitwise reproducible.
#include <hip/hip_fp16.h>

#include <map>
#include <mutex>
#include <utility>

#include "vq_device.h"
#include "vq_internal.h"

namespace vq {
namespace {

#define LDS_AS __attribute__((address_space(3)))

constexpr int SW = STREAM_WAVES;               // waves per workgroup
constexpr int STHR = 64 * SW;
constexpr int SLOT = 1280;                     // codes 1024 | scales 128 | mins 128

template <int FMT>
constexpr int ndma() { return FMT == VQ_FMT_Q4_MIN ? 3 : 2; }   // loads per slot

template <int K>
constexpr int ring_depth() { return K == 1 ? 10 : 7; }

// ----------------------------------------------------------------- stage addressing

// Rows (unpaired) or row pairs (gate|up) of global stage s: the units dealt to waves.
__device__ __forceinline__ int stage_jobs(const PassPlan& P, int s) {
    if (s == 4 * P.L) return P.V;
    switch (s & 3) {
        case 0: return P.H + 2 * P.KV;
        case 1: return P.H;
        case 2: return P.FF;
        default: return P.H;
    }
}

__device__ __forceinline__ int stage_cols(const PassPlan& P, int s) {
    return (s != 4 * P.L && (s & 3) == 3) ? P.FF : P.H;
}

// Jobs [j0, j1) of wave gw of nw (contiguous ranges, as even as integers allow).
__device__ __forceinline__ void wave_jobs(int njobs, int gw, int nw, int& j0, int& j1) {
    j0 = (int)((long)njobs * gw / nw);
    j1 = (int)((long)njobs * (gw + 1) / nw);
}

// A wave-uniform pointer pinned in scalar registers (the inline assembly takes it as a
// scalar base).
__device__ __forceinline__ const uint8_t* sgpr_ptr(const void* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Base addresses of one weight row: codes, scales, mins.
struct RowPtr {
    const uint8_t* qs;
    const uint8_t* sc;
    const uint8_t* mn;
};

// Row `job` (sub-row u of a gate|up pair) of stage s.
__device__ __forceinline__ RowPtr row_ptr(const PassPlan& P, int s, int job, int u) {
    const int l = s >> 2;
    const bool lm = s == 4 * P.L;
    const int li = l - P.layer0;
    const MatPtrs* mp;
    int lr = job;
    if (lm) {
        mp = &P.lm;
    } else {
        switch (s & 3) {
            case 0:
                if (job < P.H) mp = &P.m[li][0];
                else if (job < P.H + P.KV) { mp = &P.m[li][1]; lr = job - P.H; }
                else { mp = &P.m[li][2]; lr = job - P.H - P.KV; }
                break;
            case 1: mp = &P.m[li][3]; break;
            case 2: mp = &P.m[li][4 + u]; break;
            default: mp = &P.m[li][6]; break;
        }
    }
    const uint32_t cols = (uint32_t)stage_cols(P, s), nb = cols >> 5;
    const uint32_t ssz = P.fmt == VQ_FMT_MXFP4 ? 1u : 2u;
    RowPtr r;
    r.qs = sgpr_ptr((const uint8_t*)mp->qs + (size_t)lr * (cols >> 1));
    r.sc = sgpr_ptr((const uint8_t*)mp->sc + (size_t)lr * nb * ssz);
    r.mn = mp->mn ? sgpr_ptr((const uint8_t*)mp->mn + (size_t)lr * nb * 2) : r.sc;
    return r;
}

// What the pass needs of stage s besides its weights (the fields build_stage fills for
// the staged kernels): where its input comes from, where its outputs go.
struct StreamStage {
    int rows, cols, paired, half;
    int glue;                  // GLUE_NONE: fp16 x16; GLUE_RHO: unit-RMS columns of src
    const uint16_t* x16;
    const float* src;
    int ld;
    uint16_t* keep;            // fp16 copy of the input [K][cols]
    float* y;                  // [K][rows]
    float* sbuf;               // gate|up: silu(gate) * up [K][half]
};

__device__ __forceinline__ void stream_stage(const PassPlan& P, int s, StreamStage& S) {
    const int l = s >> 2, j = s & 3;
    const bool lm = s == 4 * P.L;
    S.cols = stage_cols(P, s);
    S.paired = !lm && j == 2;
    S.half = S.paired ? P.FF : 0;
    S.rows = lm ? P.V : j == 0 ? P.H + 2 * P.KV : j == 2 ? 2 * P.FF : P.H;
    S.keep = (uint16_t*)(lm ? P.base + P.final_in_off : P.base + (size_t)l * P.layer_bytes + P.in_off[j]);
    S.y = lm ? P.logits : (float*)(P.base + (size_t)l * P.layer_bytes + P.out_off[j]);
    S.sbuf = P.sbuf + (size_t)l * P.sbuf_stride;
    S.x16 = P.x0;
    S.src = nullptr;
    S.ld = 0;
    if (s == 0) {
        S.glue = GLUE_NONE;
    } else {
        // the previous stage's raw output: q part of q|k|v, o, silu(gate) * up, down
        const int pl = (s - 1) >> 2, pj = (s - 1) & 3;
        S.glue = GLUE_RHO;
        if (pj == 2) {
            S.src = P.sbuf + (size_t)pl * P.sbuf_stride;
            S.ld = P.FF;
        } else {
            S.src = (const float*)(P.base + (size_t)pl * P.layer_bytes + P.out_off[pj]);
            S.ld = pj == 0 ? P.H + 2 * P.KV : P.H;
        }
    }
}

// ----------------------------------------------------------------- the issue cursor

// Position of the next slot to load: stage, job, sub-row, segment, with the row's base
// addresses.  Past the end it stays on the last slot (its loads repeat harmlessly).
struct Cursor {
    int s, job, job1, u, nsub, g, nsg, nb;
    RowPtr rp;
};

__device__ __forceinline__ void cursor_stage(const PassPlan& P, Cursor& c, int s, int s1, int gw, int nw) {
    for (; s < s1; ++s) {
        int j0, j1;
        wave_jobs(stage_jobs(P, s), gw, nw, j0, j1);
        if (j0 < j1) {
            c.s = s;
            c.job = j0;
            c.job1 = j1;
            c.u = 0;
            c.nsub = (s != 4 * P.L && (s & 3) == 2) ? 2 : 1;
            c.g = 0;
            c.nb = stage_cols(P, s) >> 5;
            c.nsg = (c.nb + 63) >> 6;
            c.rp = row_ptr(P, s, j0, 0);
            return;
        }
    }
    c.s = s1;
}

__device__ __forceinline__ void cursor_next(const PassPlan& P, Cursor& c, int s1, int gw, int nw) {
    if (c.s >= s1) return;
    if (++c.g < c.nsg) return;
    c.g = 0;
    if (++c.u < c.nsub) {
        c.rp = row_ptr(P, c.s, c.job, c.u);
        return;
    }
    c.u = 0;
    if (++c.job < c.job1) {
        c.rp = row_ptr(P, c.s, c.job, 0);
        return;
    }
    const Cursor last = c;
    cursor_stage(P, c, c.s + 1, s1, gw, nw);
    if (c.s >= s1) {                              // nothing left: repeat the last slot
        c = last;
        c.s = s1;
        c.job = c.job1 - 1;
        c.u = c.nsub - 1;
        c.g = c.nsg - 1;
    }
}

// The slot's LDS-direct loads into the ring slot at LDS address `lds` (wave-uniform):
// codes of blocks 64g .. 64g + 63 (16 bytes per lane), then scales (and mins) of the
// same blocks, 4 bytes per lane over the first 32 (fp16) or 16 (E8M0) lanes.  Lanes past
// the row's last block load its last block again (their terms are masked).  M0 holds the
// LDS address of a load; it is restored afterwards.
template <int FMT>
__device__ __forceinline__ void issue_slot(const Cursor& c, uint32_t lds, int lane) {
    const uint32_t b = (uint32_t)min(64 * c.g + lane, c.nb - 1);
    uint32_t keep;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(keep)
        : "v"(16u * b), "s"(c.rp.qs), "s"(lds)
        : "memory");
    if constexpr (FMT == VQ_FMT_MXFP4) {
        const uint32_t b4 = (uint32_t)min(64 * c.g + 4 * (lane & 15), c.nb - 4);
        if (lane < 16) {
            asm volatile(
                "s_mov_b32 %0, m0\n\t"
                "s_mov_b32 m0, %3\n\t"
                "s_nop 0\n\t"
                "global_load_lds_dword %1, %2\n\t"
                "s_mov_b32 m0, %0"
                : "=&s"(keep)
                : "v"(b4), "s"(c.rp.sc), "s"(lds + 1024)
                : "memory");
        }
    } else {
        const uint32_t b2 = 2u * (uint32_t)min(64 * c.g + 2 * (lane & 31), c.nb - 2);
        if (lane < 32) {
            if constexpr (FMT == VQ_FMT_Q4_MIN) {
                asm volatile(
                    "s_mov_b32 %0, m0\n\t"
                    "s_mov_b32 m0, %3\n\t"
                    "s_nop 0\n\t"
                    "global_load_lds_dword %1, %2\n\t"
                    "s_mov_b32 m0, %5\n\t"
                    "s_nop 0\n\t"
                    "global_load_lds_dword %1, %4\n\t"
                    "s_mov_b32 m0, %0"
                    : "=&s"(keep)
                    : "v"(b2), "s"(c.rp.sc), "s"(lds + 1024), "s"(c.rp.mn), "s"(lds + 1152)
                    : "memory");
            } else {
                asm volatile(
                    "s_mov_b32 %0, m0\n\t"
                    "s_mov_b32 m0, %3\n\t"
                    "s_nop 0\n\t"
                    "global_load_lds_dword %1, %2\n\t"
                    "s_mov_b32 m0, %0"
                    : "=&s"(keep)
                    : "v"(b2), "s"(c.rp.sc), "s"(lds + 1024)
                    : "memory");
            }
        }
    }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Waits until the DONE_REPL group counters at cnt sum to `target` (thread 0 polls; the
// caller's barrier holds the other threads).  Bounded: after about a second without
// completion the error flag is raised and the pass goes on, so a launch always ends.
__device__ void wait_done(const unsigned* cnt, unsigned target, int* err) {
    if (threadIdx.x != 0) return;
    unsigned spins = 0;
    for (;;) {
        unsigned sum = 0;
#pragma unroll
        for (int r = 0; r < DONE_REPL; ++r)
            sum += __hip_atomic_load(cnt + r * DONE_STRIDE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (sum >= target) return;
        __builtin_amdgcn_s_sleep(1);
        if ((++spins & 1023u) == 0) {
            if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
            if (spins >= (1u << 20)) {
                __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return;
            }
        }
    }
}

// ----------------------------------------------------------------- stage input

// The stage's K input columns into LDS: xs[k][block][quarter ^ swizzle] in the widened
// pair order, block sums xsum[k][block] (Q4 with mins), and the fp16 copy (`keep`) by
// one workgroup.  Thread t takes quarters (8 columns) t, t + STHR, ...
template <int FMT, int K>
__device__ void stage_input(const StreamStage& A, int nbmax, bool keeper, u4_t LDS_AS* xs, float LDS_AS* xsum,
                            float LDS_AS* red) {
    constexpr int QPT = (VQ_STREAM_MAX_COLS / 8 + STHR - 1) / STHR;     // quarters per thread
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int cols = A.cols, nq = cols >> 3;
    float rs[K];
    f4_t lo[K][QPT], hi[K][QPT];
    if (A.glue == GLUE_NONE) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            rs[k] = 1.f;
#pragma unroll
            for (int i = 0; i < QPT; ++i) {
                const int qi = min((int)threadIdx.x + STHR * i, nq - 1);
                const u4_t v = ld_global<u4_t>(A.x16 + (size_t)k * cols + 8 * qi);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo[k][i][e] = half_bits_to_float(v[e >> 1] >> (16 * (e & 1)) & 0xffffu);
                    hi[k][i][e] = half_bits_to_float(v[2 + (e >> 1)] >> (16 * (e & 1)) & 0xffffu);
                }
            }
        }
    } else {
        float ss[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            ss[k] = 0.f;
#pragma unroll
            for (int i = 0; i < QPT; ++i) {
                const int q = (int)threadIdx.x + STHR * i;
                const int qi = min(q, nq - 1);
                const float* p = A.src + (size_t)k * A.ld + 8 * qi;
                lo[k][i] = ld_global<f4_t>(p);
                hi[k][i] = ld_global<f4_t>(p + 4);
                if (q < nq)
#pragma unroll
                    for (int e = 0; e < 4; ++e) ss[k] += lo[k][i][e] * lo[k][i][e] + hi[k][i][e] * hi[k][i][e];
            }
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float w = wave_sum(ss[k]);
            if (lane == 0) red[wave * K + k] = w;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < SW; ++w) t += red[w * K + k];
            rs[k] = 1.0f / __fsqrt_rn(__fdiv_rn(t, (float)cols));
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
#pragma unroll
        for (int i = 0; i < QPT; ++i) {
            const int qi = (int)threadIdx.x + STHR * i;
            if (qi < nq) {
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[e] = f2h_scaled(lo[k][i][e], rs[k]);
                    h[4 + e] = f2h_scaled(hi[k][i][e], rs[k]);
                }
                if (keeper && A.keep) {
                    u4_t v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = h[2 * e] | (h[2 * e + 1] << 16);
                    *reinterpret_cast<u4_t*>(A.keep + (size_t)k * cols + 8 * qi) = v;
                }
                u4_t pk;
#pragma unroll
                for (int t = 0; t < 4; ++t) pk[t] = h[slot_col<FMT>(2 * t)] | (h[slot_col<FMT>(2 * t + 1)] << 16);
                const int b = qi >> 2, q = qi & 3;
                xs[((size_t)k * nbmax + b) * 4 + (q ^ ((b >> 2) & 3))] = pk;
            }
        }
    }
    __syncthreads();
    if constexpr (FMT == VQ_FMT_Q4_MIN) {
        const int nb = cols >> 5;
        for (int e = threadIdx.x; e < K * nb; e += STHR) {
            const int k = e / nb, b = e - k * nb;
            float t = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u4_t pk = xs[((size_t)k * nbmax + b) * 4 + q];
                float tq = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) tq += half_bits_to_float(pk[i] & 0xffffu) + half_bits_to_float(pk[i] >> 16);
                t += tq;
            }
            xsum[k * nbmax + b] = t;
        }
        __syncthreads();
    }
}

// ----------------------------------------------------------------- the pass kernel

template <int FMT, int K>
__global__ __launch_bounds__(STHR, 1) void k_stream(const PassPlan P) {
    constexpr int D = ring_depth<K>();
    constexpr int WAITN = ndma<FMT>() * (D - 1);
    static_assert(WAITN <= 63, "vmcnt counts up to 63");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int nbmax = (P.H > P.FF ? P.H : P.FF) >> 5;
    uint8_t LDS_AS* base = (uint8_t LDS_AS*)(LDS_AS void*)smem;
    u4_t LDS_AS* xs = (u4_t LDS_AS*)(base + SW * D * SLOT);
    float LDS_AS* xsum = (float LDS_AS*)(base + SW * D * SLOT + (size_t)K * nbmax * 64);
    float LDS_AS* red = xsum + (size_t)K * nbmax;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int nwg = gridDim.x;                    // a multiple of 8
    const int grp = blockIdx.x & 7;
    const int vid = grp * (nwg >> 3) + (blockIdx.x >> 3);
    const int nw = nwg * SW, gw = vid * SW + wave;
    const uint32_t ring = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(base + wave * D * SLOT));
    const int s0 = 4 * P.layer0;
    const int s1 = 4 * (P.layer0 + P.nlayers) + (P.with_lm ? 1 : 0);

    // prime the ring: D - 1 slots ahead
    Cursor ci;
    cursor_stage(P, ci, s0, s1, gw, nw);
    if (ci.s >= s1) {                             // this wave has no rows at all: point at
        cursor_stage(P, ci, s0, s1, 0, nw);       // wave 0's first slot (repeated loads)
        ci.s = s1;
    }
    int islot = 0, cslot = 0;
#pragma unroll 1
    for (int t = 0; t < D - 1; ++t) {
        issue_slot<FMT>(ci, ring + islot * SLOT, lane);
        cursor_next(P, ci, s1, gw, nw);
        islot = islot + 1 == D ? 0 : islot + 1;
    }

#pragma unroll 1
    for (int s = s0; s < s1; ++s) {
        const int njobs = stage_jobs(P, s);
        if ((long)njobs * vid / nwg >= (long)njobs * (vid + 1) / nwg) continue;   // no rows here
        StreamStage A;
        stream_stage(P, s, A);
        if (s > s0) {
            const int pj = stage_jobs(P, s - 1);
            wait_done(P.done + (size_t)(s - 1) * DONE_WORDS, (unsigned)(pj < nwg ? pj : nwg), P.err);
        }
        __syncthreads();                          // also: every wave is done with the old input
        stage_input<FMT, K>(A, nbmax, vid == 0, xs, xsum, red);

        int j0, j1;
        wave_jobs(njobs, gw, nw, j0, j1);
        const int nb = A.cols >> 5, nsg = (nb + 63) >> 6;
        const int nsub = A.paired ? 2 : 1;
        const int rows = A.rows;
        float* const y = A.y;
#pragma unroll 1
        for (int job = j0; job < j1; ++job) {
            float g[K];
#pragma unroll 1
            for (int u = 0; u < nsub; ++u) {
                float acc[K];
#pragma unroll
                for (int k = 0; k < K; ++k) acc[k] = 0.f;
#pragma unroll 1
                for (int sg = 0; sg < nsg; ++sg) {
                    issue_slot<FMT>(ci, ring + islot * SLOT, lane);
                    cursor_next(P, ci, s1, gw, nw);
                    islot = islot + 1 == D ? 0 : islot + 1;
                    wait_vmcnt<WAITN>();          // slot cslot has landed
                    const uint8_t LDS_AS* sl = (const uint8_t LDS_AS*)(uintptr_t)(ring + cslot * SLOT);
                    cslot = cslot + 1 == D ? 0 : cslot + 1;
                    const u4_t w = *(const u4_t LDS_AS*)(sl + 16 * lane);
                    float d, m = 0.f;
                    if constexpr (FMT == VQ_FMT_MXFP4) {
                        d = e8m0_to_float(*(const uint8_t LDS_AS*)(sl + 1024 + lane));
                    } else {
                        d = half_bits_to_float(*(const uint16_t LDS_AS*)(sl + 1024 + 2 * lane));
                        if constexpr (FMT == VQ_FMT_Q4_MIN)
                            m = half_bits_to_float(*(const uint16_t LDS_AS*)(sl + 1152 + 2 * lane));
                    }
                    const int bl = 64 * sg + lane;
                    const int b = min(bl, nb - 1);
                    const float msk = bl < nb ? 1.f : 0.f;
                    h2_t p[4][4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) unpack8<FMT>(w[i], p[i]);
                    const int sw = (b >> 2) & 3;
#pragma unroll
                    for (int k = 0; k < K; ++k) {
                        float t = 0.f;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const u4_t xq = xs[((size_t)k * nbmax + b) * 4 + (i ^ sw)];
#pragma unroll
                            for (int e = 0; e < 4; ++e) t = __builtin_amdgcn_fdot2(p[i][e], as_h2(xq[e]), t, false);
                        }
                        float v = d * t;
                        if constexpr (FMT == VQ_FMT_Q4_MIN) v = fmaf(m, xsum[k * nbmax + b], v);
                        acc[k] = fmaf(v, msk, acc[k]);
                    }
                }
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const float r = wave_sum(acc[k]);
                    if (nsub == 2 && u == 0) {
                        g[k] = r;
                    } else if (lane == 0) {
                        if (nsub == 2) {
                            const int half = A.half;
                            st_shared_f32(y + (size_t)k * rows + job, g[k], true);
                            st_shared_f32(y + (size_t)k * rows + half + job, r, true);
                            st_shared_f32(A.sbuf + (size_t)k * half + job, silu_mul(g[k], r), true);
                        } else {
                            st_shared_f32(y + (size_t)k * rows + job, r, true);
                        }
                    }
                }
            }
        }
        // this workgroup's outputs of stage s are in memory: count it (every wave drains
        // its memory operations; the stores are its latest ones)
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(P.done + (size_t)s * DONE_WORDS + grp * DONE_STRIDE, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);                // ring loads still in flight land first
}

template <int FMT, int K>
const void* stream_fn() {
    return reinterpret_cast<const void*>(&k_stream<FMT, K>);
}

const void* stream_fn_of(int fmt, int K) {
    if (fmt == VQ_FMT_Q4) return K == 1 ? stream_fn<VQ_FMT_Q4, 1>() : stream_fn<VQ_FMT_Q4, 2>();
    if (fmt == VQ_FMT_Q4_MIN) return K == 1 ? stream_fn<VQ_FMT_Q4_MIN, 1>() : stream_fn<VQ_FMT_Q4_MIN, 2>();
    return K == 1 ? stream_fn<VQ_FMT_MXFP4, 1>() : stream_fn<VQ_FMT_MXFP4, 2>();
}

}  // namespace

bool stream_enabled() { return false; }

size_t stream_lds_bytes(int K, int H, int FF) {
    const int D = K == 1 ? ring_depth<1>() : ring_depth<2>();
    const size_t nbmax = (size_t)std::max(H, FF) / 32;
    return (size_t)SW * D * SLOT + (size_t)K * nbmax * 64 + (size_t)K * nbmax * 4 + (size_t)SW * K * 4;
}

int stream_supported(int fmt, int K, int H, int KV, int FF) {
    if (K < 1 || K > STREAM_MAX_K) return 0;
    if (std::max(H, FF) > VQ_STREAM_MAX_COLS) return 0;
    // whole-dword scale loads: 4-byte aligned rows of scales
    const int nbH = H / 32, nbF = FF / 32;
    if (fmt == VQ_FMT_MXFP4 ? (nbH % 4 || nbF % 4) : (nbH % 2 || nbF % 2)) return 0;
    (void)KV;
    int dev = 0, lds = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 0;
    return stream_lds_bytes(K, H, FF) <= (size_t)lds;
}

hipError_t launch_stream_segment(const PassPlan& P, hipStream_t st) {
    const void* fn = stream_fn_of(P.fmt, P.K);
    const size_t lds = stream_lds_bytes(P.K, P.H, P.FF);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    int dev = 0, cus = 0, occ = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, STHR, lds);
    if (e != hipSuccess) return e;
    if (occ < 1 || cus < 8) return hipErrorInvalidConfiguration;
    const int nwg = cus - cus % 8;
    void* args[] = {const_cast<PassPlan*>(&P)};
    // cooperative: every workgroup is resident, which the waits between stages rely on
    e = hipLaunchCooperativeKernel(fn, dim3(nwg), dim3(STHR), args, lds, st);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace vq
