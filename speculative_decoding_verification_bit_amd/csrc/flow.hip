// The verify pass's weight stream: every block-quantised weight matrix read from HBM
// once and applied to the K activation columns of the window (page "100 tokens per
// second from a 27B model on a 24 GB AMD card", sections "The wall" and "How
// speculative decoding gets past a per-token wall"; Hacker News thread 49596054: the
// window goes through each layer once).
//
// One kernel, k_flow, one workgroup per compute unit, 12 waves:
//  * waves 0..10 compute.  A stage's chunks (16 rows x 128 columns of the tiled layout:
//    1 KB of codes and the rows' block scales / mins) are split into one contiguous range
//    per workgroup, equal to within a chunk; compute wave c takes every 11th step (two
//    chunks) of its workgroup's range, keeping DEPTH steps of loads in flight in registers
//    (the loads run on across stage boundaries: weights never wait for activations).  A
//    wave's steps come from a work list built on the host (steps.h).  The 32 codes
//    of a block widen exactly to fp16 (a Q4 code n to n - 8, an E2M1 code to its value),
//    one v_mfma_f32_16x16x32_f16 per block multiplies them with the fp16 activations
//    read from LDS (products exact, fp32 sums); the block scale multiplies the fp32
//    result and, for Q4 with mins, the min multiplies the block's activation sum (a second
//    MFMA against ones), so no weight is rounded.  At the end of each unit (a tile's
//    chunks inside one column window) a wave leaves its fp32 partial in an LDS ring.
//  * wave 11 conducts.  Per stage it waits for the previous stage to complete on every
//    workgroup (device-scope counters), derives rho from the previous output's sums of
//    squares, copies the workgroup's activation windows into LDS (global_load_lds), and
//    then adds the 11 partials of every unit in wave order.  A tile that lies inside the
//    workgroup's range gets its epilogue at once; a tile split over workgroups (or column
//    windows) has its parts written to memory, and one fixed workgroup adds them in a
//    fixed order at the end of the stage.  Summation orders depend only on the shapes
//    and the grid, so every launch split of a pass gives the same bits.
//
// Stage glue of the pass (no attention, norm weights or residuals; the pages leave the
// layer internals open): a stage's input is the previous stage's fp32 output rounded to
// fp16 (the q rows of q|k|v for the o stage, silu(gate) * up for the down stage), and a
// stage scales its dot products by rho = 1 / sqrt(mean(v^2)) of that previous output v,
// so every output has the magnitude of a unit-RMS input's.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "vq_device.h"
#include "vq_internal.h"
#include "steps.h"

namespace vq {
namespace {

constexpr int NCW = FLOW_NCW;
constexpr int NTHR = 64 * (NCW + 1);
constexpr int DEPTH = ST_ROUND;         // steps (two chunks each) in flight per compute wave
constexpr unsigned SPIN_LDS = 1u << 23; // bounded waits (about a second)
constexpr unsigned SPIN_GLOBAL = 1u << 22;

// The launch's arguments, read in place from the kernel-argument segment (scalar loads;
// binding the by-value parameter to a reference would copy it to scratch memory).
typedef const __attribute__((address_space(4))) FlowArgs KArgs;
typedef __attribute__((address_space(3))) void LdsVoid;

// ------------------------------------------------------------------ small helpers

// A value every lane of the wave holds alike, kept in a scalar register.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ unsigned ld_acq(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void st_rel(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Wait until an LDS word reaches v.  A waiting wave sleeps between polls and looks at
// the abort flag only every 32 polls.  A timeout (never expected: every LDS wait is on
// work of the same workgroup or on the conductor's bounded waits) raises the error word
// and the abort flag, after which every wait returns at once, so the kernel always ends.
__device__ __forceinline__ void wait_ge(const unsigned* p, unsigned v, int* err, unsigned* abort) {
    if ((unsigned)uni((int)ld_acq(p)) >= v) return;
    unsigned n = 0;
    for (;;) {
        __builtin_amdgcn_s_sleep(2);
        if ((unsigned)uni((int)ld_acq(p)) >= v) return;
        if ((++n & 31u) == 0u) {
            if (uni((int)__hip_atomic_load(abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP))) return;
            if (n > SPIN_LDS) {
                __hip_atomic_store(abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if (err) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return;
            }
        }
    }
}

// Data other workgroups of the same launch read is written through to memory (device
// scope) and read with device-scope loads.
__device__ __forceinline__ void st_dev_f32(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u16(uint16_t* p, uint16_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev_f32(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_dev_u32(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Eight codes -> the MFMA B operand (8 fp16 in column order; the tiled layout stores the
// Q4 nibbles so that the widening below comes out in that order).
template <int FMT>
__device__ __forceinline__ h8_t widen8(uint32_t w) {
    h2_t p[4];
    unpack8<FMT>(w, p);
    h8_t r;
    r[0] = p[0][0]; r[1] = p[0][1]; r[2] = p[1][0]; r[3] = p[1][1];
    r[4] = p[2][0]; r[5] = p[2][1]; r[6] = p[3][0]; r[7] = p[3][1];
    return r;
}

// v with lane j replaced by the scalar x (v_writelane_b32; j and x wave-uniform).
__device__ __forceinline__ int writelane(int x, int j, int v) {
    x = __builtin_amdgcn_readfirstlane(x);
    j = __builtin_amdgcn_readfirstlane(j);
    // the lane select goes through M0: two SGPR operands would exceed the constant bus
    asm("s_mov_b32 m0, %2\n\tv_writelane_b32 %0, %1, m0" : "+v"(v) : "s"(x), "s"(j) : "m0");
    return v;
}

// Sum over the 16 lanes of a row of 16 (every lane gets the sum; fixed order).
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
    return v;
}

// Value of lane n + 8 (mod 16) of the lane's row of 16.
__device__ __forceinline__ float row_ror8(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
}

// ------------------------------------------------------------ stage geometry

__device__ __forceinline__ int kind_of(KArgs& A, int s) {
    if (A.linear) return SK_LIN;
    if (s == 4 * A.L) return SK_LM;
    return s & 3;
}

// Plan values of one stage kind, in scalar registers.
struct Plan {
    int T, G, nwin, gw, glast, cb, nwe, q, r, xs, rows, cols;
};
__device__ __forceinline__ Plan plan_of(KArgs& A, int kind) {
    Plan p;
    p.T = uni(A.kp[kind].T); p.G = uni(A.kp[kind].G); p.nwin = uni(A.kp[kind].nwin);
    p.gw = uni(A.kp[kind].gw); p.glast = uni(A.kp[kind].glast); p.cb = uni(A.kp[kind].cb);
    p.nwe = uni(A.kp[kind].nwe); p.q = uni(A.kp[kind].q); p.r = uni(A.kp[kind].r);
    p.xs = uni(A.kp[kind].xs); p.rows = uni(A.kp[kind].rows); p.cols = uni(A.kp[kind].cols);
    return p;
}

// Position of chunk c of a stage: window, tile, group inside the window, groups of that
// window.
struct Pos {
    int w, t, i, gl;
};
__device__ __forceinline__ Pos locate(const Plan& P, int c) {
    Pos p;
    const int span = P.T * P.gw;
    const int lastb = (P.nwin - 1) * span;
    if (c < lastb) {
        p.w = uni(c / span);
        const int r = c - p.w * span;
        p.t = uni(r / P.gw);
        p.i = r - p.t * P.gw;
        p.gl = P.gw;
    } else {
        p.w = P.nwin - 1;
        const int r = c - lastb;
        p.t = uni(r / P.glast);
        p.i = r - p.t * P.glast;
        p.gl = P.glast;
    }
    return p;
}
__device__ __forceinline__ void step_pos(const Plan& P, Pos& p, int n) {
    p.i += n;
    while (p.i >= p.gl) {
        p.i -= p.gl;
        if (++p.t == P.T) {
            p.t = 0;
            ++p.w;
            p.gl = p.w == P.nwin - 1 ? P.glast : P.gw;
        }
    }
}

// The workgroup's chunks of one stage, in processing order: segment A (the tail of its
// range when that unit continues in the next workgroup's range: done first, so that the
// workgroup finishing the tile gets both parts early), then segment B (the rest, in
// order).  Units in processing order: A's unit, then B's units in increasing index.
struct Seq {
    int n;            // chunks
    int lo, hi;       // the range [lo, hi)
    int lenA, a0;     // segment A: [a0, a0 + lenA) = [a0, hi)
    int nU;           // units
    int uA, uB0;      // flat unit (window * T + tile) of A, and of B's first
    int wlo;          // window of lo
};
__device__ __forceinline__ Seq seq_of(const Plan& P, int w) {
    Seq q;
    q.n = 0; q.lo = 0; q.hi = 0; q.lenA = 0; q.a0 = 0; q.nU = 0; q.uA = 0; q.uB0 = 0; q.wlo = 0;
    if (w >= P.nwe) return q;
    q.lo = w * P.q + (w < P.r ? w : P.r);
    q.hi = q.lo + P.q + (w < P.r ? 1 : 0);
    q.n = q.hi - q.lo;
    const Pos pl = locate(P, q.hi - 1);
    const int ustart = q.hi - 1 - pl.i;
    q.a0 = q.hi;
    if (ustart + pl.gl > q.hi) q.a0 = ustart > q.lo ? ustart : q.lo;
    q.lenA = q.hi - q.a0;
    const Pos p0 = locate(P, q.lo);
    q.wlo = p0.w;
    q.uB0 = p0.w * P.T + p0.t;
    q.uA = pl.w * P.T + pl.t;
    const int lenB = q.a0 - q.lo;
    int nb = 0;
    if (lenB > 0) {
        const Pos pb = locate(P, q.a0 - 1);
        nb = pb.w * P.T + pb.t - q.uB0 + 1;
    }
    q.nU = (q.lenA > 0 ? 1 : 0) + nb;
    return q;
}
__device__ __forceinline__ int seq_chunk(const Seq& q, int k) { return k < q.lenA ? q.a0 + k : q.lo + (k - q.lenA); }
__device__ __forceinline__ int unit_pos(const Seq& q, int U) {
    if (q.lenA > 0) return U == q.uA ? 0 : 1 + (U - q.uB0);
    return U - q.uB0;
}

// Workgroup holding chunk c.
__device__ __forceinline__ int wg_of(const Plan& P, int c) {
    const int big = P.r * (P.q + 1);
    return c < big ? c / (P.q + 1) : P.r + (c - big) / P.q;
}

// Matrix and stage input / output addresses.
__device__ __forceinline__ const uint8_t* mat_of(KArgs& A, int s, int kind) {
    if (kind == SK_LIN || kind == SK_LM) return A.lm;
    return A.w[(s >> 2) - A.l0][s & 3];
}
__device__ __forceinline__ const uint16_t* input_of(KArgs& A, int s) {
    if (s == 0 || A.linear) return A.x0;
    if (s == 4 * A.L) return (const uint16_t*)(A.ws + A.off_fx);
    return (const uint16_t*)(A.ws + (size_t)(s >> 2) * A.layer_bytes + A.off_x[s & 3]);
}

// ------------------------------------------------------------------------ kernel

template <int FMT, int KC>
__global__ void __launch_bounds__(NTHR, 1) k_flow(const FlowArgs args) {
    (void)args;
    KArgs& A = *(KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    __shared__ __attribute__((aligned(16))) uint8_t lds[FLOW_LDS];
    FlowCtrl& C = *(FlowCtrl*)(lds + FLOW_CTRL_OFF);
    const int lane = threadIdx.x & 63;
    const int wave = uni((int)(threadIdx.x >> 6));
    const int w = blockIdx.x;
    const int n16 = lane & 15, q4 = lane >> 4;
    int* const err = A.err;
    const int K = A.K;
    const int nsp = A.nsp;                  // power of two
    const int pbytes = A.pbytes;
    const int plane = pbytes >> 4;          // lanes holding partial sums (16 per 4 columns)

    if (threadIdx.x < FLOW_NSP_MAX) {
        C.pcnt[threadIdx.x] = 0;
        C.pfree[threadIdx.x] = 0;
    }
    if (threadIdx.x == 0) {
        C.xready = 0;
        C.abort = 0;
    }
    __syncthreads();

    if (wave < NCW) {
        // ============================================================ compute waves
        const int cw = wave;
        using scale_t = typename std::conditional<FMT == VQ_FMT_Q4_MIN, u4_t,
                        typename std::conditional<FMT == VQ_FMT_Q4 || FMT == VQ_FMT_Q4_K, u2_t,
                                                  uint32_t>::type>::type;
        constexpr int SB = FMT == VQ_FMT_Q4_MIN ? 16 : FMT == VQ_FMT_Q4 || FMT == VQ_FMT_Q4_K ? 8 : 4;
        const int xoff1 = A.xoff1;
        uint8_t* const ring = lds + A.ring_off;

        // The wave's work list (built on the host for this launch and grid): per step the
        // byte offset of its two chunks in the stage's matrix and a flags word (LDS offset of
        // the activations, units to close first, stage entry, valid, launch stage).  It is
        // read a round of DEPTH entries at a time, two rounds ahead, with vector loads (a
        // scalar load in flight would make every LDS wait also wait for it); the issue side
        // runs one round ahead of the consume side.
        typedef const __attribute__((address_space(4))) uint32_t CU32;
        const uint32_t first = ((CU32*)A.step_start)[w * NCW + cw];
        const uint32_t* const tab = A.steps + 2 * (size_t)first;
        // a round's 2 DEPTH words sit in lanes 0 .. 2 DEPTH - 1 of one register (one
        // dword load per lane; the other lanes load a copy)
        const int tl = lane % (2 * DEPTH);
        static_assert(2 * DEPTH <= 64, "a round fits the lanes of one register");
        uint32_t e0, e1, e2;
        auto load_round = [&](int r) __attribute__((always_inline)) -> uint32_t {
            return tab[2 * DEPTH * r + tl];
        };
        // entry u of a round: (offset, flags)
        auto ent_off = [&](uint32_t e, int u) __attribute__((always_inline)) -> uint32_t {
            return (uint32_t)__builtin_amdgcn_readlane((int)e, 2 * u);
        };
        auto ent_flags = [&](uint32_t e, int u) __attribute__((always_inline)) -> uint32_t {
            return (uint32_t)__builtin_amdgcn_readlane((int)e, 2 * u + 1);
        };
        int ib_idx = -1;                   // launch stage whose matrix ibase is
        const uint8_t* ibase = A.lm;

        f4_t acc = {0.f, 0.f, 0.f, 0.f};
        uint32_t xlane = 0;                // this lane's A-operand byte offset in a window
        unsigned useq = 0;                 // ring sequence number of the next unit to close
        // this wave's partial of the current unit into the ring (zero if it had no chunk there)
        auto close_unit = [&]() __attribute__((always_inline)) {
            const unsigned slot = useq & (unsigned)(nsp - 1), round = useq / (unsigned)nsp;
            wait_ge(&C.pfree[slot], round, err, &C.abort);
            if (lane < plane) *(f4_t*)(ring + ((int)slot * NCW + cw) * pbytes + 16 * lane) = acc;
            if (lane == 0) __hip_atomic_fetch_add(&C.pcnt[slot], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            acc = f4_t{0.f, 0.f, 0.f, 0.f};
            useq = (unsigned)uni((int)useq + 1);
        };

        // One step: two chunks (groups 2g, 2g + 1 of a tile), each 1 KB of codes and the
        // rows' scales; the second chunk follows the first.
        constexpr int CB1 = FMT == VQ_FMT_Q4_MIN ? 1280 : FMT == VQ_FMT_Q4 ? 1152 : FMT == VQ_FMT_Q4_K ? 1184 : 1088;
        u4_t rq[DEPTH][2];
        scale_t rs[DEPTH][2];
        uint32_t rk[DEPTH][2];             // Q4_K: the row's super-block D (h = 0) and Dmin (h = 1)
        // every entry names a chunk in its matrix, with or without ST_VALID: the loads are
        // unconditional, so that the wait counts of the unrolled rounds are exact
        auto issue = [&](int u, uint32_t off, uint32_t f) __attribute__((always_inline)) {
            const int idx = (int)((f >> ST_STAGE_SHIFT) & 127u);
            if (idx != ib_idx) {
                ib_idx = idx;
                const int s = A.s_begin + idx;
                ibase = mat_of(A, s, kind_of(A, s));
            }
            const uint8_t* p = ibase + off;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                rq[u][h] = ld_global_nt<u4_t>(p + h * CB1 + 16 * lane);
                rs[u][h] = ld_global_nt<scale_t>(p + h * CB1 + 1024 + SB * n16);
                if constexpr (FMT == VQ_FMT_Q4_K) rk[u][h] = ld_global_nt<uint16_t>(p + h * CB1 + 1152 + 2 * n16);
            }
        };

        // Q4 widening constants held in registers, so that each masked OR is one
        // v_and_or_b32 (a VOP3 operand cannot be a literal)
        uint32_t m_lo, m_hi, magic;
        asm volatile("s_mov_b32 %0, 0x000f000f" : "=s"(m_lo));
        asm volatile("s_mov_b32 %0, 0x00f000f0" : "=s"(m_hi));
        asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));
        // Eight codes -> the MFMA B operand (8 fp16 in column order; the tiled layout stores
        // the Q4 nibbles so that this order comes out).  A nibble OR-ed into the mantissa of
        // 1024.0 gives 1024 + n (low nibbles) or 1024 + 16 n (high nibbles); both map
        // exactly to n - 8 (Q4, Q4_MIN) or to n (Q4_K, whose codes are unsigned).
        auto widen = [&](uint32_t w) __attribute__((always_inline)) -> h8_t {
            if constexpr (FMT == VQ_FMT_MXFP4) {
                return widen8<FMT>(w);
            } else {
                constexpr float lo_off = FMT == VQ_FMT_Q4_K ? 1024.0f : 1032.0f;
                constexpr float hi_off = FMT == VQ_FMT_Q4_K ? -64.0f : -72.0f;
                const uint32_t w8 = w >> 8;
                const h2_t k1032 = {(_Float16)lo_off, (_Float16)lo_off};
                const h2_t k16 = {(_Float16)0.0625f, (_Float16)0.0625f};
                const h2_t k72 = {(_Float16)hi_off, (_Float16)hi_off};
                const h2_t p0 = as_h2((w & m_lo) | magic) - k1032;
                const h2_t p1 = as_h2((w & m_hi) | magic) * k16 + k72;
                const h2_t p2 = as_h2((w8 & m_lo) | magic) - k1032;
                const h2_t p3 = as_h2((w8 & m_hi) | magic) * k16 + k72;
                // pairs (c0, c4), (c1, c5), (c2, c6), (c3, c7) of the dword's nibbles: the
                // tiled layout puts columns 0..7 of the block quarter in that nibble order
                const u4_t r = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                                __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
                return as_h8(r);
            }
        };

        const h8_t ONES = {(_Float16)1, (_Float16)1, (_Float16)1, (_Float16)1,
                           (_Float16)1, (_Float16)1, (_Float16)1, (_Float16)1};
        constexpr int NF = KC < 4 ? KC : 4;     // accumulator elements that can hold a column < K

        auto consume = [&](int u, uint32_t f) __attribute__((always_inline)) {
            const uint32_t nclose = (f >> ST_CLOSE_SHIFT) & ST_CLOSE_MAX;
            if (__builtin_expect(nclose != 0, 0)) {
                for (uint32_t i = 0; i < nclose; ++i) close_unit();
            }
            if (!(f & ST_VALID)) return;
            if (__builtin_expect((f & ST_OPEN) != 0, 0)) {
                // the stage's activations are in LDS once the conductor says so
                const int idx = (int)((f >> ST_STAGE_SHIFT) & 127u);
                wait_ge(&C.xready, (unsigned)idx + 1u, err, &C.abort);
                const int mrow = n16 < K ? n16 : 0;
                xlane = (uint32_t)(mrow * uni(A.kp[kind_of(A, A.s_begin + idx)].xs) + 16 * q4);
            }
            const uint32_t xa = xlane + ((f & ST_XOFF_MASK) << 4);
            // Q4_K: the step is one super-block of the row; D * s and Dmin * m are exact in
            // fp32 (an fp16 times a byte)
            float kd = 0.f, kdm = 0.f;
            if constexpr (FMT == VQ_FMT_Q4_K) {
                kd = half_bits_to_float(rk[u][0]);
                kdm = -half_bits_to_float(rk[u][1]);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                h8_t a[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) a[j] = as_h8(*(const u4_t*)(lds + xa + 256 * h + 64 * j));
                const u4_t raw = rq[u][h];
                const scale_t sc = rs[u][h];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const h8_t b = widen(raw[j]);
                    const f4_t z = {0.f, 0.f, 0.f, 0.f};
                    const f4_t cj = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j], b, z, 0, 0, 0);
                    float d;
                    if constexpr (FMT == VQ_FMT_MXFP4) d = e8m0_to_float((sc >> (8 * j)) & 0xffu);
                    else if constexpr (FMT == VQ_FMT_Q4_K) d = kd * (float)((sc[0] >> (8 * j)) & 0xffu);
                    else d = half_bits_to_float((sc[j >> 1] >> ((j & 1) * 16)) & 0xffffu);
#pragma unroll
                    for (int i = 0; i < NF; ++i) acc[i] = __builtin_fmaf(d, cj[i], acc[i]);
                    if constexpr (FMT == VQ_FMT_Q4_MIN || FMT == VQ_FMT_Q4_K) {
                        // the block's min term: (sum of the column's activations) * min
                        const f4_t sj = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j], ONES, z, 0, 0, 0);
                        float mm;
                        if constexpr (FMT == VQ_FMT_Q4_K) mm = kdm * (float)((sc[1] >> (8 * j)) & 0xffu);
                        else mm = half_bits_to_float((sc[2 + (j >> 1)] >> ((j & 1) * 16)) & 0xffffu);
#pragma unroll
                        for (int i = 0; i < NF; ++i) acc[i] = __builtin_fmaf(mm, sj[i], acc[i]);
                    }
                }
            }
        };

        e0 = load_round(0);
        e1 = load_round(1);
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) issue(u, ent_off(e0, u), ent_flags(e0, u));
        for (int r = 0;; ++r) {
            e2 = load_round(r + 2);
#pragma unroll
            for (int u = 0; u < DEPTH; ++u) {
                consume(u, ent_flags(e0, u));
                issue(u, ent_off(e1, u), ent_flags(e1, u));
            }
            if (ent_flags(e0, DEPTH - 1) & ST_END) break;
            e0 = e1;
            e1 = e2;
        }
        return;
    }

    // ================================================================ conductor
    // The conductor's work (reductions, epilogues, the stage hand-over) is on the critical
    // path of every stage: it takes issue slots ahead of the compute waves on its SIMD.
    __builtin_amdgcn_s_setprio(3);
    const f4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    unsigned useq = 0;
    float stat[4];
    for (int s = A.s_begin; s < A.s_end; ++s) {
        const int idx = s - A.s_begin;
        const int kind = kind_of(A, s);
        const Plan P = plan_of(A, kind);
        const Seq q = seq_of(P, w);
        const int n_in = s == 0 ? 0 : uni(A.kp[kind].n_in);   // stage 0 is not scaled
        const bool stats_on = A.kp[kind].stats != 0;

        // -------- the previous stage complete on every workgroup
        if (n_in > 0 && idx > 0) {
            // one poll in flight (more would contend for the counters' lines); the error word
            // and the abort flag are looked at every 16 polls
            const unsigned* dn = A.done + (size_t)(s - 1) * DONE_WORDS + lane * DONE_STRIDE;
            unsigned spins = 0;
            for (;;) {
                static_assert(DONE_REPL <= 64, "one counter per lane");
                const unsigned v = lane < DONE_REPL ? ld_dev_u32(dn) : 0u;
                // a count of workgroups (<= 1024): exact as a float sum
                const unsigned sum = (unsigned)wave_sum((float)v);
                if (sum >= (unsigned)A.nwg) break;
                if ((++spins & 15u) == 0u) {
                    if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ||
                        __hip_atomic_load(&C.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP))
                        break;
                    if (spins > SPIN_GLOBAL) {
                        __hip_atomic_store(&C.abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                        __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }

        // -------- the stage's activation windows into LDS
        if (q.n > 0) {
            const uint16_t* X = input_of(A, s);
            const Pos ph = locate(P, q.hi - 1);
            for (int win = q.wlo; win <= ph.w; ++win) {
                uint8_t* xb = lds + (win - q.wlo) * A.xoff1;
                const int g0 = win * P.gw;
                const int gl = win == P.nwin - 1 ? P.glast : P.gw;
                const int c0 = g0 * STEP_COLS;
                const int cend = min(P.cols, (g0 + gl) * STEP_COLS);
                const int Rb = (cend - c0) * 2, Wb = gl * 512;
                for (int m = 0; m < K; ++m) {
                    const char* src = (const char*)(X + (size_t)m * P.cols + c0);
                    uint8_t* dst = xb + m * P.xs;
                    if (Rb >= 1024) {
                        for (int p = 0; p < Rb; p += 1024) {
                            const int o = min(p, Rb - 1024);
                            __builtin_amdgcn_global_load_lds((const void*)(src + o + 16 * lane), (LdsVoid*)(dst + o),
                                                             16, 0, 0);
                        }
                    } else if (16 * lane < Rb) {
                        *(u4_t*)(dst + 16 * lane) = *(const u4_t*)(src + 16 * lane);
                    }
                    for (int o = Rb + 16 * lane; o < Wb; o += 1024) *(u4_t*)(dst + o) = u4_t{0u, 0u, 0u, 0u};
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
        }
        // stage 0 keeps a copy of the pass input with the other stage inputs
        if (s == 0 && !A.linear && w == 0) {
            uint16_t* keep = (uint16_t*)(A.ws + A.off_x[0]);
            for (int i = lane; i < K * A.H; i += 64) keep[i] = A.x0[i];
        }
        if (lane == 0) st_rel(&C.xready, (unsigned)idx + 1u);

        // -------- rho of the previous output (only the epilogues need it: after the
        // activations are released to the compute waves)
        if (n_in > 0) {
            // sum over workgroups in a fixed order: lane l adds workgroups 4l .. 4l + 3 (and
            // 256 on), then the wave's fixed tree; the sums of one column are contiguous, so
            // every load of the stage's figures is in flight at once
            const float* st = (const float*)(A.ws + A.off_stats) + (size_t)(s - 1) * A.stats_stride;
            float a[VQ_MAX_K];
#pragma unroll
            for (int m = 0; m < VQ_MAX_K; ++m) a[m] = 0.f;
            for (int b = 0; b < A.nwg; b += 256) {
                f4_t v[VQ_MAX_K];
#pragma unroll
                for (int m = 0; m < VQ_MAX_K; ++m)
                    v[m] = *(const f4_t*)(st + (size_t)min(m, K - 1) * FLOW_MAX_WG + b + 4 * lane);
#pragma unroll
                for (int m = 0; m < VQ_MAX_K; ++m) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (b + 4 * lane + i < A.nwg) a[m] += v[m][i];
                }
            }
#pragma unroll
            for (int m = 0; m < VQ_MAX_K; ++m) {
                if (m < K) {
                    const float t = wave_sum(a[m]);
                    if (lane == 0) C.rho[m] = __frcp_rn(__fsqrt_rn(__fdiv_rn(t, (float)n_in)));
                }
            }
        } else if (lane < VQ_MAX_K) {
            C.rho[lane] = 1.0f;
        }


        // -------- units: reduce the 11 partials, then epilogue or part
        const float* rho = C.rho;
        auto epilogue = [&](int t, const f4_t& sum) __attribute__((always_inline)) {
            float sq[4] = {0.f, 0.f, 0.f, 0.f};
            const bool chain = kind != SK_LIN && kind != SK_LM;
            const bool last_down = kind == SK_DOWN && s + 1 == 4 * A.L;
            const char* lb = A.ws + (size_t)(s >> 2) * A.layer_bytes;
            const char* nb = A.ws + (size_t)((s + 1) >> 2) * A.layer_bytes;
            float* yout = chain ? (float*)(lb + A.off_y[s & 3]) : nullptr;
            uint16_t* xn = chain ? (last_down ? (uint16_t*)(A.ws + A.off_fx) : (uint16_t*)(nb + A.off_x[(s + 1) & 3]))
                                 : nullptr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * q4 + i;
                const bool mv = m < K;
                const float y = mv ? __fmul_rn(sum[i], rho[m]) : 0.f;
                if (!chain) {
                    const int r = 16 * t + n16;
                    if (mv && r < P.rows) {
                        if (kind == SK_LIN && A.y_dtype == VQ_DTYPE_F16)
                            ((uint16_t*)A.out)[(size_t)m * P.rows + r] = (uint16_t)f2h_bits(y);
                        else
                            ((float*)A.out)[(size_t)m * P.rows + r] = y;
                    }
                    continue;
                }
                if (kind == SK_GU) {
                    const int r = 8 * t + (n16 & 7);
                    if (mv) yout[(size_t)m * P.rows + (n16 < 8 ? r : A.FF + r)] = y;
                    const float u = row_ror8(y);
                    if (n16 < 8 && mv) {
                        const float sv = silu_mul(y, u);
                        st_dev_u16(xn + (size_t)m * A.FF + r, (uint16_t)f2h_bits(sv));
                        sq[i] = sv * sv;
                    }
                } else {
                    const int r = 16 * t + n16;
                    if (mv) yout[(size_t)m * P.rows + r] = y;
                    if (mv && (kind != SK_QKV || r < A.H)) {
                        st_dev_u16(xn + (size_t)m * A.H + r, (uint16_t)f2h_bits(y));
                        sq[i] = y * y;
                    }
                }
            }
            if (chain) {
#pragma unroll
                for (int i = 0; i < 4; ++i) stat[i] += row16_sum(sq[i]);
            }
        };
        // split-tile bookkeeping
        auto part_slot = [&](int U, int t, int side) __attribute__((always_inline)) -> float* {
            const int sl = P.nwin == 1 ? (idx * A.nwg + (side == 0 ? w : w - 1)) * 2 + side : 2 * U + side;
            return A.parts + (size_t)sl * (pbytes >> 2);
        };
        auto counter = [&](int t, int side) __attribute__((always_inline)) -> unsigned* {
            return A.cnt + (P.nwin == 1 ? (side == 0 ? w : w - 1) : t);
        };

#pragma unroll
        for (int i = 0; i < 4; ++i) stat[i] = 0.f;
        int npend = 0;
        int nrel = 0;                            // parts stored whose counters are not yet raised
        auto flush_rel = [&]() __attribute__((always_inline)) {
            __builtin_amdgcn_s_waitcnt(0);
            for (int j = lane; j < nrel; j += 64)
                __hip_atomic_fetch_add(A.cnt + C.rel_t[j], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            nrel = 0;
        };
        // one window: a split tile's second part is this workgroup's (kept in registers, it
        // is the first unit of its range); the first part comes from the previous workgroup.
        // Half-way through the units its counter is read once (the load stays in flight while
        // the other units are reduced), so that a part already there needs no polling.
        f4_t own = zero4;
        int own_t = -1;
        bool early = false;
        unsigned cload = 0;
        unsigned* const pcn = A.cnt + (w > 0 ? w - 1 : 0);
        int uw = 0, ut = 0;                      // window and tile of the unit at position pos
        for (int pos = 0; pos < q.nU; ++pos) {
            int U;
            if (q.lenA > 0 && pos == 0) U = q.uA;
            else U = q.uB0 + pos - (q.lenA > 0 ? 1 : 0);
            uw = uni(U / P.T);
            ut = U - uw * P.T;
            const unsigned sq_ = useq + (unsigned)pos;
            const unsigned slot = sq_ & (unsigned)(nsp - 1), round = sq_ / (unsigned)nsp;
            if (own_t >= 0 && !early && 2 * pos >= q.nU) {
                cload = ld_dev_u32(pcn);
                early = true;
            }
            wait_ge(&C.pcnt[slot], (unsigned)NCW * (round + 1u), err, &C.abort);
            f4_t sum = zero4;
            if (lane < plane) {
#pragma unroll
                for (int c = 0; c < NCW; ++c) sum += *(const f4_t*)(lds + A.ring_off + ((int)slot * NCW + c) * pbytes + 16 * lane);
            }
            // free the slot once the ring reads are done (an LDS wait only: a release here
            // would also wait for every epilogue store in flight)
            __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0)
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (lane == 0) __hip_atomic_store(&C.pfree[slot], round + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            // where this unit's chunks lie
            const int gl = uw == P.nwin - 1 ? P.glast : P.gw;
            const int f = uw * P.T * P.gw + ut * gl;
            const int l = f + gl - 1;
            const bool has_first = f >= q.lo, has_last = l < q.hi;
            if (P.nwin == 1 && has_first && has_last) {
                epilogue(ut, sum);
            } else if (P.nwin == 1 && !has_first) {
                own = sum;
                own_t = ut;
            } else {
                const int side = has_first ? 0 : 1;
                float* ps = part_slot(U, ut, side);
                if (lane < plane) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) st_dev_f32(ps + 4 * lane + i, sum[i]);
                }
                if (P.nwin == 1) {
                    // one window: the next workgroup's finisher waits for this part early
                    __builtin_amdgcn_s_waitcnt(0);
                    if (lane == 0)
                        __hip_atomic_fetch_add(counter(ut, side), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } else {
                    // several windows: the counters are raised together after the unit loop
                    // (one wait for the stores instead of one per unit)
                    if (lane == 0) C.rel_t[nrel] = ut;
                    if (++nrel == FLOW_REL_MAX) flush_rel();
                }
                // several windows: the finisher of a tile is the workgroup holding the last
                // chunk of the tile's unit in window t mod nwin
                if (P.nwin > 1) {
                    const int wf = ut % P.nwin;
                    const int glf = wf == P.nwin - 1 ? P.glast : P.gw;
                    const int lf = wf * P.T * P.gw + (ut + 1) * glf - 1;
                    if (lf >= q.lo && lf < q.hi && wf == uw && npend < FLOW_PEND_MAX) {
                        if (lane == 0) C.pend_t[npend] = ut;
                        ++npend;
                    }
                }
            }
        }
        useq += (unsigned)q.nU;
        if (nrel > 0) flush_rel();

        // -------- finish the split tiles this workgroup owns
        auto poll = [&](const unsigned* cn, unsigned expect) __attribute__((always_inline)) {
            unsigned spins = 0;
            while (ld_dev_u32(cn) < expect) {
                if ((++spins & 15u) == 0u &&
                    (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ||
                     __hip_atomic_load(&C.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)))
                    break;
                __builtin_amdgcn_s_sleep(1);
                if (spins > SPIN_GLOBAL) {
                    __hip_atomic_store(&C.abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        };
        if (own_t >= 0) {
            // the previous workgroup's part (slot side 0 of its boundary), then this one's
            if (!early || (unsigned)uni((int)cload) < 1u) poll(pcn, 1u);
            f4_t sum = zero4;
            if (lane < plane) {
                const float* p0 = A.parts + (size_t)((idx * A.nwg + w - 1) * 2) * (pbytes >> 2);
                sum = *(const f4_t*)(p0 + 4 * lane) + own;
            }
            epilogue(own_t, sum);
            if (lane == 0) __hip_atomic_store(pcn, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // several windows: the tiles listed above.  Lane j watches tile j's counter, so one
        // poll round covers them all.
        if (npend > 0) {
            int tl = 0;
            unsigned el = 0u;
            if (lane < npend) {
                tl = C.pend_t[lane];
                for (int win = 0; win < P.nwin; ++win) {
                    const int gl = win == P.nwin - 1 ? P.glast : P.gw;
                    const int f = win * P.T * P.gw + tl * gl;
                    el += wg_of(P, f) != wg_of(P, f + gl - 1) ? 2u : 1u;
                }
            }
            unsigned spins = 0;
            for (;;) {
                const unsigned v = lane < npend ? ld_dev_u32(A.cnt + tl) : el;
                if (__builtin_amdgcn_ballot_w64(v < el) == 0) break;
                if ((++spins & 15u) == 0u &&
                    (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ||
                     __hip_atomic_load(&C.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)))
                    break;
                __builtin_amdgcn_s_sleep(1);
                if (spins > SPIN_GLOBAL) {
                    __hip_atomic_store(&C.abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
        // Then each tile in list order.  Its parts are read four windows (eight parts) at a
        // time with every load in flight together: one round trip per four windows, not one
        // per part (a missing part is zero, which leaves the sum's bits as they are).
        constexpr int PW = 4;
        auto issue_parts = [&](int t, int w0, f4_t (&v)[2 * PW]) __attribute__((always_inline)) {
#pragma unroll
            for (int k = 0; k < PW; ++k) {
                v[2 * k] = zero4;
                v[2 * k + 1] = zero4;
                const int win = w0 + k;
                if (win < P.nwin && lane < plane) {
                    const int gl = win == P.nwin - 1 ? P.glast : P.gw;
                    const int f = win * P.T * P.gw + t * gl;
                    // the unit has a second part when it runs past the end of the range of
                    // the workgroup holding its first chunk (one division, not two)
                    const int i0 = wg_of(P, f);
                    const int end = (i0 + 1) * P.q + min(i0 + 1, P.r);
                    const float* ps = A.parts + (size_t)(2 * (win * P.T + t)) * (pbytes >> 2);
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[2 * k][i] = ld_dev_f32(ps + 4 * lane + i);
                    if (f + gl - 1 >= end) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) v[2 * k + 1][i] = ld_dev_f32(ps + (pbytes >> 2) + 4 * lane + i);
                    }
                }
            }
        };
        auto add_parts = [&](f4_t& sum, const f4_t (&v)[2 * PW]) __attribute__((always_inline)) {
#pragma unroll
            for (int k = 0; k < 2 * PW; ++k) sum += v[k];
        };
        for (int j = 0; j < npend; ++j) {
            const int t = uni(C.pend_t[j]);
            f4_t sum = zero4;
            for (int w0 = 0; w0 < P.nwin; w0 += PW) {
                f4_t v[2 * PW];
                issue_parts(t, w0, v);
                add_parts(sum, v);
            }
            epilogue(t, sum);
            if (lane == 0) __hip_atomic_store(A.cnt + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        // -------- report the stage: sums of squares, then the completion counter
        if (stats_on && n16 == 0) {
            float* st = (float*)(A.ws + A.off_stats) + (size_t)s * A.stats_stride + w;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * q4 + i;
                if (m < K) st_dev_f32(st + (size_t)m * FLOW_MAX_WG, stat[i]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        if (A.done && lane == 0)
            __hip_atomic_fetch_add(A.done + (size_t)s * DONE_WORDS + (w & (DONE_REPL - 1)) * DONE_STRIDE, 1u,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ------------------------------------------------------------------ tiling

// Nibble p of a Q4 code dword in the tiled layout holds column kPairSrc[p] of the 8.
__device__ __forceinline__ uint32_t q4_to_pair_order(uint32_t v) {
    uint32_t o = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int src = (p < 4) ? 2 * p : 2 * (p - 4) + 1;
        o |= ((v >> (4 * src)) & 0xFu) << (4 * p);
    }
    return o;
}

// One workgroup of 64 threads per chunk of the tiles that rows [row0, row0 + W.rows)
// touch; thread l = n + 16 q writes the lane-l codes and, for q = 0, row n's scales.
__global__ void k_tile(vq_matrix W, uint8_t* dst, int dst_rows, int order, int row0, int t0, int G, int cb) {
    const int t = t0 + blockIdx.y;
    const int g = blockIdx.x;
    const int l = threadIdx.x;
    const int n = l & 15, q = l >> 4;
    // logical row of tile row n
    int R;
    if (order == VQ_ROWS_PAIR8) R = n < 8 ? 8 * t + n : dst_rows / 2 + 8 * t + (n - 8);
    else R = 16 * t + n;
    const bool pad = R >= dst_rows;
    const bool mine = R >= row0 && R < row0 + W.rows;
    if (!pad && !mine) return;
    const int sr = R - row0;
    const int nb = W.cols / 32;
    uint8_t* chunk = dst + ((size_t)t * G + g) * cb;
    u4_t codes = {0u, 0u, 0u, 0u};
    uint32_t sc[4] = {0, 0, 0, 0}, mn[4] = {0, 0, 0, 0};
    uint32_t sup = 0;
    const bool bytes = W.format == VQ_FMT_MXFP4 || W.format == VQ_FMT_Q4_K;   // one-byte scales
    if (mine) {
        const uint8_t* qs = (const uint8_t*)W.qs + (size_t)sr * (W.cols / 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = 4 * g + j;
            if (b < nb) {
                const uint32_t v = *(const uint32_t*)(qs + 16 * b + 4 * q);
                codes[j] = W.format == VQ_FMT_MXFP4 ? v : q4_to_pair_order(v);
                if (bytes) sc[j] = ((const uint8_t*)W.scales)[(size_t)sr * nb + b];
                else sc[j] = ((const uint16_t*)W.scales)[(size_t)sr * nb + b];
                if (W.format == VQ_FMT_Q4_MIN) mn[j] = ((const uint16_t*)W.mins)[(size_t)sr * nb + b];
                if (W.format == VQ_FMT_Q4_K) mn[j] = ((const uint8_t*)W.mins)[(size_t)sr * nb + b];
            }
        }
        // Q4_K: cols % 256 == 0, so group g lies in super-block g / 2 of the row; the even
        // group's chunk carries its D, the odd group's its Dmin
        if (W.format == VQ_FMT_Q4_K)
            sup = ((const uint16_t*)W.supers)[((size_t)sr * (W.cols / 256) + g / 2) * 2 + (g & 1)];
    }
    *(u4_t*)(chunk + 16 * l) = codes;
    if (q == 0) {
        uint8_t* s = chunk + 1024;
        if (W.format == VQ_FMT_MXFP4) {
            const uint32_t e = sc[0] | (sc[1] << 8) | (sc[2] << 16) | ((uint32_t)sc[3] << 24);
            *(uint32_t*)(s + 4 * n) = e;
        } else if (W.format == VQ_FMT_Q4) {
            const u2_t v = {sc[0] | ((uint32_t)sc[1] << 16), sc[2] | ((uint32_t)sc[3] << 16)};
            *(u2_t*)(s + 8 * n) = v;
        } else if (W.format == VQ_FMT_Q4_K) {
            const u2_t v = {sc[0] | (sc[1] << 8) | (sc[2] << 16) | (sc[3] << 24),
                            mn[0] | (mn[1] << 8) | (mn[2] << 16) | (mn[3] << 24)};
            *(u2_t*)(s + 8 * n) = v;
            *(uint16_t*)(s + 128 + 2 * n) = (uint16_t)sup;
        } else {
            const u4_t v = {sc[0] | ((uint32_t)sc[1] << 16), sc[2] | ((uint32_t)sc[3] << 16),
                            mn[0] | ((uint32_t)mn[1] << 16), mn[2] | ((uint32_t)mn[3] << 16)};
            *(u4_t*)(s + 16 * n) = v;
        }
    }
}

__global__ void k_zero_u32(unsigned* p, size_t n) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

template <int FMT, int KC>
hipError_t launch_t(const FlowArgs& A, hipStream_t st) {
    const bool coop = A.s_end - A.s_begin > 1;
    if (coop) {
        void* args[] = {(void*)&A};
        return hipLaunchCooperativeKernel((const void*)k_flow<FMT, KC>, dim3(A.nwg), dim3(NTHR), args, 0, st);
    }
    k_flow<FMT, KC><<<dim3(A.nwg), dim3(NTHR), 0, st>>>(A);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_f(const FlowArgs& A, hipStream_t st) {
    if (A.K <= 1) return launch_t<FMT, 1>(A, st);
    if (A.K <= 4) return launch_t<FMT, 4>(A, st);
    return launch_t<FMT, 16>(A, st);
}

}  // namespace

hipError_t launch_tile(const vq_matrix& W, uint8_t* dst, int dst_rows, int order, int row0, hipStream_t st) {
    const int G = 2 * ((W.cols + STEP_COLS - 1) / STEP_COLS);   // even: zero chunks pad the last step
    int t0, t1;
    if (order == VQ_ROWS_PAIR8) {
        const int half = dst_rows / 2;
        const int r0 = row0 < half ? row0 : row0 - half;
        t0 = r0 / 8;
        t1 = (r0 + W.rows + 7) / 8;
    } else {
        t0 = row0 / TILE_ROWS;
        t1 = (row0 + W.rows + TILE_ROWS - 1) / TILE_ROWS;
    }
    if (t1 <= t0) return hipSuccess;
    k_tile<<<dim3(G, t1 - t0), 64, 0, st>>>(W, dst, dst_rows, order, row0, t0, G, chunk_bytes(W.format));
    return hipGetLastError();
}

hipError_t launch_zero_u32(unsigned* p, size_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    k_zero_u32<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(p, n);
    return hipGetLastError();
}

hipError_t launch_flow(const FlowArgs& A, hipStream_t st) {
    switch (A.fmt) {
        case VQ_FMT_Q4: return launch_f<VQ_FMT_Q4>(A, st);
        case VQ_FMT_Q4_MIN: return launch_f<VQ_FMT_Q4_MIN>(A, st);
        case VQ_FMT_Q4_K: return launch_f<VQ_FMT_Q4_K>(A, st);
        default: return launch_f<VQ_FMT_MXFP4>(A, st);
    }
}

int flow_grid() {
    static int n = 0;
    if (n == 0) {
        int dev = 0, cu = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cu > 0)
            n = std::min(cu, FLOW_MAX_WG);
        else
            n = 256;
    }
    return n;
}

}  // namespace vq
