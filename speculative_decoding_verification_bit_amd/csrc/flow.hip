// The verify pass's weight stream: every block-quantised weight matrix read from HBM
// once and applied to the K activation columns of the window (page "100 tokens per
// second from a 27B model on a 24 GB AMD card", sections "The wall" and "How
// speculative decoding gets past a per-token wall"; Hacker News thread 49596054: the
// window goes through each layer once).
//
// One kernel, k_flow, one workgroup per compute unit, 12 waves:
//  * waves 0..3 are loaders.  The workgroup's weights for the whole launch form one
//    sequence of chunks (16 rows x 4 blocks of 32 columns: 1 KB of codes, the 64 block
//    scales and, for Q4 with mins, the 64 mins).  Loader w streams chunks w, w+4, ... with
//    DEPTH chunks of 16-byte loads in flight in registers and copies each into a slot of
//    an LDS ring, publishing it with a release store of its sequence number.  Loaders
//    never wait for the activations, so the weight stream runs on across stage
//    boundaries while the compute waves wait for the previous stage.
//  * waves 4..11 compute.  Compute wave c takes, for every tile of 16 rows, the column
//    groups c, c+8, ... of the row, reads each chunk out of the ring and frees the slot.
//    The 32 weights of a block are widened exactly to fp16 (a Q4 code n becomes n - 8,
//    an E2M1 code its value) and one v_mfma_f32_16x16x32_f16 per block multiplies them
//    with the fp16 activations (products exact, fp32 accumulation); the block scale is
//    applied to the fp32 result, and for Q4 with mins the min times the block's input
//    sum (a second MFMA against ones) is added, so w = d q + m is never rounded.
//    A tile's 8 partial sums meet in LDS and are added in wave order by one wave,
//    which also writes the tile's outputs.
//  * the pass's stages depend on one another through the previous output; a stage's
//    workgroups count themselves on 8 completion counters (device-scope atomics) after
//    their outputs are written through to memory, and wave 4 of every workgroup waits
//    for the count before the compute waves read the stage's input.
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

namespace vq {
namespace {

constexpr int NLD = 4;                  // loader waves
constexpr int NCW = 8;                  // compute waves
constexpr int NTHR = 64 * (NLD + NCW);
constexpr int SLOT = 1280;              // bytes per ring slot: codes, scales, mins
constexpr int NSLOT = 96;               // ring slots (a multiple of NLD)
constexpr int DEPTH = 12;               // chunks in flight per loader wave
constexpr unsigned SPIN_LDS = 1u << 23; // bounded waits (about a second)
constexpr unsigned SPIN_GLOBAL = 1u << 22;

// The launch's arguments, read in place from the kernel-argument segment (scalar loads;
// binding the by-value parameter to a reference would copy it to scratch memory).
typedef const __attribute__((address_space(4))) FlowArgs KArgs;

struct Lds {
    uint8_t ring[NSLOT][SLOT];
    unsigned full[NSLOT];        // sequence number + 1 of the chunk in the slot
    unsigned cons[NSLOT];        // times the slot has been consumed
    f4_t part[2][NCW][64];       // tile partial sums, by tile parity
    unsigned pcnt[2];            // partials written (8 per tile)
    unsigned pdone[2];           // tiles of this parity reduced
    unsigned send;               // compute waves that finished the current stage
    unsigned open;               // last stage whose input may be read
    unsigned rho_seq;            // last stage whose input scale is in rho
    unsigned abort;              // set by the first wait that times out: later waits return at once
    float rho[VQ_MAX_K];
    float tstat[NCW][VQ_MAX_K];  // sums of squares per compute wave for the current stage
};

// ------------------------------------------------------------------ small helpers

// A value every lane of the wave holds alike, kept in a scalar register.  Without this the
// compiler can treat wave-uniform values (spin-loop results, the stage cursor) as per-lane
// and index the kernel arguments with vector loads, whose waits would drain the weight
// loads in flight.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ unsigned uni(unsigned v) { return (unsigned)__builtin_amdgcn_readfirstlane((int)v); }

__device__ __forceinline__ unsigned ld_acq(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void st_rel(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Wait until an LDS word reaches v.  A waiting wave sleeps between polls and looks at
// the abort flag only every 32 polls: in a stream bound by memory the consumers are
// usually early, and tight polling by many waves would take the scalar unit the loaders
// need.  A timeout (never expected: every wait is on work of the same workgroup) raises
// the error word and the workgroup's abort flag, after which every wait returns at once,
// so the kernel always ends.
__device__ __forceinline__ void wait_ge(const unsigned* p, unsigned v, int* err, unsigned* abort) {
    if (uni(ld_acq(p)) >= v) return;
    unsigned n = 0;
    for (;;) {
        __builtin_amdgcn_s_sleep(2);
        if (uni(ld_acq(p)) >= v) return;
        if ((++n & 31u) == 0u) {
            if (uni(__hip_atomic_load(abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP))) return;
            if (n > SPIN_LDS) {
                __hip_atomic_store(abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if (err) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return;
            }
        }
    }
}

// Stores of data that other workgroups of the same launch read: written through to
// memory (device scope), so that a reader's first miss finds them.
__device__ __forceinline__ void st_dev_f32(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u16(uint16_t* p, uint16_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// fp16 activations as the MFMA A operand: Q4 codes widen to the pairs (c0,c4), (c1,c5),
// (c2,c6), (c3,c7) of each 8-column group, so the activations take the same order.
__device__ __forceinline__ u4_t perm_pairs(u4_t v) {
    u4_t o;
    o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
    o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
    o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
    o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
    return o;
}

// Position of column c (0..7 of an aligned group of 8) in that order.
__device__ __forceinline__ int pair_pos(int c) { return 2 * (c & 3) + (c >> 2); }

// 4x4 transpose of dwords across the lane quarters: lane (n, q) holds the 4 dwords of
// block q of its row; afterwards register j holds dword q of block j (the 8 codes of
// k-quarter q that MFMA j needs).
__device__ __forceinline__ void quarter_transpose(u4_t v, uint32_t (&t)[4]) {
    auto a = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
    auto b = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
    auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    t[0] = c[0];
    t[1] = c[1];
    t[2] = d[0];
    t[3] = d[1];
}

// Eight codes -> the B operand (8 fp16 in k order).
template <int FMT>
__device__ __forceinline__ h8_t widen8(uint32_t w) {
    h2_t p[4];
    unpack8<FMT>(w, p);
    h8_t r;
    r[0] = p[0][0]; r[1] = p[0][1]; r[2] = p[1][0]; r[3] = p[1][1];
    r[4] = p[2][0]; r[5] = p[2][1]; r[6] = p[3][0]; r[7] = p[3][1];
    return r;
}

// Scale of block j (0..3) of the lane's row as fp32, from the 4 packed 16-bit entries.
template <int FMT>
__device__ __forceinline__ float block_scale(u2_t sc, int j) {
    const uint32_t w = (j < 2) ? sc.x : sc.y;
    const uint32_t h = (j & 1) ? (w >> 16) : (w & 0xffffu);
    if constexpr (FMT == VQ_FMT_MXFP4) return e8m0_to_float(h & 0xffu);
    else return half_bits_to_float(h);
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

// ------------------------------------------------------------ stage iteration

__device__ __forceinline__ StageGeo uni_geo(const StageGeo& g) {
    StageGeo r;
    r.kind = uni(g.kind); r.rows = uni(g.rows); r.cols = uni(g.cols); r.nb = uni(g.nb);
    r.G = uni(g.G); r.T = uni(g.T); r.n_in = uni(g.n_in);
    return r;
}

// Walks the workgroup's tiles, stage by stage: tile t of stage s belongs to workgroup
// (base_s + t) mod nwg, with base_s (from the host) advancing by each stage's tile count, so
// consecutive stages deal their tiles on from where the previous one stopped.
struct TileCursor {
    int s;          // stage (>= s_end: finished)
    int t;          // current tile of stage s
    StageGeo g;
};

// The workgroup's first tile in a stage dealt from offset base (both < nwg).
__device__ __forceinline__ int first_tile(int w, int base, int nwg) {
    const int t = w - base;
    return t < 0 ? t + nwg : t;
}

// Position the cursor on the first stage >= c.s in which the workgroup owns a tile.
__device__ __forceinline__ void seek_stage(KArgs& A, TileCursor& c, int w) {
    c.s = uni(c.s);
    while (c.s < A.s_end) {
        c.g = uni_geo(stage_geo(A, c.s));
        c.t = uni(first_tile(w, A.base[c.s - A.s_begin], A.nwg));
        if (c.t < c.g.T) return;
        c.s = uni(c.s + 1);
    }
}

__device__ __forceinline__ void next_tile(KArgs& A, TileCursor& c, int w) {
    c.t = uni(c.t + A.nwg);
    if (c.t >= c.g.T) {
        c.s = uni(c.s + 1);
        seek_stage(A, c, w);
    }
}

// Row pointers of lane n (0..15) of tile t of stage s: codes, scales, mins, and
// whether the row exists (the last tile of a stage may be partial).
struct RowPtr {
    const uint8_t* qs;
    const uint8_t* sc;
    const uint8_t* mn;
    bool valid;
};

__device__ __forceinline__ MatPtr mat_of(KArgs& A, int li, int j) {
    MatPtr r;
    if (li < 0) {
        r.qs = A.lm.qs; r.sc = A.lm.sc; r.mn = A.lm.mn;
    } else {
        r.qs = A.m[li][j].qs; r.sc = A.m[li][j].sc; r.mn = A.m[li][j].mn;
    }
    return r;
}

template <int FMT>
__device__ __forceinline__ RowPtr row_ptr(KArgs& A, const StageGeo& g, int s, int t, int n) {
    // The matrix is chosen per tile (wave-uniform: scalar loads of the kernel arguments);
    // only gate|up picks between two matrices per lane.
    MatPtr mp;
    int r;
    if (g.kind == SK_LIN || g.kind == SK_LM) {
        mp = mat_of(A, -1, 0);
        r = 16 * t + n;
    } else {
        const int li = uni((s >> 2) - A.l0);
        if (g.kind == SK_QKV) {
            const int r0 = 16 * t;      // a tile lies inside one of q, k, v (sizes multiples of 16)
            const int seg = r0 < A.H ? 0 : (r0 < A.H + A.KV ? 1 : 2);
            mp = mat_of(A, li, uni(seg));
            r = r0 - (seg == 0 ? 0 : (seg == 1 ? A.H : A.H + A.KV)) + n;
        } else if (g.kind == SK_GU) {
            const MatPtr mg = mat_of(A, li, 4), mu = mat_of(A, li, 5);
            mp.qs = n < 8 ? mg.qs : mu.qs;
            mp.sc = n < 8 ? mg.sc : mu.sc;
            mp.mn = n < 8 ? mg.mn : mu.mn;
            r = 8 * t + (n & 7);
        } else {
            mp = mat_of(A, li, g.kind == SK_O ? 3 : 6);
            r = 16 * t + n;
        }
    }
    RowPtr p;
    const int rows_here = (g.kind == SK_LIN || g.kind == SK_LM) ? g.rows : 0x7fffffff;
    p.valid = r < rows_here;
    if (!p.valid) r = rows_here - 1;
    const size_t rr = (size_t)r;
    p.qs = mp.qs + rr * (size_t)(g.cols >> 1);
    constexpr int SB = FMT == VQ_FMT_MXFP4 ? 1 : 2;
    p.sc = (const uint8_t*)mp.sc + rr * (size_t)g.nb * SB;
    p.mn = (const uint8_t*)mp.mn + rr * (size_t)g.nb * 2;
    return p;
}

// ----------------------------------------------------------------------- loader

// One chunk's loads for lane (n, q): the 16 code bytes of block 4g + q of row n, its
// scale and (Q4 with mins) its min.  Blocks past the row's end load block 0 and are
// zeroed when stored.
template <int FMT>
struct LoadCursor {
    TileCursor tc;
    int g;                    // group of the current tile
    RowPtr rp;                // the lane's row
    int nb;                   // blocks of that row
    int done;                 // 1 when the sequence is exhausted (block 0 of the last row is re-read)
};

template <int FMT>
__device__ __forceinline__ void lc_row(KArgs& A, LoadCursor<FMT>& c, int n) {
    c.rp = row_ptr<FMT>(A, c.tc.g, c.tc.s, c.tc.t, n);
    c.nb = c.tc.g.nb;
}

template <int FMT>
__device__ __forceinline__ void lc_advance(KArgs& A, LoadCursor<FMT>& c, int w, int n, int steps) {
    if (c.done) return;
    c.g = uni(c.g + steps);
    if (c.g < c.tc.g.G) return;
    while (c.g >= c.tc.g.G) {
        c.g = uni(c.g - c.tc.g.G);
        next_tile(A, c.tc, w);
        if (c.tc.s >= A.s_end) {
            c.done = 1;      // stay on the last row (a valid address to re-read)
            c.g = 0;
            return;
        }
    }
    lc_row<FMT>(A, c, n);
}

// ------------------------------------------------------------------------ kernel

template <int FMT, int KC>
__global__ void __launch_bounds__(NTHR, 1) k_flow(const FlowArgs args) {
    (void)args;
    KArgs& A = *(KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    __shared__ Lds S;
    const int lane = threadIdx.x & 63;
    const int wave = uni((int)(threadIdx.x >> 6));    // wave-uniform: scalar branches
    const int w = blockIdx.x;
    const int n16 = lane & 15, q4 = lane >> 4;
    int* const err = A.err;

    for (int i = threadIdx.x; i < NSLOT; i += NTHR) {
        S.full[i] = 0;
        S.cons[i] = 0;
    }
    if (threadIdx.x < 2) {
        S.pcnt[threadIdx.x] = 0;
        S.pdone[threadIdx.x] = 0;
    }
    if (threadIdx.x == 0) {
        S.send = 0;
        S.open = 0;
        S.rho_seq = 0;
        S.abort = 0;
    }
    __syncthreads();

    // Total chunks of this workgroup (both roles need it).
    int total = 0;
    {
        TileCursor c{A.s_begin, 0, {}};
        seek_stage(A, c, w);
        while (c.s < A.s_end) {
            total += c.g.G;
            next_tile(A, c, w);
        }
    }

    if (wave < NLD) {
        // ------------------------------------------------------------- loader
        if (total <= wave) return;
        LoadCursor<FMT> c;
        c.tc = TileCursor{A.s_begin, 0, {}};
        seek_stage(A, c.tc, w);
        c.g = 0;
        c.done = 0;
        lc_row<FMT>(A, c, n16);
        lc_advance<FMT>(A, c, w, n16, wave);

        // Blocks past the row's end re-read block 0 of the row (finite data); the compute
        // waves zero their activations, so they add exactly 0.
        using scale_t = typename std::conditional<FMT == VQ_FMT_MXFP4, uint8_t, uint16_t>::type;
        u4_t rq[DEPTH];
        scale_t rs[DEPTH];
        uint16_t rm[DEPTH];
        auto issue = [&](int u) {
            int b = 4 * c.g + q4;
            if (c.done || b >= c.nb) b = 0;
            rq[u] = ld_global_nt<u4_t>(c.rp.qs + 16 * b);
            if constexpr (FMT == VQ_FMT_MXFP4) rs[u] = ld_global_nt<uint8_t>(c.rp.sc + b);
            else rs[u] = ld_global_nt<uint16_t>(c.rp.sc + 2 * b);
            if constexpr (FMT == VQ_FMT_Q4_MIN) rm[u] = ld_global_nt<uint16_t>(c.rp.mn + 2 * b);
        };
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
            issue(u);
            lc_advance<FMT>(A, c, w, n16, NLD);
        }
        for (int k0 = wave; k0 < total; k0 += NLD * DEPTH) {
#pragma unroll
            for (int u = 0; u < DEPTH; ++u) {
                const int k = k0 + NLD * u;
                if (k >= total) break;
                const int slot = k % NSLOT;
                wait_ge(&S.cons[slot], (unsigned)(k / NSLOT), err, &S.abort);
                uint8_t* base = S.ring[slot];
                *(u4_t*)(base + 16 * lane) = rq[u];
                const int mi = 4 * n16 + q4;
                // 16 bits per scale in the slot (an E8M0 byte in the low half)
                if constexpr (FMT == VQ_FMT_MXFP4) base[1024 + 2 * mi] = rs[u];
                else ((uint16_t*)(base + 1024))[mi] = rs[u];
                if constexpr (FMT == VQ_FMT_Q4_MIN) ((uint16_t*)(base + 1152))[mi] = rm[u];
                if (lane == 0) st_rel(&S.full[slot], (unsigned)k + 1u);
                issue(u);
                lc_advance<FMT>(A, c, w, n16, NLD);
            }
        }
        return;
    }

    // ---------------------------------------------------------------- compute
    const int cw = wave - NLD;
    const h8_t ONES = {(_Float16)1, (_Float16)1, (_Float16)1, (_Float16)1,
                       (_Float16)1, (_Float16)1, (_Float16)1, (_Float16)1};
    constexpr int NF = KC < 4 ? KC : 4;      // accumulator elements that can hold a column < K
    const int K = A.K;
    float stat[4] = {0.f, 0.f, 0.f, 0.f};    // lanes n16 == 0: sums of squares of columns 4 q4 + i
    int k_tile = 0;                          // chunk index of the current tile's group 0
    unsigned tile_seq = 0;                   // tiles of this workgroup so far in the launch
    unsigned stage_seq = 0;                  // stages this workgroup has finished

    for (int s = A.s_begin; s < A.s_end; ++s) {
        const StageGeo g = uni_geo(stage_geo(A, s));
        const int t0 = first_tile(w, A.base[s - A.s_begin], A.nwg);
        int ntile = 0;
        for (int t = t0; t < g.T; t += A.nwg) ++ntile;

        // -------- the stage's input: wait for the previous stage (wave 4), read rho
        if (cw == 0) {
            if (g.n_in > 0) {
                // previous stage complete: its 8 counters sum to nwg
                const unsigned* dn = A.done + (size_t)(s - 1) * DONE_WORDS;
                unsigned spins = 0;
                for (;;) {
                    unsigned v = 0;
                    if (lane < DONE_REPL)
                        v = __hip_atomic_load(dn + lane * DONE_STRIDE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    unsigned sum = 0;
#pragma unroll
                    for (int r = 0; r < DONE_REPL; ++r) sum += __builtin_amdgcn_readlane(v, r);
                    if (sum >= (unsigned)A.nwg) break;
                    // another workgroup's timeout, or this one's: stop waiting
                    if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ||
                        __hip_atomic_load(&S.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP))
                        break;
                    __builtin_amdgcn_s_sleep(2);
                    if (++spins > SPIN_GLOBAL) {
                        __hip_atomic_store(&S.abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                        __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                }
            }
            if (lane == 0) st_rel(&S.open, (unsigned)(s - A.s_begin) + 1u);
            // rho of the previous output: sum of the per-workgroup sums of squares, in a
            // fixed order (lane l adds workgroups l, l + 64, ...; then the wave's fixed tree)
            if (g.n_in > 0) {
                const float* st = (const float*)(A.ws + A.off_stats) + (size_t)(s - 1) * A.stats_stride;
                for (int m = 0; m < K; ++m) {
                    float a = 0.f;
                    for (int ww = lane; ww < A.nwg; ww += 64)
                        a += __hip_atomic_load(st + (size_t)ww * K + m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    a = wave_sum(a);
                    if (lane == 0) S.rho[m] = __frcp_rn(__fsqrt_rn(__fdiv_rn(a, (float)g.n_in)));
                }
            } else if (lane < VQ_MAX_K) {
                S.rho[lane] = 1.0f;
            }
            if (lane == 0) st_rel(&S.rho_seq, (unsigned)(s - A.s_begin) + 1u);
        } else {
            wait_ge(&S.open, (unsigned)(s - A.s_begin) + 1u, err, &S.abort);
        }
        // -------- where this stage reads its activations
        const uint16_t* xa;
        bool natural;
        if (s == 0 || A.linear) {
            xa = A.x0;
            natural = true;
        } else if (s == 4 * A.L) {
            xa = (const uint16_t*)(A.ws + (FMT == VQ_FMT_MXFP4 ? A.off_fxn : A.off_fxp));
            natural = FMT == VQ_FMT_MXFP4;
        } else {
            const int j = s & 3;
            const char* lb = A.ws + (size_t)(s >> 2) * A.layer_bytes;
            xa = (const uint16_t*)(lb + (FMT == VQ_FMT_MXFP4 ? A.off_xn[j] : A.off_xp[j]));
            natural = FMT == VQ_FMT_MXFP4;
        }
        // stage 0 keeps a copy of the pass input with the other stage inputs
        if (s == 0 && !A.linear && w == 0) {
            uint16_t* keep = (uint16_t*)(A.ws + A.off_xn[0]);
            for (int i = cw * 64 + lane; i < K * g.cols; i += NCW * 64) keep[i] = A.x0[i];
        }

        // Activations of block 4 grp + j for lane (m = n16, quarter q4): always loaded (rows
        // past K and blocks past the row end read row 0, block 0) so that the loads can be
        // in flight while earlier chunks compute; zeroed and put in pair order at use.
        const int xrow = n16 < K ? n16 : 0;
        auto load_a = [&](int grp, int j) -> u4_t {
            int b = 4 * grp + j;
            if (b >= g.nb) b = 0;
            return *(const u4_t*)(xa + (size_t)xrow * g.cols + 32 * b + 8 * q4);
        };
        auto use_a = [&](u4_t v, int grp, int j) -> h8_t {
            const bool ok = n16 < K && 4 * grp + j < g.nb;
            if (natural && FMT != VQ_FMT_MXFP4) v = perm_pairs(v);
            const u4_t z = {0u, 0u, 0u, 0u};
            return as_h8(ok ? v : z);
        };

        // Tile epilogue (one wave): lane (n16, q4) holds rows n16 and columns 4 q4 + i of
        // the tile's sums.  Outputs are scaled by rho, stored, rounded to fp16 as the next
        // stage's input (natural order, and pair order for the Q4 formats), and their
        // squares summed per column.
        auto epilogue = [&](const StageGeo& g, int s, int t, const f4_t& sum) {
            const int kind = g.kind;
            float sq[4] = {0.f, 0.f, 0.f, 0.f};
            const bool chain = kind != SK_LIN && kind != SK_LM;
            const char* lb = A.ws + (size_t)(s >> 2) * A.layer_bytes;
            const bool last_down = (kind == SK_DOWN) && (s + 1 == 4 * A.L);
            const char* nb_ = A.ws + (size_t)((s + 1) >> 2) * A.layer_bytes;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i >= NF && KC <= 4) continue;
                const int m = 4 * q4 + i;
                const bool mv = m < K;
                const float rho = mv ? S.rho[m] : 0.f;
                const float y = mv ? __fmul_rn(sum[i], rho) : 0.f;
                if (!chain) {
                    const int r = 16 * t + n16;
                    if (mv && r < g.rows) {
                        if (kind == SK_LIN && A.y_dtype == VQ_DTYPE_F16)
                            ((uint16_t*)A.out)[(size_t)m * g.rows + r] = (uint16_t)f2h_bits(y);
                        else
                            ((float*)A.out)[(size_t)m * g.rows + r] = y;
                    }
                    continue;
                }
                float* yout = (float*)(lb + A.off_y[s & 3]);
                uint16_t* xn = last_down ? (uint16_t*)(A.ws + A.off_fxn) : (uint16_t*)(nb_ + A.off_xn[(s + 1) & 3]);
                uint16_t* xp = last_down ? (uint16_t*)(A.ws + A.off_fxp) : (uint16_t*)(nb_ + A.off_xp[(s + 1) & 3]);
                if (kind == SK_GU) {
                    const int r = 8 * t + (n16 & 7);
                    if (mv) st_dev_f32(yout + (size_t)m * g.rows + (n16 < 8 ? r : A.FF + r), y);
                    const float u = row_ror8(y);
                    if (n16 < 8 && mv) {
                        const float sv = silu_mul(y, u);
                        const uint16_t h = (uint16_t)f2h_bits(sv);
                        st_dev_u16(xn + (size_t)m * A.FF + r, h);
                        if (FMT != VQ_FMT_MXFP4) st_dev_u16(xp + (size_t)m * A.FF + (r & ~7) + pair_pos(r & 7), h);
                        sq[i] = sv * sv;
                    }
                } else {
                    const int r = 16 * t + n16;
                    if (mv) st_dev_f32(yout + (size_t)m * g.rows + r, y);
                    const bool feeds = kind != SK_QKV || r < A.H;
                    if (mv && feeds) {
                        const uint16_t h = (uint16_t)f2h_bits(y);
                        st_dev_u16(xn + (size_t)m * A.H + r, h);
                        if (FMT != VQ_FMT_MXFP4) st_dev_u16(xp + (size_t)m * A.H + (r & ~7) + pair_pos(r & 7), h);
                        sq[i] = y * y;
                    }
                }
            }
            if (chain) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (i >= NF && KC <= 4) continue;
                    stat[i] += row16_sum(sq[i]);
                }
            }
        };

        const int ng = cw < g.G ? (g.G - cw + NCW - 1) / NCW : 0;

        // one chunk: wait for the slot, read it, free it, multiply
        auto chunk = [&](int k, const u4_t (&ar)[4], int grp, f4_t& acc) {
            h8_t a[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) a[j] = use_a(ar[j], grp, j);
            const int slot = k % NSLOT;
            wait_ge(&S.full[slot], (unsigned)k + 1u, err, &S.abort);
            const uint8_t* base = S.ring[slot];
            const u4_t raw = *(const u4_t*)(base + 16 * lane);
            const u2_t scw = *(const u2_t*)(base + 1024 + 8 * n16);
            u2_t mnw = {0u, 0u};
            if constexpr (FMT == VQ_FMT_Q4_MIN) mnw = *(const u2_t*)(base + 1152 + 8 * n16);
            if (lane == 0) st_rel(&S.cons[slot], (unsigned)(k / NSLOT) + 1u);
            uint32_t t[4];
            quarter_transpose(raw, t);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const h8_t b = widen8<FMT>(t[j]);
                const f4_t z = {0.f, 0.f, 0.f, 0.f};
                const f4_t cj = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j], b, z, 0, 0, 0);
                const float d = block_scale<FMT>(scw, j);
#pragma unroll
                for (int i = 0; i < NF; ++i) acc[i] = __builtin_fmaf(d, cj[i], acc[i]);
                if constexpr (FMT == VQ_FMT_Q4_MIN) {
                    const f4_t sj = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j], ONES, z, 0, 0, 0);
                    const float mm = half_bits_to_float(((j < 2) ? mnw.x : mnw.y) >> ((j & 1) * 16) & 0xffffu);
#pragma unroll
                    for (int i = 0; i < NF; ++i) acc[i] = __builtin_fmaf(mm, sj[i], acc[i]);
                }
            }
        };

        // the tile's partial sums meet in LDS; wave (tile_seq mod 8) adds them and writes
        // the tile's outputs
        auto tile_end = [&](int jt, const f4_t& acc) {
            const int t = t0 + jt * A.nwg;
            const unsigned buf = tile_seq & 1u, round = tile_seq >> 1;
            wait_ge(&S.pdone[buf], round, err, &S.abort);
            if (lane < 16 * ((KC + 3) / 4)) S.part[buf][cw][lane] = acc;
            // one arrival per wave (lane 0's release covers the whole wave's LDS writes)
            if (lane == 0) __hip_atomic_fetch_add(&S.pcnt[buf], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            if ((int)(tile_seq % NCW) == cw) {
                wait_ge(&S.pcnt[buf], NCW * (round + 1), err, &S.abort);
                f4_t sum = {0.f, 0.f, 0.f, 0.f};
                if (lane < 16 * ((KC + 3) / 4)) {
#pragma unroll
                    for (int c = 0; c < NCW; ++c) sum += S.part[buf][c][lane];
                }
                if (lane == 0) st_rel(&S.pdone[buf], round + 1u);
                wait_ge(&S.rho_seq, (unsigned)(s - A.s_begin) + 1u, err, &S.abort);
                epilogue(g, s, t, sum);
            }
            ++tile_seq;
        };

        if (ng == 0) {
            const f4_t z = {0.f, 0.f, 0.f, 0.f};
            for (int jt = 0; jt < ntile; ++jt) tile_end(jt, z);
        } else {
            // flat loop over (tile, group) steps; the activations of step i + 2 are loaded
            // while step i computes (they depend only on the group, so they run on across
            // tile boundaries).  The loads are unconditional -- the last two steps load a
            // valid group they do not use -- so that the compiler's waits stay per step.
            const int nsteps = ntile * ng;
            u4_t ab[3][4];
            int pii = 0;
            auto prefetch = [&](u4_t (&dst)[4]) {
#pragma unroll
                for (int j = 0; j < 4; ++j) dst[j] = load_a(cw + NCW * pii, j);
                pii = (pii + 1 == ng) ? 0 : pii + 1;
            };
            prefetch(ab[0]);
            prefetch(ab[1]);
            int ii = 0, jt = 0;
            f4_t acc = {0.f, 0.f, 0.f, 0.f};
            auto step = [&](int i, u4_t (&cur)[4], u4_t (&nxt)[4]) {
                prefetch(nxt);
                chunk(k_tile + cw + NCW * ii, cur, cw + NCW * ii, acc);
                if (++ii == ng) {
                    ii = 0;
                    tile_end(jt, acc);
                    acc = f4_t{0.f, 0.f, 0.f, 0.f};
                    k_tile += g.G;
                    ++jt;
                }
            };
            for (int i = 0; i < nsteps; i += 3) {
                step(i, ab[0], ab[2]);
                if (i + 1 < nsteps) step(i + 1, ab[1], ab[0]);
                if (i + 2 < nsteps) step(i + 2, ab[2], ab[1]);
            }
        }
        if (ng == 0) k_tile += ntile * g.G;

        // -------- stage end: per-wave sums of squares, then wave 4 reports the stage
        if (lane < 64 && n16 == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * q4 + i;
                if (m < VQ_MAX_K) S.tstat[cw][m] = stat[i];
                stat[i] = 0.f;
            }
        }
        // this wave's epilogue stores (write-through) are in memory before the stage is
        // reported complete; waiting here once per stage, not per tile, keeps a reducing
        // wave from stalling the workgroup's next tiles
        __builtin_amdgcn_s_waitcnt(0);
        if (lane == 0) __hip_atomic_fetch_add(&S.send, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        ++stage_seq;
        if (cw == 0 && A.done) {
            wait_ge(&S.send, NCW * stage_seq, err, &S.abort);
            if (g.kind != SK_LIN && g.kind != SK_LM && lane < K) {
                float a = 0.f;
#pragma unroll
                for (int c = 0; c < NCW; ++c) a += S.tstat[c][lane];
                float* st = (float*)(A.ws + A.off_stats) + (size_t)s * A.stats_stride;
                st_dev_f32(st + (size_t)w * K + lane, a);
            }
            __builtin_amdgcn_s_waitcnt(0);
            if (lane == 0)
                __hip_atomic_fetch_add(A.done + (size_t)s * DONE_WORDS + (w & (DONE_REPL - 1)) * DONE_STRIDE, 1u,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

__global__ void k_zero_u32(unsigned* p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
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

hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    k_zero_u32<<<dim3((n + 255) / 256), 256, 0, st>>>(p, n);
    return hipGetLastError();
}

hipError_t launch_flow(const FlowArgs& A, hipStream_t st) {
    switch (A.fmt) {
        case VQ_FMT_Q4: return launch_f<VQ_FMT_Q4>(A, st);
        case VQ_FMT_Q4_MIN: return launch_f<VQ_FMT_Q4_MIN>(A, st);
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
