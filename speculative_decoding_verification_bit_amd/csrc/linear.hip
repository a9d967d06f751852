// Weight-streaming linear map y = W x for a K-wide verify window on gfx950.
//
// Decode reads every weight once per pass and multiplies it against the activation
// vector (page "100 tokens per second from a 27B model on a 24 GB AMD card", section
// "The wall"); verification applies the same single read to K activation columns
// (same page, section "How speculative decoding gets past a per-token wall"), layer by
// layer (Hacker News thread 49596054).
//
// One launch per stage.  A workgroup of 4 waves owns a 64-row tile and a chunk of 4
// groups of 8 quantisation blocks (one group of 256 input columns per wave):
//  * prologue: the wave issues all of its weight loads first (unconditional loads from
//    clamped addresses, so they are all in flight at once), then builds its K activation
//    columns in registers -- either the fp16 input, or the previous stage's raw output
//    scaled to unit RMS per column and rounded to fp16 (the RMS comes from per-tile sums
//    of squares the previous stage wrote);
//  * the dot products (VALU or MFMA, below);
//  * epilogue: the four waves' partials are combined in LDS in a fixed order; with more
//    than one chunk per tile, each chunk writes its partial and the last workgroup to
//    arrive at the tile's counter sums the chunks in chunk order, writes y and the tile's
//    sums of squares, and resets the counter.  Results are bitwise reproducible.
//
//  * VALU kernel (K <= 8): lane 8s + c owns block c of the wave's group for rows
//    8i + s (i = 0..7): each load instruction covers 8 rows x 128 contiguous bytes.  The
//    lane keeps its block's activations in VGPRs; codes are widened to exact fp16
//    q = n - 8 (0x6400 exponent trick, two nibbles per instruction) and fed to
//    v_dot2_f32_f16; per block y += d * sum(q x) + m * sum(x); the 8 block partials of a
//    row are summed across lanes with DPP.
//  * MFMA kernel (K <= 16): v_mfma_f32_16x16x32_f16 with the weights as B (16 rows x 32
//    columns = one quantisation block per instruction) and the K activation columns,
//    zero-padded to 16, as A.  A lane loads a whole block of one row (16 bytes);
//    permlane32/permlane16 swaps transpose 4 lanes' blocks into the k-quarters the MFMA
//    expects.  Each block's product is scaled by its scale on the accumulator; the min
//    term sum_b m_b * sum(x_b) is one more MFMA per 8 blocks with the block sums split
//    into fp16 hi + lo parts.
#include <hip/hip_fp16.h>

#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "vq_device.h"
#include "vq_internal.h"

namespace vq {
namespace {

// ------------------------------------------------------------------ rows of a tile

// Output row of local row r (0..63) of tile t.  Paired stages (gate|up) put rows
// [32t, 32t + 32) of segment 0 in r < 32 and the same rows of segment 1 in r >= 32, so
// one tile holds both factors of silu(gate) * up.
__device__ __forceinline__ int out_row(const StageArgs& A, int t, int r) {
    if (A.paired) return (r < 32 ? 0 : A.W.seg_end[0]) + 32 * t + (r & 31);
    return 64 * t + r;
}

__device__ __forceinline__ bool row_ok(const StageArgs& A, int t, int r) {
    if (A.paired) return 32 * t + (r & 31) < A.W.seg_end[0];
    return 64 * t + r < A.W.rows;
}

// A valid row standing in for (t, r): r itself, or the last row of its segment range.
__device__ __forceinline__ int clamp_row(const StageArgs& A, int t, int r) {
    if (A.paired) return (r < 32 ? 0 : A.W.seg_end[0]) + min(32 * t + (r & 31), A.W.seg_end[0] - 1);
    return min(64 * t + r, A.W.rows - 1);
}


// Base addresses of one segment (uniform); a row's data lies at 32-bit offsets from them
// (a matrix's codes stay below 2 GiB), which lets the loads take the base in scalar
// registers and only the offset in a vector register.
struct SegRef {
    const uint8_t* qs;       // codes, rows of cols / 2 bytes
    const uint8_t* sc8;      // scales, rows of nb fp16 (nb bytes for E8M0)
    const uint16_t* mn;      // mins, rows of nb fp16 (or NULL)
    int r0;                  // first row of the segment
};

__device__ __forceinline__ int tile_seg(const StageArgs& A, int t, int r) {
    if (A.paired) return r < 32 ? 0 : 1;
    const int row0 = 64 * t;
    return __builtin_amdgcn_readfirstlane(
        (A.W.nseg > 2 && row0 >= A.W.seg_end[1]) ? 2 : (A.W.nseg > 1 && row0 >= A.W.seg_end[0]) ? 1 : 0);
}

// Pins a uniform value (a segment's base or bound) into scalar registers.  Besides
// keeping the value scalar, the intrinsic stops the compiler from folding the segment
// select below into an indexed load, which would force a Mat held in registers (the
// persistent pass builds one per stage) out to scratch memory.
__device__ __forceinline__ int opaque(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
__device__ __forceinline__ T* opaque(T* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<T*>((uint64_t)lo | ((uint64_t)hi << 32));
}

// Segment `seg` (uniform) of W.
__device__ __forceinline__ SegRef seg_ref(const Mat& W, int seg) {
    const uint8_t* q[3] = {opaque(W.qs[0]), opaque(W.qs[1]), opaque(W.qs[2])};
    const void* c[3] = {opaque(W.scales[0]), opaque(W.scales[1]), opaque(W.scales[2])};
    const uint16_t* m[3] = {opaque(W.mins[0]), opaque(W.mins[1]), opaque(W.mins[2])};
    const int e0 = opaque(W.seg_end[0]), e1 = opaque(W.seg_end[1]);
    SegRef r;
    r.qs = seg == 2 ? q[2] : seg == 1 ? q[1] : q[0];
    r.sc8 = (const uint8_t*)(seg == 2 ? c[2] : seg == 1 ? c[1] : c[0]);
    r.mn = seg == 2 ? m[2] : seg == 1 ? m[1] : m[0];
    r.r0 = seg == 2 ? e1 : seg == 1 ? e0 : 0;
    return r;
}

// ------------------------------------------------------------------ stage glue

// rs[k] = 1 / sqrt(sum_i stats_in[i][k] / n_in): per-column inverse RMS of the previous
// stage's output, from its per-tile sums of squares (summed in a fixed order).
// The workgroup's sum of its threads' partial sums acc[k] (a fixed order: each wave's DPP
// tree, then the four waves), turned into the input scales rs[k] = 1 / sqrt(sum / n_in).
__device__ void rms_reduce(const StageArgs& A, const float (&acc)[VQ_MAX_K], float* rs, float* sh) {
    const int K = A.K;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < VQ_MAX_K; ++k)
        if (k < K) {
            const float w = wave_sum(acc[k]);
            if (lane == 0) sh[4 * k + wave] = w;
        }
    __syncthreads();
    if (threadIdx.x < (unsigned)K) {
        const float* t = sh + 4 * threadIdx.x;
        rs[threadIdx.x] = 1.0f / __fsqrt_rn(__fdiv_rn((t[0] + t[1]) + (t[2] + t[3]), (float)A.n_in));
    }
    __syncthreads();
}

// Thread t sums the flat entries f = t, t + 256, ... of the previous stage's sums of
// squares ([nstats_in][K], entry f belongs to column f mod K).
__device__ void stage_rms(const StageArgs& A, float* rs, float* sh) {
    if (A.glue == GLUE_NONE) return;
    const int K = A.K, n = A.nstats_in * K;
    float acc[VQ_MAX_K];
#pragma unroll
    for (int k = 0; k < VQ_MAX_K; ++k) acc[k] = 0.f;
    // entries in the same order, loaded 8 at a time (one round trip per 8, not per entry)
    for (int f0 = threadIdx.x; f0 < n; f0 += 8 * 256) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = f0 + 256 * u < n ? A.stats_in[f0 + 256 * u] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int f = f0 + 256 * u;
            const int kf = f % K;
#pragma unroll
            for (int k = 0; k < VQ_MAX_K; ++k) acc[k] += (f < n && k == kf) ? v[u] : 0.f;
        }
    }
    rms_reduce(A, acc, rs, sh);
}

// The same sums with the loads issued early (before a workgroup's weights, so that
// waiting for them does not wait for the weights too): at most NPRE entries per thread,
// loaded unconditionally from clamped addresses.  `ok` is false when the stage has more
// entries (or no input scales); stats_finish then falls back to stage_rms.
template <int NPRE>
struct StatsPre {
    float a[NPRE];
    bool ok;
};

template <int NPRE>
__device__ __forceinline__ void stats_issue(const StageArgs& A, StatsPre<NPRE>& S) {
    const int n = A.nstats_in * A.K;
    S.ok = A.glue != GLUE_NONE && n <= 256 * NPRE;
    // a readable stand-in address when there is nothing to load
    const float* p = S.ok ? A.stats_in : reinterpret_cast<const float*>(A.W.qs[0]);
    const int last = S.ok ? n - 1 : 0;
#pragma unroll
    for (int j = 0; j < NPRE; ++j) S.a[j] = ld_global<float>(p + min((int)threadIdx.x + 256 * j, last));
}

template <int NPRE>
__device__ void stats_finish(const StageArgs& A, const StatsPre<NPRE>& S, float* rs, float* sh) {
    if (A.glue == GLUE_NONE) return;
    if (!S.ok) {
        stage_rms(A, rs, sh);
        return;
    }
    const int K = A.K, n = A.nstats_in * K;
    float acc[VQ_MAX_K];
#pragma unroll
    for (int k = 0; k < VQ_MAX_K; ++k) acc[k] = 0.f;
#pragma unroll
    for (int j = 0; j < NPRE; ++j) {
        const int f = (int)threadIdx.x + 256 * j;
        const int kf = f % K;
#pragma unroll
        for (int k = 0; k < VQ_MAX_K; ++k) acc[k] += (f < n && k == kf) ? S.a[j] : 0.f;
    }
    rms_reduce(A, acc, rs, sh);
}

__device__ __forceinline__ void keep_x8(const StageArgs& A, int k, int col, const uint32_t (&h)[8]) {
    u4_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = h[2 * e] | (h[2 * e + 1] << 16);
    *reinterpret_cast<u4_t*>(A.keep + (size_t)k * A.W.cols + col) = v;
}

// ------------------------------------------------------------------ epilogue

// red[w][k][l] (w < 4 waves, k < K, l < 64 local rows) holds this workgroup's partials
// for (tile, part).  Wave w finishes columns w, w + 4, ... of the item, one lane per
// local row.  With one column the other waves return at once (in a one-item launch they
// end, which frees their registers and wave slots while wave 0 waits on memory).  Writes
// y (and the tile's sums of squares) once all parts of the tile are in.
template <int KR>
__device__ void stage_epilogue(const StageArgs& A, int tile, int part, int nparts, float (*red)[KR][65],
                               int* s_flag) {
    constexpr int NC = (KR + 3) / 4;                 // columns per wave, at most
    const int K = A.K, rows = A.W.rows;
    const bool solo = K == 1;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (solo && wave > 0) return;
    const int l = threadIdx.x & 63;
    const bool ok = row_ok(A, tile, l);
    const int orow = ok ? out_row(A, tile, l) : 0;
    float fv[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int k = wave + 4 * j;
        fv[j] = k < K ? ((red[0][k][l] + red[1][k][l]) + red[2][k][l]) + red[3][k][l] : 0.f;
    }
    if (nparts > 1) {
        // Partials, the counter and the last arriver's reads all use device-scope relaxed
        // atomics, which gfx950 performs coherently across XCDs without flushing or
        // invalidating the L2; s_waitcnt 0 makes each wave's partial stores complete
        // before the workgroup's arrival is counted.
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const int k = wave + 4 * j;
            if (k < K && ok)
                __hip_atomic_store(&A.part[((size_t)part * K + k) * rows + orow], fv[j], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_s_waitcnt(0);
        bool last;
        if (solo) {
            unsigned prev = 0u;
            if (l == 0)
                prev = __hip_atomic_fetch_add(&A.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = (unsigned)__builtin_amdgcn_readfirstlane((int)prev) == (unsigned)(nparts - 1);
        } else {
            __syncthreads();
            if (threadIdx.x == 0)
                *s_flag = __hip_atomic_fetch_add(&A.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                          (unsigned)(nparts - 1);
            __syncthreads();
            last = *s_flag != 0;
        }
        if (!last) return;
        // the parts are summed in part order; their loads go out in groups of 8, so a
        // wide stage (17 parts at 17408 columns) waits for 3 round trips, not 17
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const int k = wave + 4 * j;
            float v = 0.f;
            if (k < K && ok) {
                const float* pp = A.part + (size_t)k * rows + orow;
                const size_t pstride = (size_t)K * rows;
                for (int c0 = 0; c0 < nparts; c0 += 8) {
                    float t[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        t[u] = c0 + u < nparts ? __hip_atomic_load(pp + (size_t)(c0 + u) * pstride, __ATOMIC_RELAXED,
                                                                   __HIP_MEMORY_SCOPE_AGENT)
                                               : 0.f;
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        if (c0 + u < nparts) v += t[u];
                }
            }
            fv[j] = v;
        }
        if (threadIdx.x == 0) __hip_atomic_store(&A.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int k = wave + 4 * j;
        if (k >= K || !ok) continue;
        const size_t o = (size_t)k * rows + orow;
        if (A.y_dtype == VQ_DTYPE_F16)
            reinterpret_cast<uint16_t*>(A.y)[o] = (uint16_t)f2h_bits(fv[j]);
        else
            st_shared_f32(reinterpret_cast<float*>(A.y) + o, fv[j], A.coh);
    }
    if (A.stats_out) {
        // silu(gate) * up (paired: lane l < 32 holds gate, lane l + 32 up) and the tile's
        // sums of squares
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const int k = wave + 4 * j;
            if (k >= K) continue;
            float sq = 0.f;
            if (A.paired) {
                const float up = __shfl(fv[j], (l + 32) & 63, 64);
                if (l < 32 && ok) {
                    const float v = silu_mul(fv[j], up);
                    st_shared_f32(A.sbuf + (size_t)k * A.W.seg_end[0] + 32 * tile + l, v, A.coh);
                    sq = v * v;
                }
            } else {
                const int row = 64 * tile + l;
                if (row < A.nstat && row < rows) sq = fv[j] * fv[j];
            }
            const float ss = wave_sum(sq);
            if (l == 0) st_shared_f32(A.stats_out + (size_t)tile * K + k, ss, A.coh);
        }
    }
    if (A.done) {
        // the tile's outputs are in memory before its XCD group's counter counts it
        __builtin_amdgcn_s_waitcnt(0);
        if (!solo) __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(A.done + (blockIdx.x & 7) * DONE_STRIDE, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Waits (thread 0 polls, the workgroup waits behind it) until *flag reaches target; after
// about a second the error word is raised and the workgroup proceeds, so a launch always
// ends.
__device__ void wait_flag(const unsigned* flag, unsigned target, int* err) {
    if (threadIdx.x == 0) {
        unsigned spins = 0;
        while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins >= (1u << 22)) {
                __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

// ------------------------------------------------------------------ VALU kernel

// One wave's share of a 64-row tile: 8 rows x one block per lane.
struct WTileV {
    u4_t w[8];
    uint32_t sr[8], mr[8];
};

// Q4 with mins at K = 1 (PAIR): lanes c and c + 1 (c even) hold blocks p and p + 1 of the
// same row, so the even lane loads both blocks' scales and the odd lane both blocks' mins,
// one 4-byte load each (T.sr; T.mr unused), and compute_tile_valu swaps the halves between
// the two lanes (measured: K = 1 pass 4.63 -> 4.60 ms; at K >= 2 it was slower).  bu is the lane's block before clamping (the pair is formed from
// it, so the two lanes agree on it even past the row's end).
template <int FMT, bool PAIR>
__device__ __forceinline__ void load_tile_valu(const StageArgs& A, int tile, int s, int bcl, int bu, WTileV& T) {
    tile = opaque(tile);          // row addresses are recomputed per chunk, not kept live
    const uint32_t rowq = (uint32_t)A.W.cols >> 1, nb = (uint32_t)A.W.cols >> 5;
    const uint32_t b = (uint32_t)bcl;
    const bool odd = (threadIdx.x & 1) != 0;
    const uint32_t pb = (uint32_t)bu & ~1u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const SegRef R = seg_ref(A.W, tile_seg(A, tile, 8 * i));
        const uint32_t lr = (uint32_t)(clamp_row(A, tile, 8 * i + s) - R.r0);
        T.w[i] = ld_global_nt<u4_t>(R.qs + (lr * rowq + 16u * b));
        if constexpr (FMT == VQ_FMT_Q4_MIN && PAIR) {
            const uint8_t* src = odd ? reinterpret_cast<const uint8_t*>(R.mn) : R.sc8;
            if ((nb & 1u) == 0u) {
                // even row length: the pair is 4-byte aligned and inside the row
                const uint32_t e0 = min(pb, nb - 2u);
                T.sr[i] = ld_global<uint32_t>(src + 2u * (lr * nb + e0));
            } else {
                const uint32_t e0 = min(pb, nb - 1u), e1 = min(pb + 1u, nb - 1u);
                T.sr[i] = (uint32_t)ld_global<uint16_t>(src + 2u * (lr * nb + e0)) |
                          ((uint32_t)ld_global<uint16_t>(src + 2u * (lr * nb + e1)) << 16);
            }
            T.mr[i] = 0u;
        } else if constexpr (FMT == VQ_FMT_MXFP4) {
            T.sr[i] = ld_global<uint8_t>(R.sc8 + (lr * nb + b));
            T.mr[i] = 0u;
        } else {
            T.sr[i] = ld_global<uint16_t>(R.sc8 + 2u * (lr * nb + b));
            T.mr[i] = FMT == VQ_FMT_Q4_MIN ? (uint32_t)ld_global<uint16_t>(R.mn + (lr * nb + b)) : 0u;
        }
    }
}

// acc[k][i] += this lane's block term for row 8i + s (summed over the 8 block lanes later).
template <int FMT, int K>
__device__ __forceinline__ void compute_tile_valu(const StageArgs& A, int tile, int s, bool live, const WTileV& T,
                                                  const uint32_t (&xv)[K][16], const float (&bs)[K],
                                                  float (&acc)[K][8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float t[K];
#pragma unroll
        for (int k = 0; k < K; ++k) t[k] = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            h2_t p[4];
            unpack8<FMT>(T.w[i][q], p);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                t[k] = __builtin_amdgcn_fdot2(p[0], as_h2(xv[k][4 * q]), t[k], false);
                t[k] = __builtin_amdgcn_fdot2(p[1], as_h2(xv[k][4 * q + 1]), t[k], false);
                t[k] = __builtin_amdgcn_fdot2(p[2], as_h2(xv[k][4 * q + 2]), t[k], false);
                t[k] = __builtin_amdgcn_fdot2(p[3], as_h2(xv[k][4 * q + 3]), t[k], false);
            }
        }
        const bool ok = live && row_ok(A, tile, 8 * i + s);
        float d, m;
        if constexpr (FMT == VQ_FMT_Q4_MIN && K == 1) {
            // the pair's scales (even lane) and mins (odd lane): swap with the partner lane
            const uint32_t own = T.sr[i];
            const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)own, 0xB1, 0xF, 0xF, false);
            const bool odd = (threadIdx.x & 1) != 0;
            d = half_bits_to_float(odd ? (other >> 16) : (own & 0xffffu));
            m = half_bits_to_float(odd ? (own >> 16) : (other & 0xffffu));
        } else {
            d = FMT == VQ_FMT_MXFP4 ? e8m0_to_float(T.sr[i]) : half_bits_to_float(T.sr[i]);
            m = half_bits_to_float(T.mr[i]);
        }
        d = ok ? d : 0.f;
        m = ok ? m : 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float v = d * t[k];
            if constexpr (FMT == VQ_FMT_Q4_MIN) v = fmaf(m, bs[k], v);
            acc[k][i] += v;
        }
    }
}

// LDS of one stage item (a 64-row tile x one chunk).
template <int KR>
struct StageSmem {
    float red[4][KR][65];          // the 4 waves' partials; also the RMS reduction scratch
    float rs[VQ_MAX_K];
    int flag;
};

// One item: a 64-row tile x a run of chunks [part * cpw, part * cpw + cpw) (a chunk is
// 4 groups of 8 blocks, one group per wave).  Lane 8s + c owns block c of the wave's
// group for rows 8i + s of the tile.
//
// The weights of one chunk for this lane.
template <int FMT, bool PAIR>
__device__ __forceinline__ void prefetch_valu(const StageArgs& A, int tile, int chunk, WTileV& T) {
    const int nb = A.W.cols >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int b = (chunk * 4 + wave) * 8 + (lane & 7);
    load_tile_valu<FMT, PAIR>(A, tile, lane >> 3, b < nb ? b : nb - 1, b, T);
}

// Whether a chunk's compute overlaps the loads of the next weights (two register tiles
// per lane), or the next weights are loaded after it (one tile, more workgroups per CU).
#ifndef VQ_PREFETCH_NEXT
#define VQ_PREFETCH_NEXT 0
#endif
constexpr bool PREFETCH_NEXT = VQ_PREFETCH_NEXT != 0;

// Orders one wave's LDS writes before its later LDS reads (the wave's own region only).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One lane's share of a chunk's activations (elements 4s..4s+3 of block c of the wave's
// group, per column), before conversion.
template <int K>
struct XPre {
    uint2 r16[K];
    f4_t r32[K];
};

template <int K>
__device__ __forceinline__ void x_issue(const StageArgs& A, int nb, int ch, XPre<K>& X) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int s = lane >> 3, c = lane & 7;
    const int b = (ch * 4 + wave) * 8 + c;
    const int col = 32 * (b < nb ? b : nb - 1) + 4 * s;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (A.glue == GLUE_NONE) X.r16[k] = *reinterpret_cast<const uint2*>(A.x16 + (size_t)k * A.W.cols + col);
        else X.r32[k] = *reinterpret_cast<const f4_t*>(A.src + (size_t)k * A.ld + col);
    }
}

// On entry `cur` holds the item's first chunk and sm.rs the stage's input scales.  Each
// chunk's activations are loaded (the first chunk's may come preloaded in *pre) and
// converted, then the next weights are issued (the next chunk, else the first chunk of
// item (ntile, npart) unless ntile < 0), then the chunk is computed; on return `cur`
// holds those next weights.
template <int FMT, int K, bool MULTI, bool PREP = false>
__device__ void stage_item_valu(const StageArgs& A, const StageGeom& g, int tile, int part, StageSmem<K>& sm,
                                uint2 (&xs)[4][K][8][8], WTileV& cur, int ntile, int npart,
                                const XPre<K>* pre = nullptr) {
    float (*red)[K][65] = sm.red;
    const float* rs = sm.rs;
    const int nb = g.nb;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int s = lane >> 3, c = lane & 7;
    // MULTI = false: one chunk per item (cpw == 1), compiled without the loop, which
    // keeps far fewer registers live
    const int c0 = part * g.cpw, c1 = MULTI ? min(g.nchunks, c0 + g.cpw) : c0 + 1;
    float acc[K][8];
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[k][i] = 0.f;
    for (int ch = c0; ch < c1; ++ch) {
        const int b = (ch * 4 + wave) * 8 + c;
        const bool live = b < nb;
        const int bcl = live ? b : nb - 1;
        const int col = 32 * bcl + 4 * s;
        float bs[K];
        uint32_t xv[K][16];
        if constexpr (PREP) {
            // the stage's input converted once (prep_x_valu): block c's 32 values per
            // column in the widened pair order, and its sum
            const float* bsum = reinterpret_cast<const float*>(A.xpa);
#pragma unroll
            for (int k = 0; k < K; ++k) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u4_t v = live ? ld_global<u4_t>(A.xp + ((size_t)k * nb + b) * 4 + q) : u4_t{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int e = 0; e < 4; ++e) xv[k][4 * q + e] = v[e];
                }
                bs[k] = live ? ld_global<float>(bsum + (size_t)k * nb + b) : 0.f;
            }
        } else {
        // this chunk's activations: lane (s, c) takes elements 4s..4s+3 of block c
        XPre<K> X;
        if (pre && ch == c0) X = *pre;
        else x_issue<K>(A, nb, ch, X);
        const uint2 (&r16)[K] = X.r16;
        const f4_t (&r32)[K] = X.r32;
        // fp16 inputs; the wave shares them through LDS, so that each lane then holds its
        // block's 32 activations per column in the widened pair order
        const bool keeper = A.keep && tile == 0 && live;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            uint32_t h[4];
            if (A.glue == GLUE_NONE) {
                h[0] = r16[k].x & 0xffffu; h[1] = r16[k].x >> 16; h[2] = r16[k].y & 0xffffu; h[3] = r16[k].y >> 16;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = f2h_scaled(r32[k][e], rs[k]);
            }
            const uint2 pk = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            xs[wave][k][c][s] = pk;
            if (keeper) *reinterpret_cast<uint2*>(A.keep + (size_t)k * A.W.cols + col) = pk;
            float sum = (half_bits_to_float(h[0]) + half_bits_to_float(h[1])) +
                        (half_bits_to_float(h[2]) + half_bits_to_float(h[3]));
            sum += __shfl_xor(sum, 8, 64);
            sum += __shfl_xor(sum, 16, 64);
            sum += __shfl_xor(sum, 32, 64);
            bs[k] = live ? sum : 0.f;
        }
        wave_lds_sync();
#pragma unroll
        for (int k = 0; k < K; ++k) {
            uint32_t h[32];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint2 v = xs[wave][k][c][q];
                h[4 * q] = v.x & 0xffffu; h[4 * q + 1] = v.x >> 16;
                h[4 * q + 2] = v.y & 0xffffu; h[4 * q + 3] = v.y >> 16;
            }
#pragma unroll
            for (int gg = 0; gg < 4; ++gg)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const uint32_t lo = h[8 * gg + slot_col<FMT>(2 * t)], hi = h[8 * gg + slot_col<FMT>(2 * t + 1)];
                    xv[k][4 * gg + t] = live ? (lo | (hi << 16)) : 0u;
                }
        }
        wave_lds_sync();
        }
        if constexpr (PREFETCH_NEXT) {
            // the next weights load while this chunk is computed (issued only now: a wait
            // for the activations above would otherwise also wait for them)
            WTileV nxt;
            if (ch + 1 < c1) prefetch_valu<FMT, K == 1>(A, tile, ch + 1, nxt);
            else if (ntile >= 0) prefetch_valu<FMT, K == 1>(A, ntile, npart * g.cpw, nxt);
            compute_tile_valu<FMT, K>(A, tile, s, live, cur, xv, bs, acc);
            cur = nxt;
        } else {
            compute_tile_valu<FMT, K>(A, tile, s, live, cur, xv, bs, acc);
            if (ch + 1 < c1) prefetch_valu<FMT, K == 1>(A, tile, ch + 1, cur);
            else if (ntile >= 0) prefetch_valu<FMT, K == 1>(A, ntile, npart * g.cpw, cur);
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float v = sum8(acc[k][i]);
            if (c == 0) red[wave][k][8 * i + s] = v;
        }
    __syncthreads();
    stage_epilogue<K>(A, tile, part, g.nparts, red, &sm.flag);
}

// A 16-byte store that other XCDs read within the same launch: two device-scope 8-byte
// stores, written through past this XCD's L2, so that waiting for their completion
// (s_waitcnt) is enough before the count that publishes them (no L2 write-back).
__device__ __forceinline__ void st_through_u4(u4_t* p, const u4_t& v) {
    uint64_t* q = reinterpret_cast<uint64_t*>(p);
    __hip_atomic_store(q, (uint64_t)v[0] | ((uint64_t)v[1] << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, (uint64_t)v[2] | ((uint64_t)v[3] << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The input conversion of stage_item_valu for the whole stage, done once: wave v of the
// n_prep converting workgroups takes (column, group of 8 blocks) units v, v + 4 n_prep,
// ...; lane (s, c) converts elements 4s..4s+3 of block c with the same arithmetic and
// order as the inline conversion (the block sum by the same butterfly), so both give the
// same bits.  Writes xp ([k][block] 64 bytes: the block's 32 values in the widened pair
// order), the block sums ([k][block] floats at xpa) and the fp16 copy of the input.
// Every 16-byte slot is written whole by one lane.
template <int FMT>
__device__ void prep_x_valu(const StageArgs& A, const float* rs) {
    const int K = A.K;
    const int nb = A.W.cols >> 5;
    const int ngrp = (nb + 7) >> 3;
    const int lane = threadIdx.x & 63;
    const int s = lane >> 3, c = lane & 7;
    const int nwv = A.n_prep * 4;
    float* bsum = reinterpret_cast<float*>(A.xpa);
    for (int u = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6); u < K * ngrp; u += nwv) {
        const int k = u / ngrp, gi = u - k * ngrp;
        const int b = 8 * gi + c;
        const bool live = b < nb;
        const int col = 32 * (live ? b : nb - 1) + 4 * s;
        uint32_t h[4];
        if (A.glue == GLUE_NONE) {
            const uint2 v = *reinterpret_cast<const uint2*>(A.x16 + (size_t)k * A.W.cols + col);
            h[0] = v.x & 0xffffu; h[1] = v.x >> 16; h[2] = v.y & 0xffffu; h[3] = v.y >> 16;
        } else {
            const f4_t v = *reinterpret_cast<const f4_t*>(A.src + (size_t)k * A.ld + col);
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = f2h_scaled(v[e], rs[k]);
        }
        if (A.keep && live)
            *reinterpret_cast<uint2*>(A.keep + (size_t)k * A.W.cols + col) =
                make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        float sum = (half_bits_to_float(h[0]) + half_bits_to_float(h[1])) +
                    (half_bits_to_float(h[2]) + half_bits_to_float(h[3]));
        sum += __shfl_xor(sum, 8, 64);
        sum += __shfl_xor(sum, 16, 64);
        sum += __shfl_xor(sum, 32, 64);
        // lane s ^ 1 holds the other half of the 8-value group s >> 1
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (uint32_t)__shfl_xor((int)h[e], 8, 64);
        if ((s & 1) == 0 && live) {
            const uint32_t v8[8] = {h[0], h[1], h[2], h[3], o[0], o[1], o[2], o[3]};
            u4_t out;
#pragma unroll
            for (int t = 0; t < 4; ++t) out[t] = v8[slot_col<FMT>(2 * t)] | (v8[slot_col<FMT>(2 * t + 1)] << 16);
            st_through_u4(A.xp + ((size_t)k * nb + b) * 4 + (s >> 1), out);
        }
        if (s == 0 && live) __hip_atomic_store(bsum + (size_t)k * nb + b, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int FMT, int K, bool MULTI, bool PREP = false>
__global__ __launch_bounds__(256) void k_stage_valu(const StageArgs A, const StageGeom g) {
    __shared__ StageSmem<K> sm;
    __shared__ uint2 xs[4][K][8][8];          // [wave][column][block][quarter of 4 fp16]
    if constexpr (PREP) {
        if ((int)blockIdx.x < A.n_prep) {
            stage_rms(A, sm.rs, &sm.red[0][0][0]);
            prep_x_valu<FMT>(A, sm.rs);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (threadIdx.x == 0) __hip_atomic_fetch_add(A.xflag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        const int item = xcd_item((int)blockIdx.x - A.n_prep, (int)gridDim.x - A.n_prep);
        const int tile = item / g.nparts, part = item - tile * g.nparts;
        WTileV cur;
        prefetch_valu<FMT, K == 1>(A, tile, part, cur);
        wait_flag(A.xflag, (unsigned)A.n_prep, A.err);
        stage_item_valu<FMT, K, false, true>(A, g, tile, part, sm, xs, cur, -1, 0);
        return;
    }
    const int item = xcd_item(blockIdx.x, gridDim.x);
    const int tile = item / g.nparts, part = item - tile * g.nparts;
    WTileV cur;
    if constexpr (MULTI) {
        prefetch_valu<FMT, K == 1>(A, tile, part * g.cpw, cur);
        stage_rms(A, sm.rs, &sm.red[0][0][0]);
        stage_item_valu<FMT, K, MULTI>(A, g, tile, part, sm, xs, cur, -1, 0);
    } else {
        // the small loads first (input sums of squares, the chunk's activations), then the
        // weights: loads complete in order, so the scales and activations are ready
        // without waiting for the weights
        StatsPre<4 * K> sp;
        stats_issue<4 * K>(A, sp);
        XPre<K> xp;
        x_issue<K>(A, g.nb, part, xp);
        prefetch_valu<FMT, K == 1>(A, tile, part, cur);
        stats_finish<4 * K>(A, sp, sm.rs, &sm.red[0][0][0]);
        stage_item_valu<FMT, K, MULTI>(A, g, tile, part, sm, xs, cur, -1, 0, &xp);
    }
}

// ------------------------------------------------------------------ MFMA kernel

// Lane group g (lanes 16g..16g+15) holds R[t] = quarter t of block g; afterwards
// R[t] = quarter g of block t.  permlane32_swap exchanges the upper half of its first
// operand with the lower half of its second; permlane16_swap exchanges odd 16-lane rows
// of its first operand with even rows of its second.
__device__ __forceinline__ void transpose4(uint32_t (&R)[4]) {
    auto s02 = __builtin_amdgcn_permlane32_swap(R[0], R[2], false, false);
    auto s13 = __builtin_amdgcn_permlane32_swap(R[1], R[3], false, false);
    R[0] = s02[0];
    R[2] = s02[1];
    R[1] = s13[0];
    R[3] = s13[1];
    auto s01 = __builtin_amdgcn_permlane16_swap(R[0], R[1], false, false);
    auto s23 = __builtin_amdgcn_permlane16_swap(R[2], R[3], false, false);
    R[0] = s01[0];
    R[1] = s01[1];
    R[2] = s23[0];
    R[3] = s23[1];
}

template <int FMT>
__device__ __forceinline__ h8_t widen_block_quarter(uint32_t w) {
    h2_t p[4];
    unpack8<FMT>(w, p);
    h8_t r;
    r[0] = p[0][0]; r[1] = p[0][1];
    r[2] = p[1][0]; r[3] = p[1][1];
    r[4] = p[2][0]; r[5] = p[2][1];
    r[6] = p[3][0]; r[7] = p[3][1];
    return r;
}

// One wave's share of a 64-row tile: 4 sub-tiles of 16 rows x 8 blocks.
struct WTileM {
    u4_t n0[4], n1[4];       // blocks b0 + g and b0 + 4 + g of row j of each sub-tile
    uint32_t sv[4][4];       // scales of blocks b0..b0+7 (8 fp16 or 8 E8M0 bytes)
    uint32_t mv[4][4];       // mins of blocks b0..b0+7 (8 fp16)
};

template <int FMT>
__device__ __forceinline__ void load_tile_mfma(const StageArgs& A, int tile, int j, int gq, int b0, int nvb,
                                               bool al, WTileM& T) {
    const int nb = A.W.cols >> 5;
    const uint32_t rowq = (uint32_t)A.W.cols >> 1, unb = (uint32_t)nb;
    const int bb0 = min(b0, nb - 1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const SegRef R = seg_ref(A.W, tile_seg(A, tile, 16 * t));
        const uint32_t lr = (uint32_t)(clamp_row(A, tile, 16 * t + j) - R.r0);
        const uint32_t qrow = lr * rowq;
        T.n0[t] = ld_global_nt<u4_t>(R.qs + (qrow + 16u * (uint32_t)min(b0 + gq, nb - 1)));
        T.n1[t] = ld_global_nt<u4_t>(R.qs + (qrow + 16u * (uint32_t)min(b0 + 4 + gq, nb - 1)));
        const uint32_t srow = lr * unb * (FMT == VQ_FMT_MXFP4 ? 1u : 2u), mrow = 2u * lr * unb;
        if (al && nvb == 8) {
            if constexpr (FMT == VQ_FMT_MXFP4) {
                const u2_t v = ld_global<u2_t>(R.sc8 + (srow + (uint32_t)b0));
                T.sv[t][0] = v[0];
                T.sv[t][1] = v[1];
                T.sv[t][2] = T.sv[t][3] = 0u;
            } else {
                const u4_t v = ld_global<u4_t>(R.sc8 + (srow + 2u * (uint32_t)b0));
#pragma unroll
                for (int e = 0; e < 4; ++e) T.sv[t][e] = v[e];
            }
            if constexpr (FMT == VQ_FMT_Q4_MIN) {
                const u4_t v = ld_global<u4_t>(reinterpret_cast<const uint8_t*>(R.mn) + (mrow + 2u * (uint32_t)b0));
#pragma unroll
                for (int e = 0; e < 4; ++e) T.mv[t][e] = v[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) T.mv[t][e] = 0u;
            }
        } else {
            // ragged group: one element load per block
            uint32_t sb[8], mb[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t bb = (uint32_t)min(bb0 + i, nb - 1);
                if constexpr (FMT == VQ_FMT_MXFP4) sb[i] = ld_global<uint8_t>(R.sc8 + (srow + bb));
                else sb[i] = ld_global<uint16_t>(R.sc8 + (srow + 2u * bb));
                if constexpr (FMT == VQ_FMT_Q4_MIN)
                    mb[i] = ld_global<uint16_t>(reinterpret_cast<const uint8_t*>(R.mn) + (mrow + 2u * bb));
                else
                    mb[i] = 0u;
                if (i >= nvb) sb[i] = mb[i] = 0u;
            }
            if constexpr (FMT == VQ_FMT_MXFP4) {
                T.sv[t][0] = sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
                T.sv[t][1] = sb[4] | (sb[5] << 8) | (sb[6] << 16) | (sb[7] << 24);
                T.sv[t][2] = T.sv[t][3] = 0u;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) T.sv[t][e] = sb[2 * e] | (sb[2 * e + 1] << 16);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) T.mv[t][e] = mb[2 * e] | (mb[2 * e + 1] << 16);
        }
    }
}

template <int FMT>
__device__ __forceinline__ void compute_tile_mfma(const WTileM& T, int gq, int nvb, const h8_t (&a)[8], h8_t am,
                                                  f4_t (&acc)[4]) {
    const f4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t T0[4] = {T.n0[t][0], T.n0[t][1], T.n0[t][2], T.n0[t][3]};
        uint32_t T1[4] = {T.n1[t][0], T.n1[t][1], T.n1[t][2], T.n1[t][3]};
        transpose4(T0);
        transpose4(T1);
        float d[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (FMT == VQ_FMT_MXFP4) d[i] = e8m0_to_float((T.sv[t][i >> 2] >> (8 * (i & 3))) & 0xffu);
            else d[i] = half_bits_to_float((T.sv[t][i >> 1] >> (16 * (i & 1))) & 0xffffu);
        }
        if constexpr (FMT != VQ_FMT_Q4_MIN) {
            // one product at a time: batched, these formats' kernels take far more
            // registers (the E8M0 one drops from 5 waves per SIMD to 2: measured slower)
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                if (tt < nvb) {
                    const h8_t B = widen_block_quarter<FMT>(tt < 4 ? T0[tt] : T1[tt - 4]);
                    const f4_t D = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[tt], B, zero, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[t][v] = fmaf(d[tt], D[v], acc[t][v]);
                }
            }
        } else {
            // all 8 block products first (independent MFMAs, issued back to back), then
            // the scales in block order; blocks past the row's end have zero A operands
            // and zero scales, so they add exactly nothing
            f4_t D[8];
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                const h8_t B = widen_block_quarter<FMT>(tt < 4 ? T0[tt] : T1[tt - 4]);
                D[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[tt], B, zero, 0, 0, 0);
            }
#pragma unroll
            for (int tt = 0; tt < 8; ++tt)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[t][v] = fmaf(d[tt], D[tt][v], acc[t][v]);
        }
        if constexpr (FMT == VQ_FMT_Q4_MIN) {
            u4_t mm;
#pragma unroll
            for (int e = 0; e < 4; ++e) mm[e] = gq < 2 ? T.mv[t][e] : 0u;
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(am, as_h8(mm), acc[t], 0, 0, 0);
        }
    }
}

// One item: a 64-row tile (4 sub-tiles of 16 rows) x one chunk (4 groups of 8 blocks,
// one per wave).  Lane (j = lane % 16, g = lane / 16): weight row j of a sub-tile and
// k-quarter g of each block; as the A operand, activation column j.
template <int FMT>
__device__ __forceinline__ void prefetch_mfma(const StageArgs& A, int tile, int chunk, WTileM& T) {
    const int nb = A.W.cols >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int b0 = (chunk * 4 + wave) * 8;
    load_tile_mfma<FMT>(A, tile, lane & 15, lane >> 4, b0, max(0, min(8, nb - b0)), (nb & 7) == 0, T);
}

// As stage_item_valu (the same chunk run, load order and next-weights contract); the
// MFMA accumulators carry the sums across the run.
// One lane's raw activations of a chunk for the MFMA A operands: column j = lane mod 16,
// k-quarter gq = lane / 16 of each of the wave's 8 blocks (8 fp16 of the input, or 8 f32
// of the previous output).
struct MPre {
    f4_t raw[8][2];
};

__device__ __forceinline__ void mraw_issue(const StageArgs& A, int nb, int ch, MPre& X) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, gq = lane >> 4;
    const int kk = j < A.K ? j : 0;
    const int bb0 = min((ch * 4 + wave) * 8, nb - 1);
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
        const int col = 32 * min(bb0 + tt, nb - 1) + 8 * gq;
        if (A.glue == GLUE_NONE) {
            X.raw[tt][0] = __builtin_bit_cast(f4_t, *reinterpret_cast<const u4_t*>(A.x16 + (size_t)kk * A.W.cols + col));
            X.raw[tt][1] = X.raw[tt][0];
        } else {
            const float* p = A.src + (size_t)kk * A.ld + col;
            X.raw[tt][0] = *reinterpret_cast<const f4_t*>(p);
            X.raw[tt][1] = *reinterpret_cast<const f4_t*>(p + 4);
        }
    }
}

template <int FMT, bool MULTI, bool PREP = false>
__device__ void stage_item_mfma(const StageArgs& A, const StageGeom& g, int tile, int part, StageSmem<16>& sm,
                                WTileM& cur, int ntile, int npart, const MPre* pre = nullptr) {
    float (*red)[16][65] = sm.red;
    const float* rs = sm.rs;
    const int K = A.K;
    const int nb = g.nb;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, gq = lane >> 4;
    const bool col_live = j < K;
    const int kk = col_live ? j : 0;
    const bool keeper = A.keep && tile == 0 && col_live;
    const float r = A.glue == GLUE_NONE ? 1.f : rs[kk];
    const int c0 = part * g.cpw, c1 = MULTI ? min(g.nchunks, c0 + g.cpw) : c0 + 1;
    const f4_t zero = {0.f, 0.f, 0.f, 0.f};
    f4_t acc[4] = {zero, zero, zero, zero};
    for (int ch = c0; ch < c1; ++ch) {
        const int b0 = (ch * 4 + wave) * 8;
        const int nvb = max(0, min(8, nb - b0));      // blocks of this group (wave-uniform)
        const int bb0 = min(b0, nb - 1);
        h8_t a[8];
        h8_t am = h8_t{};
        if constexpr (PREP) {
            // operands converted once for the whole stage (prep_x_mfma)
#pragma unroll
            for (int tt = 0; tt < 8; ++tt)
                a[tt] = tt < nvb ? as_h8(ld_global<u4_t>(A.xp + (size_t)(b0 + tt) * 64 + lane)) : h8_t{};
            if constexpr (FMT == VQ_FMT_Q4_MIN) {
                const h8_t v = nvb > 0 ? as_h8(ld_global<u4_t>(A.xpa + (size_t)(b0 >> 3) * 64 + lane)) : h8_t{};
#pragma unroll
                for (int tt = 0; tt < 8; ++tt) am[tt] = tt < nvb ? v[tt] : (_Float16)0.0f;
            }
        } else {
        // A operands: activation column j, k-quarter gq of each block of the group (raw
        // values first: 8 fp16 of the input, or 8 f32 of the previous output)
        MPre X;
        if (pre && ch == c0) X = *pre;
        else mraw_issue(A, nb, ch, X);
        const f4_t (&raw)[8][2] = X.raw;
        float bsum[8];
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
            uint32_t h[8];
            if (A.glue == GLUE_NONE) {
                const u4_t v = __builtin_bit_cast(u4_t, raw[tt][0]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[2 * e] = v[e] & 0xffffu;
                    h[2 * e + 1] = v[e] >> 16;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[e] = f2h_scaled(raw[tt][0][e], r);
                    h[4 + e] = f2h_scaled(raw[tt][1][e], r);
                }
            }
            if (keeper && tt < nvb) keep_x8(A, kk, 32 * (bb0 + tt) + 8 * gq, h);
            float sum = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) sum += half_bits_to_float(h[e]);
            h8_t v;
#pragma unroll
            for (int p = 0; p < 8; ++p) v[p] = __builtin_bit_cast(_Float16, (uint16_t)h[slot_col<FMT>(p)]);
            const bool use = col_live && tt < nvb;
            a[tt] = use ? v : h8_t{};
            bsum[tt] = use ? sum : 0.f;
        }
        if constexpr (FMT == VQ_FMT_Q4_MIN) {
            // block sums over the 4 k-quarters (lanes j, j+16, j+32, j+48), then fp16 hi / lo
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                float v = bsum[tt];
                v += __shfl_xor(v, 16, 64);
                v += __shfl_xor(v, 32, 64);
                const _Float16 hi = (_Float16)v;
                const _Float16 lo = (_Float16)(v - (float)hi);
                am[tt] = gq == 0 ? hi : (gq == 1 ? lo : (_Float16)0.0f);
            }
        }
        }
        if constexpr (PREFETCH_NEXT) {
            // the next weights load while this chunk is computed (issued only now: a wait
            // for the activations above would otherwise also wait for them)
            WTileM nxt;
            if (ch + 1 < c1) prefetch_mfma<FMT>(A, tile, ch + 1, nxt);
            else if (ntile >= 0) prefetch_mfma<FMT>(A, ntile, npart * g.cpw, nxt);
            compute_tile_mfma<FMT>(cur, gq, nvb, a, am, acc);
            cur = nxt;
        } else {
            compute_tile_mfma<FMT>(cur, gq, nvb, a, am, acc);
            if (ch + 1 < c1) prefetch_mfma<FMT>(A, tile, ch + 1, cur);
            else if (ntile >= 0) prefetch_mfma<FMT>(A, ntile, npart * g.cpw, cur);
        }
    }
    // lane (j, gq) holds D[4 gq + v][j] = column 4 gq + v of row 16 t + j
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][4 * gq + v][16 * t + j] = acc[t][v];
    __syncthreads();
    stage_epilogue<16>(A, tile, part, g.nparts, red, &sm.flag);
}

// The input conversion of stage_item_mfma for the whole stage, done once: wave v of
// the n_prep converting workgroups takes groups of 8 blocks v, v + 4 n_prep, ...; lane
// (j, gq) converts k-quarter gq of column j of each block with the same arithmetic and
// order as the inline conversion, so both give the same bits.  Every 16-byte slot of xp
// and xpa (hence every cache line a reader loads) is written whole by one wave: a line
// assembled from several writers could leave a partly written copy in one XCD's L2.
// Also writes the fp16 copy of the input (if any).
template <int FMT>
__device__ void prep_x_mfma(const StageArgs& A, const float* rs) {
    const int K = A.K;
    const int nb = A.W.cols >> 5;
    const int ngrp = (nb + 7) >> 3;
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, gq = lane >> 4;
    const bool col_live = j < K;
    const int kk = col_live ? j : 0;
    const float r = A.glue == GLUE_NONE ? 1.f : rs[kk];
    const int nwv = A.n_prep * 4;
    for (int gi = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6); gi < ngrp; gi += nwv) {
        const int nvb = min(8, nb - 8 * gi);
        u4_t am = {0u, 0u, 0u, 0u};
        for (int tt = 0; tt < nvb; ++tt) {
            const int b = 8 * gi + tt;
            const int col = 32 * b + 8 * gq;
            uint32_t h[8];
            if (A.glue == GLUE_NONE) {
                const u4_t v = *reinterpret_cast<const u4_t*>(A.x16 + (size_t)kk * A.W.cols + col);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[2 * e] = v[e] & 0xffffu;
                    h[2 * e + 1] = v[e] >> 16;
                }
            } else {
                const float* p = A.src + (size_t)kk * A.ld + col;
                const f4_t x0 = *reinterpret_cast<const f4_t*>(p), x1 = *reinterpret_cast<const f4_t*>(p + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[e] = f2h_scaled(x0[e], r);
                    h[4 + e] = f2h_scaled(x1[e], r);
                }
            }
            if (A.keep && col_live) keep_x8(A, kk, col, h);
            float sum = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) sum += half_bits_to_float(h[e]);
            u4_t v;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                v[q] = col_live ? h[slot_col<FMT>(2 * q)] | (h[slot_col<FMT>(2 * q + 1)] << 16) : 0u;
            A.xp[(size_t)b * 64 + lane] = v;
            if constexpr (FMT == VQ_FMT_Q4_MIN) {
                float t = col_live ? sum : 0.f;
                t += __shfl_xor(t, 16, 64);
                t += __shfl_xor(t, 32, 64);
                const _Float16 hi = (_Float16)t;
                const _Float16 lo = (_Float16)(t - (float)hi);
                const uint32_t e = __builtin_bit_cast(uint16_t, gq == 0 ? hi : (gq == 1 ? lo : (_Float16)0.0f));
                am[tt >> 1] |= e << (16 * (tt & 1));
            }
        }
        if constexpr (FMT == VQ_FMT_Q4_MIN) A.xpa[(size_t)gi * 64 + lane] = am;
    }
}

template <int FMT, bool MULTI, bool PREP = false>
__global__ __launch_bounds__(256) void k_stage_mfma(const StageArgs A, const StageGeom g) {
    __shared__ StageSmem<16> sm;
    if constexpr (PREP) {
        if ((int)blockIdx.x < A.n_prep) {
            // convert the stage's input, publish it (written back past this XCD's L2
            // before the count), count this workgroup
            stage_rms(A, sm.rs, &sm.red[0][0][0]);
            prep_x_mfma<FMT>(A, sm.rs);
            // plain stores written back by a fence before the count (measured faster here
            // than write-through stores; the VALU conversion measured the other way)
            __threadfence();
            __syncthreads();
            if (threadIdx.x == 0) __hip_atomic_fetch_add(A.xflag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        const int item = xcd_item((int)blockIdx.x - A.n_prep, (int)gridDim.x - A.n_prep);
        const int tile = item / g.nparts, part = item - tile * g.nparts;
        WTileM cur;
        prefetch_mfma<FMT>(A, tile, part * g.cpw, cur);
        wait_flag(A.xflag, (unsigned)A.n_prep, A.err);
        stage_item_mfma<FMT, MULTI, true>(A, g, tile, part, sm, cur, -1, 0);
        return;
    }
    const int item = xcd_item(blockIdx.x, gridDim.x);
    const int tile = item / g.nparts, part = item - tile * g.nparts;
    WTileM cur;
    // the small loads first, then the weights, as in the VALU kernel: the input sums of
    // squares always; the first chunk's activations too for one-chunk items (with chunk
    // runs they would hold too many registers across the weight loads)
    StatsPre<8> sp;
    stats_issue<8>(A, sp);
    if constexpr (MULTI) {
        prefetch_mfma<FMT>(A, tile, part * g.cpw, cur);
        stats_finish<8>(A, sp, sm.rs, &sm.red[0][0][0]);
        stage_item_mfma<FMT, MULTI>(A, g, tile, part, sm, cur, -1, 0);
    } else {
        MPre xp;
        mraw_issue(A, g.nb, part, xp);
        prefetch_mfma<FMT>(A, tile, part, cur);
        stats_finish<8>(A, sp, sm.rs, &sm.red[0][0][0]);
        stage_item_mfma<FMT, MULTI>(A, g, tile, part, sm, cur, -1, 0, &xp);
    }
}


// ------------------------------------------------------------------ row-strip VALU kernel
//
// One item = R consecutive output rows (gate|up: rows h of both halves for R / 2 values
// of h) over all columns, so no partial sum leaves the workgroup.  The whole row's
// activations (K x cols fp16) sit in LDS, converted once per stage and workgroup, in the
// widened pair order (quarters swizzled against bank conflicts).  Wave w computes the
// item's local rows 4j + w (j < RW); lane l takes block 64s + l of each of the row's NSG
// 64-block segments, so a wave reads 1 KB of one row's codes per load instruction.  The
// code is specialised on NSG so that all loads and block terms are straight-line, which
// lets the compiler wait for exactly the item being computed while the next item's
// loads are in flight (lanes past the row's last block re-read that block, which the
// wave's load merges, and drop the term).  A block term is d * sum q x (+ m * sum x),
// with q widened exactly to fp16 as in the tile kernel, so a row of zero codes or zero
// scales gives exactly 0.

struct RowSmem {
    u4_t xs[ROWS_X_BYTES / 16];      // [k][block][quarter] fp16 x, quarters swizzled
    float scratch[ROWS_X_BYTES / 16 > ROWS_MAX_K * 256 ? ROWS_X_BYTES / 16 : ROWS_MAX_K * 256];
                                     // RMS reduction (K x 256) / quarter sums (K x xwb x 4)
    float xb[ROWS_X_BYTES / 64];     // [k][block] sums of x (Q4 with mins)
    float fin[16][ROWS_MAX_K];       // the item's outputs [R][K]
    float rs[VQ_MAX_K];
};

// Local row lr of an item: its matrix row, whether it exists, and its segment.
struct RowRef {
    int row;
    bool ok;
    int seg;
};

__device__ __forceinline__ RowRef rows_ref(const StageArgs& A, const StageGeom& g, int item, int lr) {
    RowRef r;
    if (A.paired) {
        const int hr = g.R >> 1, half = A.W.seg_end[0];
        const int up = lr >= hr;
        const int h = item * hr + (up ? lr - hr : lr);
        r.ok = h < half;
        r.row = (up ? half : 0) + min(h, half - 1);
        r.seg = up;
    } else {
        const int row = item * g.R + lr;
        r.ok = row < A.W.rows;
        r.row = min(row, A.W.rows - 1);
        const int row0 = item * g.R;        // items never straddle a segment boundary
        r.seg = (A.W.nseg > 2 && row0 >= A.W.seg_end[1]) ? 2 : (A.W.nseg > 1 && row0 >= A.W.seg_end[0]) ? 1 : 0;
    }
    return r;
}

// The stage's (up to three) segment bases, pinned in scalar registers once per stage.
struct StageSegs {
    SegRef s[MAX_SEG];
    __device__ __forceinline__ const SegRef& get(int seg) const { return seg == 2 ? s[2] : seg == 1 ? s[1] : s[0]; }
};

__device__ __forceinline__ StageSegs stage_segs(const StageArgs& A) {
    StageSegs r;
#pragma unroll
    for (int i = 0; i < MAX_SEG; ++i) r.s[i] = seg_ref(A.W, i);
    return r;
}

// Converts the activations into LDS (and, for item 0's owner, the fp16 copy of the stage
// input), with the sum of every block (for the min term).  Thread t takes quarters t,
// t + 256, ... (8 columns each).
template <int FMT, int K>
__device__ void rows_stage_x(const StageArgs& A, const StageGeom& g, bool keeper, RowSmem& sm) {
    constexpr int QMAX = ROWS_X_BYTES / 16 / 256;      // quarters per thread at most
    constexpr bool Q4F = FMT == VQ_FMT_Q4_MIN;
    const int nb = g.nb;
    const int nq = K * nb * 4;
    f4_t ra[QMAX], rb[QMAX];
#pragma unroll
    for (int i = 0; i < QMAX; ++i) {
        const int qi = threadIdx.x + 256 * i;
        if (qi < nq) {
            const int k = qi / (nb * 4), rem = qi - k * nb * 4;
            const int col = 8 * rem;
            if (A.glue == GLUE_NONE) {
                ra[i] = __builtin_bit_cast(f4_t, *reinterpret_cast<const u4_t*>(A.x16 + (size_t)k * A.W.cols + col));
            } else {
                const float* p = A.src + (size_t)k * A.ld + col;
                ra[i] = *reinterpret_cast<const f4_t*>(p);
                rb[i] = *reinterpret_cast<const f4_t*>(p + 4);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < QMAX; ++i) {
        const int qi = threadIdx.x + 256 * i;
        if (qi < nq) {
            const int k = qi / (nb * 4), rem = qi - k * nb * 4;
            const int b = rem >> 2, q = rem & 3;
            uint32_t h[8];
            if (A.glue == GLUE_NONE) {
                const u4_t v = __builtin_bit_cast(u4_t, ra[i]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[2 * e] = v[e] & 0xffffu;
                    h[2 * e + 1] = v[e] >> 16;
                }
            } else {
                const float r = sm.rs[k];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[e] = f2h_scaled(ra[i][e], r);
                    h[4 + e] = f2h_scaled(rb[i][e], r);
                }
            }
            if (keeper) {
                u4_t v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = h[2 * e] | (h[2 * e + 1] << 16);
                *reinterpret_cast<u4_t*>(A.keep + (size_t)k * A.W.cols + 8 * rem) = v;
            }
            u4_t pk;
#pragma unroll
            for (int t = 0; t < 4; ++t) pk[t] = h[slot_col<FMT>(2 * t)] | (h[slot_col<FMT>(2 * t + 1)] << 16);
            sm.xs[(k * g.xwb + b) * 4 + (q ^ ((b >> 2) & 3))] = pk;
            if constexpr (Q4F) {
                float f[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = half_bits_to_float(h[e]);
                sm.scratch[(k * g.xwb + b) * 4 + q] = ((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7]));
            }
        }
    }
    __syncthreads();
    if constexpr (Q4F) {
        for (int t = threadIdx.x; t < K * nb; t += 256) {
            const int k = t / nb, b = t - k * nb;
            const float* q4 = &sm.scratch[(k * g.xwb + b) * 4];
            sm.xb[k * g.xwb + b] = (q4[0] + q4[1]) + (q4[2] + q4[3]);
        }
        __syncthreads();
    }
}

template <int N>
struct WRowN {
    u4_t w[N];
    uint32_t sr[N], mr[N];
};

template <int NSG>
struct RowShape {
    static constexpr int RW = rows_per_wave(NSG);      // rows per wave
    static constexpr int N = RW * NSG;                 // loads per lane
};

// The weights of item `item` for this lane; idle = true issues the same loads, all lanes
// of a wave on the first block of each row (a cheap stand-in when there is no next
// item, which keeps the compiler's load-counter waits exact).
template <int FMT, int NSG>
__device__ __forceinline__ void rows_load_s(const StageArgs& A, const StageGeom& g, const StageSegs& S, int item,
                                            WRowN<RowShape<NSG>::N>& T, bool idle) {
    constexpr int RW = RowShape<NSG>::RW;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const uint32_t rowq = (uint32_t)A.W.cols >> 1, nb = (uint32_t)g.nb;
#pragma unroll
    for (int j = 0; j < RW; ++j) {
        const RowRef rr = rows_ref(A, g, item, 4 * j + wave);
        const SegRef& R = S.get(__builtin_amdgcn_readfirstlane(rr.seg));
        const uint32_t lr = (uint32_t)(rr.row - R.r0);
#pragma unroll
        for (int sg = 0; sg < NSG; ++sg) {
            const int u = j * NSG + sg;
            const uint32_t b = idle ? 0u : min((uint32_t)(64 * sg + lane), nb - 1u);
            T.w[u] = ld_global_nt<u4_t>(R.qs + (lr * rowq + 16u * b));
            if constexpr (FMT == VQ_FMT_MXFP4) {
                T.sr[u] = ld_global<uint8_t>(R.sc8 + (lr * nb + b));
                T.mr[u] = 0u;
            } else {
                T.sr[u] = ld_global<uint16_t>(R.sc8 + 2u * (lr * nb + b));
                T.mr[u] = FMT == VQ_FMT_Q4_MIN ? (uint32_t)ld_global<uint16_t>(R.mn + (lr * nb + b)) : 0u;
            }
        }
    }
}

// acc[j][k] += this lane's block terms of local row 4j + wave.
template <int FMT, int K, int NSG>
__device__ __forceinline__ void rows_compute_s(const StageArgs& A, const StageGeom& g, int item,
                                               const WRowN<RowShape<NSG>::N>& T, const RowSmem& sm,
                                               float (&acc)[RowShape<NSG>::RW][K]) {
    constexpr int RW = RowShape<NSG>::RW;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    bool ok[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) ok[j] = rows_ref(A, g, item, 4 * j + wave).ok;
#pragma unroll
    for (int sg = 0; sg < NSG; ++sg) {
        // the segment's activations serve all RW rows of the wave
        const int bl = 64 * sg + lane;
        const bool in = bl < g.nb;
        const int blc = min(bl, g.nb - 1);
        const int sw = (blc >> 2) & 3;
        // 1 for a lane's own block of an existing row, 0 for a repeated one (a factor,
        // not a branch: every lane computes a finite term either way)
        float msk[RW];
#pragma unroll
        for (int j = 0; j < RW; ++j) msk[j] = (in && ok[j]) ? 1.f : 0.f;
        u4_t xq[K][4];
        float xs[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int xb = (k * g.xwb + blc) * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) xq[k][i] = sm.xs[xb + (i ^ sw)];
            xs[k] = FMT == VQ_FMT_Q4_MIN ? sm.xb[k * g.xwb + blc] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const int u = j * NSG + sg;
            const float d = FMT == VQ_FMT_MXFP4 ? e8m0_to_float(T.sr[u]) : half_bits_to_float(T.sr[u]);
            const float m = FMT == VQ_FMT_Q4_MIN ? half_bits_to_float(T.mr[u]) : 0.f;
            h2_t p[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) unpack8<FMT>(T.w[u][i], p[i]);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float t = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) t = __builtin_amdgcn_fdot2(p[i][e], as_h2(xq[k][i][e]), t, false);
                float v = d * t;
                if constexpr (FMT == VQ_FMT_Q4_MIN) v = fmaf(m, xs[k], v);
                acc[j][k] = fmaf(v, msk[j], acc[j][k]);
            }
        }
    }
}


// Outputs, sums of squares and silu(gate) * up of an item whose results are in sm.fin.
template <int K>
__device__ __forceinline__ void rows_epilogue(const StageArgs& A, const StageGeom& g, int item, RowSmem& sm) {
    const int rows = A.W.rows;
    for (int e = threadIdx.x; e < g.R * K; e += 256) {
        const int lr = e / K, k = e - lr * K;
        const RowRef rr = rows_ref(A, g, item, lr);
        if (!rr.ok) continue;
        const size_t o = (size_t)k * rows + rr.row;
        if (A.y_dtype == VQ_DTYPE_F16)
            reinterpret_cast<uint16_t*>(A.y)[o] = (uint16_t)f2h_bits(sm.fin[lr][k]);
        else
            st_shared_f32(reinterpret_cast<float*>(A.y) + o, sm.fin[lr][k], A.coh);
    }
    if (A.stats_out && threadIdx.x < (unsigned)K) {
        const int k = threadIdx.x;
        float ss = 0.f;
        if (A.paired) {
            const int hr = g.R >> 1, half = A.W.seg_end[0];
            for (int l = 0; l < hr; ++l) {
                const int h = item * hr + l;
                if (h >= half) break;
                const float v = silu_mul(sm.fin[l][k], sm.fin[hr + l][k]);
                st_shared_f32(A.sbuf + (size_t)k * half + h, v, A.coh);
                ss += v * v;
            }
        } else {
            for (int l = 0; l < g.R; ++l) {
                const int row = item * g.R + l;
                if (row < A.nstat && row < rows) ss += sm.fin[l][k] * sm.fin[l][k];
            }
        }
        st_shared_f32(A.stats_out + (size_t)item * K + k, ss, A.coh);
    }
}

// Items vid, vid + nwg, ... of a stage; `cur` holds the first one's weights, already
// issued.  The stage's input scales and activations are prepared once; each item's
// weights are issued before the previous item is computed.
template <int FMT, int K, int NSG>
__device__ void rows_run_s(const StageArgs& A, const StageGeom& g, const StageSegs& S, int vid, int nwg,
                           RowSmem& sm, WRowN<RowShape<NSG>::N>& cur) {
    constexpr int RW = RowShape<NSG>::RW;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    stage_rms(A, sm.rs, sm.scratch);
    rows_stage_x<FMT, K>(A, g, A.keep && vid == 0, sm);
    for (int it = vid; it < g.nitems; it += nwg) {
        const int nx = it + nwg;
        const bool more = nx < g.nitems;
        WRowN<RowShape<NSG>::N> nxt;
        rows_load_s<FMT, NSG>(A, g, S, more ? nx : it, nxt, !more);
        float acc[RW][K];
#pragma unroll
        for (int j = 0; j < RW; ++j)
#pragma unroll
            for (int k = 0; k < K; ++k) acc[j][k] = 0.f;
        rows_compute_s<FMT, K, NSG>(A, g, it, cur, sm, acc);
#pragma unroll
        for (int j = 0; j < RW; ++j)
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float v = wave_sum(acc[j][k]);
                if (lane == 0) sm.fin[4 * j + wave][k] = v;
            }
        __syncthreads();
        rows_epilogue<K>(A, g, it, sm);
        cur = nxt;
        __syncthreads();                      // fin is reused by the next item
    }
}

template <int FMT, int K, int NSG>
__global__ __launch_bounds__(256) void k_rows_s(const StageArgs A, const StageGeom g) {
    __shared__ RowSmem sm;
    const int nwg = gridDim.x;
    const int vid = xcd_item(blockIdx.x, nwg);
    const StageSegs S = stage_segs(A);
    WRowN<RowShape<NSG>::N> cur;
    rows_load_s<FMT, NSG>(A, g, S, vid, cur, false);
    rows_run_s<FMT, K, NSG>(A, g, S, vid, nwg, sm, cur);
}

// ------------------------------------------------------------------ persistent pass

// Waits until the DONE_REPL group counters at cnt (DONE_STRIDE words apart) sum to
// `target`: thread 0 polls, the workgroup waits at the barrier behind it.  The wait is
// bounded: after about a second without completion the error flag is raised and the
// workgroup proceeds, so a launch always ends.
__device__ void wait_count(const unsigned* cnt, unsigned target, int* err) {
    if (threadIdx.x == 0) {
        unsigned spins = 0;
        for (;;) {
            unsigned sum = 0;
#pragma unroll
            for (int r = 0; r < DONE_REPL; ++r)
                sum += __hip_atomic_load(cnt + r * DONE_STRIDE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (sum >= target) break;
            __builtin_amdgcn_s_sleep(1);
            if ((++spins & 1023u) == 0) {
                // another workgroup gave up: do not wait either
                if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
                if (spins >= (1u << 20)) {
                    __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
    }
    __syncthreads();
}

// The stages of a plan segment in one launch, with the plan's geometry (the same items
// as one launch per stage, so the same sums in the same order).  A stage's items are
// dealt round-robin to the workgroups (those of one XCD take consecutive items, so a
// tile's parts meet in one L2).  There is no grid-wide barrier: a workgroup with items in
// stage s issues its first item's weight loads, then waits until every tile of stage
// s - 1 has counted itself complete, then reads that stage's outputs.  Workgroups without items in a stage go straight on to the next one.
template <int FMT, int K, bool MFMA>
__global__ __launch_bounds__(256) void k_pass(const PassPlan P) {
    struct Smem {
        StageSmem<MFMA ? 16 : K> st;
        uint2 xs[4][MFMA ? 1 : K][8][8];
    };
    __shared__ Smem sm;
    const int nwg = gridDim.x;                // a multiple of 8
    const int grp = blockIdx.x & 7;
    const int vid = grp * (nwg >> 3) + (blockIdx.x >> 3);
    const int s0 = 4 * P.layer0;
    const int s1 = 4 * (P.layer0 + P.nlayers) + (P.with_lm ? 1 : 0);
    auto kind = [&](int stage) { return stage == 4 * P.L ? 4 : stage & 3; };
    for (int stage = s0; stage < s1; ++stage) {
        StageArgs A;
        build_stage(P, stage, A);
        const StageGeom& g = P.geo[kind(stage)];
        if (vid >= g.nitems) continue;
        using Tile = typename std::conditional<MFMA, WTileM, WTileV>::type;
        const int nitems = g.ntiles * g.nparts;
        Tile cur;
        {
            const int tile = vid / g.nparts, part = vid - tile * g.nparts;
            if constexpr (MFMA) prefetch_mfma<FMT>(A, tile, part * g.cpw, cur);
            else prefetch_valu<FMT, K == 1>(A, tile, part * g.cpw, cur);
        }
        if (stage > s0)
            wait_count(P.done + (size_t)(stage - 1) * DONE_WORDS, (unsigned)P.geo[kind(stage - 1)].nstat, P.err);
        stage_rms(A, sm.st.rs, &sm.st.red[0][0][0]);
        for (int it = vid; it < nitems; it += nwg) {
            const int tile = it / g.nparts, part = it - tile * g.nparts;
            const int nx = it + nwg;
            const int ntile = nx < nitems ? nx / g.nparts : -1;
            const int npart = nx < nitems ? nx - ntile * g.nparts : 0;
            if constexpr (MFMA) stage_item_mfma<FMT, true>(A, g, tile, part, sm.st, cur, ntile, npart);
            else stage_item_valu<FMT, K, true>(A, g, tile, part, sm.st, sm.xs, cur, ntile, npart);
            __syncthreads();                  // LDS is reused by the next item
        }
    }
}

template <int FMT, int K, bool MFMA>
const void* pass_fn() {
    return reinterpret_cast<const void*>(&k_pass<FMT, K, MFMA>);
}

template <int FMT>
const void* pass_fn_k(int K, bool mfma) {
    if (mfma) return pass_fn<FMT, 1, true>();
    switch (K) {
        case 1: return pass_fn<FMT, 1, false>();
        case 2: return pass_fn<FMT, 2, false>();
        case 3: return pass_fn<FMT, 3, false>();
        case 4: return pass_fn<FMT, 4, false>();
        case 5: return pass_fn<FMT, 5, false>();
        case 6: return pass_fn<FMT, 6, false>();
        case 7: return pass_fn<FMT, 7, false>();
        default: return pass_fn<FMT, 8, false>();
    }
}

constexpr int PERSIST_WGS_PER_CU = 4;

__global__ void k_zero_u32(unsigned* p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

template <int FMT, int K>
void launch_valu_k(const StageArgs& A, int tg, const StageGeom& g, hipStream_t st) {
    // staged VALU launches take one chunk per item (the plan never gives them runs)
    if (A.n_prep > 0) k_stage_valu<FMT, K, false, true><<<dim3(tg * g.nparts + A.n_prep), 256, 0, st>>>(A, g);
    else k_stage_valu<FMT, K, false><<<dim3(tg * g.nparts), 256, 0, st>>>(A, g);
}

template <int FMT>
void launch_mfma_f(const StageArgs& A, const dim3& grid, const StageGeom& g, hipStream_t st) {
    if (A.n_prep > 0 && g.cpw > 1) k_stage_mfma<FMT, true, true><<<dim3(grid.x + A.n_prep), 256, 0, st>>>(A, g);
    else if (A.n_prep > 0) k_stage_mfma<FMT, false, true><<<dim3(grid.x + A.n_prep), 256, 0, st>>>(A, g);
    else if (g.cpw > 1) k_stage_mfma<FMT, true><<<grid, 256, 0, st>>>(A, g);
    else k_stage_mfma<FMT, false><<<grid, 256, 0, st>>>(A, g);
}

template <int FMT>
void launch_valu_f(const StageArgs& A, int tg, const StageGeom& g, hipStream_t st) {
    switch (A.K) {
        case 1: launch_valu_k<FMT, 1>(A, tg, g, st); break;
        case 2: launch_valu_k<FMT, 2>(A, tg, g, st); break;
        case 3: launch_valu_k<FMT, 3>(A, tg, g, st); break;
        case 4: launch_valu_k<FMT, 4>(A, tg, g, st); break;
        case 5: launch_valu_k<FMT, 5>(A, tg, g, st); break;
        case 6: launch_valu_k<FMT, 6>(A, tg, g, st); break;
        case 7: launch_valu_k<FMT, 7>(A, tg, g, st); break;
        default: launch_valu_k<FMT, 8>(A, tg, g, st); break;
    }
}

}  // namespace

// ------------------------------------------------------------------ host side

// Split-K partials [parts][K][rows] and tile arrival counters, with room for the most
// parts any tile geometry of the stage has: one chunk per item (parts = chunks).
size_t stage_scratch_bytes(int rows, int cols, int K, int paired, int half) {
    const StageGeom g = stage_geom_cpw(rows, cols, paired, half, 1);
    return align_up((size_t)max_parts(cols) * K * rows * 4, 256) + align_up((size_t)g.ntiles * 4, 256);
}

void stage_scratch_carve(void* base, int rows, int cols, int K, int paired, int half, StageArgs* A) {
    (void)paired;
    (void)half;
    A->part = (float*)base;
    A->counters = (unsigned*)((char*)base + align_up((size_t)max_parts(cols) * K * rows * 4, 256));
}

hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    k_zero_u32<<<dim3((n + 255) / 256), 256, 0, st>>>(p, n);
    return hipGetLastError();
}

// Resident workgroups of a kernel on this device (queried once per kernel and device).
int resident_wgs(const void* fn) {
    static std::mutex mu;
    static std::map<std::pair<const void*, int>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find({fn, dev});
    if (it != cache.end()) return it->second;
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, 256, 0) != hipSuccess || occ < 1)
        occ = 1, cus = cus > 0 ? cus : 256;
    const int n = cus * occ;
    cache[{fn, dev}] = n;
    return n;
}

template <int FMT, int K, int NSG>
void launch_rows_s(const StageArgs& A, const StageGeom& g, hipStream_t st) {
    if constexpr (rows_fit(K, NSG)) {
        // one workgroup per item while they all fit at once, else as many as fit (each
        // then streams several items)
        const int nwg = std::min(g.nitems, resident_wgs(reinterpret_cast<const void*>(&k_rows_s<FMT, K, NSG>)));
        k_rows_s<FMT, K, NSG><<<dim3(nwg), 256, 0, st>>>(A, g);
    }
}

template <int FMT, int K>
void launch_rows_k(const StageArgs& A, const StageGeom& g, hipStream_t st) {
    switch (g.xwb / 64) {
        case 1: launch_rows_s<FMT, K, 1>(A, g, st); break;
        case 2: launch_rows_s<FMT, K, 2>(A, g, st); break;
        case 3: launch_rows_s<FMT, K, 3>(A, g, st); break;
        case 4: launch_rows_s<FMT, K, 4>(A, g, st); break;
        case 5: launch_rows_s<FMT, K, 5>(A, g, st); break;
        case 6: launch_rows_s<FMT, K, 6>(A, g, st); break;
        case 7: launch_rows_s<FMT, K, 7>(A, g, st); break;
        case 8: launch_rows_s<FMT, K, 8>(A, g, st); break;
        default: launch_rows_s<FMT, K, 9>(A, g, st); break;
    }
}

template <int FMT>
void launch_rows_f(const StageArgs& A, const StageGeom& g, hipStream_t st) {
    switch (A.K) {
        case 1: launch_rows_k<FMT, 1>(A, g, st); break;
        case 2: launch_rows_k<FMT, 2>(A, g, st); break;
        case 3: launch_rows_k<FMT, 3>(A, g, st); break;
        default: launch_rows_k<FMT, 4>(A, g, st); break;
    }
}

hipError_t launch_stage(const StageArgs& A, const StageGeom& g, bool mfma, hipStream_t st) {
    if (g.rk) {
        switch (A.W.fmt) {
            case VQ_FMT_Q4: launch_rows_f<VQ_FMT_Q4>(A, g, st); break;
            case VQ_FMT_Q4_MIN: launch_rows_f<VQ_FMT_Q4_MIN>(A, g, st); break;
            default: launch_rows_f<VQ_FMT_MXFP4>(A, g, st); break;
        }
        return hipGetLastError();
    }
    // one workgroup per item (a tile and a run of its chunks); the partials were sized
    // for at most max_parts parts
    if (g.nparts < 1 || g.nparts > max_parts(A.W.cols) || g.cpw < 1) return hipErrorInvalidValue;
    const int tg = g.ntiles;
    const dim3 grid(tg * g.nparts);
    if (mfma) {
        switch (A.W.fmt) {
            case VQ_FMT_Q4: launch_mfma_f<VQ_FMT_Q4>(A, grid, g, st); break;
            case VQ_FMT_Q4_MIN: launch_mfma_f<VQ_FMT_Q4_MIN>(A, grid, g, st); break;
            default: launch_mfma_f<VQ_FMT_MXFP4>(A, grid, g, st); break;
        }
    } else {
        switch (A.W.fmt) {
            case VQ_FMT_Q4: launch_valu_f<VQ_FMT_Q4>(A, tg, g, st); break;
            case VQ_FMT_Q4_MIN: launch_valu_f<VQ_FMT_Q4_MIN>(A, tg, g, st); break;
            default: launch_valu_f<VQ_FMT_MXFP4>(A, tg, g, st); break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_pass_segment(const PassPlan& P, bool mfma, hipStream_t st) {
    // tile geometries only, within the partial buffers' room
    const int gcols[5] = {P.H, P.H, P.H, P.FF, P.H};
    for (int j = 0; j < 5; ++j)
        if (P.geo[j].rk || P.geo[j].nparts < 1 || P.geo[j].nparts > max_parts(gcols[j]) || P.geo[j].cpw < 1)
            return hipErrorInvalidValue;
    const void* fn = P.fmt == VQ_FMT_Q4 ? pass_fn_k<VQ_FMT_Q4>(P.K, mfma)
                     : P.fmt == VQ_FMT_Q4_MIN ? pass_fn_k<VQ_FMT_Q4_MIN>(P.K, mfma)
                                              : pass_fn_k<VQ_FMT_MXFP4>(P.K, mfma);
    int dev = 0, cus = 0, occ = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, 256, 0);
    if (e != hipSuccess) return e;
    int nwg = cus * std::min(occ, PERSIST_WGS_PER_CU);
    nwg -= nwg % 8;
    if (nwg < 8) return hipErrorInvalidConfiguration;
    void* args[] = {const_cast<PassPlan*>(&P)};
    // cooperative: the runtime refuses the launch unless every workgroup is resident,
    // which the waits between stages rely on
    e = hipLaunchCooperativeKernel(fn, dim3(nwg), dim3(256), args, 0, st);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace vq
