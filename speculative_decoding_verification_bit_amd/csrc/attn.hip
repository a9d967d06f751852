// The window's attention in one layer over a block-quantised KV cache: the K query rows of
// the verify window read the cache once per layer ("Decode is memory-bound ...", section
// "The ceiling": at long context the cache joins the weights in what every pass reads;
// "100 tokens per second ...", section "The wall": the target's cache kept at q8_0 / q4_0).
//
// Cache: blocks of 32 along the head dimension D = 128 with an fp16 scale each; q8_0 codes
// are int8 (value d * c), q4_0 codes nibbles (value d * (n - 8), low nibble first).  Layout
// per kv head g: codes [L][D] (q8_0) or [L][D/2] (q4_0), scales [L][D/32].  Query head h
// reads kv head h / G (G = Hq / Hkv).  The window is the cache's last K positions; window
// row i sees positions 0 .. L - K + i.
//
// k_attn_part: one workgroup of 4 waves per (span of positions, kv head, group of up to 3
// row tiles); each wave takes a quarter of the span in tiles of 16 positions, with the
// next tiles' loads in flight in registers.  Scores on the f16 matrix instruction over the
// exactly widened key codes (the key scale applied to each 32-dimension block's fp32
// result), an online softmax in log2 units, and p v on the fp32 matrix instruction over
// the values dequantised exactly in fp32.  The waves' results are merged in LDS, and
// k_attn_reduce combines the spans of a head in a fixed order:
// out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, M = max_s m_s.
#include <hip/hip_runtime.h>

#include "vq_device.h"
#include "vq_internal.h"

namespace vq {
namespace {

constexpr int AT_THREADS = 256;
constexpr int AT_WAVES = AT_THREADS / 64;
constexpr int AT_D = 128;            // head dimension
// Waves per SIMD the registers must allow: two with one row tile (each wave keeps one
// pair of tiles in flight ahead), one with more (the accumulators take the registers).
#define AT_WAVES_EU(rtm) ((rtm) == 1 ? 2 : 1)

struct AttnArgs {
    const uint8_t* kc;
    const uint16_t* ks;
    const uint8_t* vc;
    const uint16_t* vs;
    int kfmt, vfmt;
    const uint16_t* q;       // [K][Hq][D]
    float* part_o;           // [Hkv][S][M][D]
    float* part_ml;          // [Hkv][S][M][2]: running maximum (log2 units) and sum
    float* out;              // [K][Hq][D]
    int Hkv, Hq, G, K, L;
    int S, span;             // spans per head, positions per span (a multiple of 64)
};

// Eight q8_0 codes (two dwords, k = 0..7) -> the MFMA operand as exact fp16 pairs
// (c0, c2), (c1, c3), (c4, c6), (c5, c7): an offset byte u = c + 128 OR-ed into the
// mantissa of 1024.0 gives 1024 + u, and (1024 + u) - 1152 = c.
__device__ __forceinline__ h8_t widen_q8(u2_t w) {
    const uint32_t MAGIC = 0x64006400u;
    const h2_t k1152 = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t u0 = w[0] ^ 0x80808080u, u1 = w[1] ^ 0x80808080u;
    const h2_t p0 = as_h2((u0 & 0x00FF00FFu) | MAGIC) - k1152;
    const h2_t p1 = as_h2(((u0 >> 8) & 0x00FF00FFu) | MAGIC) - k1152;
    const h2_t p2 = as_h2((u1 & 0x00FF00FFu) | MAGIC) - k1152;
    const h2_t p3 = as_h2(((u1 >> 8) & 0x00FF00FFu) | MAGIC) - k1152;
    const u4_t r = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                    __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
    return as_h8(r);
}
// Dimension (0..7 within the lane's eight) held by slot p of the widened operand.
__device__ __forceinline__ int slot_dim(bool k8, int p) {
    return k8 ? 4 * (p >> 2) + 2 * (p & 1) + ((p >> 1) & 1) : (p >> 1) + 4 * (p & 1);
}

// fp16 pair (x, y), each rounded toward zero.
__device__ __forceinline__ uint32_t pk_rtz(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x, y));
}
// x - half H of the fp16 pair hb, in one mixed FMA (exact when that half is x rounded
// toward zero: the residual has at most 13 significant bits).
template <int H>
__device__ __forceinline__ float resid(float x, uint32_t hb) {
    float r;
    if constexpr (H == 0) asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(hb), "v"(x));
    else asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(hb), "v"(x));
    return r;
}
// Eight fp32 values as fp16 hi + lo operands (hi rounded toward zero, lo the rounded
// residual): hi + lo equals each value to within 2^-22 of it (2^-25 absolute below 2^-3).
__device__ __forceinline__ void split8(const float (&x)[8], h8_t& hi, h8_t& lo) {
    u4_t h, l;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        h[k] = pk_rtz(x[2 * k], x[2 * k + 1]);
        l[k] = pk_rtz(resid<0>(x[2 * k], h[k]), resid<1>(x[2 * k + 1], h[k]));
    }
    hi = as_h8(h);
    lo = as_h8(l);
}

// RTM: row tiles of this workgroup (at most, 1..3); K8 / V8: q8_0 keys / values (else q4_0).
//
// Wave w of workgroup (s, g) takes positions [w0, w1) (a quarter of the workgroup's span)
// in tiles of 16, one tile's loads in flight while the previous one is used.  Per tile:
//  * scores, transposed: S^T[pos][r] = sum_b d_k[pos][b] (codes_b[pos] . q_b[r]), one
//    v_mfma_f32_16x16x32_f16 per 32-dimension block b (A: lane (pos i, kq) holds 8 key
//    codes widened exactly to fp16; B: lane (row n, kq) the query's 8 matching fp16
//    values; fp32 sums), the key scale applied to each block's fp32 result.  Output lane
//    (row n, q) holds positions 4 q .. 4 q + 3 of row n, in log2 units (times log2(e) /
//    sqrt(128));
//  * online softmax per row: the tile's maximum over the 4 lanes of the row, the running
//    output and sum scaled by 2^(m_old - m_new), p = 2^(s - m_new);
//  * O^T[dim][r] += V^T[dim][pos] P^T[pos][r] on v_mfma_f32_16x16x4f32 (fp32 operands:
//    the values d * code exact in fp32, p as computed).  Step t of the tile takes
//    positions 4 kq + t, so lane (row n, kq)'s own score for position 4 kq + t is its B
//    element; output tile dt's row i is dimension 8 i + dt, so lane (i, kq) loads the
//    8 consecutive dimensions 8 i .. 8 i + 7 of its 4 positions.
// The 4 waves' results are merged in LDS in wave order; the span's partial (m, l, O) of
// every row goes to memory.
template <int RTM, bool K8, bool V8>
__global__ void __launch_bounds__(AT_THREADS) __attribute__((amdgpu_waves_per_eu(AT_WAVES_EU(RTM), 8)))
k_attn_part(AttnArgs A) {
    __shared__ u4_t qb[RTM][4][64];                          // scores' B operand per row tile, block
    __shared__ float wm[AT_WAVES][16 * RTM], wl[AT_WAVES][16 * RTM];
    __shared__ __attribute__((aligned(16))) float ob[16 * RTM][AT_D + 4];

    const int s = blockIdx.x, g = blockIdx.y;
    // the wave index in a scalar register, so that the control flow that depends on it is
    // uniform (no exec masking around the accumulators)
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, q4 = lane >> 4;
    const int M = A.G * A.K;
    // this workgroup's row tiles: RTM of them from tile blockIdx.z * RTM (fewer at the end)
    const int mt0 = blockIdx.z * RTM, rt = min(RTM, (M + 15) / 16 - mt0);
    constexpr int kbytes = K8 ? AT_D : AT_D / 2, vbytes = V8 ? AT_D : AT_D / 2;

    // the queries as B operands: lane (n, kq) of tile mt, block b holds row 16 mt + n's
    // dimensions 32 b + 8 kq + slot_dim(p), p = 0..7 (zero rows past M)
    for (int e = tid; e < RTM * 4 * 64; e += AT_THREADS) {
        const int l = e & 63, b = (e >> 6) & 3, mt = e >> 8;
        const int r = 16 * (mt0 + mt) + (l & 15), kq = l >> 4;
        u4_t v = {0u, 0u, 0u, 0u};
        if (r < M) {
            const int i = r / A.G, hh = r - i * A.G;
            const uint16_t* src = A.q + ((size_t)i * A.Hq + g * A.G + hh) * AT_D + 32 * b + 8 * kq;
#pragma unroll
            for (int p = 0; p < 8; p += 2)
                v[p >> 1] = (uint32_t)src[slot_dim(K8, p)] | ((uint32_t)src[slot_dim(K8, p + 1)] << 16);
        }
        qb[mt][b][l] = v;
    }
    __syncthreads();

    const int p0 = s * A.span, p1 = min(p0 + A.span, A.L);
    const int wsp = A.span / AT_WAVES;
    const int w0 = min(p0 + wave * wsp, p1), w1 = min(w0 + wsp, p1);
    const size_t head = (size_t)g * A.L;
    const float C = 1.4426950408889634f * 0.08838834764831845f;   // log2(e) / sqrt(128)

    // last visible position of each of the lane's rows (rows past M see everything: their
    // queries are zero and their results are dropped)
    int lim[RTM];
#pragma unroll
    for (int mt = 0; mt < RTM; ++mt) {
        const int r = 16 * (mt0 + mt) + n16;
        lim[mt] = r < M ? A.L - A.K + r / A.G : A.L;
    }

    f4_t o[RTM][8];
    float m_run[RTM], l_run[RTM];
#pragma unroll
    for (int mt = 0; mt < RTM; ++mt) {
        m_run[mt] = -INFINITY;
        l_run[mt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[mt][dt] = f4_t{0.f, 0.f, 0.f, 0.f};
    }

    // one tile's loads: key codes of position pb + n16 (block b at 8 / 4 bytes per lane),
    // key scales of positions pb + 4 q4 + j, value codes of dimensions 8 n16 .. + 7 and
    // their block's scale for positions pb + 4 q4 + t.
    struct Tile {
        u2_t kc[4];
        u2_t ks[4];
        u2_t vc[4];
        uint32_t vs[4];
    };
    // the lane's addresses at position 0 of the head; a tile adds pb rows (a scalar)
    const uint8_t* kl = (const uint8_t*)A.kc + head * kbytes + n16 * kbytes + (K8 ? 8 : 4) * q4;
    const uint8_t* ksl = (const uint8_t*)A.ks + (head + 4 * q4) * 8;
    const uint8_t* vl = (const uint8_t*)A.vc + (head + 4 * q4) * vbytes + (V8 ? 8 : 4) * n16;
    const uint8_t* vsl = (const uint8_t*)A.vs + (head + 4 * q4) * 8 + 2 * (n16 >> 2);
    // a tile whose 16 positions all lie in the cache: fixed offsets from the lane's base
    auto load_fast = [&](Tile& T, int pb) __attribute__((always_inline)) {
        const uint8_t* kp = kl + (size_t)pb * kbytes;
        const uint8_t* ksp = ksl + (size_t)pb * 8;
        const uint8_t* vp = vl + (size_t)pb * vbytes;
        const uint8_t* vsp = vsl + (size_t)pb * 8;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if constexpr (K8) T.kc[b] = ld_global<u2_t>(kp + 32 * b);
            else T.kc[b] = u2_t{ld_global<uint32_t>(kp + 16 * b), 0u};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            T.ks[j] = ld_global<u2_t>(ksp + 8 * j);
            if constexpr (V8) T.vc[j] = ld_global<u2_t>(vp + vbytes * j);
            else T.vc[j] = u2_t{ld_global<uint32_t>(vp + vbytes * j), 0u};
            T.vs[j] = ld_global<uint16_t>(vsp + 8 * j);
        }
    };
    // the tile that runs past the cache's end: those positions read its last position
    // (they are masked), one clamped address per position
    auto load_tail = [&](Tile& T, int pb) __attribute__((always_inline)) {
        const int pk = min(pb + n16, A.L - 1);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint8_t* kp = kl + (ptrdiff_t)(pk - n16) * kbytes;
            if constexpr (K8) T.kc[b] = ld_global<u2_t>(kp + 32 * b);
            else T.kc[b] = u2_t{ld_global<uint32_t>(kp + 16 * b), 0u};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pj = min(pb + 4 * q4 + j, A.L - 1) - 4 * q4;   // rows past the lane's base
            T.ks[j] = ld_global<u2_t>(ksl + (ptrdiff_t)pj * 8);
            if constexpr (V8) T.vc[j] = ld_global<u2_t>(vl + (ptrdiff_t)pj * vbytes);
            else T.vc[j] = u2_t{ld_global<uint32_t>(vl + (ptrdiff_t)pj * vbytes), 0u};
            T.vs[j] = ld_global<uint16_t>(vsl + (ptrdiff_t)pj * 8);
        }
    };

    // the queries' operands in registers for the whole span
    u4_t qr[RTM][4];
#pragma unroll
    for (int mt = 0; mt < RTM; ++mt) {
#pragma unroll
        for (int b = 0; b < 4; ++b) qr[mt][b] = qb[mt][b][lane];
    }
    // last position the lane's row may see in this wave's range, less 4 q4 (so that
    // position pb + 4 q4 + j is visible iff j <= vis_lim - pb)
    int vlim[RTM];
#pragma unroll
    for (int mt = 0; mt < RTM; ++mt) vlim[mt] = min(w1 - 1, lim[mt]) - 4 * q4;

    // A tile's values in a compact exact form: per position t, q4_0 nibbles as fp16 n - 8
    // in the pairs (c, c + 4) of the lane's 8 dimensions, or q8_0 bytes offset to c + 128;
    // the scale as fp16.  value(t, dim) is then one (mixed) FMA, exact in fp32.
    struct Vals {
        uint32_t w[4][4];
        uint32_t d[4];
    };
    auto vals = [&](const Tile& T, Vals& V) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            V.d[t] = T.vs[t];
            if constexpr (V8) {
                V.w[t][0] = T.vc[t][0] ^ 0x80808080u;
                V.w[t][1] = T.vc[t][1] ^ 0x80808080u;
            } else {
                h2_t pp[4];
                unpack_q4(T.vc[t][0], pp);
#pragma unroll
                for (int c = 0; c < 4; ++c) V.w[t][c] = __builtin_bit_cast(uint32_t, pp[c]);
            }
        }
    };
    auto value = [&](const Vals& V, int t, int dim) __attribute__((always_inline)) -> float {
        const _Float16 dh = __builtin_bit_cast(_Float16, (uint16_t)V.d[t]);
        if constexpr (V8) {
            const float u = (float)((V.w[t][dim >> 2] >> (8 * (dim & 3))) & 0xFFu);
            return __builtin_fmaf(u, (float)dh, -128.0f * (float)dh);
        } else {
            const h2_t pr = __builtin_bit_cast(h2_t, V.w[t][dim & 3]);
            return __builtin_fmaf((float)pr[dim >> 2], (float)dh, 0.0f);
        }
    };
    // scores (log2 units, -inf where not visible) of positions pb + 4 q4 + j for the
    // lane's row of tile mt
    auto scores = [&](const Tile& T, int mt, int pb) __attribute__((always_inline)) -> f4_t {
        f4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            h8_t ka;
            if constexpr (K8) {
                ka = widen_q8(T.kc[b]);
            } else {
                h2_t pp[4];
                unpack_q4(T.kc[b][0], pp);
                const u4_t r = {__builtin_bit_cast(uint32_t, pp[0]), __builtin_bit_cast(uint32_t, pp[1]),
                                __builtin_bit_cast(uint32_t, pp[2]), __builtin_bit_cast(uint32_t, pp[3])};
                ka = as_h8(r);
            }
            const f4_t z = {0.f, 0.f, 0.f, 0.f};
            const f4_t part = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, as_h8(qr[mt][b]), z, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float dk = half_bits_to_float((T.ks[j][b >> 1] >> (16 * (b & 1))) & 0xFFFFu);
                sc[j] = __builtin_fmaf(dk, part[j], sc[j]);
            }
        }
        const int rel = vlim[mt] - pb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v = sc[j] * C;
            asm volatile("" : "+v"(v));                          // computed for every lane, then selected
            sc[j] = j <= rel ? v : -INFINITY;
        }
        return sc;
    };

    // Two tiles (32 positions) per step.  p v on the f16 matrix instruction: slot s of the
    // lane's 8 k values is position 4 q4 + s of tile a (s < 4) or 4 q4 + s - 4 of tile b,
    // which is where the lane's values and scores of those positions already are.  Values
    // and 2^7 p go in as fp16 hi + lo (hi hi + hi lo + lo hi; the lo lo term is below
    // 2^-22 of the product); 2^7 p <= 2^15 stays in fp16 range, and the factor cancels
    // between the sums and the outputs.
    auto step2 = [&](const Tile& Ta, const Tile& Tb, int pb) __attribute__((always_inline)) {
        Vals va, vb;
        vals(Ta, va);
        vals(Tb, vb);
        // the values' hi + lo operands of dimension tile dt: made where they are used with
        // one row tile, once per pair (kept for every row tile) with more
        auto vsplit = [&](int dt, h8_t& vh, h8_t& vl) __attribute__((always_inline)) {
            const float x[8] = {value(va, 0, dt), value(va, 1, dt), value(va, 2, dt), value(va, 3, dt),
                                value(vb, 0, dt), value(vb, 1, dt), value(vb, 2, dt), value(vb, 3, dt)};
            split8(x, vh, vl);
        };
        constexpr int NV = RTM == 1 ? 1 : 8;
        h8_t vhs[NV], vls[NV];
        if constexpr (RTM > 1) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) vsplit(dt, vhs[dt], vls[dt]);
        }
#pragma unroll
        for (int mt = 0; mt < RTM; ++mt) {
            if (mt < rt) {
                const f4_t sa = scores(Ta, mt, pb), sb = scores(Tb, mt, pb + 16);
                float mx = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(sa[0], sa[1]), __builtin_fmaxf(sa[2], sa[3])),
                                           __builtin_fmaxf(__builtin_fmaxf(sb[0], sb[1]), __builtin_fmaxf(sb[2], sb[3])));
                mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16));
                mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
                // The reference maximum moves only when a row's scores exceed it by more
                // than 2^8 (p <= 256 otherwise); then every row of the tile moves to its
                // running maximum and the tile's sums and outputs are scaled to match.
                if (__builtin_amdgcn_ballot_w64(mx > m_run[mt] + 8.0f) != 0) {
                    const float mn = __builtin_fmaxf(m_run[mt], mx);
                    const float alpha = m_run[mt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[mt] - mn);
                    l_run[mt] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) o[mt][dt] *= alpha;
                    m_run[mt] = mn;
                }
                // 2^7 p; a row with no visible position yet has every score -inf (p = 0)
                const float mu = (m_run[mt] == -INFINITY ? 0.f : m_run[mt]) - 7.0f;
                float pv[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pv[j] = __builtin_amdgcn_exp2f(sa[j] - mu);
                    pv[4 + j] = __builtin_amdgcn_exp2f(sb[j] - mu);
                }
                l_run[mt] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
                h8_t ph, pl;
                split8(pv, ph, pl);
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    h8_t vh, vl;
                    if constexpr (RTM == 1) {
                        vsplit(dt, vh, vl);
                    } else {
                        vh = vhs[dt];
                        vl = vls[dt];
                    }
                    o[mt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, ph, o[mt][dt], 0, 0, 0);
                    o[mt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, pl, o[mt][dt], 0, 0, 0);
                    o[mt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl, ph, o[mt][dt], 0, 0, 0);
                }
            }
        }
    };

    // tiles of the wave's range in pairs (a pair's second tile may lie past the range: its
    // positions are masked); only the cache's last pair can run past the cache's end.  A
    // ring of NP pairs in registers keeps the next NP - 1 pairs' loads in flight (as many
    // as the registers left by the row tiles' accumulators allow).
    const int nt = (w1 - w0 + 15) / 16;
    const int np = (nt + 1) / 2;
    const bool tail = np > 0 && w0 + 32 * np > A.L;
    const int nf = np - (tail ? 1 : 0);                      // pairs read without clamping
    constexpr int NP = 2;
    Tile ring[2 * NP];
#pragma unroll
    for (int u = 0; u < NP - 1; ++u) {
        if (u < nf) {
            load_fast(ring[2 * u], w0 + 32 * u);
            load_fast(ring[2 * u + 1], w0 + 32 * u + 16);
        }
    }
    for (int q0 = 0; q0 < nf; q0 += NP) {
#pragma unroll
        for (int u = 0; u < NP; ++u) {
            const int q = q0 + u;
            if (q < nf) {
                const int ahead = q + NP - 1, slot = (u + NP - 1) % NP;
                if (ahead < nf) {
                    load_fast(ring[2 * slot], w0 + 32 * ahead);
                    load_fast(ring[2 * slot + 1], w0 + 32 * ahead + 16);
                }
                step2(ring[2 * u], ring[2 * u + 1], w0 + 32 * q);
            }
        }
    }
    if (tail) {
        load_tail(ring[0], w0 + 32 * nf);
        load_tail(ring[1], w0 + 32 * nf + 16);
        step2(ring[0], ring[1], w0 + 32 * nf);
    }

    // merge the 4 waves in wave order: M = max m_w, each wave's l and O times 2^(m_w - M)
#pragma unroll
    for (int mt = 0; mt < RTM; ++mt) {
        float l = l_run[mt];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (q4 == 0) {
            wm[wave][16 * mt + n16] = m_run[mt];
            wl[wave][16 * mt + n16] = l;
        }
    }
    __syncthreads();
    float sw[RTM], mrow[RTM];
#pragma unroll
    for (int mt = 0; mt < RTM; ++mt) {
        const int r = 16 * mt + n16;                         // local row
        const float mx = __builtin_fmaxf(__builtin_fmaxf(wm[0][r], wm[1][r]), __builtin_fmaxf(wm[2][r], wm[3][r]));
        mrow[mt] = mx;
        sw[mt] = m_run[mt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[mt] - mx);
    }
    for (int w = 0; w < AT_WAVES; ++w) {
        if (wave == w) {
#pragma unroll
            for (int mt = 0; mt < RTM; ++mt) {
                if (mt < rt) {
                    const int r = 16 * mt + n16, rg = 16 * (mt0 + mt) + n16;   // local, global row
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float* dst = &ob[r][8 * (4 * q4 + j)];
                        f4_t a, b;
#pragma unroll
                        for (int dt = 0; dt < 4; ++dt) {
                            a[dt] = o[mt][dt][j] * sw[mt];
                            b[dt] = o[mt][dt + 4][j] * sw[mt];
                        }
                        if (w > 0) {
                            a += *(const f4_t*)dst;
                            b += *(const f4_t*)(dst + 4);
                        }
                        if (w < AT_WAVES - 1) {
                            *(f4_t*)dst = a;
                            *(f4_t*)(dst + 4) = b;
                        } else if (rg < M) {
                            const size_t base = ((size_t)g * A.S + s) * M + rg;
                            float* po = A.part_o + base * AT_D + 8 * (4 * q4 + j);
                            *(f4_t*)po = a;
                            *(f4_t*)(po + 4) = b;
                        }
                    }
                    if (w == AT_WAVES - 1 && q4 == 0 && rg < M) {
                        float l = 0.f;
#pragma unroll
                        for (int v = 0; v < AT_WAVES; ++v) {
                            const float mv = wm[v][r];
                            l += mv == -INFINITY ? 0.f : wl[v][r] * __builtin_amdgcn_exp2f(mv - mrow[mt]);
                        }
                        const size_t base = ((size_t)g * A.S + s) * M + rg;
                        A.part_ml[2 * base] = mrow[mt];
                        A.part_ml[2 * base + 1] = l;
                    }
                }
            }
        }
        __syncthreads();
    }
}

// One workgroup per (row r, kv head g) merges the head's S spans: the weights
// w_s = 2^(m_s - max m) (0 for a span the row sees none of) go to LDS with their fixed-
// order sums; then wave w adds w_s o_s over the spans s = w, w + 4, ... for dimensions
// 2 lane, 2 lane + 1, and the 4 waves' sums are added in wave order.
constexpr int AT_MAX_S = 1024;       // spans per head (attn_plan keeps S below this)

__global__ void __launch_bounds__(AT_THREADS) k_attn_reduce(AttnArgs A) {
    __shared__ float wts[AT_MAX_S];
    __shared__ float red[AT_THREADS];
    __shared__ float wsum[AT_WAVES][AT_D];
    const int r = blockIdx.x, g = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int M = A.G * A.K;
    const size_t first = (size_t)g * A.S * M + r;            // span 0's entry; span s adds s M
    float mx = -INFINITY;
    for (int s = tid; s < A.S; s += AT_THREADS) mx = __builtin_fmaxf(mx, A.part_ml[2 * (first + (size_t)s * M)]);
    red[tid] = mx;
    __syncthreads();
    for (int h = AT_THREADS / 2; h > 0; h >>= 1) {
        if (tid < h) red[tid] = __builtin_fmaxf(red[tid], red[tid + h]);
        __syncthreads();
    }
    mx = red[0];
    __syncthreads();
    float den = 0.f;
    for (int s = tid; s < A.S; s += AT_THREADS) {
        const size_t base = first + (size_t)s * M;
        const float m = A.part_ml[2 * base];
        const float w = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mx);
        wts[s] = w;
        den = __builtin_fmaf(w, A.part_ml[2 * base + 1], den);
    }
    red[tid] = den;
    __syncthreads();
    for (int h = AT_THREADS / 2; h > 0; h >>= 1) {
        if (tid < h) red[tid] += red[tid + h];
        __syncthreads();
    }
    den = red[0];
    float n0 = 0.f, n1 = 0.f;
#pragma unroll 8
    for (int s = wave; s < A.S; s += AT_WAVES) {
        const float2 o = *(const float2*)(A.part_o + (first + (size_t)s * M) * AT_D + 2 * lane);
        const float w = wts[s];
        n0 = __builtin_fmaf(w, o.x, n0);
        n1 = __builtin_fmaf(w, o.y, n1);
    }
    wsum[wave][2 * lane] = n0;
    wsum[wave][2 * lane + 1] = n1;
    __syncthreads();
    if (wave == 0) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int w = 0; w < AT_WAVES; ++w) {
            a0 += wsum[w][2 * lane];
            a1 += wsum[w][2 * lane + 1];
        }
        const int i = r / A.G, h = g * A.G + (r - i * A.G);
        float* o = A.out + ((size_t)i * A.Hq + h) * AT_D;
        o[2 * lane] = a0 / den;
        o[2 * lane + 1] = a1 / den;
    }
}

template <int RTM>
hipError_t launch_part(const AttnArgs& A, int nz, hipStream_t st) {
    const dim3 grid(A.S, A.Hkv, nz);
    const bool k8 = A.kfmt == VQ_KV_Q8_0, v8 = A.vfmt == VQ_KV_Q8_0;
    if (k8 && v8) k_attn_part<RTM, true, true><<<grid, AT_THREADS, 0, st>>>(A);
    else if (k8) k_attn_part<RTM, true, false><<<grid, AT_THREADS, 0, st>>>(A);
    else if (v8) k_attn_part<RTM, false, true><<<grid, AT_THREADS, 0, st>>>(A);
    else k_attn_part<RTM, false, false><<<grid, AT_THREADS, 0, st>>>(A);
    return hipGetLastError();
}

}  // namespace

void attn_plan(int Hkv, int L, int M, int nwg, int* S, int* span) {
    // one round of workgroups: as many per compute unit as waves per SIMD fit;
    // spans of whole 64-position quarters (16-position tiles per wave)
    const int rt = (M + 15) / 16, nz = (rt + 2) / 3;
    const int target = AT_WAVES_EU(rt) * nwg;
    const int s = std::min(AT_MAX_S, std::max(1, target / std::max(1, Hkv * nz)));
    int sp = (L + s - 1) / s;
    sp = std::max(64, (sp + 63) / 64 * 64);
    *span = sp;
    *S = (L + sp - 1) / sp;
}

static size_t attn_part_o_bytes(int Hkv, int S, size_t M) { return align_up((size_t)Hkv * S * M * AT_D * 4, 256); }

size_t attn_workspace_bytes(int Hkv, int Hq, int L, int K, int nwg) {
    int S, span;
    const size_t M = (size_t)(Hq / Hkv) * K;
    attn_plan(Hkv, L, (int)M, nwg, &S, &span);
    return attn_part_o_bytes(Hkv, S, M) + align_up((size_t)Hkv * S * M * 2 * 4, 256);
}

hipError_t launch_attention(const vq_attention& C, const void* q, int K, float* out, uint8_t* ws, int nwg,
                            hipStream_t st) {
    AttnArgs A;
    A.kc = (const uint8_t*)C.k_codes;
    A.ks = (const uint16_t*)C.k_scales;
    A.vc = (const uint8_t*)C.v_codes;
    A.vs = (const uint16_t*)C.v_scales;
    A.kfmt = C.k_format;
    A.vfmt = C.v_format;
    A.q = (const uint16_t*)q;
    A.Hkv = C.n_kv_heads;
    A.Hq = C.n_q_heads;
    A.G = A.Hq / A.Hkv;
    A.K = K;
    A.L = C.length;
    const int M = A.G * K;
    attn_plan(A.Hkv, A.L, M, nwg, &A.S, &A.span);
    A.part_o = (float*)ws;
    A.part_ml = (float*)(ws + attn_part_o_bytes(A.Hkv, A.S, (size_t)M));
    A.out = out;
    // row tiles per workgroup: at most 3 (their accumulators, the tiles in flight and the
    // value operands fill the registers); more rows take several workgroups per span,
    // each reading the span
    const int rt = (M + 15) / 16, nz = (rt + 2) / 3, per = (rt + nz - 1) / nz;
    hipError_t e;
    if (rt > 8) return hipErrorInvalidValue;
    if (per == 1) e = launch_part<1>(A, nz, st);
    else if (per == 2) e = launch_part<2>(A, nz, st);
    else e = launch_part<3>(A, nz, st);
    if (e != hipSuccess) return e;
    k_attn_reduce<<<dim3(M, A.Hkv), AT_THREADS, 0, st>>>(A);
    return hipGetLastError();
}

}  // namespace vq
