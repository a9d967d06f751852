// Weight-streaming linear map y = W x for a K-wide verify window on gfx950.
//
// Decode reads every weight once per pass and multiplies it against the activation
// vector (page "100 tokens per second from a 27B model on a 24 GB AMD card", section
// "The wall"); verification applies the same single read to K activation columns
// (same page, section "How speculative decoding gets past a per-token wall").
//
// Two kernels share one work decomposition: a workgroup of 4 waves owns a 64-row tile
// and a chunk of 4 groups of 8 blocks (256 input columns per wave).  Each wave reads
// its 64 rows x 256 columns of 4-bit codes exactly once, with 16-byte loads, and the
// four waves' partial sums are combined in LDS in a fixed order.  Chunks of one tile
// are written as split-K partials and summed in fixed order by the finalize kernel,
// so results are bitwise reproducible.
//
//  * VALU kernel (K <= 8): lane = weight row, all 64 lanes at the same input columns,
//    so the activations are wave-uniform and feed v_dot2_f32_f16 from scalar
//    registers.  Codes are widened to exact fp16 q = n - 8 with the 0x6400 exponent
//    trick (two nibbles per instruction); the block scale and min are applied once
//    per 32 columns: y += d * sum(q x) + m * sum(x).
//  * MFMA kernel (K <= 16): v_mfma_f32_16x16x32_f16 with the weights as the B operand
//    (16 rows x 32 columns = one quantisation block per instruction) and the K
//    activation columns, zero-padded to 16, as A.  A lane loads a whole block of one
//    row (16 bytes); permlane32/permlane16 swaps transpose 4 lanes' blocks into the
//    k-quarters the MFMA expects.  Each block's product is scaled by its fp16 scale
//    on the accumulator; the min term sum_b m_b * sum(x_b) is one more MFMA per
//    8 blocks with the block sums split into fp16 hi + lo parts.
#include <hip/hip_fp16.h>

#include "vq_internal.h"

namespace vq {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ uint32_t h2_bits(h2_t h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// E8M0 (OCP MX v1.0): 2^(E-127); E = 0 is 2^-127 (an fp32 subnormal), E = 255 NaN.
__device__ __forceinline__ float e8m0_to_float(uint32_t e) {
    if (e == 0u) return __uint_as_float(0x00400000u);
    if (e == 255u) return __uint_as_float(0x7fc00000u);
    return __uint_as_float(e << 23);
}

// Eight 4-bit codes of columns c0..c7 (c0 in bits 0..3) -> exact fp16 q = n - 8 as the
// pairs (c0,c4), (c1,c5), (c2,c6), (c3,c7).  OR-ing a nibble into the mantissa of
// 1024.0 (0x6400) gives 1024 + n; a nibble in bits 4..7 gives 1024 + 16 n.
__device__ __forceinline__ void unpack_q4(uint32_t w, h2_t (&p)[4]) {
    const uint32_t MAGIC = 0x64006400u;
    const uint32_t a = (w & 0x000F000Fu) | MAGIC;
    const uint32_t b = (w & 0x00F000F0u) | MAGIC;
    const uint32_t w8 = w >> 8;
    const uint32_t c = (w8 & 0x000F000Fu) | MAGIC;
    const uint32_t d = (w8 & 0x00F000F0u) | MAGIC;
    const h2_t k1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2_t k16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2_t k72 = {(_Float16)-72.0f, (_Float16)-72.0f};
    p[0] = as_h2(a) - k1032;        // (1024 + n) - 1032 = n - 8, exact
    p[1] = as_h2(b) * k16 + k72;    // (1024 + 16 n) / 16 - 72 = n - 8, exact
    p[2] = as_h2(c) - k1032;
    p[3] = as_h2(d) * k16 + k72;
}

// Eight E2M1 codes (c0 in bits 0..3) -> fp16 values in natural column order
// (c0,c1), (c2,c3), (c4,c5), (c6,c7), by the gfx950 scaled FP4 conversion (scale 1).
__device__ __forceinline__ void unpack_fp4(uint32_t w, h2_t (&p)[4]) {
    p[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    p[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    p[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    p[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
}

template <int FMT>
__device__ __forceinline__ void unpack8(uint32_t w, h2_t (&p)[4]) {
    if constexpr (FMT == VQ_FMT_MXFP4) unpack_fp4(w, p);
    else unpack_q4(w, p);
}

// Position of column c (0..7) of an 8-column group in the widened order above.
__host__ __device__ __forceinline__ int q4_slot(int c) { return (c & 3) * 2 + (c >> 2); }

// Scales (and mins) of blocks [rb, rb + nvb) of one row; rb = row * nb + b0.
template <int FMT, bool AL>
__device__ __forceinline__ void load_scales(const void* scales, const uint16_t* mins, size_t rb,
                                            int nvb, float (&d)[8], float (&m)[8]) {
    if constexpr (FMT == VQ_FMT_MXFP4) {
        const uint8_t* s = (const uint8_t*)scales + rb;
        if (AL) {
            const uint2 v = *reinterpret_cast<const uint2*>(s);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                d[i] = e8m0_to_float((v.x >> (8 * i)) & 0xffu);
                d[i + 4] = e8m0_to_float((v.y >> (8 * i)) & 0xffu);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) d[i] = i < nvb ? e8m0_to_float(s[i]) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) m[i] = 0.f;
    } else {
        const uint16_t* s = (const uint16_t*)scales + rb;
        if (AL) {
            const uint4 v = *reinterpret_cast<const uint4*>(s);
            const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                d[2 * i] = half_bits_to_float(vv[i] & 0xffffu);
                d[2 * i + 1] = half_bits_to_float(vv[i] >> 16);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) d[i] = i < nvb ? half_bits_to_float(s[i]) : 0.f;
        }
        if constexpr (FMT == VQ_FMT_Q4_MIN) {
            const uint16_t* mm = mins + rb;
            if (AL) {
                const uint4 v = *reinterpret_cast<const uint4*>(mm);
                const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    m[2 * i] = half_bits_to_float(vv[i] & 0xffffu);
                    m[2 * i + 1] = half_bits_to_float(vv[i] >> 16);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) m[i] = i < nvb ? half_bits_to_float(mm[i]) : 0.f;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) m[i] = 0.f;
        }
    }
}


// Segment of the 64-row tile starting at row r0 (tiles never straddle segments).
struct SegRef {
    const uint8_t* qs;
    const void* scales;
    const uint16_t* mins;
    int row0;   // first row of the segment
};

__device__ __forceinline__ SegRef seg_of(const Mat& W, int r0) {
    int s = 0;
    if (W.nseg > 1 && r0 >= W.seg_end[0]) s = 1;
    if (W.nseg > 2 && r0 >= W.seg_end[1]) s = 2;
    SegRef g;
    g.qs = W.qs[s];
    g.scales = W.scales[s];
    g.mins = W.mins[s];
    g.row0 = s ? W.seg_end[s - 1] : 0;
    return g;
}

// ------------------------------------------------------------------ VALU kernel

template <int FMT, int K, bool AL>
__global__ __launch_bounds__(256) void k_lin_valu(const Mat W, const uint32_t* __restrict__ xp,
                                                  const float* __restrict__ bsum,
                                                  float* __restrict__ part) {
    __shared__ float red[4][K][64];
    const int rows = W.rows, cols = W.cols;
    const SegRef sg = seg_of(W, blockIdx.x * 64);
    const int nb = cols >> 5;
    const int ngroups = (nb + 7) >> 3;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int grp = blockIdx.y * 4 + wave;
    const int row = blockIdx.x * 64 + lane;
    const int hc = cols >> 1;
    float acc[K];
#pragma unroll
    for (int k = 0; k < K; ++k) acc[k] = 0.f;
    if (grp < ngroups && row < rows) {
        const int b0 = grp * 8;
        const int nvb = min(8, nb - b0);
        const int lr = row - sg.row0;
        const u4_t* qp = reinterpret_cast<const u4_t*>(sg.qs + (size_t)lr * (size_t)hc) + b0;
        u4_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < nvb) w[i] = __builtin_nontemporal_load(qp + i);
        float d[8], m[8];
        load_scales<FMT, AL>(sg.scales, sg.mins, (size_t)lr * nb + b0, nvb, d, m);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i < nvb) {
                const int b = b0 + i;
                const uint32_t wd[4] = {w[i][0], w[i][1], w[i][2], w[i][3]};
                float t[K];
#pragma unroll
                for (int k = 0; k < K; ++k) t[k] = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    h2_t p[4];
                    unpack8<FMT>(wd[q], p);
#pragma unroll
                    for (int k = 0; k < K; ++k) {
                        const uint4 xv = *reinterpret_cast<const uint4*>(
                            xp + (size_t)k * hc + (size_t)b * 16 + q * 4);
                        t[k] = __builtin_amdgcn_fdot2(p[0], as_h2(xv.x), t[k], false);
                        t[k] = __builtin_amdgcn_fdot2(p[1], as_h2(xv.y), t[k], false);
                        t[k] = __builtin_amdgcn_fdot2(p[2], as_h2(xv.z), t[k], false);
                        t[k] = __builtin_amdgcn_fdot2(p[3], as_h2(xv.w), t[k], false);
                    }
                }
#pragma unroll
                for (int k = 0; k < K; ++k) acc[k] = fmaf(d[i], t[k], acc[k]);
                if constexpr (FMT == VQ_FMT_Q4_MIN) {
#pragma unroll
                    for (int k = 0; k < K; ++k) acc[k] = fmaf(m[i], bsum[(size_t)k * nb + b], acc[k]);
                }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) red[wave][k][lane] = acc[k];
    __syncthreads();
    for (int e = threadIdx.x; e < K * 64; e += 256) {
        const int k = e >> 6, l = e & 63;
        const int r = blockIdx.x * 64 + l;
        if (r < rows) {
            const float s = ((red[0][k][l] + red[1][k][l]) + red[2][k][l]) + red[3][k][l];
            part[((size_t)blockIdx.y * K + k) * (size_t)rows + r] = s;
        }
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

__device__ __forceinline__ h8_t as_h8(uint4 v) { return __builtin_bit_cast(h8_t, v); }

template <int FMT, bool AL>
__global__ __launch_bounds__(256) void k_lin_mfma(const Mat W, const uint4* __restrict__ afrag,
                                                  const uint4* __restrict__ mfrag,
                                                  float* __restrict__ part, int K) {
    __shared__ float red[4][16][65];
    const int rows = W.rows, cols = W.cols;
    const SegRef sg = seg_of(W, blockIdx.x * 64);
    const int nb = cols >> 5;
    const int ngroups = (nb + 7) >> 3;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, gq = lane >> 4;
    const int grp = blockIdx.y * 4 + wave;
    const int rbase = blockIdx.x * 64;
    const int hc = cols >> 1;
    f4_t acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f4_t{0.f, 0.f, 0.f, 0.f};
    if (grp < ngroups) {
        const int b0 = grp * 8;
        const int nvb = min(8, nb - b0);
        h8_t a[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = h8_t{};
            if (i < nvb) a[i] = as_h8(afrag[(size_t)(b0 + i) * 64 + lane]);
        }
        h8_t am = h8_t{};
        if constexpr (FMT == VQ_FMT_Q4_MIN) am = as_h8(mfrag[(size_t)grp * 64 + lane]);
        const f4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int row = rbase + 16 * t + j;
            const bool rv = row < rows;
            const int lr = row - sg.row0;
            const u4_t* qp = reinterpret_cast<const u4_t*>(sg.qs + (size_t)lr * (size_t)hc) + b0;
            u4_t n0 = {0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
            u4_t n1 = n0;
            if (rv && gq < nvb) n0 = __builtin_nontemporal_load(qp + gq);
            if (rv && 4 + gq < nvb) n1 = __builtin_nontemporal_load(qp + 4 + gq);
            float d[8], m[8];
            if (rv) {
                load_scales<FMT, AL>(sg.scales, sg.mins, (size_t)lr * nb + b0, nvb, d, m);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) d[i] = m[i] = 0.f;
            }
            uint32_t T0[4] = {n0[0], n0[1], n0[2], n0[3]};
            uint32_t T1[4] = {n1[0], n1[1], n1[2], n1[3]};
            transpose4(T0);
            transpose4(T1);
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                if (tt < nvb) {
                    const h8_t B = widen_block_quarter<FMT>(tt < 4 ? T0[tt] : T1[tt - 4]);
                    const f4_t D = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[tt], B, zero, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[t][v] = fmaf(d[tt], D[v], acc[t][v]);
                }
            }
            if constexpr (FMT == VQ_FMT_Q4_MIN) {
                h8_t Bm = h8_t{};
                if (rv && gq < 2) {
                    const uint16_t* mp = sg.mins + (size_t)lr * nb + b0;
                    if (AL) {
                        Bm = as_h8(*reinterpret_cast<const uint4*>(mp));
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            if (i < nvb) Bm[i] = __builtin_bit_cast(_Float16, mp[i]);
                    }
                }
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(am, Bm, acc[t], 0, 0, 0);
            }
        }
    }
    // lane (j, gq) holds D[4 gq + v][j]: activation column 4 gq + v, weight row 16 t + j
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][4 * gq + v][16 * t + j] = acc[t][v];
    __syncthreads();
    for (int e = threadIdx.x; e < K * 64; e += 256) {
        const int k = e >> 6, l = e & 63;
        const int r = rbase + l;
        if (r < rows) {
            const float s = ((red[0][k][l] + red[1][k][l]) + red[2][k][l]) + red[3][k][l];
            part[((size_t)blockIdx.y * K + k) * (size_t)rows + r] = s;
        }
    }
}

// ------------------------------------------------------------- activation layouts

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Source of activation (k, c) for the prep kernels.
struct XSrc {
    const uint16_t* x16;   // plain fp16 input [K][cols], or NULL
    const float* src;      // raw fp32 stage output
    int ld, up_off, mode;
    const float* stats;
    int nstats;
    uint16_t* keep;        // fp16 copy of the prepared input [K][cols], or NULL
};

// Inverse RMS of each activation column from per-block partial sums of squares.
__device__ void glue_scales(const XSrc& S, int K, int n, float* rs) {
    if (S.mode != GLUE_NONE && threadIdx.x < (unsigned)K) {
        float ss = 0.f;
        for (int i = 0; i < S.nstats; ++i) ss += S.stats[(size_t)i * K + threadIdx.x];
        rs[threadIdx.x] = 1.0f / __fsqrt_rn(__fdiv_rn(ss, (float)n));
    }
    __syncthreads();
}

// Loads the 32 activations of block b of column k as fp16 bits, applying the glue.
__device__ __forceinline__ void load_block_x(const XSrc& S, int cols, int k, int b, float r,
                                             uint16_t (&h)[32]) {
    if (S.mode == GLUE_NONE) {
        const uint4* p = reinterpret_cast<const uint4*>(S.x16 + (size_t)k * cols + (size_t)b * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 v = p[i];
            const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h[i * 8 + 2 * e] = vv[e] & 0xffffu;
                h[i * 8 + 2 * e + 1] = vv[e] >> 16;
            }
            if (S.keep)
                reinterpret_cast<uint4*>(S.keep + (size_t)k * cols + (size_t)b * 32)[i] = v;
        }
        return;
    }
    const float* src = S.src + (size_t)k * S.ld + (size_t)b * 32;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        float v = src[c];
        if (S.mode == GLUE_RHO_SILU) v = silu_mul(v, src[S.up_off + c]);
        h[c] = __builtin_bit_cast(uint16_t, (_Float16)(v * r));
    }
    if (S.keep) {
        uint4* kp = reinterpret_cast<uint4*>(S.keep + (size_t)k * cols + (size_t)b * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = h[i * 8 + 2 * e] | ((uint32_t)h[i * 8 + 2 * e + 1] << 16);
            kp[i] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

// VALU layout: xp[k][b*16 + g*4 + t] = half2 pair t of 8-column group g of block b
// (Q4: (x[8g+t], x[8g+4+t]); MXFP4: (x[8g+2t], x[8g+2t+1])) and bsum[k][b] = sum x.
template <int FMT>
__global__ __launch_bounds__(256) void k_prep_valu(XSrc S, int K, int cols, uint32_t* __restrict__ xp,
                                                   float* __restrict__ bsum) {
    __shared__ float rs[VQ_MAX_K];
    const int nb = cols >> 5;
    glue_scales(S, K, S.mode == GLUE_NONE ? 1 : cols, rs);
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= K * nb) return;
    const int k = idx / nb, b = idx % nb;
    uint16_t h[32];
    load_block_x(S, cols, k, b, S.mode == GLUE_NONE ? 1.f : rs[k], h);
    uint32_t out[16];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint32_t lo, hi;
            if (FMT == VQ_FMT_MXFP4) {
                lo = h[8 * g + 2 * t];
                hi = h[8 * g + 2 * t + 1];
            } else {
                lo = h[8 * g + t];
                hi = h[8 * g + 4 + t];
            }
            out[g * 4 + t] = lo | (hi << 16);
        }
    uint4* dst = reinterpret_cast<uint4*>(xp + (size_t)k * (cols >> 1) + (size_t)b * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
    if (bsum) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 32; ++c) s += (float)__builtin_bit_cast(_Float16, h[c]);
        bsum[(size_t)k * nb + b] = s;
    }
}

// MFMA layout: afrag[b][16 g + i] = the 8 activations of column i (0 when i >= K) at
// block b, columns 8g..8g+7 in the widened order; mfrag[grp][16 g + i] holds, for g = 0
// and 1, the fp16 hi and lo parts of the block sums of column i over blocks 8 grp..+7
// (zero for g = 2, 3, for i >= K and for blocks past the row end).
template <int FMT>
__global__ __launch_bounds__(256) void k_prep_mfma(XSrc S, int K, int cols, uint4* __restrict__ afrag,
                                                   uint16_t* __restrict__ mfrag) {
    __shared__ float rs[VQ_MAX_K];
    const int nb = cols >> 5;
    const int ngroups = (nb + 7) >> 3;
    glue_scales(S, K, S.mode == GLUE_NONE ? 1 : cols, rs);
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= 16 * ngroups * 8) return;
    const int i = idx & 15, b = idx >> 4;
    uint16_t h[32];
    const bool live = i < K && b < nb;
    if (live) {
        load_block_x(S, cols, i, b, S.mode == GLUE_NONE ? 1.f : rs[i], h);
    } else {
#pragma unroll
        for (int c = 0; c < 32; ++c) h[c] = 0;
    }
    if (b < nb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint32_t w[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                uint32_t lo, hi;
                if (FMT == VQ_FMT_MXFP4) {
                    lo = h[8 * g + 2 * s];
                    hi = h[8 * g + 2 * s + 1];
                } else {
                    // widened order: slot 2s holds column s, slot 2s+1 column s+4
                    lo = h[8 * g + s];
                    hi = h[8 * g + s + 4];
                }
                w[s] = lo | (hi << 16);
            }
            afrag[(size_t)b * 64 + 16 * g + i] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
    if (mfrag) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 32; ++c) s += (float)__builtin_bit_cast(_Float16, h[c]);
        const _Float16 hi = (_Float16)s;
        const _Float16 lo = (_Float16)(s - (float)hi);
        uint16_t* base = mfrag + ((size_t)(b >> 3) * 64) * 8 + (b & 7);
        base[(size_t)(0 * 16 + i) * 8] = __builtin_bit_cast(uint16_t, hi);
        base[(size_t)(1 * 16 + i) * 8] = __builtin_bit_cast(uint16_t, lo);
        base[(size_t)(2 * 16 + i) * 8] = 0;
        base[(size_t)(3 * 16 + i) * 8] = 0;
    }
}

// ------------------------------------------------------------------ finalize

__global__ __launch_bounds__(256) void k_finalize(const float* __restrict__ part, int C, int K,
                                                  int rows, void* __restrict__ y, int y_dtype) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)K * rows) return;
    const int k = (int)(idx / rows);
    const int r = (int)(idx % rows);
    float s = 0.f;
    for (int c = 0; c < C; ++c) s += part[((size_t)c * K + k) * rows + r];
    if (y_dtype == VQ_DTYPE_F16)
        reinterpret_cast<uint16_t*>(y)[idx] = __builtin_bit_cast(uint16_t, (_Float16)s);
    else
        reinterpret_cast<float*>(y)[idx] = s;
}

__device__ float block_sum_256(float v, float* sh) {
    sh[threadIdx.x] = v;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (threadIdx.x < (unsigned)s) sh[threadIdx.x] += sh[threadIdx.x + s];
        __syncthreads();
    }
    const float r = sh[0];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(256) void k_finalize_stats(const float* __restrict__ part, int C, int K,
                                                        int rows, float* __restrict__ y, int nstat,
                                                        int silu, float* __restrict__ stats) {
    __shared__ float sh[256];
    const int half = silu ? rows / 2 : rows;
    const int r = blockIdx.x * 256 + threadIdx.x;
    for (int k = 0; k < K; ++k) {
        float sq = 0.f;
        if (r < half) {
            float s = 0.f;
            for (int c = 0; c < C; ++c) s += part[((size_t)c * K + k) * rows + r];
            y[(size_t)k * rows + r] = s;
            if (silu) {
                float u = 0.f;
                for (int c = 0; c < C; ++c) u += part[((size_t)c * K + k) * rows + half + r];
                y[(size_t)k * rows + half + r] = u;
                const float v = silu_mul(s, u);
                sq = v * v;
            } else if (r < nstat) {
                sq = s * s;
            }
        }
        const float t = block_sum_256(sq, sh);
        if (threadIdx.x == 0) stats[(size_t)blockIdx.x * K + k] = t;
    }
}

template <typename F>
hipError_t launch_checked(F f) {
    f();
    return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------------ host side

size_t lin_scratch_bytes(int fmt, int rows, int cols, int K, bool mfma) {
    const LinGeom g = lin_geom(rows, cols);
    size_t n = 0;
    if (mfma) {
        n += align_up((size_t)g.nb * 64 * 16, 256);
        if (fmt == VQ_FMT_Q4_MIN) n += align_up((size_t)g.ngroups * 64 * 16, 256);
    } else {
        n += align_up((size_t)K * cols * 2, 256);
        if (fmt == VQ_FMT_Q4_MIN) n += align_up((size_t)K * g.nb * 4, 256);
    }
    n += align_up((size_t)g.nchunks * K * rows * 4, 256);
    return n;
}

void lin_scratch_carve(void* base, int fmt, int rows, int cols, int K, bool mfma, LinScratch* s) {
    const LinGeom g = lin_geom(rows, cols);
    char* p = (char*)base;
    s->xlay = p;
    p += mfma ? align_up((size_t)g.nb * 64 * 16, 256) : align_up((size_t)K * cols * 2, 256);
    s->aux = nullptr;
    if (fmt == VQ_FMT_Q4_MIN) {
        s->aux = p;
        p += mfma ? align_up((size_t)g.ngroups * 64 * 16, 256) : align_up((size_t)K * g.nb * 4, 256);
    }
    s->part = (float*)p;
}

static hipError_t launch_prep(const Mat& W, const XSrc& S, int K, bool mfma, const LinScratch& s,
                              hipStream_t st) {
    const LinGeom g = lin_geom(W.rows, W.cols);
    if (mfma) {
        const int n = 16 * g.ngroups * 8;
        dim3 grid((n + 255) / 256);
        switch (W.fmt) {
            case VQ_FMT_Q4:
                k_prep_mfma<VQ_FMT_Q4><<<grid, 256, 0, st>>>(S, K, W.cols, (uint4*)s.xlay, nullptr);
                break;
            case VQ_FMT_Q4_MIN:
                k_prep_mfma<VQ_FMT_Q4_MIN><<<grid, 256, 0, st>>>(S, K, W.cols, (uint4*)s.xlay,
                                                                 (uint16_t*)s.aux);
                break;
            default:
                k_prep_mfma<VQ_FMT_MXFP4><<<grid, 256, 0, st>>>(S, K, W.cols, (uint4*)s.xlay, nullptr);
        }
    } else {
        const int n = K * g.nb;
        dim3 grid((n + 255) / 256);
        switch (W.fmt) {
            case VQ_FMT_Q4:
                k_prep_valu<VQ_FMT_Q4><<<grid, 256, 0, st>>>(S, K, W.cols, (uint32_t*)s.xlay, nullptr);
                break;
            case VQ_FMT_Q4_MIN:
                k_prep_valu<VQ_FMT_Q4_MIN><<<grid, 256, 0, st>>>(S, K, W.cols, (uint32_t*)s.xlay,
                                                                 (float*)s.aux);
                break;
            default:
                k_prep_valu<VQ_FMT_MXFP4><<<grid, 256, 0, st>>>(S, K, W.cols, (uint32_t*)s.xlay, nullptr);
        }
    }
    return hipGetLastError();
}

hipError_t launch_prep_plain(const Mat& W, const uint16_t* x, int K, bool mfma, const LinScratch& s,
                             uint16_t* x_keep, hipStream_t st) {
    XSrc S{x, nullptr, 0, 0, GLUE_NONE, nullptr, 0, x_keep};
    return launch_prep(W, S, K, mfma, s, st);
}

hipError_t launch_prep_glue(const Mat& W, const float* src, int ld, int up_off, int mode,
                            const float* stats, int nstats, int K, bool mfma, uint16_t* x_keep,
                            const LinScratch& s, hipStream_t st) {
    XSrc S{nullptr, src, ld, up_off, mode, stats, nstats, x_keep};
    return launch_prep(W, S, K, mfma, s, st);
}

template <int FMT, int K, bool AL>
static void launch_valu_k(const Mat& W, const LinScratch& s, dim3 grid, hipStream_t st) {
    k_lin_valu<FMT, K, AL><<<grid, 256, 0, st>>>(W, (const uint32_t*)s.xlay, (const float*)s.aux, s.part);
}

template <int FMT, bool AL>
static void launch_valu_f(const Mat& W, int K, const LinScratch& s, dim3 grid, hipStream_t st) {
    switch (K) {
        case 1: launch_valu_k<FMT, 1, AL>(W, s, grid, st); break;
        case 2: launch_valu_k<FMT, 2, AL>(W, s, grid, st); break;
        case 3: launch_valu_k<FMT, 3, AL>(W, s, grid, st); break;
        case 4: launch_valu_k<FMT, 4, AL>(W, s, grid, st); break;
        case 5: launch_valu_k<FMT, 5, AL>(W, s, grid, st); break;
        case 6: launch_valu_k<FMT, 6, AL>(W, s, grid, st); break;
        case 7: launch_valu_k<FMT, 7, AL>(W, s, grid, st); break;
        default: launch_valu_k<FMT, 8, AL>(W, s, grid, st); break;
    }
}

template <int FMT, bool AL>
static void launch_mfma_f(const Mat& W, int K, const LinScratch& s, dim3 grid, hipStream_t st) {
    k_lin_mfma<FMT, AL><<<grid, 256, 0, st>>>(W, (const uint4*)s.xlay, (const uint4*)s.aux, s.part, K);
}

hipError_t launch_linear_main(const Mat& W, int K, bool mfma, const LinScratch& s, hipStream_t st) {
    const LinGeom g = lin_geom(W.rows, W.cols);
    dim3 grid(g.ntiles, g.nchunks);
    const bool al = (g.nb % 8) == 0;
    if (mfma) {
        switch (W.fmt * 2 + (al ? 1 : 0)) {
            case 0: launch_mfma_f<VQ_FMT_Q4, false>(W, K, s, grid, st); break;
            case 1: launch_mfma_f<VQ_FMT_Q4, true>(W, K, s, grid, st); break;
            case 2: launch_mfma_f<VQ_FMT_Q4_MIN, false>(W, K, s, grid, st); break;
            case 3: launch_mfma_f<VQ_FMT_Q4_MIN, true>(W, K, s, grid, st); break;
            case 4: launch_mfma_f<VQ_FMT_MXFP4, false>(W, K, s, grid, st); break;
            default: launch_mfma_f<VQ_FMT_MXFP4, true>(W, K, s, grid, st); break;
        }
    } else {
        switch (W.fmt * 2 + (al ? 1 : 0)) {
            case 0: launch_valu_f<VQ_FMT_Q4, false>(W, K, s, grid, st); break;
            case 1: launch_valu_f<VQ_FMT_Q4, true>(W, K, s, grid, st); break;
            case 2: launch_valu_f<VQ_FMT_Q4_MIN, false>(W, K, s, grid, st); break;
            case 3: launch_valu_f<VQ_FMT_Q4_MIN, true>(W, K, s, grid, st); break;
            case 4: launch_valu_f<VQ_FMT_MXFP4, false>(W, K, s, grid, st); break;
            default: launch_valu_f<VQ_FMT_MXFP4, true>(W, K, s, grid, st); break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_finalize(const Mat& W, int K, const LinScratch& s, void* y, int y_dtype,
                           hipStream_t st) {
    const LinGeom g = lin_geom(W.rows, W.cols);
    const size_t n = (size_t)K * W.rows;
    k_finalize<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(s.part, g.nchunks, K, W.rows, y, y_dtype);
    return hipGetLastError();
}

int finalize_stats_blocks(int rows, int silu) {
    const int half = silu ? rows / 2 : rows;
    return (half + 255) / 256;
}

hipError_t launch_finalize_stats(const Mat& W, int K, const LinScratch& s, float* y, int nstat,
                                 int silu, float* stats, hipStream_t st) {
    const LinGeom g = lin_geom(W.rows, W.cols);
    k_finalize_stats<<<dim3(finalize_stats_blocks(W.rows, silu)), 256, 0, st>>>(
        s.part, g.nchunks, K, W.rows, y, nstat, silu, stats);
    return hipGetLastError();
}

}  // namespace vq
