// The CDNA4 scaled matrix path for MXFP4 weights: y ~= W x with the activations first
// converted to the 8-bit MX format E4M3 (one E8M0 scale per 32 values, as the OCP
// Microscaling Formats v1.0 specification converts a block), then one
// v_mfma_scale_f32_16x16x128_f8f6f4 per 128 columns of a 16-row tile, the E2M1 weight
// codes and both sets of block scales going into the instruction as they are.  The
// activation conversion makes this an approximation of W x; it is offered beside the exact
// fp16 path for the K = 16 window of MXFP4 weights (the dense case named for evaluating
// CDNA4's MXFP4 instructions), not in its place.
//
// Operand order of the instruction (16 x 16 x 128, A = activations E4M3, B = weights E2M1),
// established on this GPU with single-element probes:
//   * lane l = i + 16 q: A row i, B column i; the output lane holds rows 4 q .. 4 q + 3 of
//     column i (row = activation column, column = weight row);
//   * B (4 registers, 32 codes): the 32 values k = 32 q .. 32 q + 31, low nibble first;
//   * A (8 registers, 32 bytes): bytes 0..15 are k = 16 q .. 16 q + 15, bytes 16..31 are
//     k = 64 + 16 q .. 64 + 16 q + 15;
//   * the scale byte of lane i + 16 q (A and B alike) multiplies the 32 values of block q,
//     k = 32 q .. 32 q + 31, of row / column i.
#include <hip/hip_runtime.h>

#include "vq_internal.h"

namespace vq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

constexpr int MX_THREADS = 256;      // 4 waves per workgroup
constexpr int MX_DEPTH = 4;          // chunks of loads in flight per wave

// E4M3 code of v (to nearest, ties to the even mantissa, saturating at 448; the sign bit
// is v's).  v = x * 2^-E is exact in fp32 for the fp16 x and shared exponents E that occur.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const uint32_t sign = (__builtin_bit_cast(uint32_t, v) >> 24) & 0x80u;
    const float a = __builtin_fabsf(v);
    uint32_t code;
    if (a >= 448.0f) {
        code = 0x7Eu;
    } else if (a < 0.015625f) {                       // below 2^-6: steps of 2^-9
        code = (uint32_t)__builtin_rintf(a * 512.0f);   // 0 .. 8 (8 is the smallest normal)
    } else {
        const int e = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xFFu) - 127;   // -6 .. 8
        const float f = __builtin_ldexpf(a, -e);        // [1, 2), exact
        uint32_t m = (uint32_t)__builtin_rintf((f - 1.0f) * 8.0f);
        int ee = e;
        if (m == 8u) {
            m = 0u;
            ++ee;
        }
        code = ((uint32_t)(ee + 7) << 3) | m;
    }
    return code | sign;
}

// One thread per block of 32 activations of one column: the shared E8M0 scale and the 32
// E4M3 codes.  Columns K .. 15 are zero (codes 0, scale byte 0).
__global__ void k_mx_quant(const uint16_t* x, int K, int cols, uint8_t* xq, uint8_t* xs) {
    const int nb = cols / 32;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= 16 * nb) return;
    const int m = i / nb, b = i - m * nb;
    uint8_t* q = xq + (size_t)m * cols + 32 * b;
    if (m >= K) {
        for (int j = 0; j < 32; j += 16) *(u4v*)(q + j) = u4v{0u, 0u, 0u, 0u};
        xs[i] = 0;
        return;
    }
    const uint16_t* src = x + (size_t)m * cols + 32 * b;
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        v[j] = (float)__builtin_bit_cast(_Float16, src[j]);
        amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j]));
    }
    int E = -127;
    if (amax > 0.0f) E = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFFu) - 127 - 8;
    xs[i] = (uint8_t)(E + 127);
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t d = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) d |= e4m3_code(__builtin_ldexpf(v[4 * j + t], -E)) << (8 * t);
        w[j] = d;
    }
    *(u4v*)q = u4v{w[0], w[1], w[2], w[3]};
    *(u4v*)(q + 16) = u4v{w[4], w[5], w[6], w[7]};
}

struct MxArgs {
    const uint8_t* qs;      // E2M1 codes [rows][cols / 2]
    const uint8_t* sc;      // E8M0 [rows][cols / 32]
    const uint8_t* xq;      // E4M3 [16][cols]
    const uint8_t* xs;      // E8M0 [16][cols / 32]
    float* out;             // S == 1: y [K][rows]; else parts [S][K][rows]
    int rows, cols, K;
    int T, C;               // tiles of 16 rows, chunks of 128 columns
    int S, cps;             // splits of a tile's chunks, chunks per split
};

// Work item i = (tile t, split s): chunks [s cps, min((s + 1) cps, C)) of tile t, one wave.
// The wave's items are i = wave, wave + waves, ...; loads run MX_DEPTH chunks ahead.
__global__ void __launch_bounds__(MX_THREADS) k_mx_lin(MxArgs A) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, q = lane >> 4;
    const int waves = gridDim.x * (MX_THREADS / 64);
    const int gw = blockIdx.x * (MX_THREADS / 64) + (threadIdx.x >> 6);
    const size_t rb = (size_t)A.cols / 2;           // bytes per weight row
    const int nbr = A.cols / 32;                     // scale bytes per row
    for (int it = gw; it < A.T * A.S; it += waves) {
        const int t = it / A.S, s = it - t * A.S;
        const int c0 = s * A.cps, c1 = min(c0 + A.cps, A.C);
        const int row = min(16 * t + n, A.rows - 1);    // rows past the matrix re-read its last
        const uint8_t* wrow = A.qs + (size_t)row * rb + 16 * q;
        const uint8_t* srow = A.sc + (size_t)row * nbr + q;
        const uint8_t* xrow = A.xq + (size_t)n * A.cols + 16 * q;
        const uint8_t* xsrow = A.xs + (size_t)n * nbr + q;
        u4v rb4[MX_DEPTH], ra0[MX_DEPTH], ra1[MX_DEPTH];
        int rsb[MX_DEPTH], rsa[MX_DEPTH];
        auto issue = [&](int u, int c) __attribute__((always_inline)) {
            c = min(c, c1 - 1);                          // past the end: re-read the last chunk
            rb4[u] = *(const u4v*)(wrow + 64 * (size_t)c);
            rsb[u] = srow[4 * c];
            ra0[u] = *(const u4v*)(xrow + 128 * (size_t)c);
            ra1[u] = *(const u4v*)(xrow + 128 * (size_t)c + 64);
            rsa[u] = xsrow[4 * c];
        };
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < MX_DEPTH; ++u) issue(u, c0 + u);
        for (int c = c0; c < c1; c += MX_DEPTH) {
#pragma unroll
            for (int u = 0; u < MX_DEPTH; ++u) {
                if (c + u < c1) {
                    const v8i a = {(int)ra0[u][0], (int)ra0[u][1], (int)ra0[u][2], (int)ra0[u][3],
                                   (int)ra1[u][0], (int)ra1[u][1], (int)ra1[u][2], (int)ra1[u][3]};
                    const v8i b = {(int)rb4[u][0], (int)rb4[u][1], (int)rb4[u][2], (int)rb4[u][3], 0, 0, 0, 0};
                    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 4, 0, rsa[u], 0, rsb[u]);
                }
                issue(u, c + u + MX_DEPTH);
            }
        }
        const int r = 16 * t + n;
        if (r < A.rows) {
            float* o = A.out + (A.S > 1 ? (size_t)s * A.K * A.rows : 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * q + i;
                if (m < A.K) o[(size_t)m * A.rows + r] = acc[i];
            }
        }
    }
}

// y[m][r] = sum over splits s, in order, of parts[s][m][r].
__global__ void k_mx_reduce(const float* parts, float* y, int n, int S) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float v = parts[i];
    for (int s = 1; s < S; ++s) v += parts[(size_t)s * n + i];
    y[i] = v;
}

}  // namespace

void mx_plan(int rows, int cols, int nwg, int* T, int* C, int* S, int* cps) {
    *T = (rows + 15) / 16;
    *C = cols / 128;
    const int waves = nwg * (MX_THREADS / 64);
    int s = (4 * waves + *T - 1) / *T;
    s = std::max(1, std::min(s, *C));
    *cps = (*C + s - 1) / s;
    *S = (*C + *cps - 1) / *cps;
}

hipError_t launch_mx_linear(const vq_matrix& W, const void* x, int K, float* y, uint8_t* ws, int nwg, hipStream_t st) {
    int T, C, S, cps;
    mx_plan(W.rows, W.cols, nwg, &T, &C, &S, &cps);
    uint8_t* xq = ws;
    uint8_t* xs = ws + align_up((size_t)16 * W.cols, 256);
    float* parts = (float*)(xs + align_up((size_t)16 * (W.cols / 32), 256));
    const int nq = 16 * (W.cols / 32);
    k_mx_quant<<<dim3((nq + 255) / 256), 256, 0, st>>>((const uint16_t*)x, K, W.cols, xq, xs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    MxArgs A;
    A.qs = (const uint8_t*)W.qs;
    A.sc = (const uint8_t*)W.scales;
    A.xq = xq;
    A.xs = xs;
    A.out = S > 1 ? parts : y;
    A.rows = W.rows;
    A.cols = W.cols;
    A.K = K;
    A.T = T;
    A.C = C;
    A.S = S;
    A.cps = cps;
    k_mx_lin<<<dim3(nwg), MX_THREADS, 0, st>>>(A);
    e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    const int n = K * W.rows;
    k_mx_reduce<<<dim3((n + 255) / 256), 256, 0, st>>>(parts, y, n, S);
    return hipGetLastError();
}

size_t mx_workspace_bytes(int rows, int cols, int K, int nwg) {
    int T, C, S, cps;
    mx_plan(rows, cols, nwg, &T, &C, &S, &cps);
    return align_up((size_t)16 * cols, 256) + align_up((size_t)16 * (cols / 32), 256) +
           (S > 1 ? align_up((size_t)S * K * rows * 4, 256) : 0);
}

}  // namespace vq
