// Device helpers shared by the weight-streaming kernels of libvq (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/vq.h"

namespace vq {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ h8_t as_h8(u4_t v) { return __builtin_bit_cast(h8_t, v); }

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ uint32_t f2h_bits(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);   // round to nearest even
}

// fp16(v * r) with the product rounded to fp32 first.  The explicit product keeps the
// compiler from fusing the multiply and the narrowing into one mixed-precision FMA in
// some kernels and not in others (a single rounding from the exact product can differ
// from the two-step one by an fp16 ulp), so every kernel converts stage inputs alike.
__device__ __forceinline__ uint32_t f2h_scaled(float v, float r) {
    return f2h_bits(__fmul_rn(v, r));
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

// Column held by slot p (0..7) of an 8-column group in the widened order above.
template <int FMT>
__device__ __forceinline__ int slot_col(int p) {
    if constexpr (FMT == VQ_FMT_MXFP4) return p;
    else return (p >> 1) + 4 * (p & 1);
}

// Work item of workgroup `id` in a 1-D grid of n items.  Workgroups are dealt to the
// 8 XCDs round-robin by id; id -> (id % 8) * (n / 8) + id / 8 gives each XCD a run of
// consecutive items, so the chunks of one row tile (which share the lines holding the
// tile's block scales and mins) meet in one L2 and are in flight together.
__device__ __forceinline__ int xcd_item(int id, int n) {
    const int full = n & ~7;
    if (id >= full) return id;
    return (id & 7) * (full >> 3) + (id >> 3);
}

// Sum over the 8 lanes 8s..8s+7 (a fixed butterfly: every lane gets the same result).
__device__ __forceinline__ float sum8(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    return v;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Data one workgroup writes and another reads within the same launch (the persistent
// pass) is stored with device-scope relaxed atomics, which write through to memory past
// the XCD's own L2.  The readers use plain loads: every such buffer is written once per
// pass at an address no workgroup has read since the launch began (the launch starts
// with clean caches), so a load cannot hit a stale line, and after the first miss the
// XCD's other workgroups find the line in their L2.
__device__ __forceinline__ void st_shared_f32(float* p, float v, bool coh) {
    if (coh) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}

// Loads through global (not flat) pointers.  The compiler cannot always prove that a
// weight pointer is global; a flat load would also count against the LDS / scalar-load
// counter, so every LDS wait would wait for the weights in flight as well.
#define GLOBAL_AS __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ T ld_global(const void* p) {
    return *(const GLOBAL_AS T*)p;          // an address-space cast (no instruction)
}
template <typename T>
__device__ __forceinline__ T ld_global_nt(const void* p) {
    return __builtin_nontemporal_load((const GLOBAL_AS T*)p);
}

// Sum over the 64 lanes of a wave, the same in every lane (a fixed order: DPP sums over
// 8 and 16 lanes, then the four 16-lane rows).
__device__ __forceinline__ float wave_sum(float v) {
    v = sum8(v);
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return ((r0 + r1) + r2) + r3;
}

}  // namespace vq
