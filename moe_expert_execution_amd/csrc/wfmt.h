// Weight-chunk decoding shared by the expert kernels (device code).
//
// A chunk is 16 bytes of one weight row (K contiguous): 8 bf16 values, 16
// e4m3fn codes (scale: one fp32 per 128x128 block) or 32 e2m1 codes (scale:
// one e8m0 per 32 along K).  Block-FP8 and MXFP4 banks are the quantised
// formats the pages list for slot records ("The Expert Cache That Follows the
// Router", section "One logical expert, two physical levels of memory").
#pragma once
#include "common.h"

namespace ftmoe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // a 16-byte chunk held in registers

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// exact bf16 of a float whose value needs at most 8 significant bits
__device__ __forceinline__ uint32_t pack_bf16_trunc(float lo, float hi) {
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    return e == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

template <int FMT>
struct WF;

template <>
struct WF<FT_FMT_BF16> {
    static constexpr int EPC = 8;                                   // elements per 16-byte chunk
    __device__ static int64_t row_bytes(int K) { return 2ll * K; }
    // 8 weights -> 4 packed bf16 pairs (already bf16)
    __device__ static void to_bf16(const uint4 c, float, uint32_t* out) {
        out[0] = c.x; out[1] = c.y; out[2] = c.z; out[3] = c.w;
    }
};

template <>
struct WF<FT_FMT_FP8_B128> {
    static constexpr int EPC = 16;
    __device__ static int64_t row_bytes(int K) { return (int64_t)K; }
    __device__ static void to_f32(const uint4 c, float* v) { to_f32(u32x4_t{c.x, c.y, c.z, c.w}, v); }
    __device__ static void to_f32(const u32x4_t c, float* v) {
        const uint32_t w[4] = {c[0], c[1], c[2], c[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
            f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
            v[4 * i + 0] = lo[0];
            v[4 * i + 1] = lo[1];
            v[4 * i + 2] = hi[0];
            v[4 * i + 3] = hi[1];
        }
    }
};

template <>
struct WF<FT_FMT_MXFP4_B32> {
    static constexpr int EPC = 32;
    __device__ static int64_t row_bytes(int K) { return (int64_t)K / 2; }
    // 32 codes, low nibble first, times `scale` (exact: a power of two)
    __device__ static void to_f32(const uint4 c, float scale, float* v) {
        to_f32(u32x4_t{c.x, c.y, c.z, c.w}, scale, v);
    }
    __device__ static void to_f32(const u32x4_t c, float scale, float* v) {
        const uint32_t w[4] = {c[0], c[1], c[2], c[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], scale, 0);
            const f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], scale, 1);
            const f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], scale, 2);
            const f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], scale, 3);
            v[8 * i + 0] = p0[0];
            v[8 * i + 1] = p0[1];
            v[8 * i + 2] = p1[0];
            v[8 * i + 3] = p1[1];
            v[8 * i + 4] = p2[0];
            v[8 * i + 5] = p2[1];
            v[8 * i + 6] = p3[0];
            v[8 * i + 7] = p3[1];
        }
    }
};

}  // namespace ftmoe
