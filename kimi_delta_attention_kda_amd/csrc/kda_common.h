// kda_common.h -- device-side types and helpers shared by the libkda kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] B[32x16], fp32 accumulate.
// Lane l (g = l/16, li = l%16): A slot s = A[li][8g+s], B slot s = B[8g+s][li],
// D slot s = D[4g+s][li].  Only the pairing of A slot (g,s) with B slot (g,s)
// matters for the contraction, so a consistent relabelling of k is allowed.
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Two fp32 values rounded to bf16 (nearest even) into one packed register, and the
// two halves widened back exactly (a bf16 is the upper half of an fp32).  Written on the
// packed word so that one conversion serves a pair and the widening is a shift or a mask.
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, b2));
}
__device__ __forceinline__ float bf_lo(uint32_t p) { return __builtin_bit_cast(float, p << 16); }
__device__ __forceinline__ float bf_hi(uint32_t p) { return __builtin_bit_cast(float, p & 0xffff0000u); }

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x4 bf4(f32x4 x) {
    return __builtin_bit_cast(bf16x4, u32x2{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3])});
}

__device__ __forceinline__ f32x4 f4(bf16x4 x) {
    const u32x2 p = __builtin_bit_cast(u32x2, x);
    return f32x4{bf_lo(p[0]), bf_hi(p[0]), bf_lo(p[1]), bf_hi(p[1])};
}

// hi = RNE(x), lo = RNE(x - hi): x ~= hi + lo to about 16 significant bits.
__device__ __forceinline__ void split4(f32x4 x, bf16x4 &hi, bf16x4 &lo) {
    const uint32_t h0 = pack_bf2(x[0], x[1]), h1 = pack_bf2(x[2], x[3]);
    hi = __builtin_bit_cast(bf16x4, u32x2{h0, h1});
    lo = __builtin_bit_cast(bf16x4, u32x2{pack_bf2(x[0] - bf_lo(h0), x[1] - bf_hi(h0)),
                                          pack_bf2(x[2] - bf_lo(h1), x[3] - bf_hi(h1))});
}

__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
    u32x4 h, l;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t p = pack_bf2(x[2 * s], x[2 * s + 1]);
        h[s] = p;
        l[s] = pack_bf2(x[2 * s] - bf_lo(p), x[2 * s + 1] - bf_hi(p));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ float softplus_f(float x) {
    // max(x,0) + log1p(exp(-|x|)) in fp32
    return fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x)));
}

}  // namespace kda
