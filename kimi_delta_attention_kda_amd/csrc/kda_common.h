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

__device__ __forceinline__ bf16x4 bf4(f32x4 x) {
    bf16x4 r;
    r[0] = (bf16_t)x[0];
    r[1] = (bf16_t)x[1];
    r[2] = (bf16_t)x[2];
    r[3] = (bf16_t)x[3];
    return r;
}

__device__ __forceinline__ f32x4 f4(bf16x4 x) {
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}

// hi = RNE(x), lo = RNE(x - hi): x ~= hi + lo to about 16 significant bits.
__device__ __forceinline__ void split4(f32x4 x, bf16x4 &hi, bf16x4 &lo) {
    hi = bf4(x);
    lo = bf4(x - f4(hi));
}

__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        bf16_t h = (bf16_t)x[s];
        hi[s] = h;
        lo[s] = (bf16_t)(x[s] - (float)h);
    }
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ float softplus_f(float x) {
    // max(x,0) + log1p(exp(-|x|)) in fp32
    return fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x)));
}

}  // namespace kda
