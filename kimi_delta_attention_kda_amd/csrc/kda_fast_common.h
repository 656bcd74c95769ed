// kda_fast_common.h -- device helpers of the bf16 chunk kernel (kda_fast.hip).
#pragma once

#include "kda_common.h"

namespace kda {
namespace fk {

typedef _Float16 f16_t;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16h(f16x4 a, f16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma32h(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 cath(f16x4 a, f16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Key channel held in row rho of the state's 16-row tile ct.  Tiles 2kb and 2kb+1 hold
// channels 32kb + 8(rho/4) + {0..3} and {4..7}: the k slots s of lane group g in the
// products with the state are then channels 32kb + 8g + s.
__device__ __forceinline__ int key_row(int ct, int rho) {
    return 32 * (ct >> 1) + 8 * (rho >> 2) + 4 * (ct & 1) + (rho & 3);
}
// Inverse: the tile row (16 ct + rho) of key channel c.  Khat^T is stored in this row
// order so that the state update reads 16 consecutive rows per fragment.
__device__ __forceinline__ int tile_row(int c) {
    return 16 * (2 * (c >> 5) + ((c >> 2) & 1)) + 4 * ((c >> 3) & 3) + (c & 3);
}

// fp16 A-operand fragment whose k slots follow the accumulator row order of two 16-row
// tiles: slot s<4 -> column k0+4g+s, slot s>=4 -> column k0+16+4g+(s-4).
__device__ __forceinline__ f16x8 fragA_perm_h(const f16_t *base, int pitch, int row, int k0, int g) {
    const f16_t *p = base + row * pitch + k0 + 4 * g;
    return cath(*(const f16x4 *)p, *(const f16x4 *)(p + 16));
}

// x = hi + lo to about 22 significant bits: hi = fp16(x) and lo = fp16(x - hi), both
// rounded to nearest even.  hi is formed two at a time by the packed conversion; lo by
// the mixed-precision FMA, which reads hi from its fp16 half and computes x - hi (exact
// in fp32) before rounding it to fp16 -- one instruction per element instead of a
// widening, a subtraction and a narrowing.
__device__ __forceinline__ uint32_t pk_h2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, h2));
}
// The -1 is passed in a register (an inline constant in this encoding is not read as an
// fp32 -1).  The compiler does not count the wait states an MFMA needs after a VALU
// instruction it sees only as inline asm writes one of its operands, so the second
// instruction ends with its own wait.
__device__ __forceinline__ uint32_t lo_h2(uint32_t hp, float a, float b) {
    uint32_t r;
    const float m1 = -1.f;
    asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(hp), "v"(m1), "v"(a));
    asm("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\ts_nop 4"
        : "+v"(r) : "v"(hp), "v"(m1), "v"(b));
    return r;
}
__device__ __forceinline__ void split_h(f32x4 x, f16x4 &hi, f16x4 &lo) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const uint32_t h0 = pk_h2(x[0], x[1]), h1 = pk_h2(x[2], x[3]);
    hi = __builtin_bit_cast(f16x4, u2{h0, h1});
    lo = __builtin_bit_cast(f16x4, u2{lo_h2(h0, x[0], x[1]), lo_h2(h1, x[2], x[3])});
}

// alpha = exp(-A softplus(x)) = (1 + e^x)^(-A), computed as 2^(-A log2(1 + 2^(x log2 e)));
// the safe gate's floor on log alpha is a floor exp(bound) on alpha.  Branch-free: the
// three transcendentals are the hardware base-2 exp/log.
__device__ __forceinline__ float gate_alpha(float raw, float dtb_l2e, float negA, float amin) {
    // dtb_l2e = dt_bias * log2(e): one FMA forms (raw + dt_bias) log2(e)
    const float t = __builtin_amdgcn_exp2f(fmaf(raw, 1.44269504088896341f, dtb_l2e));
    const float a = __builtin_amdgcn_exp2f(negA * __builtin_amdgcn_logf(1.f + t));
    return fmaxf(a, amin);
}

// compile-time integer (template arguments of lambdas)
template <int N>
struct IC {
    static constexpr int value = N;
};

// value held by lane q of this lane's quad (DPP quad permutation [q, q, q, q])
template <int Q>
__device__ __forceinline__ float quad_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), Q * 0x55, 0xF, 0xF, false));
}

// Maximum of a non-negative float over the wave, in a scalar register: lane exchanges
// inside each row of 16 lanes (DPP, no LDS round trip), then the four row maxima read
// into scalar registers, where non-negative floats order like their bit patterns.
__device__ __forceinline__ float wave_max_nonneg(float x) {
    auto dpp_max = [](float v, auto ctrl) {
        const int m = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), decltype(ctrl)::value, 0xF, 0xF, false);
        return fmaxf(v, __builtin_bit_cast(float, m));
    };
    x = dpp_max(x, IC<0xB1>{});   // quad_perm [1,0,3,2]
    x = dpp_max(x, IC<0x4E>{});   // quad_perm [2,3,0,1]
    x = dpp_max(x, IC<0x141>{});  // row_half_mirror
    x = dpp_max(x, IC<0x140>{});  // row_mirror
    const unsigned b = __builtin_bit_cast(unsigned, x);
    const unsigned m = max(max(__builtin_amdgcn_readlane(b, 0), __builtin_amdgcn_readlane(b, 16)),
                           max(__builtin_amdgcn_readlane(b, 32), __builtin_amdgcn_readlane(b, 48)));
    return __builtin_bit_cast(float, m);
}

// Step K of the quad-parallel unit-lower substitution (and the following steps): broadcast
// acc_K from quad lane K/4, fold x_K = -acc_K into this lane's four rows.
template <int K>
__device__ __forceinline__ void inv_step(float (&acc)[4], const float *At, int q) {
    const f32x4 ak = *(const f32x4 *)(At + K * 20 + 4 * q);
    const float yk = quad_bcast<(K >> 2)>(acc[K & 3]);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = fmaf(-ak[j], yk, acc[j]);
    if constexpr (K < 15) inv_step<K + 1>(acc, At, q);
}

}  // namespace fk
}  // namespace kda
