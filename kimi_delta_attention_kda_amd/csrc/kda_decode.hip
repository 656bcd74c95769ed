// kda_decode.hip -- one recurrent step per sequence (single-token decode).
//
// The token recurrence of the nx_nofloat_kda.nx source (kda_step: decay, delta-write,
// read) applied once to each sequence's pool slot:
//     S' = Diag(alpha) S,  pred = S'^T k,  delta = beta (v - pred),
//     S'' = S' + k delta^T,  o = scale S''^T q = scale (S'^T q + (q . k) delta).
// One workgroup per (sequence, head): thread (row group rg, column j) keeps its rows of
// column j of the decayed state in registers between the two passes, so the fp32 state
// is read once and written once -- the step is bound by those 2 dk dv 4 bytes of HBM
// traffic per (sequence, head).
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

namespace dec {

constexpr int NT = 256;

template <typename T>
__device__ __forceinline__ float ld(const T *p) { return (float)*p; }

template <int DK, int DV, typename T>
__global__ __launch_bounds__(NT) void kda_decode_kernel(DecodeArgs a) {
    constexpr int RG = NT / DV;   // row groups
    constexpr int NR = DK / RG;   // rows per thread
    __shared__ float sA[DK], sK[DK], sQ[DK];
    __shared__ float sPred[RG][DV], sQs[RG][DV];
    __shared__ float sDelta[DV];
    __shared__ float sQK;

    const int b = blockIdx.x / a.H, h = blockIdx.x - b * a.H;
    const int t = threadIdx.x, j = t % DV, rg = t / DV;
    const int slot = a.state_indices[b];
    float *S = a.state_pool + ((int64_t)slot * a.H + h) * DK * DV;

    // ---- gate, key and query of the token (log alpha = -e^{a_log} softplus(raw + dt_bias))
    if (t < DK) {
        const float x = a.raw_gate[((int64_t)b * a.H + h) * DK + t] + a.dt_bias[h * DK + t];
        const float sp = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
        float la = -expf(a.a_log[h]) * sp;
        if (a.gate_mode == 1) la = fmaxf(la, a.lb);
        sA[t] = expf(la);
        const int hk = h / (a.H / a.Hk);  // key head of value head h
        sK[t] = ld((const T *)a.k + ((int64_t)b * a.Hk + hk) * DK + t);
        sQ[t] = ld((const T *)a.q + ((int64_t)b * a.Hk + hk) * DK + t);
    }
    __syncthreads();
    if (t < 64) {  // q . k
        float p = 0.f;
        for (int i = t; i < DK; i += 64) p += sQ[i] * sK[i];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) p += __shfl_xor(p, o);
        if (t == 0) sQK = p;
    }

    // ---- decay this thread's rows of column j; partial S'^T k and S'^T q
    float s[NR];
    const int i0 = rg * NR;
    if (a.v_first) {
        const float *c = S + (int64_t)j * DK + i0;
#pragma unroll
        for (int r = 0; r < NR; r += 4) {
            const f32x4 x = *(const f32x4 *)(c + r);
            s[r] = x[0];
            s[r + 1] = x[1];
            s[r + 2] = x[2];
            s[r + 3] = x[3];
        }
    } else {
#pragma unroll
        for (int r = 0; r < NR; ++r) s[r] = S[(int64_t)(i0 + r) * DV + j];
    }
    float pk = 0.f, pq = 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        s[r] *= sA[i0 + r];
        pk = fmaf(sK[i0 + r], s[r], pk);
        pq = fmaf(sQ[i0 + r], s[r], pq);
    }
    sPred[rg][j] = pk;
    sQs[rg][j] = pq;
    __syncthreads();

    // ---- delta and output of column j
    if (rg == 0) {
        float pred = 0.f, qs = 0.f;
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            pred += sPred[g][j];
            qs += sQs[g][j];
        }
        const float bl = a.beta_logits[(int64_t)b * a.H + h];
        const float beta = a.beta_mode == 0 ? 1.f / (1.f + expf(-bl)) : bl;
        const float delta = beta * (ld((const T *)a.v + ((int64_t)b * a.H + h) * DV + j) - pred);
        sDelta[j] = delta;
        ((T *)a.out)[((int64_t)b * a.H + h) * DV + j] = (T)(a.scale * fmaf(sQK, delta, qs));
    }
    __syncthreads();

    // ---- S'' = S' + k delta^T
    const float dj = sDelta[j];
    if (a.v_first) {
        float *c = S + (int64_t)j * DK + i0;
#pragma unroll
        for (int r = 0; r < NR; r += 4)
            *(f32x4 *)(c + r) = f32x4{fmaf(sK[i0 + r], dj, s[r]), fmaf(sK[i0 + r + 1], dj, s[r + 1]),
                                      fmaf(sK[i0 + r + 2], dj, s[r + 2]), fmaf(sK[i0 + r + 3], dj, s[r + 3])};
    } else {
#pragma unroll
        for (int r = 0; r < NR; ++r) S[(int64_t)(i0 + r) * DV + j] = fmaf(sK[i0 + r], dj, s[r]);
    }
}

}  // namespace dec

hipError_t launch_decode(const DecodeArgs &a, int dk, bool bf16, hipStream_t stream) {
    const dim3 grid(a.B * a.H), block(dec::NT);
    if (dk == 128) {
        if (bf16) hipLaunchKernelGGL((dec::kda_decode_kernel<128, 128, bf16_t>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((dec::kda_decode_kernel<128, 128, float>), grid, block, 0, stream, a);
    } else {
        if (bf16) hipLaunchKernelGGL((dec::kda_decode_kernel<64, 64, bf16_t>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((dec::kda_decode_kernel<64, 64, float>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace kda
