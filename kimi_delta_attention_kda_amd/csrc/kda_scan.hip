// kda_scan.hip -- ordered exclusive prefix of affine segment maps, gfx950.
//
// KDA Context Parallelism ("Incoming and outgoing states", "Implementation order"):
// per head, W = S_init; for each segment in order the incoming state is W, then
// W <- M_i W + U_i is the outgoing state; the last W is the final state.  The state
// multiplies on the left, so the columns of W are independent: one workgroup owns
// one head and 16 state columns and walks the segments in order.  Products and sums
// are fp32 throughout.
//  - dk in {64, 128}: fp32 16x16x4 MFMAs.  Each lane holds its rows of M_i in registers
//    (the next segment's M and U are loaded while the current step computes), W sits in
//    LDS, and the column blocks of one head run on one XCD so M_i comes from HBM once.
//  - dk in {16, 32}: fp32 FMA with M_i staged in LDS.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

constexpr int SCAN_NT = 256;
constexpr int SCAN_DKMAX = 128;

__global__ __launch_bounds__(SCAN_NT) void kda_affine_scan_kernel(int n_seg, int H, int dk, int dv,
                                                                  const float *__restrict__ M,
                                                                  const float *__restrict__ U,
                                                                  const float *__restrict__ S_init,
                                                                  float *incoming, float *outgoing,
                                                                  float *final_state) {
    __shared__ float sM[SCAN_DKMAX * (SCAN_DKMAX + 1)];
    __shared__ float sW[SCAN_DKMAX * 16];
    const int n_cb = dv / 16;
    const int h = blockIdx.x / n_cb, cb = blockIdx.x - h * n_cb;
    const int t = threadIdx.x;
    const int pm = dk + 1;
    const int tpr = SCAN_NT / dk;        // threads per state row
    const int cpt = 16 / tpr;            // columns per thread
    const int r = t / tpr, cl = (t - r * tpr) * cpt;
    const bool active = r < dk;

    for (int e = t; e < dk * 16; e += SCAN_NT) {
        const int i = e >> 4, j = e & 15;
        sW[e] = S_init[((int64_t)h * dk + i) * dv + 16 * cb + j];
    }
    __syncthreads();
    for (int s = 0; s < n_seg; ++s) {
        const int64_t mb = ((int64_t)s * H + h) * dk * dk;
        const int64_t ub = ((int64_t)s * H + h) * dk * dv;
        for (int e = t; e < dk * dk; e += SCAN_NT) sM[(e / dk) * pm + (e % dk)] = M[mb + e];
        for (int e = t; e < dk * 16; e += SCAN_NT) {
            const int i = e >> 4, j = e & 15;
            incoming[ub + (int64_t)i * dv + 16 * cb + j] = sW[e];
        }
        __syncthreads();
        float acc[16];
        if (active) {
#pragma unroll 16
            for (int q = 0; q < 16; ++q)
                if (q < cpt) acc[q] = U[ub + (int64_t)r * dv + 16 * cb + cl + q];
            for (int c = 0; c < dk; ++c) {
                const float m = sM[r * pm + c];
#pragma unroll 16
                for (int q = 0; q < 16; ++q)
                    if (q < cpt) acc[q] = fmaf(m, sW[c * 16 + cl + q], acc[q]);
            }
        }
        __syncthreads();
        if (active) {
#pragma unroll 16
            for (int q = 0; q < 16; ++q)
                if (q < cpt) {
                    sW[r * 16 + cl + q] = acc[q];
                    outgoing[ub + (int64_t)r * dv + 16 * cb + cl + q] = acc[q];
                }
        }
        __syncthreads();
    }
    for (int e = t; e < dk * 16; e += SCAN_NT) {
        const int i = e >> 4, j = e & 15;
        final_state[((int64_t)h * dk + i) * dv + 16 * cb + j] = sW[e];
    }
}

// MFMA walk for dk in {64, 128}.  Wave w owns rows RW w .. RW w + RW - 1 (RW = dk/4, TT =
// dk/64 tiles of 16 rows); lane (g, li) holds rows RW w + 16tt + 4g + s of column li, the
// accumulator layout.  MFMA step (q, e) on lane quarter g contracts index KQ g + 4q + e
// (KQ = dk/4): A is one entry of the lane's row of M_i, B one entry of a column of W from
// LDS, skewed by 16 floats per quarter so the four quarters read distinct banks.
__device__ __forceinline__ f32x4 mfma_f32x4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
template <int DK>
__device__ __forceinline__ int wx_at(int k, int c) { return 16 * k + c + 16 * (k / (DK / 4)); }

template <int DK>
__global__ __launch_bounds__(SCAN_NT) void kda_affine_scan_mfma(int n_seg, int H, int dv,
                                                                const float *__restrict__ M,
                                                                const float *__restrict__ U,
                                                                const float *__restrict__ S_init,
                                                                float *incoming, float *outgoing,
                                                                float *final_state) {
    constexpr int TT = DK / 64, RW = DK / 4, KQ = DK / 4;
    __shared__ float sx[16 * DK + 16 * 4];
    const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 4, li = l & 15;
    const int ncb = dv / 16;
    const int n_lin = (H * ncb + 8 * ncb - 1) / (8 * ncb) * (8 * ncb);
    for (int lin = blockIdx.x; lin < n_lin; lin += gridDim.x) {
        // workgroups are dealt to the 8 XCDs round-robin: lin & 7 picks the XCD
        const int cb = (lin >> 3) % ncb, h = (lin / (8 * ncb)) * 8 + (lin & 7);
        if (h >= H) continue;  // uniform over the workgroup
        const int col = 16 * cb + li;
        auto row = [&](int tt, int s) { return RW * w + 16 * tt + 4 * g + s; };
        f32x4 x[TT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int s = 0; s < 4; ++s) x[tt][s] = S_init[((int64_t)h * DK + row(tt, s)) * dv + col];
        f32x4 ma[TT][KQ / 4], ua[TT];
        auto load = [&](int i) {
            const int64_t kh = (int64_t)i * H + h;
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                const float *Mr = M + (kh * DK + RW * w + 16 * tt + li) * DK + KQ * g;
#pragma unroll
                for (int q = 0; q < KQ / 4; ++q) ma[tt][q] = *(const f32x4 *)(Mr + 4 * q);
#pragma unroll
                for (int s = 0; s < 4; ++s) ua[tt][s] = U[(kh * DK + row(tt, s)) * dv + col];
            }
        };
        load(0);
        for (int i = 0; i < n_seg; ++i) {
            const int64_t kh = (int64_t)i * H + h;
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int s = 0; s < 4; ++s) incoming[(kh * DK + row(tt, s)) * dv + col] = x[tt][s];
            __syncthreads();  // every wave is done reading the previous W from LDS
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int s = 0; s < 4; ++s) sx[wx_at<DK>(row(tt, s), li)] = x[tt][s];
            __syncthreads();
            f32x4 mc[TT][KQ / 4], acc[TT];
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                acc[tt] = ua[tt];
#pragma unroll
                for (int q = 0; q < KQ / 4; ++q) mc[tt][q] = ma[tt][q];
            }
            if (i + 1 < n_seg) load(i + 1);  // in flight during this step
#pragma unroll
            for (int q = 0; q < KQ / 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float bx = sx[wx_at<DK>(KQ * g + 4 * q + e, li)];
#pragma unroll
                    for (int tt = 0; tt < TT; ++tt) acc[tt] = mfma_f32x4(mc[tt][q][e], bx, acc[tt]);
                }
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                x[tt] = acc[tt];
#pragma unroll
                for (int s = 0; s < 4; ++s) outgoing[(kh * DK + row(tt, s)) * dv + col] = x[tt][s];
            }
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int s = 0; s < 4; ++s) final_state[((int64_t)h * DK + row(tt, s)) * dv + col] = x[tt][s];
        __syncthreads();  // the next task's first W store waits for this one's readers
    }
}

hipError_t launch_affine_scan(int n_seg, int H, int dk, int dv, const float *M, const float *U,
                              const float *S_init, float *incoming, float *outgoing, float *final_state,
                              hipStream_t stream) {
    if (dk == 128 || dk == 64) {
        const int ncb = dv / 16;
        const dim3 grid((H * ncb + 8 * ncb - 1) / (8 * ncb) * (8 * ncb));
        if (dk == 128)
            hipLaunchKernelGGL(kda_affine_scan_mfma<128>, grid, dim3(SCAN_NT), 0, stream, n_seg, H, dv, M, U,
                               S_init, incoming, outgoing, final_state);
        else
            hipLaunchKernelGGL(kda_affine_scan_mfma<64>, grid, dim3(SCAN_NT), 0, stream, n_seg, H, dv, M, U,
                               S_init, incoming, outgoing, final_state);
        return hipGetLastError();
    }
    const dim3 grid(H * (dv / 16));
    hipLaunchKernelGGL(kda_affine_scan_kernel, grid, dim3(SCAN_NT), 0, stream, n_seg, H, dk, dv, M, U,
                       S_init, incoming, outgoing, final_state);
    return hipGetLastError();
}

}  // namespace kda
