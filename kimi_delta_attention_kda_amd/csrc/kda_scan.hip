// kda_scan.hip -- ordered exclusive prefix of affine segment maps, gfx950.
//
// KDA Context Parallelism ("Incoming and outgoing states", "Implementation order"):
// per head, W = S_init; for each segment in order the incoming state is W, then
// W <- M_i W + U_i is the outgoing state; the last W is the final state.  The state
// multiplies on the left, so the columns of W are independent: one workgroup owns
// one head and 16 state columns and walks the segments in order, with the current
// M_i staged in LDS and W held in LDS between segments.  fp32 FMA throughout.
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

hipError_t launch_affine_scan(int n_seg, int H, int dk, int dv, const float *M, const float *U,
                              const float *S_init, float *incoming, float *outgoing, float *final_state,
                              hipStream_t stream) {
    const dim3 grid(H * (dv / 16));
    hipLaunchKernelGGL(kda_affine_scan_kernel, grid, dim3(SCAN_NT), 0, stream, n_seg, H, dk, dv, M, U,
                       S_init, incoming, outgoing, final_state);
    return hipGetLastError();
}

}  // namespace kda
