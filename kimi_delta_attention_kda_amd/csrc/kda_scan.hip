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
#include <algorithm>

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
// W in LDS column by column: column c of the workgroup's 16 CT at c (DK + 4), so that a
// lane reads the four contraction entries of an MFMA group with one 16-byte read, and the
// 16 lanes of a read phase (16 columns, pitch 132 floats) start in distinct groups of
// four banks; a lane writes its four consecutive state rows with one 16-byte write.
template <int DK>
__device__ __forceinline__ int wx_at(int k, int c) { return c * (DK + 4) + k; }

// What one launch of the walk does.  The composition is associative (KDA Context
// Parallelism, "Theory"), so the ordered prefix may be regrouped into blocks of blk
// segments:
//   WALK_COMPOSE  task b < n_blocks - 1: the composite of block b's maps, walked on the
//                 augmented state [A | B] = [I | 0] with maps X <- M_s X + [0 | U_s],
//                 stored to comp[b] = [A_b | B_b] ([H, dk, dk + dv] per block);
//   WALK_BLOCKS   one task: W = S_init, W <- A_b W + B_b for b = 0 .. n_blocks - 2, each W
//                 stored as the incoming state of block b + 1;
//   WALK_SEGMENTS task b: block b's segments walked from its incoming state (S_init for
//                 block 0), incoming and outgoing stored, the last block's W as final.
// The plain ordered walk is WALK_SEGMENTS with one block of n_seg segments.
enum { WALK_SEGMENTS = 0, WALK_COMPOSE = 1, WALK_BLOCKS = 2 };
struct ScanWalk {
    int mode, n_seg, H, dv, blk, n_task;
    int width;  // state columns walked: dv, or dk + dv for WALK_COMPOSE
    const float *M, *U, *S_init;
    float *incoming, *outgoing, *final_state;
    float *comp;  // block composites (WALK_COMPOSE writes, WALK_BLOCKS reads)
};

// A workgroup walks 16 CT state columns of one (task, head).  CT = 1 when few workgroups
// run (the ordered walk is a chain of dependent steps: more, narrower workgroups shorten
// each step); CT = 4 when the tasks fill the chip many times over, so that a map's rows,
// loaded once per step, serve 64 columns (four times fewer reads of each map from L2).
template <int DK, int MODE, int CT>
__global__ __launch_bounds__(SCAN_NT) void kda_affine_scan_mfma(ScanWalk a) {
    constexpr int TT = DK / 64, RW = DK / 4, KQ = DK / 4;
    __shared__ __attribute__((aligned(16))) float sx[16 * CT * (DK + 4)];
    const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 4, li = l & 15;
    const int H = a.H, dv = a.dv;
    const int ncb = a.width / (16 * CT), n_hh = (H + 7) / 8;
    const int64_t n_lin = 8 * (int64_t)a.n_task * n_hh * ncb;
    for (int64_t lin = blockIdx.x; lin < n_lin; lin += gridDim.x) {
        // workgroups are dealt to the 8 XCDs round-robin: lin & 7 picks the XCD, and every
        // column block of a head runs on the same one, so each map comes from HBM once
        // (a grid stride that is a multiple of 8 keeps each workgroup on its XCD)
        const int64_t r = lin >> 3;
        const int cb = (int)(r % ncb), hh = (int)((r / ncb) % n_hh), task = (int)(r / (ncb * n_hh));
        const int h = 8 * hh + (lin & 7);
        if (h >= H) continue;  // uniform over the workgroup
        const int col = 16 * CT * cb + li;  // column of tile c: col + 16 c
        auto row = [&](int tt, int s) { return RW * w + 16 * tt + 4 * g + s; };
        // Addresses are a wave-uniform base per step (scalar) plus 32-bit lane offsets:
        // step i reads the M rows of its map at mb(i) (row pitch ldm) and U column ucol at
        // ub(i) (row pitch ldu), and writes state rows at sb(i) (row pitch dv).
        const int s0 = MODE == WALK_BLOCKS ? 0 : task * a.blk;
        const int n_steps = MODE == WALK_BLOCKS ? (a.n_seg + a.blk - 1) / a.blk - 1 : min(a.blk, a.n_seg - s0);
        const int ldm = MODE == WALK_BLOCKS ? DK + dv : DK, ldu = MODE == WALK_BLOCKS ? DK + dv : dv;
        const int64_t hs = (int64_t)H * DK;  // one step of a [*, H, DK, ...] stack, in rows
        const float *m0, *u0;
        int64_t m_step, u_step;
        int ucol = col;
        bool has_u = true;
        if constexpr (MODE == WALK_BLOCKS) {
            m0 = a.comp + (int64_t)h * DK * (DK + dv);
            u0 = m0 + DK;
            m_step = u_step = hs * (DK + dv);
        } else {
            m0 = a.M + ((int64_t)s0 * H + h) * DK * DK;
            u0 = a.U + ((int64_t)s0 * H + h) * DK * dv;
            m_step = hs * DK;
            u_step = hs * dv;
            if constexpr (MODE == WALK_COMPOSE) {
                // the workgroup's 16 CT columns are all M or all U columns: 16 CT divides DK
                ucol = max(col - DK, 0);  // in bounds even where no U is read
                has_u = col >= DK;
            }
        }
        const int mo = (RW * w + li) * ldm + KQ * g;      // + 16 tt ldm + 4 q
        const int uo = (RW * w + 4 * g) * ldu + ucol;     // + (16 tt + s) ldu + 16 c
        const int so = (RW * w + 4 * g) * dv + col;       // + (16 tt + s) dv + 16 c
        float *const inc0 = a.incoming + ((int64_t)s0 * H + h) * DK * dv;
        float *const out0 = a.outgoing + ((int64_t)s0 * H + h) * DK * dv;
        const int64_t s_step = hs * dv;
        f32x4 x[TT][CT];
        {
            const float *src = MODE == WALK_SEGMENTS && s0 > 0 ? inc0 : a.S_init + (int64_t)h * DK * dv;
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int c = 0; c < CT; ++c)
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        if constexpr (MODE == WALK_COMPOSE)
                            x[tt][c][s] = row(tt, s) == col + 16 * c ? 1.f : 0.f;
                        else
                            x[tt][c][s] = src[so + (16 * tt + s) * dv + 16 * c];
                    }
        }
        f32x4 ma[TT][KQ / 4], ua[TT][CT];
        auto load = [&](int i) {
            const float *mb = m0 + i * m_step, *ub = u0 + i * u_step;
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
                for (int q = 0; q < KQ / 4; ++q) ma[tt][q] = *(const f32x4 *)(mb + mo + 16 * tt * ldm + 4 * q);
#pragma unroll
                for (int c = 0; c < CT; ++c)
#pragma unroll
                    for (int s = 0; s < 4; ++s) ua[tt][c][s] = has_u ? ub[uo + (16 * tt + s) * ldu + 16 * c] : 0.f;
            }
        };
        load(0);
        for (int i = 0; i < n_steps; ++i) {
            if constexpr (MODE == WALK_SEGMENTS) {
                float *ib = inc0 + i * s_step;
#pragma unroll
                for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                    for (int c = 0; c < CT; ++c)
#pragma unroll
                        for (int s = 0; s < 4; ++s) ib[so + (16 * tt + s) * dv + 16 * c] = x[tt][c][s];
            }
            __syncthreads();  // every wave is done reading the previous W from LDS
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int c = 0; c < CT; ++c) *(f32x4 *)(sx + wx_at<DK>(row(tt, 0), 16 * c + li)) = x[tt][c];
            __syncthreads();
            f32x4 mc[TT][KQ / 4], acc[TT][CT];
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
                for (int c = 0; c < CT; ++c) acc[tt][c] = ua[tt][c];
#pragma unroll
                for (int q = 0; q < KQ / 4; ++q) mc[tt][q] = ma[tt][q];
            }
            if (i + 1 < n_steps) load(i + 1);  // in flight during this step
#pragma unroll
            for (int q = 0; q < KQ / 4; ++q)
#pragma unroll
                for (int c = 0; c < CT; ++c) {
                    const f32x4 bx = *(const f32x4 *)(sx + wx_at<DK>(KQ * g + 4 * q, 16 * c + li));
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int tt = 0; tt < TT; ++tt) acc[tt][c] = mfma_f32x4(mc[tt][q][e], bx[e], acc[tt][c]);
                }
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int c = 0; c < CT; ++c) x[tt][c] = acc[tt][c];
            if constexpr (MODE == WALK_SEGMENTS) {
                float *ob = out0 + i * s_step;
#pragma unroll
                for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                    for (int c = 0; c < CT; ++c)
#pragma unroll
                        for (int s = 0; s < 4; ++s) ob[so + (16 * tt + s) * dv + 16 * c] = x[tt][c][s];
            } else if constexpr (MODE == WALK_BLOCKS) {
                // incoming state of block i + 1
                float *ib = a.incoming + ((int64_t)((i + 1) * a.blk) * H + h) * DK * dv;
#pragma unroll
                for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                    for (int c = 0; c < CT; ++c)
#pragma unroll
                        for (int s = 0; s < 4; ++s) ib[so + (16 * tt + s) * dv + 16 * c] = x[tt][c][s];
            }
        }
        if constexpr (MODE == WALK_COMPOSE) {
            float *cp = a.comp + ((int64_t)task * H + h) * DK * (DK + dv);
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int c = 0; c < CT; ++c)
#pragma unroll
                    for (int s = 0; s < 4; ++s) cp[(int64_t)row(tt, s) * (DK + dv) + col + 16 * c] = x[tt][c][s];
        } else if (MODE == WALK_SEGMENTS && s0 + n_steps == a.n_seg) {
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int c = 0; c < CT; ++c)
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        a.final_state[((int64_t)h * DK + row(tt, s)) * dv + col + 16 * c] = x[tt][c][s];
        }
        __syncthreads();  // the next task's first W store waits for this one's readers
    }
}

template <int DK, int CT>
static hipError_t launch_walk_ct(const ScanWalk &a, hipStream_t stream) {
    // one workgroup per (task, head, 16 CT columns), at most 2^20 at once (the kernel strides)
    const int64_t n_lin = 8 * (int64_t)a.n_task * ((a.H + 7) / 8) * (a.width / (16 * CT));
    const dim3 grid((unsigned)std::min<int64_t>(n_lin, (int64_t)1 << 20));
    if (a.mode == WALK_COMPOSE)
        hipLaunchKernelGGL((kda_affine_scan_mfma<DK, WALK_COMPOSE, CT>), grid, dim3(SCAN_NT), 0, stream, a);
    else if (a.mode == WALK_BLOCKS)
        hipLaunchKernelGGL((kda_affine_scan_mfma<DK, WALK_BLOCKS, CT>), grid, dim3(SCAN_NT), 0, stream, a);
    else
        hipLaunchKernelGGL((kda_affine_scan_mfma<DK, WALK_SEGMENTS, CT>), grid, dim3(SCAN_NT), 0, stream, a);
    return hipGetLastError();
}

// The blocks' segment walk takes 64-column workgroups when 16-column ones would number
// four per CU or more (and the width allows it): at 256 segments x 8 heads it took 196
// against 239 us.  The compose walk stays at 16 columns, whose two workgroups per CU
// measured as fast or faster (87 against 97 us at 64 segments, 335 against 331 us at 256).
template <int DK>
static hipError_t launch_walk(const ScanWalk &a, hipStream_t stream) {
    const int64_t wg16 = (int64_t)a.n_task * a.H * (a.width / 16);
    if (a.mode == WALK_SEGMENTS && a.width % 64 == 0 && wg16 >= 4 * 256) return launch_walk_ct<DK, 4>(a, stream);
    return launch_walk_ct<DK, 1>(a, stream);
}

static hipError_t launch_walk_dk(int dk, const ScanWalk &a, hipStream_t stream) {
    return dk == 128 ? launch_walk<128>(a, stream) : launch_walk<64>(a, stream);
}

hipError_t launch_affine_scan(int n_seg, int H, int dk, int dv, const float *M, const float *U,
                              const float *S_init, float *incoming, float *outgoing, float *final_state,
                              hipStream_t stream) {
    if (dk == 128 || dk == 64) {
        const ScanWalk a{WALK_SEGMENTS, n_seg, H, dv, n_seg, 1, dv, M, U, S_init, incoming, outgoing,
                         final_state, nullptr};
        return launch_walk_dk(dk, a, stream);
    }
    const dim3 grid(H * (dv / 16));
    hipLaunchKernelGGL(kda_affine_scan_kernel, grid, dim3(SCAN_NT), 0, stream, n_seg, H, dk, dv, M, U,
                       S_init, incoming, outgoing, final_state);
    return hipGetLastError();
}

int scan_block_size(int n_seg, int dk, int dv, int blk) {
    if (blk <= 0) {
        // three launches and about three times the work: below 32 segments the ordered
        // walk is faster (16 segments x 8 heads at dk = dv = 128: 0.054 against 0.080 ms);
        // above, a critical path of ~2 blk + n_seg / blk steps wants blk ~ sqrt(n_seg / 2)
        if (n_seg < 32) return n_seg;
        blk = 1;
        while (2 * blk * blk < n_seg) ++blk;
    }
    // the block composites [dk, dk + dv] per block and head are kept in the outgoing
    // stack (n_seg [dk, dv] per head) until the last launch overwrites it
    const int min_blk = 1 + (dk + dv - 1) / dv;
    blk = max(blk, min_blk);
    return blk >= n_seg ? n_seg : blk;
}

hipError_t launch_affine_scan_blocked(int n_seg, int H, int dk, int dv, int blk, const float *M,
                                      const float *U, const float *S_init, float *incoming,
                                      float *outgoing, float *final_state, hipStream_t stream) {
    if (!(dk == 128 || dk == 64))
        return launch_affine_scan(n_seg, H, dk, dv, M, U, S_init, incoming, outgoing, final_state, stream);
    blk = scan_block_size(n_seg, dk, dv, blk);
    const int n_blocks = (n_seg + blk - 1) / blk;
    hipError_t e = hipSuccess;
    if (n_blocks > 1) {
        const ScanWalk c{WALK_COMPOSE, n_seg, H, dv, blk, n_blocks - 1, dk + dv, M, U, S_init, incoming,
                         outgoing, final_state, outgoing};
        e = launch_walk_dk(dk, c, stream);
        if (e != hipSuccess) return e;
        const ScanWalk b{WALK_BLOCKS, n_seg, H, dv, blk, 1, dv, M, U, S_init, incoming, outgoing,
                         final_state, outgoing};
        e = launch_walk_dk(dk, b, stream);
        if (e != hipSuccess) return e;
    }
    const ScanWalk s{WALK_SEGMENTS, n_seg, H, dv, blk, n_blocks, dv, M, U, S_init, incoming, outgoing,
                     final_state, nullptr};
    return launch_walk_dk(dk, s, stream);
}

}  // namespace kda
