// kda_pipe.hip -- bf16 chunk-parallel KDA prefill at dk = dv = 128 on gfx950 (MI355X), with
// the work of a chunk split between two wave groups that run one chunk apart.
//
// The arithmetic is that of kda_fast.hip (the token recurrence
// S_t = (I - b k k^T) Diag(alpha) S_{t-1} + b k v^T, o_t = scale q^T S_t of the
// nx_nofloat_kda.nx source, over 64-token chunks, with the same stable 16-row decay
// factorisation, operand precisions and guards); what differs is who does it and when.
// A chunk's work falls into two kinds:
//   * per-chunk preparation that does not depend on the state: the gate, decay factors
//     (running products of alpha), the decayed score blocks A and P, the inverses of the
//     diagonal blocks of I + A, and the chain operands Kg = K e^G, Qbar = Q e^G,
//     Khat = K e^{G_last - G}, V^T, beta, e^{G_last} -- VALU-heavy, independent of the
//     previous chunk;
//   * the state chain: Y = Kg S, R = beta (V - Y), the triangular solve for U, the output
//     O = scale (Qbar S + P U) and the update S <- e^{G_last} S + Khat^T U -- MFMA and
//     LDS work, sequential over chunks.
// Waves 4..11 (the producer) prepare chunk c+1 while waves 0..3 (the chain) run chunk c:
// every SIMD holds one chain wave and two producer waves, so the producer's VALU work
// overlaps the chain's MFMA and LDS work and the producer's own latencies overlap each
// other.  Chain wave w owns state columns 32w .. 32w+31 (two 16-column MFMA tiles, fp32 in
// accumulators for the whole unit); producer wave p owns rows 16 (p/2) .. 16 (p/2) + 15
// and key channels 64 (p%2) .. 64 (p%2) + 63 of a chunk.
//
// Each chunk takes two barrier intervals.  Arrays the chain reads in its first interval
// (Kg, V^T, beta, -A off the diagonal, the diagonal inverses) are written by the
// producer in the second, and arrays it reads in its second interval (Qbar, Khat^T, P)
// are written in the first, so every LDS array has one copy; only e^{G_last}, read in
// both, alternates between two.
//
// Lane-dependent values are re-derived from an opaque copy of the lane id in every chunk
// and unit (lane_ids): otherwise the compiler hoists dozens of per-lane addresses and
// constants out of the loops and keeps them live, which spills.
#include "kda_common.h"
#include "kda_fast_common.h"
#include "kda_launch.h"

namespace kda {

namespace pipe {

using namespace fk;

constexpr int DK = 128, DV = 128;
#ifndef NCC_CFG
#define NCC_CFG 2
#endif
constexpr int NCC = NCC_CFG;       // 16-column state tiles per chain wave
constexpr int NCW = 8 / NCC;       // chain waves
constexpr int NT = 64 * (NCW + 8); // chain waves, then 8 producer waves
constexpr int PK = DK + 8;  // 16-bit element pitch of [64][DK] arrays
// 16-bit element pitch of [*][64] arrays: 136-byte rows.  A wave's 8-byte accesses of
// 16 consecutive rows then fall into distinct LDS banks, and so do the producer's
// transposed 8-byte stores of V^T and Khat^T, whose lanes step 8 rows (a 144-byte pitch
// puts all of those in the same banks).
constexpr int PJ = 64 + 4;
constexpr int PD = 20;      // 16-bit element pitch of the diagonal inverses (40-byte rows)

struct Lds {
    static constexpr int ROWS = 64 * PK * 2;
    // chain operands of the first interval, written by the producer in the second
    static constexpr int KG = 0;                       // Kg        bf16 [64][PK]
    static constexpr int VT = KG + ROWS;               // V^T       bf16 [DV][PJ]
    static constexpr int AO = VT + DV * PJ * 2;        // -A off-diagonal blocks f16 [64][PJ]
    static constexpr int D = AO + 64 * PJ * 2;         // (I + A_II)^-1  f16 [4][16][PD]
    static constexpr int BETA = D + 4 * 16 * PD * 2;   // f32 [64]
    // chain operands of the second interval, written by the producer in the first
    static constexpr int QB = BETA + 64 * 4;           // Qbar      bf16 [64][PK]
    static constexpr int KH = QB + ROWS;               // Khat^T    f16 [DK][PJ] (tile-row order)
    static constexpr int P = KH + DK * PJ * 2;         // P         f16 [64][PJ]
    static constexpr int EG = P + 64 * PJ * 2;         // e^{G_last} f32 [2][DK], by chunk parity
    // producer-private
    static constexpr int KR = EG + 2 * DK * 4;         // Kr        bf16 [64][PK], scores
    static constexpr int QR = KR + ROWS;               // Qr        bf16 [64][PK], scores
    static constexpr int KC = QR + ROWS;               // Kc        bf16 [64][PK], scores
    static constexpr int E = KC + ROWS;                // block decays   f32 [4][DK]
    static constexpr int IE = E + 4 * DK * 4;          // 1 / block decays f32 [4][DK]
    static constexpr int AD = IE + 4 * DK * 4;         // A diagonal blocks^T f32 [4][16][20]
    static constexpr int BETAP = AD + 4 * 16 * 20 * 4; // beta, producer copy f32 [64]
    static constexpr int DTB = BETAP + 64 * 4;         // dt_bias log2(e), one copy per producer wave f32 [8][DK/2]
    static constexpr int BYTES = DTB + 8 * (DK / 2) * 4;
};
static_assert(Lds::BYTES <= 160 * 1024, "LDS");

// Score block pairs (I, J <= I) of producer wave p: waves 0..3 the diagonal pair (p, p)
// (their inverse follows), waves 4..7 the off-diagonal pairs {(1,0),(2,1)}, {(2,0),(3,2)},
// {(3,0)}, {(3,1)}.
__device__ __forceinline__ int n_pairs(int p) { return (p == 4 || p == 5) ? 2 : 1; }
__device__ __forceinline__ void pair_of(int p, int pp, int &bI, int &bJ) {
    if (p < 4) {
        bI = p;
        bJ = p;
    } else if (p == 4) {
        bI = 1 + pp;
        bJ = pp;
    } else if (p == 5) {
        bI = 2 + pp;
        bJ = 2 * pp;
    } else {
        bI = 3;
        bJ = p - 6;
    }
}

__device__ __forceinline__ bf16x8 bf8(f32x4 a, f32x4 b) { return cat(bf4(a), bf4(b)); }

// Products of the decays of the whole blocks before / after block I, for key channels
// c0 .. c0+3 (selects on the uniform block index, no branches).
__device__ __forceinline__ f32x4 decay_before(const float *sE, int c0, int I) {
    f32x4 f = f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int J = 0; J < 3; ++J) {
        const f32x4 ev = *(const f32x4 *)(sE + J * DK + c0);
        f = (J < I) ? f * ev : f;
    }
    return f;
}
__device__ __forceinline__ f32x4 decay_after(const float *sE, int c0, int I) {
    f32x4 f = f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int J = 1; J < 4; ++J) {
        const f32x4 ev = *(const f32x4 *)(sE + J * DK + c0);
        f = (J > I) ? f * ev : f;
    }
    return f;
}

// Half hf (elements 4 hf .. 4 hf + 3) of an 8-element group, read or written in place.
__device__ __forceinline__ f16x4 half_of(f16x8 x, int hf) {
    return hf ? __builtin_shufflevector(x, x, 4, 5, 6, 7) : __builtin_shufflevector(x, x, 0, 1, 2, 3);
}
__device__ __forceinline__ void set_half(f16x8 &x, int hf, f16x4 v) {
#pragma unroll
    for (int s = 0; s < 4; ++s) x[4 * hf + s] = v[s];
}

// Lane ids from a copy of the lane index the compiler cannot see through, so that what
// is derived from them is recomputed where used instead of hoisted out of the loops.
struct Lane {
    int l, g, li;  // MFMA layout: lane l = 16 g + li
    int rq, cq;    // producer: row quarter, 4-channel group (4 cq .. 4 cq + 3 of the wave's half)
};
__device__ __forceinline__ float sgpr_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

__device__ __forceinline__ Lane lane_ids() {
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    return Lane{l, l >> 4, l & 15, l & 3, l >> 2};
}

template <bool GQA>
__global__ __launch_bounds__(NT, 1) void kda_pipe_kernel(ChainArgs a) {
    using L = Lds;
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    bf16_t *sKG = (bf16_t *)(smem + L::KG);
    bf16_t *sVT = (bf16_t *)(smem + L::VT);
    f16_t *sAO = (f16_t *)(smem + L::AO);
    f16_t *sD = (f16_t *)(smem + L::D);
    float *sBeta = (float *)(smem + L::BETA);
    bf16_t *sQB = (bf16_t *)(smem + L::QB);
    f16_t *sKH = (f16_t *)(smem + L::KH);
    f16_t *sP = (f16_t *)(smem + L::P);
    float *sEG = (float *)(smem + L::EG);
    bf16_t *sKR = (bf16_t *)(smem + L::KR);
    bf16_t *sQR = (bf16_t *)(smem + L::QR);
    bf16_t *sKC = (bf16_t *)(smem + L::KC);
    float *sE = (float *)(smem + L::E);
    float *sIE = (float *)(smem + L::IE);
    float *sAD = (float *)(smem + L::AD);
    float *sBetaP = (float *)(smem + L::BETAP);

    const int H = a.H;
    const int t = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const bool chain = w < NCW;
    const int cw = w;              // chain wave: state columns 16 NCC cw .. 16 NCC (cw + 1) - 1
    const int pw = w - NCW;        // producer wave:
    const int pI = pw >> 1;        //   rows 16 pI .. 16 pI + 15 (block pI),
    const int ch0 = 64 * (pw & 1); //   key channels ch0 .. ch0 + 63
    float *sDTB = (float *)(smem + L::DTB) + (pw & 7) * (DK / 2);  // this producer wave's copy
    // alpha floor of the safe gate; wave-uniform values computed by vector instructions
    // are moved to scalar registers, which the producer's vector registers cannot spare
    const float amin = sgpr_f(a.gate_mode == 1 ? expf(a.lb) : 0.f);
    const int xcd = blockIdx.x & 7;

    // strictly-upper blocks of P are never written below
    for (int e = t; e < 64 * 64; e += NT) {
        const int i = e >> 6, j = e & 63;
        if ((j >> 4) > (i >> 4)) sP[i * PJ + j] = (f16_t)0.f;
    }
    __shared__ int s_next;

    for (int pass = 0;; ++pass) {
        int t_begin, t_end, h, init;
        bool vf = false, has_v;
        float *fin;
        bf16_t *obase = (bf16_t *)a.out;
        int64_t orow = 0;  // token of obase's row 0 (W rows of a later piece start at its own)
        if (!a.plan) {
            if (pass > 0) break;
            const int unit = (blockIdx.x >> 3) * 8 + xcd;
            if (unit >= a.n_items * H) break;
            const int item = unit / H;
            h = unit - item * H;
            t_begin = a.offsets[item];
            t_end = a.offsets[item + 1];
            fin = a.state_pool + ((int64_t)a.state_indices[item] * H + h) * DK * DV;
            init = 0;
            vf = a.v_first;
            has_v = true;
        } else {
            if (t == 0) s_next = atomicAdd((int *)&a.plan->ctr, 1);
            __syncthreads();
            const int u = __builtin_amdgcn_readfirstlane(s_next);
            __syncthreads();
            if (u >= a.plan->qlen) break;
            const int2 qe = a.queue[u];
            const int qx = __builtin_amdgcn_readfirstlane(qe.x), qy = __builtin_amdgcn_readfirstlane(qe.y);
            if (qy < 0) continue;  // skip slot
            const int4 en = a.ent[qx];
            const int seq = __builtin_amdgcn_readfirstlane(en.x), cbeg = __builtin_amdgcn_readfirstlane(en.y);
            const int cend = __builtin_amdgcn_readfirstlane(en.z), piece = __builtin_amdgcn_readfirstlane(en.w);
            h = qy & 0xffff;
            const int role = qy >> 16;
            const int sb = a.offsets[seq], se = a.offsets[seq + 1];
            t_begin = sb + 64 * cbeg;
            t_end = min(se, sb + 64 * cend);
            if (role == ROLE_WHOLE) {
                fin = a.state_pool + ((int64_t)a.state_indices[seq] * H + h) * DK * DV;
                init = 0;
                vf = a.v_first;
                has_v = true;
            } else if (role == ROLE_M) {
                fin = a.ws_M + ((int64_t)piece * H + h) * DK * DV;
                init = 1;
                has_v = false;
                obase = (bf16_t *)a.ws_W;
                orow = t_begin - 64 * (int64_t)__builtin_amdgcn_readfirstlane(a.ws_piece[piece].w);
            } else {
                fin = a.ws_U + ((int64_t)piece * H + h) * DK * DV;
                init = 2;
                has_v = true;
            }
        }
        const int len = t_end - t_begin;
        if (len <= 0) continue;
        const int hk = GQA ? h / (H / a.Hk) : h;
        const int n_chunks = (len + 63) / 64;
        const int rstride = vf ? 1 : DV;

        if (chain) {
            // ================================ the state chain ================================
            // Tile (ct, cc): lane (g, li) holds key rows key_row(ct, 4g + s) of column
            // 32 cw + 16 cc + li, i.e. rows 8g + 32 (ct / 2) + 4 (ct % 2) + s.
            f32x4 S[8][NCC];
            {
                const Lane ln = lane_ids();
#pragma unroll
                for (int cc = 0; cc < NCC; ++cc) {
                    const int col = 16 * NCC * cw + 16 * cc + ln.li;
                    const float *sp = vf ? fin + col * DK + 8 * ln.g : fin + 8 * ln.g * DV + col;
#pragma unroll
                    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            const int rr = 32 * (ct >> 1) + 4 * (ct & 1) + s;
                            S[ct][cc][s] = init == 0 ? sp[rr * rstride]
                                                     : ((init == 1 && 8 * ln.g + rr == col) ? 1.f : 0.f);
                        }
                }
            }
            __syncthreads();  // producer: chunk 0's gate and factors
            __syncthreads();  // producer: chunk 0's scores and chain operands

            for (int ck = 0; ck < n_chunks; ++ck) {
                const Lane ln = lane_ids();
                const int g = ln.g, li = ln.li;
                const int t0 = t_begin + ck * 64;
                const int n = min(64, t_end - t0);
                const float *eg = sEG + (ck & 1) * DK;
                // ---- first interval: Y = Kg S, R = beta (V - Y), (I + A) U = R
                f32x4 Y[4][NCC];
                {
                    bf16x8 Sb[4][NCC];
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                        for (int cc = 0; cc < NCC; ++cc) Sb[kb][cc] = bf8(S[2 * kb][cc], S[2 * kb + 1][cc]);
                    // one row tile at a time, the next tile's operands requested before the
                    // current tile's products: fenced so that the scheduler does not request
                    // every fragment up front and run out of registers
                    bf16x8 kg[4], kgn[4];
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) kg[kb] = *(const bf16x8 *)(sKG + li * PK + 32 * kb + 8 * g);
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) {
                        if (rt < 3)
#pragma unroll
                            for (int kb = 0; kb < 4; ++kb)
                                kgn[kb] = *(const bf16x8 *)(sKG + (16 * rt + 16 + li) * PK + 32 * kb + 8 * g);
#pragma unroll
                        for (int cc = 0; cc < NCC; ++cc) {
                            Y[rt][cc] = zero4();
#pragma unroll
                            for (int kb = 0; kb < 4; ++kb) Y[rt][cc] = mfma(kg[kb], Sb[kb][cc], Y[rt][cc]);
                        }
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) kg[kb] = kgn[kb];
                    }
                    // The rounding of S to bf16 in Kg S is forgotten with the state when the
                    // chunk decays it, but accumulates to ~1e-3 of the state where a key
                    // channel barely decays: chunks in which some channel keeps more than
                    // 1/16 of its state add the product with the rounding residual of S.
                    if (wave_max_nonneg(fmaxf(eg[ln.l], eg[ln.l + 64])) > 0x1p-4f) {
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) {
                            bf16x8 sl[NCC];
#pragma unroll
                            for (int cc = 0; cc < NCC; ++cc) {
                                const bf16x8 sh = Sb[kb][cc];
                                sl[cc] = bf8(S[2 * kb][cc] - f4(bf16x4{sh[0], sh[1], sh[2], sh[3]}),
                                             S[2 * kb + 1][cc] - f4(bf16x4{sh[4], sh[5], sh[6], sh[7]}));
                            }
#pragma unroll
                            for (int rt = 0; rt < 4; ++rt) {
                                const bf16x8 kg = *(const bf16x8 *)(sKG + (16 * rt + li) * PK + 32 * kb + 8 * g);
#pragma unroll
                                for (int cc = 0; cc < NCC; ++cc) Y[rt][cc] = mfma(kg, sl[cc], Y[rt][cc]);
                            }
                        }
                    }
                }
                float rmax = 0.f;
#pragma unroll
                for (int bI = 0; bI < 4; ++bI) {
                    const f32x4 bb = *(const f32x4 *)(sBeta + 16 * bI + 4 * g);
#pragma unroll
                    for (int cc = 0; cc < NCC; ++cc) {
                        const int vcol = 16 * NCC * cw + 16 * cc + li;
                        const f32x4 vv = f4(*(const bf16x4 *)(sVT + vcol * PJ + 16 * bI + 4 * g));
                        Y[bI][cc] = bb * (vv - Y[bI][cc]);
                        const f32x4 y = Y[bI][cc];
                        rmax = fmaxf(rmax, fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3]))));
                    }
                }
                // U travels as fp16 hi + lo, exact to ~2^-22 of its largest entry only while
                // that entry is near 1, and finite only below 65504: a wave whose R is small
                // (tiny beta and a vanished state) or large (large values or states) scales R,
                // hence U, by a power of two that brings max |R| into [1/4, 1/2), undone
                // exactly in the output scale and around the state update.
                float usc, iusc;
                rmax = wave_max_nonneg(rmax);
                if ((rmax < 0x1p-8f && rmax > 0.f) || (rmax >= 0x1p6f && rmax < 0x1p127f)) {
                    const int k = max(-126, min(64, -2 - ((int)(__builtin_bit_cast(unsigned, rmax) >> 23) - 127)));
                    usc = __builtin_bit_cast(float, (k + 127) << 23);
                    iusc = __builtin_bit_cast(float, (127 - k) << 23);
#pragma unroll
                    for (int bI = 0; bI < 4; ++bI)
#pragma unroll
                        for (int cc = 0; cc < NCC; ++cc) Y[bI][cc] *= usc;
                } else {
                    usc = 1.f;
                    iusc = 1.f;
                }
                // U (hi and lo parts) of row blocks 2 jb and 2 jb + 1 share one 8-element
                // register group: the halves feed the solve's 16x16x16 products, the whole
                // the 16x16x32 products of the output and the state update, without copies
                f16x8 Uh[2][NCC], Ul[2][NCC];
#pragma unroll
                for (int bI = 0; bI < 4; ++bI) {
                    f32x4 acc[NCC];
#pragma unroll
                    for (int cc = 0; cc < NCC; ++cc) acc[cc] = Y[bI][cc];
#pragma unroll
                    for (int bJ = 0; bJ < bI; ++bJ) {
                        const f16x4 ao = *(const f16x4 *)(sAO + (16 * bI + li) * PJ + 16 * bJ + 4 * g);
#pragma unroll
                        for (int cc = 0; cc < NCC; ++cc) {
                            acc[cc] = mfma16h(ao, half_of(Uh[bJ >> 1][cc], bJ & 1), acc[cc]);
                            acc[cc] = mfma16h(ao, half_of(Ul[bJ >> 1][cc], bJ & 1), acc[cc]);
                        }
                    }
                    const f16x4 dd = *(const f16x4 *)(sD + (bI * 16 + li) * PD + 4 * g);
#pragma unroll
                    for (int cc = 0; cc < NCC; ++cc) {
                        f16x4 wh, wl, uh, ul;
                        split_h(acc[cc], wh, wl);
                        f32x4 u = mfma16h(dd, wh, zero4());
                        u = mfma16h(dd, wl, u);
                        split_h(u, uh, ul);
                        set_half(Uh[bI >> 1][cc], bI & 1, uh);
                        set_half(Ul[bI >> 1][cc], bI & 1, ul);
                    }
                }
                __syncthreads();

                // ---- second interval: O^T = S^T Qbar^T + U^T P^T (Qbar and P carry the query
                // scale), S <- e^{G_last} S + Khat^T U
                {
                    const Lane lm = lane_ids();
                    // Qbar and P arrive multiplied by the query scale (in the producer), so the
                    // output needs no multiplier unless R was rescaled
                    bf16x8 Sb[4][NCC];
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                        for (int cc = 0; cc < NCC; ++cc) Sb[kb][cc] = bf8(S[2 * kb][cc], S[2 * kb + 1][cc]);
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) {
                        f32x4 Z[NCC];
#pragma unroll
                        for (int cc = 0; cc < NCC; ++cc) Z[cc] = zero4();
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) {
                            const bf16x8 qb = *(const bf16x8 *)(sQB + (16 * rt + lm.li) * PK + 32 * kb + 8 * lm.g);
                            // output transposed, O^T = S^T Qbar^T: the state tile is the A operand
#pragma unroll
                            for (int cc = 0; cc < NCC; ++cc) Z[cc] = mfma(Sb[kb][cc], qb, Z[cc]);
                        }
                        if (usc != 1.f)
#pragma unroll
                            for (int cc = 0; cc < NCC; ++cc) Z[cc] *= usc;
#pragma unroll
                        for (int jb = 0; jb <= (rt >> 1); ++jb) {
                            const f16x8 pf = fragA_perm_h(sP, PJ, 16 * rt + lm.li, 32 * jb, lm.g);
#pragma unroll
                            for (int cc = 0; cc < NCC; ++cc)
                                Z[cc] = mfma32h(Uh[jb][cc], pf, Z[cc]);
                        }
                        if (usc != 1.f)
#pragma unroll
                            for (int cc = 0; cc < NCC; ++cc) Z[cc] *= iusc;
                        // lane holds O[token 16 rt + li][columns 32 cw + 16 cc + 4g .. +3]
                        const int i = 16 * rt + lm.li;
                        if (i < n) {
                            bf16_t *op = obase + ((t0 - orow) * H + h) * DV + (unsigned)(i * (H * DV) + 16 * NCC * cw + 4 * lm.g);
#pragma unroll
                            for (int cc = 0; cc < NCC; ++cc) *(bf16x4 *)(op + 16 * cc) = bf4(Z[cc]);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    f16x8 kh[2], khn[2];
                    f32x4 e4 = *(const f32x4 *)(eg + key_row(0, 4 * lm.g)), e4n;
                    if (usc != 1.f)
#pragma unroll
                        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                            for (int cc = 0; cc < NCC; ++cc) S[ct][cc] *= usc;
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb) kh[jb] = fragA_perm_h(sKH, PJ, lm.li, 32 * jb, lm.g);
#pragma unroll
                    for (int ct = 0; ct < 8; ++ct) {
                        if (ct < 7) {
                            e4n = *(const f32x4 *)(eg + key_row(ct + 1, 4 * lm.g));
#pragma unroll
                            for (int jb = 0; jb < 2; ++jb) khn[jb] = fragA_perm_h(sKH, PJ, 16 * ct + 16 + lm.li, 32 * jb, lm.g);
                        }
#pragma unroll
                        for (int cc = 0; cc < NCC; ++cc) S[ct][cc] *= e4;
#pragma unroll
                        for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
                            for (int cc = 0; cc < NCC; ++cc) {
                                S[ct][cc] = mfma32h(kh[jb], Uh[jb][cc], S[ct][cc]);
                                S[ct][cc] = mfma32h(kh[jb], Ul[jb][cc], S[ct][cc]);
                            }
                        }
                        if (usc != 1.f)
#pragma unroll
                            for (int cc = 0; cc < NCC; ++cc) S[ct][cc] *= iusc;
                        __builtin_amdgcn_sched_barrier(0);
                        e4 = e4n;
#pragma unroll
                        for (int jb = 0; jb < 2; ++jb) kh[jb] = khn[jb];
                    }
                }
                __syncthreads();
            }
            // ---- final state of this wave's columns
            {
                const Lane ln = lane_ids();
#pragma unroll
                for (int cc = 0; cc < NCC; ++cc) {
                    const int col = 16 * NCC * cw + 16 * cc + ln.li;
                    float *fp = vf ? fin + col * DK + 8 * ln.g : fin + 8 * ln.g * DV + col;
#pragma unroll
                    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                        for (int s = 0; s < 4; ++s) fp[(32 * (ct >> 1) + 4 * (ct & 1) + s) * rstride] = S[ct][cc][s];
                }
            }
        } else {
            // ================================ the producer ================================
            // lane: rows 16 pI + 4 rq + [0, 4), key channels c0 .. c0 + 3 (c0 = ch0 + 4 cq)
            const float negA = sgpr_f(-expf(a.a_log[h]));
            {
                // each producer wave keeps its own copy of its channels' dt_bias (scaled by
                // log2 e) in LDS: read back by the same wave only, no barrier needed, and no
                // global load inside the chunk loop (whose wait would drain the prefetch)
                const Lane ln = lane_ids();
                sDTB[ln.l] = a.dt_bias[h * DK + ch0 + ln.l] * 1.44269504088896341f;
            }

            // prefetch registers: 4 rows x 4 channels of raw/k/q/v, one beta logit (wave 4)
            f32x4 praw[4];
            bf16x4 pk[4], pq[4], pv[4];
            float pbl = 0.f;
            // Loads of chunk ck in four groups (one row each, beta with the last), issued
            // between pieces of VALU work: all at once they fill the CU's memory request
            // queue and hold the issuing wave until every workgroup's requests drain.
            // Every load is unconditional (ck is clamped to the unit's last chunk, V is
            // read even where a unit does not use it): a load under a condition leaves the
            // register merged with its old value, a copy that waits for the load to land.
            auto issue_raw = [&](int ck, const Lane &ln) {
                ck = min(ck, n_chunks - 1);
                const int rbase = 16 * pI + 4 * ln.rq, c0 = ch0 + 4 * ln.cq;
                const int tq = t_begin + ck * 64;
                const int nq = min(64, t_end - tq);
                const int64_t rb = (int64_t)tq * H + h;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    praw[r] = *(const f32x4 *)(a.raw_gate + rb * DK + (unsigned)(min(rbase + r, nq - 1) * (H * DK) + c0));
            };
            auto issue = [&](int ck, int r, const Lane &ln) {
                ck = min(ck, n_chunks - 1);
                const int rbase = 16 * pI + 4 * ln.rq, c0 = ch0 + 4 * ln.cq;
                const int tq = t_begin + ck * 64;
                const int nq = min(64, t_end - tq);
                const int64_t rb = (int64_t)tq * H + h;
                const int64_t rbk = GQA ? (int64_t)tq * a.Hk + hk : rb;
                const unsigned ro = (unsigned)(min(rbase + r, nq - 1) * (H * DK) + c0);
                const unsigned rok = GQA ? (unsigned)(min(rbase + r, nq - 1) * (a.Hk * DK) + c0) : ro;
                pk[r] = *(const bf16x4 *)((const bf16_t *)a.k + rbk * DK + rok);
                pq[r] = *(const bf16x4 *)((const bf16_t *)a.q + rbk * DK + rok);
                pv[r] = *(const bf16x4 *)((const bf16_t *)a.v + rb * DV + ro);
                if (r == 3) pbl = a.beta_logits[rb + (unsigned)(min(ln.l, nq - 1) * H)];
            };

            // the gate of chunk ck, in place over its raw pre-activations (praw then holds alpha);
            // rows past the sequence end hold a copy of its last row: only their gate (alpha =
            // 1) and beta (0) are masked; with beta = 0 they add nothing to A, R, U or the
            // state, and their outputs are never stored
            auto gate_of = [&](int ck, const Lane &ln) {
                ck = min(ck, n_chunks - 1);
                const int nq = min(64, t_end - (t_begin + ck * 64)), rbase = 16 * pI + 4 * ln.rq;
                const f32x4 dtb = *(const f32x4 *)(sDTB + 4 * ln.cq);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float floor_r = rbase + r < nq ? amin : 1.f;
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc) praw[r][cc] = gate_alpha(praw[r][cc], dtb[cc], negA, floor_r);
                }
                // pinned here: the compiler would otherwise sink this work past the barrier
                // that follows, next to its use
#pragma unroll
                for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(praw[r]));
            };

            // ---- first half of the preparation of chunk ck (gate, running products):
            // Kr, Qr, Kc (bf16, for the scores) and the block decays to LDS; Kr, Qr, Kc in
            // fp32, V and beta kept in registers for the chain operands
            f32x4 kc[4], kr[4], qr[4];  // fp32 Kc, Kr, Qr of the chunk being prepared
            bf16x4 hv[4];
            float hbeta = 0.f;
            auto prep0 = [&](int ck, const Lane &ln) {
                const int rq = ln.rq, c0 = ch0 + 4 * ln.cq, rbase = 16 * pI + 4 * rq;
                const int nq = min(64, t_end - (t_begin + ck * 64));
                float al[4][4], kf[4][4], qf[4][4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc) {
                        al[r][cc] = praw[r][cc];  // alpha, from gate_of
                        kf[r][cc] = (float)pk[r][cc];
                        qf[r][cc] = (float)pq[r][cc];
                    }
                }
                f32x4 E, pre, suf;
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    float p = 1.f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) p *= al[r][cc];
                    const float q0 = quad_bcast<0>(p), q1 = quad_bcast<1>(p);
                    const float q2 = quad_bcast<2>(p), q3 = quad_bcast<3>(p);
                    E[cc] = ((q0 * q1) * q2) * q3;  // same operation order in every lane
                    pre[cc] = (rq >= 1 ? q0 : 1.f) * (rq >= 2 ? q1 : 1.f) * (rq >= 3 ? q2 : 1.f);
                    suf[cc] = (rq <= 2 ? q3 : 1.f) * (rq <= 1 ? q2 : 1.f) * (rq <= 0 ? q1 : 1.f);
                }
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    // forward: Kr_i = K_i e^{G_i - G_(16I-1)}
                    float rr = pre[cc];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        rr *= al[r][cc];
                        kr[r][cc] = kf[r][cc] * rr;
                        qr[r][cc] = qf[r][cc] * rr;
                    }
                    // backward: Kc_j = K_j e^{G_(16I+15) - G_j}
                    float cb = suf[cc];
#pragma unroll
                    for (int r = 3; r >= 0; --r) {
                        kc[r][cc] = kf[r][cc] * cb;
                        cb *= al[r][cc];
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = rbase + r;
                    *(bf16x4 *)(sKR + i * PK + c0) = bf4(kr[r]);
                    *(bf16x4 *)(sQR + i * PK + c0) = bf4(qr[r]);
                    *(bf16x4 *)(sKC + i * PK + c0) = bf4(kc[r]);
                    hv[r] = has_v ? pv[r] : bf16x4{};  // a transition chain has no values
                }
                if (rq == 0) {
                    *(f32x4 *)(sE + pI * DK + c0) = E;
                    // 1/E <= e^{16 |bound|}: finite under the safe gate
                    *(f32x4 *)(sIE + pI * DK + c0) = f32x4{__builtin_amdgcn_rcpf(E[0]), __builtin_amdgcn_rcpf(E[1]),
                                                          __builtin_amdgcn_rcpf(E[2]), __builtin_amdgcn_rcpf(E[3])};
                }
                if (pw == 0) {
                    // the hardware reciprocal, not an IEEE division, and selects, no branch
                    const float sig = __builtin_amdgcn_rcpf(1.f + __expf(-pbl));
                    hbeta = ln.l < nq ? (a.beta_mode == 0 ? sig : pbl) : 0.f;
                    sBetaP[ln.l] = hbeta;
                }
            };

            // ---- second half of the preparation of chunk ck: chain operands and scores.
            // Writes Kg, V^T, beta, e^{G_last}, -A and the diagonal inverses; keeps P in
            // registers (written in the next interval, with Qbar and Khat^T).
            f16x4 ph[2];
            auto prep1 = [&](int ck, const Lane &ln, int nxt) {
                // nxt: the chunk whose loads go out in groups 1..3 between the parts below
                const int c0 = ch0 + 4 * ln.cq, rbase = 16 * pI + 4 * ln.rq;
                const int g = ln.g, li = ln.li;
                {
                    // Kg = K e^{G}: Kr times the decays of the earlier blocks
                    const f32x4 fI = decay_before(sE, c0, pI);
#pragma unroll
                    for (int r = 0; r < 4; ++r) *(bf16x4 *)(sKG + (rbase + r) * PK + c0) = bf4(kr[r] * fI);
                }
                issue(nxt, 1, ln);
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
                    *(bf16x4 *)(sVT + (c0 + cc) * PJ + rbase) = bf16x4{hv[0][cc], hv[1][cc], hv[2][cc], hv[3][cc]};
                if (pw == 0) {
                    sBeta[ln.l] = hbeta;
                    // e^{G_last} of channels 2l, 2l+1
                    float e0 = 1.f, e1 = 1.f;
#pragma unroll
                    for (int J = 0; J < 4; ++J) {
                        e0 *= sE[J * DK + 2 * ln.l];
                        e1 *= sE[J * DK + 2 * ln.l + 1];
                    }
                    *(float2 *)(sEG + (ck & 1) * DK + 2 * ln.l) = float2{e0, e1};
                }
                // ---- decayed scores of this wave's block pairs (bf16 16x16x32 MFMA)
                const int np = n_pairs(pw);
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    if (pp >= np) break;
                    int bI, bJ;
                    pair_of(pw, pp, bI, bJ);
                    f32x4 accA = zero4(), accP = zero4();
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) {
                        const int cc = 32 * kb + 8 * g;
                        const bf16x8 aK = *(const bf16x8 *)(sKR + (16 * bI + li) * PK + cc);
                        const bf16x8 aQ = *(const bf16x8 *)(sQR + (16 * bI + li) * PK + cc);
                        const bf16x8 kcv = *(const bf16x8 *)(sKC + (16 * bJ + li) * PK + cc);
                        // e^{G_(16I-1) - G_(16J+15)}: 1/E_I on the diagonal, else the decays of
                        // the whole blocks strictly between J and I (none for adjacent blocks)
                        bf16x8 bK = kcv;
                        if (bI != bJ + 1) {
                            f32x4 m0, m1;
                            if (bI == bJ) {
                                m0 = *(const f32x4 *)(sIE + bI * DK + cc);
                                m1 = *(const f32x4 *)(sIE + bI * DK + cc + 4);
                            } else {
                                m0 = *(const f32x4 *)(sE + (bJ + 1) * DK + cc);
                                m1 = *(const f32x4 *)(sE + (bJ + 1) * DK + cc + 4);
                                if (bI == bJ + 3) {
                                    m0 *= *(const f32x4 *)(sE + (bJ + 2) * DK + cc);
                                    m1 *= *(const f32x4 *)(sE + (bJ + 2) * DK + cc + 4);
                                }
                            }
                            bK = bf8(f4(bf16x4{kcv[0], kcv[1], kcv[2], kcv[3]}) * m0,
                                     f4(bf16x4{kcv[4], kcv[5], kcv[6], kcv[7]}) * m1);
                        }
                        accA = mfma(aK, bK, accA);
                        accP = mfma(aQ, bK, accP);
                    }
                    f32x4 at;  // diagonal block, stored transposed: column li, rows 4g .. 4g+3
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int ri = 4 * g + s, i = 16 * bI + ri, j = 16 * bJ + li;
                        const float av = sBetaP[i] * accA[s];
                        at[s] = (li < ri) ? av : 0.f;
                        if (bI != bJ) sAO[i * PJ + j] = (f16_t)(-av);
                        ph[pp][s] = (f16_t)((j <= i) ? a.scale * accP[s] : 0.f);
                    }
                    if (bI == bJ) *(f32x4 *)(sAD + (bI * 16 + li) * 20 + 4 * g) = at;
                }
                issue(nxt, 2, ln);
                if (pw < 4) {
                    // (I + A_pw)^-1 by right-looking substitution: column c = l/4 of the
                    // inverse on the four lanes of a quad, lane quarter q = l%4 holding rows
                    // 4q .. 4q+3
                    const int c = ln.l >> 2, q = ln.l & 3;
                    const float *At = sAD + pw * 16 * 20;
                    float acc[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[j] = (4 * q + j == c) ? -1.f : 0.f;
                    inv_step<0>(acc, At, q);
#pragma unroll
                    for (int j = 0; j < 4; ++j) sD[(pw * 16 + 4 * q + j) * PD + c] = (f16_t)(0.f - acc[j]);
                }
                issue(nxt, 3, ln);
                // the gate of chunk nxt, a chunk ahead of its running products: its raw
                // pre-activations went out before this interval
                gate_of(nxt, ln);
            };
            // ---- the arrays the chain reads in its second interval: Qbar and Khat^T, formed
            // here from Qr, Kc and the block decays before the next chunk's preparation
            // overwrites them, and P from registers
            auto store_second = [&](const Lane &ln) {
                const int c0 = ch0 + 4 * ln.cq, rbase = 16 * pI + 4 * ln.rq;
                {
                    // Qbar = scale Q e^{G} (Qr times the earlier blocks' decays),
                    // Khat_j = K_j e^{G_last - G_j} (Kc times the later blocks' decays)
                    const f32x4 fI = decay_before(sE, c0, pI), qS = decay_after(sE, c0, pI);
                    const f32x4 fIs = fI * a.scale;  // with the query scale
#pragma unroll
                    for (int r = 0; r < 4; ++r) *(bf16x4 *)(sQB + (rbase + r) * PK + c0) = bf4(qr[r] * fIs);
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc)
                        *(f16x4 *)(sKH + tile_row(c0 + cc) * PJ + rbase) =
                            f16x4{(f16_t)(kc[0][cc] * qS[cc]), (f16_t)(kc[1][cc] * qS[cc]),
                                  (f16_t)(kc[2][cc] * qS[cc]), (f16_t)(kc[3][cc] * qS[cc])};
                }
                const int np = n_pairs(pw);
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    if (pp >= np) break;
                    int bI, bJ;
                    pair_of(pw, pp, bI, bJ);
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        sP[(16 * bI + 4 * ln.g + s) * PJ + 16 * bJ + ln.li] = ph[pp][s];
                }
            };

            {
                const Lane ln = lane_ids();
                issue_raw(0, ln);
#pragma unroll
                for (int r = 0; r < 4; ++r) issue(0, r, ln);
                gate_of(0, ln);
                prep0(0, ln);
                issue_raw(1, ln);
                issue(1, 0, ln);
            }
            __syncthreads();
            prep1(0, lane_ids(), 1);
            __syncthreads();
            // The last chunk is peeled off, so that the loop body has no branch: with one,
            // the load-wait bookkeeping merges the paths and makes prep1 wait for every
            // load in flight, the next chunk's first group included.
            for (int ck = 0; ck + 1 < n_chunks; ++ck) {
                // first interval of chunk ck: the chain's Y, R and solve
                {
                    const Lane ln = lane_ids();
                    store_second(ln);
                    prep0(ck + 1, ln);
                    issue_raw(ck + 2, ln);
                    issue(ck + 2, 0, ln);
                }
                __syncthreads();
                // second interval: the chain's output and state update
                prep1(ck + 1, lane_ids(), ck + 2);
                __syncthreads();
            }
            store_second(lane_ids());
            __syncthreads();
            __syncthreads();
        }
    }  // units
}

}  // namespace pipe

hipError_t launch_pipe(const ChainArgs &a, dim3 grid, hipStream_t stream) {
    if (a.Hk != a.H)
        hipLaunchKernelGGL(pipe::kda_pipe_kernel<true>, grid, dim3(pipe::NT), 0, stream, a);
    else
        hipLaunchKernelGGL(pipe::kda_pipe_kernel<false>, grid, dim3(pipe::NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kda
