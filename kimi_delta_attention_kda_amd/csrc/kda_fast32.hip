// kda_fast32.hip -- bf16 chunk-parallel KDA prefill (dk = dv = 128) with 32-token chunks
// and two chains per compute unit.
//
// The chunk algebra is that of kda_fast.hip (the token recurrence of the
// nx_nofloat_kda.nx source rewritten over chunks; see there), organised so that a
// workgroup needs about 74 KB of LDS and 4 waves: two workgroups, i.e. two independent
// (sequence, head) chains, share each CU and fill each other's barrier waits and
// dependency stalls.
//  * Wave w owns state columns 32w .. 32w+31 (two 16-column tiles) for the whole unit, so
//    every Kg / Qbar / Khat^T operand fragment read from LDS feeds two MFMAs.
//  * A 32-token chunk is two 16-row blocks: scores are the two diagonal blocks (waves 0
//    and 1, which also invert them) and the adjacent pair (1, 0) (wave 2 its A block,
//    wave 3 its P block); adjacent blocks need no cross-block decay factor.
//  * Prep threads own 4 channels x 4 rows as in kda_fast.hip; the gate and decay products
//    of chunk c+1 are computed in the last segment of chunk c (software pipeline), after
//    its outputs and state update.
#include "kda_common.h"
#include "kda_fast_common.h"
#include "kda_launch.h"

namespace kda {

namespace fast32 {

using namespace fk;

constexpr int NT = 256;      // 4 waves
constexpr int CS = 32;       // tokens per chunk
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int PK = DK + 8;   // 16-bit element pitch of [CS][DK] arrays
constexpr int PJ = CS + 8;   // 16-bit element pitch of [*][CS] arrays

struct Lds {
    static constexpr int ROWS = CS * PK * 2;   // one [CS][PK] 16-bit array
    static constexpr int KR = 0;               // Kr              bf16, scores
    static constexpr int QR = KR + ROWS;       // Qr              bf16, scores
    static constexpr int KC = QR + ROWS;       // Kc              bf16, scores
    static constexpr int KG = KC + ROWS;       // Kg              bf16, chain
    static constexpr int QB = KG + ROWS;       // Qbar            bf16, chain
    static constexpr int KH = QB + ROWS;       // Khat^T          f16 [DK][PJ], tile_row order
    static constexpr int VT = KH + DK * PJ * 2;  // V^T           bf16 [DV][PJ]
    static constexpr int AO = VT + DV * PJ * 2;  // -A off-diag   f16 [CS][PJ]
    static constexpr int P = AO + CS * PJ * 2;   // P             f16 [CS][PJ]
    static constexpr int AD = P + CS * PJ * 2;   // A diag^T      f32 [2][16][20]
    static constexpr int D = AD + 2 * 16 * 20 * 4;  // (I+A_II)^-1 f16 [2][16][24]
    static constexpr int BETA = D + 2 * 16 * 24 * 2;  // f32 [CS]
    static constexpr int E = BETA + CS * 4;      // block decays  f32 [2][DK]
    static constexpr int IE = E + 2 * DK * 4;    // 1/decays      f32 [2][DK]
    static constexpr int EG = IE + 2 * DK * 4;   // e^{G_last}    f32 [DK]
    static constexpr int BYTES = EG + DK * 4;
};
static_assert(2 * (Lds::BYTES + 16) <= 160 * 1024, "two workgroups per CU");

__global__ __launch_bounds__(NT, 2) void kda_fast32_kernel(ChainArgs a) {
    using L = Lds;
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    bf16_t *sKR = (bf16_t *)(smem + L::KR);
    bf16_t *sQR = (bf16_t *)(smem + L::QR);
    bf16_t *sKC = (bf16_t *)(smem + L::KC);
    bf16_t *sKG = (bf16_t *)(smem + L::KG);
    bf16_t *sQB = (bf16_t *)(smem + L::QB);
    f16_t *sKH = (f16_t *)(smem + L::KH);
    bf16_t *sVT = (bf16_t *)(smem + L::VT);
    f16_t *sAO = (f16_t *)(smem + L::AO);
    f16_t *sP = (f16_t *)(smem + L::P);
    float *sAD = (float *)(smem + L::AD);
    f16_t *sD = (f16_t *)(smem + L::D);
    float *sBeta = (float *)(smem + L::BETA);
    float *sE = (float *)(smem + L::E);
    float *sIE = (float *)(smem + L::IE);
    float *sEG = (float *)(smem + L::EG);

    const int H = a.H;
    const int t = threadIdx.x, l = t & 63, g = l >> 4, li = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index, in a scalar register
    // prep role: block I, key channels c0 .. c0+3, rows 16I + 4rq + [0, 4)
    const int I = __builtin_amdgcn_readfirstlane(t >> 7), rq = t & 3, c0 = 4 * ((t >> 2) & 31);
    const int rbase = 16 * I + 4 * rq;
    const float amin = a.gate_mode == 1 ? expf(a.lb) : 0.f;  // alpha floor of the safe gate
    const int xcd = blockIdx.x & 7;  // workgroups are dealt to the 8 XCDs round-robin

    // strictly-upper block (0, 1) of P is never written below
    for (int e = t; e < 16 * 16; e += NT) sP[(e >> 4) * PJ + 16 + (e & 15)] = (f16_t)0.f;
    __shared__ int s_next;

    // One unit per pass: one (item, head) of the grid, or one queued unit of a plan.
    for (int pass = 0;; ++pass) {
        int t_begin, t_end, h;
        int init;         // 0: load the state from fin, 1: identity, 2: zero
        bool vf = false;  // fin is a pool slot stored [DV][DK]
        bool has_v;
        float *fin;       // [DK][DV] state of this unit: initial (init 0) and final
        bf16_t *obase = (bf16_t *)a.out;
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
            if (t == 0) s_next = atomicAdd((int *)&a.plan->ctr[xcd], 1);
            __syncthreads();
            // every value of the unit is wave-uniform: keep it in scalar registers
            const int u = __builtin_amdgcn_readfirstlane(s_next);
            __syncthreads();
            if (u >= a.plan->qlen[xcd]) break;
            const int2 qe = a.queue[xcd * a.qcap + u];
            const int qx = __builtin_amdgcn_readfirstlane(qe.x), qy = __builtin_amdgcn_readfirstlane(qe.y);
            if (qy < 0) continue;  // skip slot
            const int4 en = a.ent[qx];
            const int seq = __builtin_amdgcn_readfirstlane(en.x), cbeg = __builtin_amdgcn_readfirstlane(en.y);
            const int cend = __builtin_amdgcn_readfirstlane(en.z), piece = __builtin_amdgcn_readfirstlane(en.w);
            h = qy & 0xffff;
            const int role = qy >> 16;
            const int sb = a.offsets[seq], se = a.offsets[seq + 1];
            t_begin = sb + CS * cbeg;
            t_end = min(se, sb + CS * cend);
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
            } else {
                fin = a.ws_U + ((int64_t)piece * H + h) * DK * DV;
                init = 2;
                has_v = true;
            }
        }
        const int len = t_end - t_begin;
        if (len <= 0) continue;
        const int n_chunks = (len + CS - 1) / CS;
        const float negA = -expf(a.a_log[h]);
        const f32x4 dtb = *(const f32x4 *)(a.dt_bias + h * DK + c0) * 1.44269504088896341f;

    // ---- state tiles of wave w: S[m][ct] holds key rows key_row(ct, 4g + s) =
    // 8g + (32(ct/2) + 4(ct%2) + s) of column 32w + 16m + li.  One lane pointer per unit
    // plus row offsets times the row stride (DV for [DK][DV] storage, 1 for a V_FIRST slot).
    f32x4 S[2][8];
    const int rstride = vf ? 1 : DV;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int col = 32 * w + 16 * m + li;
        const float *sp = vf ? fin + col * DK + 8 * g : fin + 8 * g * DV + col;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int rr = 32 * (ct >> 1) + 4 * (ct & 1) + s;
                S[m][ct][s] = init == 0 ? sp[rr * rstride] : ((init == 1 && 8 * g + rr == col) ? 1.f : 0.f);
            }
    }

    // ---- prefetch registers: 4 rows x 4 channels of raw/k/q/v, one beta logit
    f32x4 praw[4];
    bf16x4 pk[4], pq[4], pv[4];
    float pbl = 0.f;
    if (!has_v)
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[r] = bf16x4{};
    // Loads of chunk ck in six small groups (q = 0..5), spread over the previous chunk.
    // Addresses: a scalar base per chunk (its first token, this head) plus 32-bit lane
    // offsets; the four row offsets of a chunk are formed once, at its first group.
    unsigned roff[4];
    auto issue = [&](int ck, int q) {
        const int t0 = t_begin + ck * CS;
        const int64_t rb = (int64_t)t0 * H + h;
        if (q == 0) {
            const int n = min(CS, t_end - t0);
#pragma unroll
            for (int r = 0; r < 4; ++r) roff[r] = (unsigned)(min(rbase + r, n - 1) * (H * DK) + c0);
        }
        const float *rg = a.raw_gate + rb * DK;
        const bf16_t *kp = (const bf16_t *)a.k + rb * DK;
        const bf16_t *qp = (const bf16_t *)a.q + rb * DK;
        const bf16_t *vp = (const bf16_t *)a.v + rb * DV;
        if (q == 0) {
            praw[0] = *(const f32x4 *)(rg + roff[0]);
            praw[1] = *(const f32x4 *)(rg + roff[1]);
        } else if (q == 1) {
            praw[2] = *(const f32x4 *)(rg + roff[2]);
            praw[3] = *(const f32x4 *)(rg + roff[3]);
            pbl = a.beta_logits[rb + (unsigned)(min(l & (CS - 1), t_end - t0 - 1) * H)];
        } else if (q == 2) {
#pragma unroll
            for (int r = 0; r < 3; ++r) pk[r] = *(const bf16x4 *)(kp + roff[r]);
        } else if (q == 3) {
            pk[3] = *(const bf16x4 *)(kp + roff[3]);
            pq[0] = *(const bf16x4 *)(qp + roff[0]);
            pq[1] = *(const bf16x4 *)(qp + roff[1]);
        } else if (q == 4) {
            pq[2] = *(const bf16x4 *)(qp + roff[2]);
            pq[3] = *(const bf16x4 *)(qp + roff[3]);
            if (has_v) pv[0] = *(const bf16x4 *)(vp + roff[0]);
        } else {
            if (has_v)
#pragma unroll
                for (int r = 1; r < 4; ++r) pv[r] = *(const bf16x4 *)(vp + roff[r]);
        }
    };
    // ---- gate and decay products of chunk ck (branch-free VALU work).  Rows past the
    // sequence end hold a copy of its last row: only their gate (alpha = 1) and beta (0)
    // are masked; with beta = 0 they add nothing to A, R, U or the state, and their outputs
    // are never stored.
    bf16x4 kr4[4], qr4[4];
    float kc[4][4];
    auto prep0 = [&](int ck) {
        const int n = min(CS, t_end - (t_begin + ck * CS));
        // one channel at a time: few values live at once
        float floor_r[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) floor_r[r] = rbase + r < n ? amin : 1.f;  // alpha <= 1: padded rows get 1
        f32x4 E;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            float al[4], kf[4], qf[4];
            float p = 1.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                al[r] = gate_alpha(praw[r][cc], dtb[cc], negA, floor_r[r]);
                kf[r] = (float)pk[r][cc];
                qf[r] = (float)pq[r][cc];
                p *= al[r];
            }
            // products over this quarter block, then over the other quarters (quad lanes)
            const float q0 = quad_bcast<0>(p), q1 = quad_bcast<1>(p);
            const float q2 = quad_bcast<2>(p), q3 = quad_bcast<3>(p);
            E[cc] = ((q0 * q1) * q2) * q3;  // same operation order in every lane
            // forward: Kr_i = K_i e^{G_i - G_(16I-1)}
            float rr = (rq >= 1 ? q0 : 1.f) * (rq >= 2 ? q1 : 1.f) * (rq >= 3 ? q2 : 1.f);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                rr *= al[r];
                kr4[r][cc] = (bf16_t)(kf[r] * rr);
                qr4[r][cc] = (bf16_t)(qf[r] * rr);
            }
            // backward: Kc_j = K_j e^{G_(16I+15) - G_j}
            float cb = (rq <= 2 ? q3 : 1.f) * (rq <= 1 ? q2 : 1.f) * (rq <= 0 ? q1 : 1.f);
#pragma unroll
            for (int r = 3; r >= 0; --r) {
                kc[r][cc] = kf[r] * cb;
                cb *= al[r];
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = rbase + r;
            *(bf16x4 *)(sKR + i * PK + c0) = kr4[r];
            *(bf16x4 *)(sQR + i * PK + c0) = qr4[r];
            bf16x4 kcb;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) kcb[cc] = (bf16_t)kc[r][cc];
            *(bf16x4 *)(sKC + i * PK + c0) = kcb;
        }
        // the four lanes of a quad hold the same E: unconditional identical stores
        *(f32x4 *)(sE + I * DK + c0) = E;
        // 1/E <= e^{16 |bound|}: finite under the safe gate
        *(f32x4 *)(sIE + I * DK + c0) = f32x4{__builtin_amdgcn_rcpf(E[0]), __builtin_amdgcn_rcpf(E[1]),
                                             __builtin_amdgcn_rcpf(E[2]), __builtin_amdgcn_rcpf(E[3])};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            bf16x4 v4;
#pragma unroll
            for (int r = 0; r < 4; ++r) v4[r] = pv[r][cc];
            *(bf16x4 *)(sVT + (c0 + cc) * PJ + rbase) = v4;
        }
        // every wave holds the beta of the chunk's rows (identical stores)
        const int rb = l & (CS - 1);
        sBeta[rb] = rb < n ? (a.beta_mode == 0 ? 1.f / (1.f + __expf(-pbl)) : pbl) : 0.f;
    };
    if (n_chunks > 0) {
#pragma unroll
        for (int q = 0; q < 6; ++q) issue(0, q);
        prep0(0);
        __syncthreads();
        if (n_chunks > 1) {
            issue(1, 0);
            issue(1, 1);
            issue(1, 2);
        }
    }

    for (int ck = 0; ck < n_chunks; ++ck) {
        const int t0 = t_begin + ck * CS;
        const int n = min(CS, t_end - t0);
        const bool more = ck + 1 < n_chunks;

        // ============ P1: cross-block factors, chain operands Kg, Qbar, Khat^T ============
        {
            const f32x4 E0 = *(const f32x4 *)(sE + c0), E1 = *(const f32x4 *)(sE + DK + c0);
            const f32x4 ones = f32x4{1.f, 1.f, 1.f, 1.f};
            const f32x4 pI = I ? E0 : ones;  // decay of the blocks before block I
            const f32x4 qS = I ? ones : E1;  // decay of the blocks after block I
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = rbase + r;
                bf16x4 x, y;
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    x[cc] = (bf16_t)((float)kr4[r][cc] * pI[cc]);  // Kg = K e^{G}
                    y[cc] = (bf16_t)((float)qr4[r][cc] * pI[cc]);  // Qbar = Q e^{G}
                }
                *(bf16x4 *)(sKG + i * PK + c0) = x;
                *(bf16x4 *)(sQB + i * PK + c0) = y;
            }
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                f16x4 h4;  // Khat_j = K_j e^{G_last - G_j}
#pragma unroll
                for (int r = 0; r < 4; ++r) h4[r] = (f16_t)(kc[r][cc] * qS[cc]);
                *(f16x4 *)(sKH + tile_row(c0 + cc) * PJ + rbase) = h4;
            }
            *(f32x4 *)(sEG + c0) = E0 * E1;  // identical stores from every block and quad lane
        }
        // (no barrier: Kg, Qbar, Khat^T and e^{G_last} are first read in the chain step)
        if (more) issue(ck + 1, 3);

        // ============ P2: decayed scores; the diagonal waves also invert their block ============
        if (w < 2) {
            // diagonal block w: factor e^{G_(16w-1) - G_(16w+15)} = 1/E_w on the B side
            f32x4 accA = zero4(), accP = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int cc = 32 * kb + 8 * g;
                const bf16x8 kcv = *(const bf16x8 *)(sKC + (16 * w + li) * PK + cc);
                const f32x4 m0 = *(const f32x4 *)(sIE + w * DK + cc), m1 = *(const f32x4 *)(sIE + w * DK + cc + 4);
                bf16x8 bK;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    bK[s] = (bf16_t)((float)kcv[s] * m0[s]);
                    bK[s + 4] = (bf16_t)((float)kcv[s + 4] * m1[s]);
                }
                accA = mfma(*(const bf16x8 *)(sKR + (16 * w + li) * PK + cc), bK, accA);
                accP = mfma(*(const bf16x8 *)(sQR + (16 * w + li) * PK + cc), bK, accP);
            }
            f32x4 at;  // stored transposed: column li, rows 4g .. 4g+3
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int ri = 4 * g + s, i = 16 * w + ri;
                at[s] = (li < ri) ? sBeta[i] * accA[s] : 0.f;
                sP[i * PJ + 16 * w + li] = (f16_t)((li <= ri) ? accP[s] : 0.f);
            }
            *(f32x4 *)(sAD + (w * 16 + li) * 20 + 4 * g) = at;
        } else {
            // pair (1, 0), adjacent: no factor.  Wave 2 builds A, wave 3 builds P.
            const bf16_t *lhs = w == 2 ? sKR : sQR;
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int cc = 32 * kb + 8 * g;
                acc = mfma(*(const bf16x8 *)(lhs + (16 + li) * PK + cc), *(const bf16x8 *)(sKC + li * PK + cc), acc);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int i = 16 + 4 * g + s;
                if (w == 2) sAO[i * PJ + li] = (f16_t)(-sBeta[i] * acc[s]);
                else sP[i * PJ + li] = (f16_t)acc[s];
            }
        }
        if (more) issue(ck + 1, 4);
        if (w < 2) {
            // (I + A_ww)^-1 by right-looking substitution on all 64 lanes (see kda_fast.hip)
            const int c = l >> 2, q = l & 3;
            const float *At = sAD + w * 16 * 20;
            float acc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = (4 * q + j == c) ? -1.f : 0.f;
            inv_step<0>(acc, At, q);
#pragma unroll
            for (int j = 0; j < 4; ++j) sD[(w * 16 + 4 * q + j) * 24 + c] = (f16_t)(0.f - acc[j]);
        }
        if (more) issue(ck + 1, 5);
        __syncthreads();

        // ============ chain step, first half: Y = Kg S, Z = S^T Qbar^T, R, forward substitution ============
        f32x4 Z[2][2];
        f16x4 Uh[2][2], Ul[2][2];  // [row block][column tile]
        {
            bf16x8 Sb[2][4];
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) Sb[m][kb] = cat(bf4(S[m][2 * kb]), bf4(S[m][2 * kb + 1]));
            f32x4 Y[2][2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    Y[rt][m] = zero4();
                    Z[rt][m] = zero4();
                }
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const bf16x8 kg = *(const bf16x8 *)(sKG + (16 * rt + li) * PK + 32 * kb + 8 * g);
                    const bf16x8 qb = *(const bf16x8 *)(sQB + (16 * rt + li) * PK + 32 * kb + 8 * g);
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        Y[rt][m] = mfma(kg, Sb[m][kb], Y[rt][m]);
                        // output transposed, O^T = S^T Qbar^T: the state tile is the A operand
                        Z[rt][m] = mfma(Sb[m][kb], qb, Z[rt][m]);
                    }
                }
            }
            // R = beta (V - Kg S); solve (I + A) U = R block by block
            const f16x4 ao = *(const f16x4 *)(sAO + (16 + li) * PJ + 4 * g);
            const f16x4 dd0 = *(const f16x4 *)(sD + li * 24 + 4 * g);
            const f16x4 dd1 = *(const f16x4 *)(sD + (16 + li) * 24 + 4 * g);
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int vcol = 32 * w + 16 * m + li;
#pragma unroll
                for (int bI = 0; bI < 2; ++bI) {
                    const f32x4 vv = f4(*(const bf16x4 *)(sVT + vcol * PJ + 16 * bI + 4 * g));
                    const f32x4 bb = *(const f32x4 *)(sBeta + 16 * bI + 4 * g);
                    f32x4 acc = bb * (vv - Y[bI][m]);
                    if (bI == 1) {
                        acc = mfma16h(ao, Uh[0][m], acc);
                        acc = mfma16h(ao, Ul[0][m], acc);
                    }
                    f16x4 wh, wl;
                    split_h(acc, wh, wl);
                    const f16x4 dd = bI ? dd1 : dd0;
                    f32x4 u = mfma16h(dd, wh, zero4());
                    u = mfma16h(dd, wl, u);
                    split_h(u, Uh[bI][m], Ul[bI][m]);
                }
            }
        }
        __syncthreads();

        // ============ chain step, second half: outputs and state update of chunk ck,
        // interleaved with the gate and decay products of chunk ck + 1 ============
        {
            const f16x8 pf0 = fragA_perm_h(sP, PJ, li, 0, g), pf1 = fragA_perm_h(sP, PJ, 16 + li, 0, g);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int i = 16 * rt + li;
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    // O^T += U^T P^T; lane holds O[token 16rt + li][columns 32w + 16m + 4g .. +3]
                    Z[rt][m] = mfma32h(cath(Uh[0][m], Uh[1][m]), rt ? pf1 : pf0, Z[rt][m]);
                    if (i < n)
                        *(bf16x4 *)(obase + ((int64_t)t0 * H + h) * DV +
                                    (unsigned)(i * (H * DV) + 32 * w + 16 * m + 4 * g)) = bf4(a.scale * Z[rt][m]);
                }
            }
            // S <- Diag(e^{G_last}) S + Khat^T U
            const f16x8 uh0 = cath(Uh[0][0], Uh[1][0]), ul0 = cath(Ul[0][0], Ul[1][0]);
            const f16x8 uh1 = cath(Uh[0][1], Uh[1][1]), ul1 = cath(Ul[0][1], Ul[1][1]);
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                const f32x4 eg = *(const f32x4 *)(sEG + key_row(ct, 4 * g));
                const f16x8 kh = fragA_perm_h(sKH, PJ, 16 * ct + li, 0, g);
                S[0][ct] *= eg;
                S[1][ct] *= eg;
                S[0][ct] = mfma32h(kh, uh0, S[0][ct]);
                S[1][ct] = mfma32h(kh, uh1, S[1][ct]);
                S[0][ct] = mfma32h(kh, ul0, S[0][ct]);
                S[1][ct] = mfma32h(kh, ul1, S[1][ct]);
            }
            // After the state update, so U and the outputs are dead while it runs (the other
            // workgroup on the CU fills the gaps).  Unconditional: past the last chunk every
            // row is padding and nothing it writes is read again.
            prep0(ck + 1);
        }
        if (ck + 2 < n_chunks) {
            issue(ck + 2, 0);
            issue(ck + 2, 1);
            issue(ck + 2, 2);
        }
        __syncthreads();
    }

    // ---- final state of this wave's tiles
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int col = 32 * w + 16 * m + li;
        float *fp = vf ? fin + col * DK + 8 * g : fin + 8 * g * DV + col;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int s = 0; s < 4; ++s) fp[(32 * (ct >> 1) + 4 * (ct & 1) + s) * rstride] = S[m][ct][s];
    }
    }  // units
}

}  // namespace fast32

hipError_t launch_fast32(const ChainArgs &a, hipStream_t stream) {
    const int n_units = a.n_items * a.H;
    const dim3 grid(8 * ((n_units + 7) / 8));
    hipLaunchKernelGGL(fast32::kda_fast32_kernel, grid, dim3(fast32::NT), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fast32_planned(const ChainArgs &a, int n_slots, hipStream_t stream) {
    // persistent: two workgroups per CU, drained queues end them
    const dim3 grid(8 * ((n_slots + 7) / 8));
    hipLaunchKernelGGL(fast32::kda_fast32_kernel, grid, dim3(fast32::NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kda
