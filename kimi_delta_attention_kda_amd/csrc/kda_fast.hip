// kda_fast.hip -- bf16 chunk-parallel KDA prefill for dk = dv in {64, 128} on gfx950 (MI355X).
//
// Same chunk algebra as the precise walk in kda_chain.hip (the token recurrence
// S_t = (I - b k k^T) Diag(alpha) S_{t-1} + b k v^T, o_t = scale q^T S_t of the
// nx_nofloat_kda.nx source rewritten over 64-token chunks), organised for throughput.
//
// Stable exponent differences.  Products e^{G_i - G_j} (j <= i, G the running sum of
// log alpha) never form e^{-G}: the chunk is cut into four 16-row blocks; row i of block
// I is scaled by e^{G_i - G_(16I-1)} <= 1, row j of block J by e^{G_(16J+15) - G_j} <= 1,
// and the remaining per-channel factor e^{G_(16I-1) - G_(16J+15)} is a product of
// whole-block decays (<= 1) for J < I, or the reciprocal of block I's decay for J = I.
// That reciprocal is <= e^{16 |bound|}, finite in fp32 and bf16 while 16 |bound| < 85:
// the reason this kernel takes the safe gate only (max.nn.state_space.kda_chunk: the
// gfx950 pipeline requires gate_mode "safe").  Every factor is a running product of
// alpha, so the gate's own three transcendentals are the only ones per element.
//
//
//  * one workgroup of dv/16 waves (8 at dv = 128, 4 at dv = 64) owns one (sequence, head)
//    and all value columns, so the dv-independent work of a chunk (gate, decay factors,
//    scores, inverses) is done once; each wave owns one 16-column tile of the fp32 state
//    (dk x 16, in MFMA accumulators) for the whole sequence;
//  * prep threads own 4 adjacent key channels x 4 rows of one 16-row block: the gate
//    pre-activations arrive as 16-byte loads, k/q/v as 8-byte loads, operand rows leave
//    as 8-byte LDS stores; decay factors are running products of alpha (no exp of
//    differences), completed across the four quarter blocks with quad lane broadcasts;
//  * decayed scores come from bf16 MFMAs on 16x16 blocks whose operands carry factors
//    <= 1, times one per-channel factor per block pair (above);
//  * (I + A) U = R is solved per wave by blocked forward substitution with fp16
//    16x16x16 MFMAs: 16x16 diagonal-block inverses (fp32 right-looking substitution,
//    once per chunk) and the right-hand side split into fp16 hi + lo;
//  * the state update uses fp16 Khat (|Khat| <= 1) against fp16 hi + lo U; products
//    with the state itself (Kg S, Qbar S) are bf16, whose range matches fp32;
//  * the key channels of the state are stored in a permuted row order inside its MFMA
//    tiles (key_row below), so that a lane's eight k slots of Kg S and Qbar S are eight
//    consecutive channels and each operand fragment is one 16-byte LDS read;
//  * global loads of chunk c+1 are issued before the scores of chunk c are built and
//    land in plain 32-bit registers, so nothing waits on them until chunk c+1.
#include "kda_common.h"
#include "kda_fast_common.h"
#include "kda_launch.h"

namespace kda {

namespace fast {

using namespace fk;

constexpr int PJ = 64 + 8;  // 16-bit element pitch of [*][64] arrays

// dk = dv = DKT in {64, 128}: DKT/16 waves, each owning 16 state columns.
template <int DKT>
struct Geo {
    static constexpr int DK = DKT, DV = DKT;
    static constexpr int NW = DV / 16;      // waves
    static constexpr int NT = 64 * NW;      // threads
    static constexpr int NCT = DK / 16;     // 16-row state tiles per wave
    static constexpr int NKB = DK / 32;     // 32-channel blocks of a score or Kg S product
    static constexpr int PK = DK + 8;       // 16-bit element pitch of [64][DK] arrays
};

template <int DKT, int MODE>
struct Lds {
    static constexpr int DK = DKT, DV = DKT, PK = Geo<DKT>::PK;
    static constexpr bool FW = MODE == MODE_FWD;
    static constexpr int ROWS = 64 * PK * 2;              // one [64][PK] 16-bit array
    static constexpr int KR = 0;                          // Kr            bf16, scores
    static constexpr int QR = KR + ROWS;                  // Qr (FWD)      bf16, scores
    static constexpr int KC = QR + (FW ? ROWS : 0);       // Kc            bf16, scores
    static constexpr int KG = KC + ROWS;                  // Kg            bf16, chain
    static constexpr int QB = KG + ROWS;                  // Qbar (FWD)    bf16, chain
    static constexpr int KH = QB + (FW ? ROWS : 0);       // Khat^T        f16 [DK][PJ]
    static constexpr int VT = KH + DK * PJ * 2;           // V^T           bf16 [DV][PJ]
    static constexpr int AO = VT + DV * PJ * 2;           // -A off-diag   f16 [64][PJ]
    static constexpr int P = AO + 64 * PJ * 2;            // P (FWD)       f16 [64][PJ]
    static constexpr int AD = P + (FW ? 64 * PJ * 2 : 0); // A diag blocks^T f32 [4][16][20]
    static constexpr int D = AD + 4 * 16 * 20 * 4;        // (I+A_II)^-1   f16 [4][16][24]
    static constexpr int BETA = D + 4 * 16 * 24 * 2;      // f32 [64]
    static constexpr int E = BETA + 64 * 4;               // block decays  f32 [4][DK]
    static constexpr int IE = E + 4 * DK * 4;             // 1/decays      f32 [4][DK]
    static constexpr int EG = IE + 4 * DK * 4;            // e^{G_last}    f32 [DK]
    static constexpr int BYTES = EG + DK * 4;
};

// Block pairs (I, J <= I) of the 4x4 grid of 16x16 score blocks handled by wave w in the
// score phase.  With 8 waves: waves 0-3 take the diagonal pair (w, w); waves 4..7 take
// the off-diagonal pairs {(1,0),(2,1)}, {(2,0),(3,2)}, {(3,0)}, {(3,1)}.  With 4 waves,
// wave w takes (w, w) and then the off-diagonal pairs of wave w + 4.  Arithmetic, so that
// no memory access (and no wait on the in-flight prefetch) is needed to find them.
__device__ __forceinline__ int n_offdiag(int v) { return (v == 4 || v == 5) ? 2 : 1; }
__device__ __forceinline__ void offdiag(int v, int pp, int &bI, int &bJ) {
    if (v == 4) { bI = 1 + pp; bJ = pp; return; }
    if (v == 5) { bI = 2 + pp; bJ = 2 * pp; return; }
    bI = 3;
    bJ = v - 6;
}
template <int NW>
__device__ __forceinline__ int n_pairs_of_wave(int w) {
    if constexpr (NW == 8) return w < 4 ? 1 : n_offdiag(w);
    else return 1 + n_offdiag(w + 4);
}
template <int NW>
__device__ __forceinline__ void pair_of_wave(int w, int pp, int &bI, int &bJ) {
    if constexpr (NW == 8) {
        if (w < 4) { bI = w; bJ = w; return; }
        offdiag(w, pp, bI, bJ);
    } else {
        if (pp == 0) { bI = w; bJ = w; return; }
        offdiag(w + 4, pp - 1, bI, bJ);
    }
}

// GQA: fewer key heads than value heads (a.Hk < a.H); q and k rows then have their own
// stride and head.  The equal-heads instantiation keeps one set of row offsets.
template <int DKT, int MODE, bool GQA>
__global__ __launch_bounds__(Geo<DKT>::NT, 1) void kda_fast_kernel(ChainArgs a) {
    using L = Lds<DKT, MODE>;
    using Gm = Geo<DKT>;
    constexpr int DK = Gm::DK, DV = Gm::DV, NW = Gm::NW, NT = Gm::NT, NCT = Gm::NCT, NKB = Gm::NKB;
    constexpr int PK = Gm::PK;
    constexpr bool FW = MODE == MODE_FWD;
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
    const int I = __builtin_amdgcn_readfirstlane(t / (NT / 4)), rq = t & 3, c0 = 4 * ((t >> 2) & (DK / 4 - 1));
    const int rbase = 16 * I + 4 * rq;
    const float amin = a.gate_mode == 1 ? expf(a.lb) : 0.f;  // alpha floor of the safe gate
    const int xcd = blockIdx.x & 7;  // workgroups are dealt to the 8 XCDs round-robin

    if (FW) {  // strictly-upper blocks of P are never written below
        for (int e = t; e < 64 * 64; e += NT) {
            const int i = e >> 6, j = e & 63;
            if ((j >> 4) > (i >> 4)) sP[i * PJ + j] = (f16_t)0.f;
        }
    }
    __shared__ int s_next;

    // One unit per pass: one (item, head) of the grid, or one queued unit of a plan.
    for (int pass = 0;; ++pass) {
        int t_begin, t_end, h;
        int init;      // 0: load the state from fin, 1: identity, 2: zero
        bool vf = false;  // fin is a pool slot stored [DV][DK]
        bool has_v;
        float *fin;    // [DK][DV] state of this unit: initial (init 0) and final
        bf16_t *obase = (bf16_t *)a.out;
        int64_t orow = 0;  // token of obase's row 0 (W rows of a later piece start at its own)
        if (!a.plan) {
            if (pass > 0) break;
            const int jx = blockIdx.x >> 3;
            const int slice = jx % a.n_slices;
            const int unit = (jx / a.n_slices) * 8 + xcd;
            if (unit >= a.n_items * H) break;
            const int item = unit / H;
            h = unit - item * H;
            t_begin = a.offsets[item];
            t_end = a.offsets[item + 1];
            if (FW) {
                fin = a.state_pool + ((int64_t)a.state_indices[item] * H + h) * DK * DV;
                init = 0;
                vf = a.v_first;
                has_v = true;
            } else {  // slice 0: transition columns M, slice 1: contribution columns U
                const bool isM = slice == 0;
                fin = (isM ? a.M : a.U) + ((int64_t)item * H + h) * DK * DV;
                init = isM ? 1 : 2;
                has_v = !isM;
            }
        } else {
            if (t == 0) s_next = atomicAdd((int *)&a.plan->ctr, 1);
            __syncthreads();
            // every value of the unit is wave-uniform: keep it in scalar registers
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
        if (FW && len <= 0) continue;
        const int hk = GQA ? h / (H / a.Hk) : h;  // key head of value head h
        const int n_chunks = len > 0 ? (len + 63) / 64 : 0;
        const float negA = -expf(a.a_log[h]);
        const f32x4 dtb = *(const f32x4 *)(a.dt_bias + h * DK + c0) * 1.44269504088896341f;

    // ---- state tile of wave w: rows 16ct+4g+s, column 16w + li
    // Lane (g, li) holds key rows key_row(ct, 4g + s) = 8g + (32(ct/2) + 4(ct%2) + s) of
    // column 16w + li: one lane pointer per unit plus row offsets times the row stride
    // (DV for [DK][DV] storage, 1 for a V_FIRST slot).
    f32x4 S[NCT];
    const float *sp = vf ? fin + (16 * w + li) * DK + 8 * g : fin + 8 * g * DV + 16 * w + li;
    const int rstride = vf ? 1 : DV;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int rr = 32 * (ct >> 1) + 4 * (ct & 1) + s;
            S[ct][s] = init == 0 ? sp[rr * rstride] : ((init == 1 && 8 * g + rr == 16 * w + li) ? 1.f : 0.f);
        }

    // ---- prefetch registers: 4 rows x 4 channels of raw/k/q/v, one beta logit
    f32x4 praw[4];
    bf16x4 pk[4], pq[4], pv[4];
    float pbl = 0.f;
    if (!has_v)
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[r] = bf16x4{};
    // Loads of chunk ck in six small groups (q = 0..5).  Issued a few at a time across
    // the previous chunk's compute, they never fill the memory request queue at once,
    // so the waves issuing them are not held up while every workgroup's loads drain.
    // Addresses: a scalar base per chunk (its first token, this head) plus 32-bit lane
    // offsets; the four row offsets of a chunk are formed once, at its first group.
    unsigned roff[4], roffk[4];  // roffk: q/k rows (GQA only)
    auto issue = [&](int ck, int q) {
        const int t0 = t_begin + ck * 64;
        const int64_t rb = (int64_t)t0 * H + h;
        const int64_t rbk = GQA ? (int64_t)t0 * a.Hk + hk : rb;
        if (q == 0) {
            const int n = min(64, t_end - t0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                roff[r] = (unsigned)(min(rbase + r, n - 1) * (H * DK) + c0);
                if constexpr (GQA) roffk[r] = (unsigned)(min(rbase + r, n - 1) * (a.Hk * DK) + c0);
            }
        }
        const unsigned *ko = GQA ? roffk : roff;
        const float *rg = a.raw_gate + rb * DK;
        const bf16_t *kp = (const bf16_t *)a.k + rbk * DK;
        const bf16_t *qp = (const bf16_t *)a.q + rbk * DK;
        const bf16_t *vp = (const bf16_t *)a.v + rb * DV;
        if (q == 0) {
            praw[0] = *(const f32x4 *)(rg + roff[0]);
            praw[1] = *(const f32x4 *)(rg + roff[1]);
        } else if (q == 1) {
            praw[2] = *(const f32x4 *)(rg + roff[2]);
            praw[3] = *(const f32x4 *)(rg + roff[3]);
            pbl = a.beta_logits[rb + (unsigned)(min(l, t_end - t0 - 1) * H)];
        } else if (q == 2) {
#pragma unroll
            for (int r = 0; r < 3; ++r) pk[r] = *(const bf16x4 *)(kp + ko[r]);
        } else if (q == 3) {
            pk[3] = *(const bf16x4 *)(kp + ko[3]);
            if (FW) {
                pq[0] = *(const bf16x4 *)(qp + ko[0]);
                pq[1] = *(const bf16x4 *)(qp + ko[1]);
            }
        } else if (q == 4) {
            if (FW) {
                pq[2] = *(const bf16x4 *)(qp + ko[2]);
                pq[3] = *(const bf16x4 *)(qp + ko[3]);
            }
            if (has_v) pv[0] = *(const bf16x4 *)(vp + roff[0]);
        } else {
            if (has_v)
#pragma unroll
                for (int r = 1; r < 4; ++r) pv[r] = *(const bf16x4 *)(vp + roff[r]);
        }
    };
    // ---- software pipeline over chunks: the gate and decay products of chunk c+1 (VALU
    // work, branch-free) are computed while the outputs and the state update of chunk c
    // (MFMA and LDS work) run.  They write only arrays that the rest of chunk c no longer
    // reads (Kr, Qr, Kc, block decays, V^T, beta).
    bf16x4 kr4[4], qr4[4];
    float kc[4][4];
    auto prep0 = [&](int ck) {
        const int n = min(64, t_end - (t_begin + ck * 64));
        {
            // Rows past the sequence end hold a copy of its last row: only their gate
            // (alpha = 1) and beta (0) are masked; with beta = 0 they add nothing to A, R, U
            // or the state, and their outputs are never stored.
            float al[4][4], kf[4][4], qf[4][4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float floor_r = rbase + r < n ? amin : 1.f;  // alpha <= 1: padded rows get 1
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    al[r][cc] = gate_alpha(praw[r][cc], dtb[cc], negA, floor_r);
                    kf[r][cc] = (float)pk[r][cc];
                    qf[r][cc] = FW ? (float)pq[r][cc] : 0.f;
                }
            }
            // products over this quarter block, then over the other quarters (quad lanes)
            f32x4 E, pre, suf;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                float p = 1.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) p *= al[r][cc];
                const float q0 = quad_bcast<0>(p), q1 = quad_bcast<1>(p);
                const float q2 = quad_bcast<2>(p), q3 = quad_bcast<3>(p);
                E[cc] = ((q0 * q1) * q2) * q3;  // same operation order in every lane
                // decay of the quarters before / after this lane's quarter (selects, no branches)
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
                    kr4[r][cc] = (bf16_t)(kf[r][cc] * rr);
                    qr4[r][cc] = (bf16_t)(qf[r][cc] * rr);
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
                *(bf16x4 *)(sKR + i * PK + c0) = kr4[r];
                if (FW) *(bf16x4 *)(sQR + i * PK + c0) = qr4[r];
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
            // every wave holds the 64 betas of the chunk (identical stores); the hardware
            // reciprocal, not an IEEE division, and selects rather than a branch
            const float sig = __builtin_amdgcn_rcpf(1.f + __expf(-pbl));
            sBeta[l] = l < n ? (a.beta_mode == 0 ? sig : pbl) : 0.f;
        }
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
        const int t0 = t_begin + ck * 64;
        const int n = min(64, t_end - t0);
        const bool more = ck + 1 < n_chunks;

        // ============ P1: cross-block factors, chain operands Kg, Qbar, Khat^T ============
        {
            f32x4 Ev[4];
#pragma unroll
            for (int J = 0; J < 4; ++J) Ev[J] = *(const f32x4 *)(sE + J * DK + c0);
            f32x4 pI = f32x4{1.f, 1.f, 1.f, 1.f}, qS = pI;
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                if (J < I) pI *= Ev[J];
                if (J > I) qS *= Ev[J];
            }
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
                if (FW) *(bf16x4 *)(sQB + i * PK + c0) = y;
            }
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                f16x4 h4;  // Khat_j = K_j e^{G_last - G_j}
#pragma unroll
                for (int r = 0; r < 4; ++r) h4[r] = (f16_t)(kc[r][cc] * qS[cc]);
                *(f16x4 *)(sKH + tile_row(c0 + cc) * PJ + rbase) = h4;
            }
            if (I == 0 && rq == 0) *(f32x4 *)(sEG + c0) = ((Ev[0] * Ev[1]) * Ev[2]) * Ev[3];
        }
        // (no barrier: Kg, Qbar, Khat^T and e^{G_last} are first read in the chain step)

        // next chunk's loads fly while this chunk is computed
        if (more) issue(ck + 1, 3);

        // ============ P2: decayed scores; diagonal waves also invert their block ============
        {
            const int np = n_pairs_of_wave<NW>(w);
            for (int pp = 0; pp < np; ++pp) {
                int bI, bJ;
                pair_of_wave<NW>(w, pp, bI, bJ);
                f32x4 accA = zero4(), accP = zero4();
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const int cc = 32 * kb + 8 * g;
                    const bf16x8 aK = *(const bf16x8 *)(sKR + (16 * bI + li) * PK + cc);
                    const bf16x8 kcv = *(const bf16x8 *)(sKC + (16 * bJ + li) * PK + cc);
                    // e^{G_(16I-1) - G_(16J+15)}: 1/E_I on the diagonal, else the product of
                    // the decays of the whole blocks strictly between J and I (at most two);
                    // adjacent blocks have none, factor 1 (the pair is wave-uniform)
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
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            bK[s] = (bf16_t)((float)kcv[s] * m0[s]);
                            bK[s + 4] = (bf16_t)((float)kcv[s + 4] * m1[s]);
                        }
                    }
                    accA = mfma(aK, bK, accA);
                    if (FW) accP = mfma(*(const bf16x8 *)(sQR + (16 * bI + li) * PK + cc), bK, accP);
                }
                f32x4 at;  // diagonal block, stored transposed: column li, rows 4g .. 4g+3
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int ri = 4 * g + s, i = 16 * bI + ri, j = 16 * bJ + li;
                    const float av = sBeta[i] * accA[s];
                    at[s] = (li < ri) ? av : 0.f;
                    if (bI != bJ) sAO[i * PJ + j] = (f16_t)(-av);
                    if (FW) sP[i * PJ + j] = (f16_t)((j <= i) ? accP[s] : 0.f);
                }
                if (bI == bJ) *(f32x4 *)(sAD + (bI * 16 + li) * 20 + 4 * g) = at;
            }
            if (more) issue(ck + 1, 4);
            if (w < 4) {
                // (I + A_ww)^-1 by right-looking substitution, column c = l/4 of the inverse
                // on the four lanes of a quad, lane quarter q = l%4 holding rows 4q .. 4q+3.
                // acc_r = sum_j A_rj x_j - delta_rc, so x_k = -acc_k once rows < k are folded
                // in; step k broadcasts acc_k across the quad and folds x_k into every row
                // (rows <= k have A_rk = 0).  A is stored transposed: row k of sAD holds
                // column k, so a lane reads its four A_rk at once.
                const int c = l >> 2, q = l & 3;
                const float *At = sAD + w * 16 * 20;
                float acc[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = (4 * q + j == c) ? -1.f : 0.f;
                inv_step<0>(acc, At, q);
#pragma unroll
                for (int j = 0; j < 4; ++j) sD[(w * 16 + 4 * q + j) * 24 + c] = (f16_t)(0.f - acc[j]);
            }
        }
        if (more) issue(ck + 1, 5);
        __syncthreads();

        // ============ chain step, first half: Y = Kg S, Z = S^T Qbar^T, R, forward substitution ============
        f32x4 Z[4];
        f16x4 Uh[4], Ul[4];
        float usc, iusc;  // power-of-two scale of this wave's U and its inverse
        {
            bf16x8 Sb[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) Sb[kb] = cat(bf4(S[2 * kb]), bf4(S[2 * kb + 1]));
            f32x4 Y[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                Y[rt] = zero4();
                Z[rt] = zero4();
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    Y[rt] = mfma(*(const bf16x8 *)(sKG + (16 * rt + li) * PK + 32 * kb + 8 * g), Sb[kb], Y[rt]);
                    // output transposed, O^T = S^T Qbar^T: the state tile is the A operand
                    if (FW)
                        Z[rt] = mfma(Sb[kb], *(const bf16x8 *)(sQB + (16 * rt + li) * PK + 32 * kb + 8 * g), Z[rt]);
                }
            }
            // The rounding of S to bf16 in the prediction Kg S is forgotten with the state
            // when the chunk decays it, but accumulates to ~1e-3 of the state where a key
            // channel barely decays.  Chunks in which some channel keeps more than 1/16 of
            // its state over the chunk add the product with the rounding residual of S.
            if (wave_max_nonneg(DK == 128 ? fmaxf(sEG[l], sEG[l + 64]) : sEG[l]) > 0x1p-4f) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const bf16x8 sh = Sb[kb];
                    const bf16x8 sl = cat(bf4(S[2 * kb] - f4(bf16x4{sh[0], sh[1], sh[2], sh[3]})),
                                          bf4(S[2 * kb + 1] - f4(bf16x4{sh[4], sh[5], sh[6], sh[7]})));
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt)
                        Y[rt] = mfma(*(const bf16x8 *)(sKG + (16 * rt + li) * PK + 32 * kb + 8 * g), sl, Y[rt]);
                }
            }
            // R = beta (V - Kg S); solve (I + A) U = R block by block
            const int vcol = 16 * w + li;
            float rmax = 0.f;
#pragma unroll
            for (int bI = 0; bI < 4; ++bI) {
                const f32x4 vv = f4(*(const bf16x4 *)(sVT + vcol * PJ + 16 * bI + 4 * g));
                const f32x4 bb = *(const f32x4 *)(sBeta + 16 * bI + 4 * g);
                Y[bI] = bb * (vv - Y[bI]);
                rmax = fmaxf(rmax, fmaxf(fmaxf(fabsf(Y[bI][0]), fabsf(Y[bI][1])), fmaxf(fabsf(Y[bI][2]), fabsf(Y[bI][3]))));
            }
            // U is carried as fp16 hi + lo, exact to ~2^-22 of its largest entry only while
            // that entry is near 1, and finite only below 65504: a wave whose R is small
            // (tiny beta and a vanished state) or large (large values or states) scales R,
            // hence U, by a power of two, undone exactly in the output scale and the state
            // update below.
            rmax = wave_max_nonneg(rmax);
            if ((rmax < 0x1p-8f && rmax > 0.f) || (rmax >= 0x1p6f && rmax < 0x1p127f)) {
                // 2^k with rmax 2^k in [1/4, 1/2)
                const int k = max(-126, min(64, -2 - ((int)(__builtin_bit_cast(unsigned, rmax) >> 23) - 127)));
                usc = __builtin_bit_cast(float, (k + 127) << 23);
                iusc = __builtin_bit_cast(float, (127 - k) << 23);
#pragma unroll
                for (int bI = 0; bI < 4; ++bI) Y[bI] *= usc;
            } else {
                usc = 1.f;
                iusc = 1.f;
            }
#pragma unroll
            for (int bI = 0; bI < 4; ++bI) {
                f32x4 acc = Y[bI];
#pragma unroll
                for (int bJ = 0; bJ < bI; ++bJ) {
                    const f16x4 ao = *(const f16x4 *)(sAO + (16 * bI + li) * PJ + 16 * bJ + 4 * g);
                    acc = mfma16h(ao, Uh[bJ], acc);
                    acc = mfma16h(ao, Ul[bJ], acc);
                }
                f16x4 wh, wl;
                split_h(acc, wh, wl);
                const f16x4 dd = *(const f16x4 *)(sD + (bI * 16 + li) * 24 + 4 * g);
                f32x4 u = mfma16h(dd, wh, zero4());
                u = mfma16h(dd, wl, u);
                split_h(u, Uh[bI], Ul[bI]);
            }
        }
        __syncthreads();

        // ============ chain step, second half: outputs and state update of chunk ck,
        // interleaved with the gate and decay products of chunk ck + 1 ============
        {
            if (FW) {
                if (usc != 1.f)
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) Z[rt] *= usc;
                const float osc = a.scale * iusc;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    // O^T += U^T P^T
#pragma unroll
                    for (int jb = 0; jb <= (rt >> 1); ++jb)
                        Z[rt] = mfma32h(cath(Uh[2 * jb], Uh[2 * jb + 1]),
                                        fragA_perm_h(sP, PJ, 16 * rt + li, 32 * jb, g), Z[rt]);
                    // lane holds O[token 16rt + li][columns 16w + 4g .. +3]: one 8-byte store
                    const int i = 16 * rt + li;
                    if (i < n)
                        *(bf16x4 *)(obase + ((t0 - orow) * H + h) * DV + (unsigned)(i * (H * DV) + 16 * w + 4 * g)) =
                            bf4(osc * Z[rt]);
                }
            }
            // unconditional, so that it shares a basic block with the state update: past the
            // last chunk every row is padding and nothing it writes is read again
            prep0(ck + 1);
            // S <- Diag(e^{G_last}) S + Khat^T U
            if (usc != 1.f)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) S[ct] *= usc;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                S[ct] *= *(const f32x4 *)(sEG + key_row(ct, 4 * g));
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    const f16x8 kh = fragA_perm_h(sKH, PJ, 16 * ct + li, 32 * jb, g);
                    S[ct] = mfma32h(kh, cath(Uh[2 * jb], Uh[2 * jb + 1]), S[ct]);
                    S[ct] = mfma32h(kh, cath(Ul[2 * jb], Ul[2 * jb + 1]), S[ct]);
                }
            }
            if (usc != 1.f)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) S[ct] *= iusc;
        }
        if (ck + 2 < n_chunks) {
            issue(ck + 2, 0);
            issue(ck + 2, 1);
            issue(ck + 2, 2);
        }
        __syncthreads();
    }

    // ---- final state of this tile
    {
        float *fp = vf ? fin + (16 * w + li) * DK + 8 * g : fin + 8 * g * DV + 16 * w + li;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int s = 0; s < 4; ++s) fp[(32 * (ct >> 1) + 4 * (ct & 1) + s) * rstride] = S[ct][s];
    }
    }  // units
}

}  // namespace fast

namespace {
template <int DKT, bool GQA>
void launch_fast_dk_g(const ChainArgs &a, int mode, dim3 grid, hipStream_t stream) {
    const dim3 block(fast::Geo<DKT>::NT);
    if (mode == MODE_FWD)
        hipLaunchKernelGGL((fast::kda_fast_kernel<DKT, MODE_FWD, GQA>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((fast::kda_fast_kernel<DKT, MODE_SUMMARY, GQA>), grid, block, 0, stream, a);
}
template <int DKT>
void launch_fast_dk(const ChainArgs &a, int mode, dim3 grid, hipStream_t stream) {
    if (a.Hk != a.H)
        launch_fast_dk_g<DKT, true>(a, mode, grid, stream);
    else
        launch_fast_dk_g<DKT, false>(a, mode, grid, stream);
}
}  // namespace

hipError_t launch_fast(const ChainArgs &a, int dk, int mode, hipStream_t stream) {
    const int n_units = a.n_items * a.H;
    const dim3 grid(8 * a.n_slices * ((n_units + 7) / 8));
    if (dk == 128 && mode == MODE_FWD)
        return launch_pipe(a, grid, stream);
    if (dk == 128)
        launch_fast_dk<128>(a, mode, grid, stream);
    else if (dk == 64)
        launch_fast_dk<64>(a, mode, grid, stream);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_fast_planned(const ChainArgs &a, int dk, int n_cu, hipStream_t stream) {
    // persistent: one workgroup per CU (LDS allows no second one), drained queues end it
    const dim3 grid(8 * ((n_cu + 7) / 8));
    if (dk == 128)
        return launch_pipe(a, grid, stream);
    else if (dk == 64)
        launch_fast_dk<64>(a, MODE_FWD, grid, stream);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace kda
