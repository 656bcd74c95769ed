// kda_fast.hip -- bf16 chunk-parallel KDA prefill for dk = dv = 128 on gfx950 (MI355X).
//
// Same chunk algebra as the chunk walk in kda_chain.hip (the token recurrence
// S_t = (I - b k k^T) Diag(alpha) S_{t-1} + b k v^T, o_t = scale q^T S_t of the
// nx_nofloat_kda.nx source rewritten over 64-token chunks), organised for throughput:
//
//  * one workgroup of 8 waves owns one (sequence, head) and all 128 value columns, so
//    the dv-independent work of a chunk (gate, decay factors, scores, inverses) is done
//    once; each wave owns one 16-column tile of the fp32 state (128 x 16, in MFMA
//    accumulators) for the whole sequence;
//  * the gate is computed by one thread per (16-row block, key channel); decay factors
//    are running products of alpha along the block (no exp of differences at all);
//  * decayed scores come from bf16 MFMAs on 16x16 blocks whose operands carry factors
//    <= 1, plus one precomputed per-channel factor per block pair (see kda_chain.hip);
//  * the unit lower-triangular system (I + A) U = R is solved per wave by blocked
//    forward substitution: 16x16 diagonal-block inverses (fp32 substitution, once per
//    chunk) and 16x16x16 bf16 MFMAs with the right-hand side split hi+lo;
//  * global loads of chunk c+1 are issued before the scores of chunk c are built, so
//    their latency hides behind the chunk's compute.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

namespace fast {

constexpr int NT = 512;  // 8 waves
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int PK = DK + 8;  // bf16 pitch of [64][DK] arrays
constexpr int PJ = 64 + 8;  // bf16 pitch of [*][64] arrays

template <int MODE>
struct Lds {
    static constexpr bool FW = MODE == MODE_FWD;
    static constexpr int KR = 0;                          // Kr, then Kg           bf16 [64][PK]
    static constexpr int QR = KR + 64 * PK * 2;           // Qr, then Qbar (FWD)   bf16 [64][PK]
    static constexpr int KC = QR + (FW ? 64 * PK * 2 : 0);// Kc                   bf16 [64][PK]
    static constexpr int KHH = KC + 64 * PK * 2;          // Khat^T hi            bf16 [DK][PJ]
    static constexpr int KHL = KHH + DK * PJ * 2;         // Khat^T lo
    static constexpr int VT = KHL + DK * PJ * 2;          // V^T                   bf16 [DV][PJ]
    static constexpr int AO = VT + DV * PJ * 2;           // -A, off-diagonal blocks bf16 [64][PJ]
    static constexpr int P = AO + 64 * PJ * 2;            // P (FWD)               bf16 [64][PJ]
    static constexpr int AD = P + (FW ? 64 * PJ * 2 : 0); // A, diagonal blocks    f32 [4][16][17]
    static constexpr int D = AD + 4 * 16 * 17 * 4;        // (I + A_II)^-1         bf16 [4][16][24]
    static constexpr int BETA = D + 4 * 16 * 24 * 2;      // f32 [64]
    static constexpr int E = BETA + 64 * 4;               // block decays          f32 [4][DK]
    static constexpr int MF = E + 4 * DK * 4;             // pair factors          f32 [10][DK]
    static constexpr int EG = MF + 10 * DK * 4;           // e^{G_last}            f32 [DK]
    static constexpr int BYTES = EG + DK * 4;
};

__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 fragA_perm(const bf16_t *base, int pitch, int row, int k0, int g) {
    const bf16_t *p = base + row * pitch + k0 + 4 * g;
    return cat(*(const bf16x4 *)p, *(const bf16x4 *)(p + 16));
}

__device__ __forceinline__ float gate_alpha(float raw, float dtb, float Ah, int safe, float lb) {
    float la = -Ah * softplus_f(raw + dtb);
    if (safe) la = fmaxf(la, lb);
    return __expf(la);
}

// block pairs (I, J<=I): diagonal pairs 0..3, then the off-diagonal ones
__device__ __constant__ int kPairI[10] = {0, 1, 2, 3, 1, 2, 2, 3, 3, 3};
__device__ __constant__ int kPairJ[10] = {0, 1, 2, 3, 0, 0, 1, 0, 1, 2};

template <int MODE>
__global__ __launch_bounds__(NT, 1) void kda_fast_kernel(ChainArgs a) {
    using L = Lds<MODE>;
    constexpr bool FW = MODE == MODE_FWD;
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    bf16_t *sKR = (bf16_t *)(smem + L::KR);
    bf16_t *sQR = (bf16_t *)(smem + L::QR);
    bf16_t *sKC = (bf16_t *)(smem + L::KC);
    bf16_t *sKHH = (bf16_t *)(smem + L::KHH);
    bf16_t *sKHL = (bf16_t *)(smem + L::KHL);
    bf16_t *sVT = (bf16_t *)(smem + L::VT);
    bf16_t *sAO = (bf16_t *)(smem + L::AO);
    bf16_t *sP = (bf16_t *)(smem + L::P);
    float *sAD = (float *)(smem + L::AD);
    bf16_t *sD = (bf16_t *)(smem + L::D);
    float *sBeta = (float *)(smem + L::BETA);
    float *sE = (float *)(smem + L::E);
    float *sMF = (float *)(smem + L::MF);
    float *sEG = (float *)(smem + L::EG);

    // ---- work item (XCD-aware: the slices of one (item, head) share an XCD)
    const int H = a.H;
    const int n_units = a.n_items * H;
    const int lin = blockIdx.x;
    const int xcd = lin & 7, jx = lin >> 3;
    const int slice = jx % a.n_slices;
    const int unit = (jx / a.n_slices) * 8 + xcd;
    if (unit >= n_units) return;
    const int item = unit / H, h = unit - item * H;
    const int t_begin = a.offsets[item], t_end = a.offsets[item + 1];
    const int len = t_end - t_begin;
    if (FW && len <= 0) return;
    const int n_chunks = len > 0 ? (len + 63) / 64 : 0;
    const int aug0 = slice * 128;
    const bool isM = (!FW) && aug0 < DK;
    const int col0 = (FW || isM) ? aug0 : aug0 - DK;
    const bool has_v = FW || !isM;

    const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 4, li = l & 15;
    const int I = t >> 7, c = t & 127;   // prep role: 16-row block I, key channel c (value column c for V)
    const int safe = a.gate_mode == 1;
    const float lb = a.lb;
    const float Ah = expf(a.a_log[h]);
    const float dtb = a.dt_bias[h * DK + c];

    // ---- state tile of wave w: rows 16ct+4g+s, column col0 + 16w + li
    f32x4 S[8];
    int slot = 0;
    if (FW) slot = a.state_indices[item];
    {
        const int col = col0 + 16 * w + li;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int r = 16 * ct + 4 * g + s;
                S[ct][s] = FW ? a.state_pool[(((int64_t)slot * H + h) * DK + r) * DV + col]
                              : ((isM && r == col) ? 1.f : 0.f);
            }
    }
    if (FW) {  // strictly-upper blocks of P are never written below
        for (int e = t; e < 64 * 64; e += NT) {
            const int i = e >> 6, j = e & 63;
            if ((j >> 4) > (i >> 4)) sP[i * PJ + j] = (bf16_t)0.f;
        }
    }

    const bf16_t *kb16 = (const bf16_t *)a.k;
    const bf16_t *qb16 = (const bf16_t *)a.q;
    const bf16_t *vb16 = (const bf16_t *)a.v;

    // ---- prefetch registers: this thread's 16 rows of raw/k/q/v and one beta logit
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    float praw[16];
    bf16x2 pk[8], pq[8], pv[8];  // two rows per register
    float pbl = 0.f;
    auto issue = [&](int ck) {
        const int t0 = t_begin + ck * 64;
        const int n = min(64, t_end - t0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = t0 + min(16 * I + r, n - 1);
            const int64_t base = ((int64_t)row * H + h) * DK + c;
            praw[r] = a.raw_gate[base];
            pk[r >> 1][r & 1] = kb16[base];
            if (FW) pq[r >> 1][r & 1] = qb16[base];
            if (has_v) pv[r >> 1][r & 1] = vb16[((int64_t)row * H + h) * DV + col0 + c];
        }
        if (t < 64) pbl = a.beta_logits[(int64_t)(t0 + min(t, n - 1)) * H + h];
    };
    if (n_chunks > 0) issue(0);

    for (int ck = 0; ck < n_chunks; ++ck) {
        const int t0 = t_begin + ck * 64;
        const int n = min(64, t_end - t0);

        // ============ P0: gate, in-block running products, operand rows ============
        float kc[16];
        {
            float al[16], kf[16], qf[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const bool valid = 16 * I + r < n;
                al[r] = valid ? gate_alpha(praw[r], dtb, Ah, safe, lb) : 1.f;
                kf[r] = valid ? (float)pk[r >> 1][r & 1] : 0.f;
                qf[r] = (FW && valid) ? (float)pq[r >> 1][r & 1] : 0.f;
            }
            float rr = 1.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {  // Kr_i = K_i e^{G_i - G_(16I-1)}
                rr *= al[r];
                const int i = 16 * I + r;
                sKR[i * PK + c] = (bf16_t)(kf[r] * rr);
                if (FW) sQR[i * PK + c] = (bf16_t)(qf[r] * rr);
            }
            sE[I * DK + c] = rr;
            float cb = 1.f;
#pragma unroll
            for (int r = 15; r >= 0; --r) {  // Kc_j = K_j e^{G_(16I+15) - G_j}
                kc[r] = kf[r] * cb;
                sKC[(16 * I + r) * PK + c] = (bf16_t)kc[r];
                cb *= al[r];
            }
            bf16x8 v0, v1;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const bf16_t x = (has_v && 16 * I + r < n) ? pv[r >> 1][r & 1] : (bf16_t)0.f;
                if (r < 8) v0[r] = x; else v1[r - 8] = x;
            }
            *(bf16x8 *)(sVT + c * PJ + 16 * I) = v0;
            *(bf16x8 *)(sVT + c * PJ + 16 * I + 8) = v1;
            if (t < 64) sBeta[t] = (t < n) ? (a.beta_mode == 0 ? 1.f / (1.f + __expf(-pbl)) : pbl) : 0.f;
        }
        __syncthreads();

        // ============ P1: cross-block factors, Khat^T, pair factors ============
        float pI = 1.f;
        {
            float Ev[4];
#pragma unroll
            for (int J = 0; J < 4; ++J) Ev[J] = sE[J * DK + c];
            float qS = 1.f;
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                if (J < I) pI *= Ev[J];
                if (J > I) qS *= Ev[J];
            }
            bf16x8 hh[2], hl[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float kh = kc[r] * qS;  // Khat_j = K_j e^{G_last - G_j}
                const bf16_t hb = (bf16_t)kh;
                hh[r >> 3][r & 7] = hb;
                hl[r >> 3][r & 7] = (bf16_t)(kh - (float)hb);
            }
            *(bf16x8 *)(sKHH + c * PJ + 16 * I) = hh[0];
            *(bf16x8 *)(sKHH + c * PJ + 16 * I + 8) = hh[1];
            *(bf16x8 *)(sKHL + c * PJ + 16 * I) = hl[0];
            *(bf16x8 *)(sKHL + c * PJ + 16 * I + 8) = hl[1];
            if (I == 0) {
                sEG[c] = Ev[0] * Ev[1] * Ev[2] * Ev[3];
            } else if (I == 1) {
                // factor e^{G_(16I-1) - G_(16J+15)}: 1/E_I on the diagonal, else the
                // product of the whole blocks strictly between J and I
#pragma unroll
                for (int p = 0; p < 10; ++p) {
                    const int bI = kPairI[p], bJ = kPairJ[p];
                    float f;
                    if (bI == bJ) {
                        f = 1.f / Ev[bI];
                    } else {
                        f = 1.f;
#pragma unroll
                        for (int K = 0; K < 4; ++K)
                            if (K > bJ && K < bI) f *= Ev[K];
                    }
                    sMF[p * DK + c] = f;
                }
            }
        }
        __syncthreads();

        // next chunk's loads fly while this chunk is computed
        if (ck + 1 < n_chunks) issue(ck + 1);

        // ============ P2: decayed scores; diagonal waves also invert their block ============
        {
            const int np = w < 4 ? 1 : (w < 6 ? 2 : 1);
            const int p0 = w < 4 ? w : (w == 4 ? 4 : (w == 5 ? 5 : w + 2));
            // waves 4,5 take pairs (4,6),(5,7); waves 6,7 take pairs 8,9
            for (int pp = 0; pp < np; ++pp) {
                const int p = p0 + 2 * pp;
                const int bI = kPairI[p], bJ = kPairJ[p];
                f32x4 accA = zero4(), accP = zero4();
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const int cc = 32 * kb + 8 * g;
                    const bf16x8 aK = *(const bf16x8 *)(sKR + (16 * bI + li) * PK + cc);
                    const bf16x8 kcv = *(const bf16x8 *)(sKC + (16 * bJ + li) * PK + cc);
                    const f32x4 m0 = *(const f32x4 *)(sMF + p * DK + cc);
                    const f32x4 m1 = *(const f32x4 *)(sMF + p * DK + cc + 4);
                    bf16x8 bK;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        bK[s] = (bf16_t)((float)kcv[s] * m0[s]);
                        bK[s + 4] = (bf16_t)((float)kcv[s + 4] * m1[s]);
                    }
                    accA = mfma(aK, bK, accA);
                    if (FW) {
                        const bf16x8 aQ = *(const bf16x8 *)(sQR + (16 * bI + li) * PK + cc);
                        accP = mfma(aQ, bK, accP);
                    }
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int ri = 4 * g + s, i = 16 * bI + ri, j = 16 * bJ + li;
                    const float av = sBeta[i] * accA[s];
                    if (bI == bJ)
                        sAD[(bI * 16 + ri) * 17 + li] = (li < ri) ? av : 0.f;
                    else
                        sAO[i * PJ + j] = (bf16_t)(-av);
                    if (FW) sP[i * PJ + j] = (bf16_t)((j <= i) ? accP[s] : 0.f);
                }
            }
            if (w < 4 && l < 16) {
                // (I + A_ww)^-1 by forward substitution, one column per lane
                const int col = l;
                const float *Ab = sAD + w * 16 * 17;
                float x[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] = (r == col) ? 1.f : 0.f;
#pragma unroll
                for (int r = 1; r < 16; ++r) {
                    float s = 0.f;
#pragma unroll
                    for (int kk = 0; kk < r; ++kk) s += (kk >= col) ? Ab[r * 17 + kk] * x[kk] : 0.f;
                    if (r > col) x[r] = -s;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) sD[(w * 16 + r) * 24 + col] = (bf16_t)x[r];
            }
        }
        __syncthreads();

        // ============ P3: Kg = Kr e^{G_(16I-1)} and Qbar = Qr e^{G_(16I-1)} in place ============
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 16 * I + r;
            sKR[i * PK + c] = (bf16_t)((float)sKR[i * PK + c] * pI);
            if (FW) sQR[i * PK + c] = (bf16_t)((float)sQR[i * PK + c] * pI);
        }
        __syncthreads();

        // ============ P4: chain step of value tile w ============
        {
            bf16x8 Sb[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) Sb[kb] = cat(bf4(S[2 * kb]), bf4(S[2 * kb + 1]));
            f32x4 Y[4], Z[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                Y[rt] = zero4();
                Z[rt] = zero4();
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    Y[rt] = mfma(fragA_perm(sKR, PK, 16 * rt + li, 32 * kb, g), Sb[kb], Y[rt]);
                    if (FW) Z[rt] = mfma(fragA_perm(sQR, PK, 16 * rt + li, 32 * kb, g), Sb[kb], Z[rt]);
                }
            }
            // R = beta (V - Kg S); solve (I + A) U = R block by block
            const int vcol = 16 * w + li;
            bf16x4 Uh[4], Ul[4];
#pragma unroll
            for (int bI = 0; bI < 4; ++bI) {
                const f32x4 vv = f4(*(const bf16x4 *)(sVT + vcol * PJ + 16 * bI + 4 * g));
                const f32x4 bb = *(const f32x4 *)(sBeta + 16 * bI + 4 * g);
                f32x4 acc = bb * (vv - Y[bI]);
#pragma unroll
                for (int bJ = 0; bJ < bI; ++bJ) {
                    const bf16x4 ao = *(const bf16x4 *)(sAO + (16 * bI + li) * PJ + 16 * bJ + 4 * g);
                    acc = mfma16(ao, Uh[bJ], acc);
                    acc = mfma16(ao, Ul[bJ], acc);
                }
                bf16x4 wh, wl;
                split4(acc, wh, wl);
                const bf16x4 dd = *(const bf16x4 *)(sD + (bI * 16 + li) * 24 + 4 * g);
                f32x4 u = mfma16(dd, wh, zero4());
                u = mfma16(dd, wl, u);
                split4(u, Uh[bI], Ul[bI]);
            }
            if (FW) {
                bf16_t *outp = (bf16_t *)a.out;
                const int col = col0 + vcol;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
                    for (int jb = 0; jb <= (rt >> 1); ++jb)
                        Z[rt] = mfma(fragA_perm(sP, PJ, 16 * rt + li, 32 * jb, g), cat(Uh[2 * jb], Uh[2 * jb + 1]),
                                     Z[rt]);
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int i = 16 * rt + 4 * g + s;
                        if (i < n) outp[((int64_t)(t0 + i) * H + h) * DV + col] = (bf16_t)(a.scale * Z[rt][s]);
                    }
                }
            }
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                S[ct] *= *(const f32x4 *)(sEG + 16 * ct + 4 * g);
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    const bf16x8 ah = fragA_perm(sKHH, PJ, 16 * ct + li, 32 * jb, g);
                    const bf16x8 alo = fragA_perm(sKHL, PJ, 16 * ct + li, 32 * jb, g);
                    const bf16x8 bh = cat(Uh[2 * jb], Uh[2 * jb + 1]);
                    const bf16x8 bl = cat(Ul[2 * jb], Ul[2 * jb + 1]);
                    S[ct] = mfma(ah, bh, S[ct]);
                    S[ct] = mfma(ah, bl, S[ct]);
                    S[ct] = mfma(alo, bh, S[ct]);
                }
            }
        }
        __syncthreads();
    }

    // ---- final state of this tile
    {
        const int col = col0 + 16 * w + li;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int r = 16 * ct + 4 * g + s;
                if (FW)
                    a.state_pool[(((int64_t)slot * H + h) * DK + r) * DV + col] = S[ct][s];
                else if (isM)
                    a.M[(((int64_t)item * H + h) * DK + r) * DK + col] = S[ct][s];
                else
                    a.U[(((int64_t)item * H + h) * DK + r) * DV + col] = S[ct][s];
            }
    }
}

}  // namespace fast

hipError_t launch_fast(const ChainArgs &a, int mode, hipStream_t stream) {
    const int n_units = a.n_items * a.H;
    const dim3 grid(8 * a.n_slices * ((n_units + 7) / 8));
    if (mode == MODE_FWD)
        hipLaunchKernelGGL(fast::kda_fast_kernel<MODE_FWD>, grid, dim3(fast::NT), 0, stream, a);
    else
        hipLaunchKernelGGL(fast::kda_fast_kernel<MODE_SUMMARY>, grid, dim3(fast::NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kda
