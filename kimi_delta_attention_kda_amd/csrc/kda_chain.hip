// kda_chain.hip -- chunk-parallel KDA prefill and segment summaries for gfx950 (MI355X).
//
// One workgroup (4 waves) owns one (sequence-or-segment, head, value slice) and walks its
// 64-token chunks in order.  For each chunk it
//   1. computes the gate (log alpha = -exp(a_log) softplus(raw + dt_bias), optionally
//      clamped from below) and beta, and the decay factors of the chunk;
//   2. builds the decayed key-key scores A (strictly lower) and query-key scores P (lower);
//   3. inverts the unit lower-triangular I + A in LDS;
//   4. with the fp32 state slice S [dk, 16-column tiles] resident in MFMA accumulators:
//        U  = (I + A)^-1 Diag(beta) (V - (K o e^G) S)
//        O  = scale ((Q o e^G) S + P U)
//        S <- Diag(e^{G_last}) S + (K o e^{G_last - G})^T U
// where G is the running sum of log alpha from the chunk start.  This is the token
// recurrence S_t = (I - b k k^T) Diag(alpha) S_{t-1} + b k v^T, o_t = scale q^T S_t
// (nx_nofloat_kda.nx source: kda_gate, kda_write, kda_forward) rewritten over a chunk;
// the chunked method's ingredients -- prefix scan of log gates, triangular inverse,
// stable decayed scores -- are those named by "GStar Assignment 2: Build Kimi Delta
// Attention", Learning path (P4, P6, P8, P9).
//
// Stable exponent differences.  Products e^{G_i - G_j} (j <= i) never form e^{-G}: the
// chunk is cut into four 16-row blocks; row i of block I is scaled by
// e^{G_i - G_(16I-1)} <= 1, row j of block J by e^{G_(16J+15) - G_j} <= 1, and the
// remaining per-channel factor e^{G_(16I-1) - G_(16J+15)} is a product of whole-block
// decays (<= 1) for J < I, or the reciprocal of block I's decay for J = I.  That
// reciprocal is <= e^{16 |bound|}, finite in fp32/bf16 when the safe-gate bound
// satisfies 16 |bound| < 85 -- the reason this fast path requires the safe gate
// (max.nn.state_space.kda_chunk: the AMD gfx950 pipeline requires gate_mode "safe").
// All factors are running products of alpha, so the only transcendentals per element
// are the three of the gate itself.
//
// Two arithmetic variants share the chunk walk:
//   FAST    (bf16 q/k/v, safe gate): bf16 MFMA operands prepared once per chunk in LDS;
//           the right-hand side of U = T R and both operands of K^T U are split into
//           bf16 hi+lo pairs, which keeps the fp32 state within ~1e-5 of fp64.
//   PRECISE (fp32 q/k/v, either gate): operands formed on the fly from fp32 K, Q and G
//           with direct exp of non-positive differences; every MFMA product is split
//           three ways (hi*hi + hi*lo + lo*hi); the diagonal blocks need no factoring.
// Segment summaries run the same walk on the augmented state X = [M | U] with
// X_0 = [I | 0] and value rows [0 | V] (KDA Context Parallelism, "Theory").
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

constexpr int CH = 64;   // tokens per chunk
constexpr int NT = 256;  // threads per workgroup (4 waves of 64)

template <int DK, int DVS, bool PRECISE, int MODE>
struct Lds {
    static constexpr bool FW = (MODE == MODE_FWD);
    static constexpr int PK = DK + 8;    // bf16 pitch, [64][DK]
    static constexpr int PJ = 64 + 8;    // bf16 pitch, [*][64]
    static constexpr int PF = 64 + 4;    // fp32 pitch, [*][64]
    static constexpr int PKF = DK + 4;   // fp32 pitch, [64][DK]
    static constexpr int cmax(int a, int b) { return a > b ? a : b; }

    // ---- FAST layout
    static constexpr int F_KR = 0;                                   // Kr -> Kg (bf16)
    static constexpr int F_QR = F_KR + 64 * PK * 2;                  // Qr -> Qbar (bf16)
    static constexpr int F_KC = F_QR + (FW ? 64 * PK * 2 : 0);       // Kc (bf16) -> T scratch (f32)
    static constexpr int F_KHH = F_KC + cmax(64 * PK * 2, 64 * PF * 4);  // Khat^T hi [DK][64]
    static constexpr int F_KHL = F_KHH + DK * PJ * 2;                // Khat^T lo
    static constexpr int F_A = F_KHL + DK * PJ * 2;                  // A (f32)
    static constexpr int F_P = F_A + 64 * PF * 4;                    // P (bf16)
    static constexpr int F_T = F_P + (FW ? 64 * PJ * 2 : 0);         // T = (I+A)^-1, bf16 hi
    static constexpr int F_TL = F_T + 64 * PJ * 2;                   // and lo
    static constexpr int F_VT = F_TL + 64 * PJ * 2;                  // V^T slice (bf16)
    static constexpr int F_BETA = F_VT + DVS * PJ * 2;
    static constexpr int F_E = F_BETA + 64 * 4;                      // block decays [4][DK]
    static constexpr int F_PI = F_E + 4 * DK * 4;                    // e^{G_(16I-1)} [4][DK]
    static constexpr int F_EG = F_PI + 4 * DK * 4;                   // e^{G_last} [DK]
    static constexpr int F_X = F_EG + DK * 4;                        // inverse scratch [3][16][17]
    static constexpr int F_BYTES = F_X + 3 * 16 * 17 * 4;

    // ---- PRECISE layout
    static constexpr int P_K = 0;                                    // K (f32)
    static constexpr int P_Q = P_K + 64 * PKF * 4;                   // Q (f32)
    static constexpr int P_G = P_Q + (FW ? 64 * PKF * 4 : 0);        // G (f32)
    static constexpr int P_A = P_G + 64 * PKF * 4;
    static constexpr int P_P = P_A + 64 * PF * 4;
    static constexpr int P_T = P_P + (FW ? 64 * PF * 4 : 0);
    static constexpr int P_VT = P_T + 64 * PF * 4;
    static constexpr int P_BETA = P_VT + DVS * PF * 4;
    static constexpr int P_EG = P_BETA + 64 * 4;
    static constexpr int P_X = P_EG + DK * 4;
    static constexpr int P_BYTES = P_X + 3 * 16 * 17 * 4;

    static constexpr int BYTES = PRECISE ? P_BYTES : F_BYTES;
};

__device__ __forceinline__ float gate_log_alpha(float raw, float dtb, float Ah, int safe, float lb) {
    float la = -Ah * softplus_f(raw + dtb);
    return safe ? fmaxf(la, lb) : la;
}

__device__ __forceinline__ float beta_of(float x, int beta_mode) {
    return beta_mode == 0 ? 1.f / (1.f + __expf(-x)) : x;
}

// A-operand fragment whose k slots follow the accumulator row order of a pair of
// 16-row tiles: slot s<4 -> column k0+4g+s, slot s>=4 -> column k0+16+4g+(s-4).
__device__ __forceinline__ bf16x8 fragA_perm(const bf16_t *base, int pitch, int row, int k0, int g) {
    const bf16_t *p = base + row * pitch + k0 + 4 * g;
    return cat(*(const bf16x4 *)p, *(const bf16x4 *)(p + 16));
}

__device__ __forceinline__ void load_perm_f32(const float *base, int pitch, int row, int k0, int g,
                                              float *x) {
    const float *p = base + row * pitch + k0 + 4 * g;
    f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 16);
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}

__device__ __forceinline__ int perm_k(int g, int s) { return s < 4 ? 4 * g + s : 16 + 4 * g + (s - 4); }

// acc += A B with optional hi/lo splits of either operand (lo*lo dropped).
__device__ __forceinline__ f32x4 mma3(f32x4 acc, bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl,
                                      bool split_a, bool split_b) {
    acc = mfma(ah, bh, acc);
    if (split_b) acc = mfma(ah, bl, acc);
    if (split_a) acc = mfma(al, bh, acc);
    return acc;
}

// Inverse of the unit lower-triangular 64x64 matrix I + A (A strictly lower, f32 in LDS,
// pitch PF) into Tf (f32, pitch PF): 16x16 diagonal blocks by forward substitution, then
// off-diagonal blocks by increasing distance: T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ.
template <int PF>
__device__ __forceinline__ void invert_unit_lower(const float *sA, float *Tf, float *sX, int t) {
    const int w = t >> 6, l = t & 63;
    // zero the strictly upper blocks
    for (int e = t; e < 6 * 256; e += NT) {
        const int blk = e >> 8;  // (0,1),(0,2),(0,3),(1,2),(1,3),(2,3)
        const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
        const int bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
        Tf[(16 * bi + ((e >> 4) & 15)) * PF + 16 * bj + (e & 15)] = 0.f;
    }
    if (l < 16) {
        const int I = w, col = l;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == col) ? 1.f : 0.f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            const float *arow = sA + (16 * I + r) * PF + 16 * I;
            float s = 0.f;
#pragma unroll
            for (int kk = 0; kk < r; ++kk) s += (kk >= col) ? arow[kk] * x[kk] : 0.f;
            if (r > col) x[r] = -s;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Tf[(16 * I + r) * PF + 16 * I + col] = x[r];
    }
    __syncthreads();
    for (int d = 1; d < 4; ++d) {
        const int nent = (4 - d) * 256;
        for (int e = t; e < nent; e += NT) {
            const int J = e >> 8, I = J + d, r = (e >> 4) & 15, c = e & 15;
            float s = 0.f;
            for (int K = J; K < I; ++K) {
                const float *arow = sA + (16 * I + r) * PF + 16 * K;
                const float *tcol = Tf + (16 * K) * PF + 16 * J + c;
#pragma unroll
                for (int kk = 0; kk < 16; ++kk) s += arow[kk] * tcol[kk * PF];
            }
            sX[(J * 16 + r) * 17 + c] = s;
        }
        __syncthreads();
        for (int e = t; e < nent; e += NT) {
            const int J = e >> 8, I = J + d, r = (e >> 4) & 15, c = e & 15;
            const float *trow = Tf + (16 * I + r) * PF + 16 * I;
            float s = 0.f;
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) s += (kk <= r) ? trow[kk] * sX[(J * 16 + kk) * 17 + c] : 0.f;
            Tf[(16 * I + r) * PF + 16 * J + c] = -s;
        }
        __syncthreads();
    }
}

template <int DK, int DVS, bool PRECISE, int MODE>
__global__ __launch_bounds__(NT, 1) void kda_chain_kernel(ChainArgs a) {
    using L = Lds<DK, DVS, PRECISE, MODE>;
    constexpr bool FW = (MODE == MODE_FWD);
    constexpr int DV = DK;           // equal head dims
    constexpr int NVT = DVS / 64;    // 16-column value tiles per wave
    constexpr int NCT = DK / 16;     // 16-row key tiles of the state
    constexpr int NKB = DK / 32;     // 32-wide k blocks over the key dim
    constexpr int PK = L::PK, PJ = L::PJ, PF = L::PF, PKF = L::PKF;
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

    // ---- work item: XCD-aware order keeps the slices of one (item, head) on one XCD
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
    if (FW && len <= 0) return;  // empty sequence: slot untouched, no rows
    const int n_chunks = len > 0 ? (len + CH - 1) / CH : 0;

    const int aug0 = slice * DVS;            // first state column of this slice
    const bool isM = (!FW) && aug0 < DK;     // summary: transition-matrix columns
    const int col0 = (FW || isM) ? aug0 : aug0 - DK;
    const bool has_v = FW || !isM;

    const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 4, li = l & 15;
    const int safe = a.gate_mode == 1;
    const float lb = a.lb;
    const float Ah = expf(a.a_log[h]);

    // ---- state slice: S[m][ct] holds rows 16ct+4g+s, column col0 + 16(w*NVT+m) + li
    f32x4 S[NVT][NCT];
    int slot = 0;
    if (FW) slot = a.state_indices[item];
#pragma unroll
    for (int m = 0; m < NVT; ++m) {
        const int col = col0 + 16 * (w * NVT + m) + li;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int c = 16 * ct + 4 * g + s;
                float val;
                if (FW)
                    val = a.state_pool[a.v_first ? (((int64_t)slot * H + h) * DV + col) * DK + c
                                                  : (((int64_t)slot * H + h) * DK + c) * DV + col];
                else
                    val = (isM && c == col) ? 1.f : 0.f;
                S[m][ct][s] = val;
            }
    }

    float *sBeta = (float *)(smem + (PRECISE ? L::P_BETA : L::F_BETA));
    float *sEG = (float *)(smem + (PRECISE ? L::P_EG : L::F_EG));
    float *sX = (float *)(smem + (PRECISE ? L::P_X : L::F_X));
    float *sA = (float *)(smem + (PRECISE ? L::P_A : L::F_A));

    if constexpr (!PRECISE && FW) {  // P upper blocks are never written below
        bf16_t *sP = (bf16_t *)(smem + L::F_P);
        for (int e = t; e < 64 * 64; e += NT) {
            const int i = e >> 6, j = e & 63;
            if ((j >> 4) > (i >> 4)) sP[i * PJ + j] = (bf16_t)0.f;
        }
    }

    const bf16_t *kb16 = (const bf16_t *)a.k;
    const bf16_t *qb16 = (const bf16_t *)a.q;
    const bf16_t *vb16 = (const bf16_t *)a.v;
    const float *kf32 = (const float *)a.k;
    const float *qf32 = (const float *)a.q;
    const float *vf32 = (const float *)a.v;

    for (int ck = 0; ck < n_chunks; ++ck) {
        const int t0 = t_begin + ck * CH;
        const int n = min(CH, t_end - t0);

        // beta of the chunk rows (0 beyond the sequence end)
        if (t < 64) {
            const float x = a.beta_logits[(int64_t)(t0 + min(t, n - 1)) * H + h];
            sBeta[t] = (t < n) ? beta_of(x, a.beta_mode) : 0.f;
        }

        if constexpr (!PRECISE) {
            // ================= FAST: gate, decay factors, operands =================
            constexpr int CPT = DK / 64;  // channels per thread
            bf16_t *sKR = (bf16_t *)(smem + L::F_KR);
            bf16_t *sQR = (bf16_t *)(smem + L::F_QR);
            bf16_t *sKC = (bf16_t *)(smem + L::F_KC);
            bf16_t *sKHH = (bf16_t *)(smem + L::F_KHH);
            bf16_t *sKHL = (bf16_t *)(smem + L::F_KHL);
            bf16_t *sP = (bf16_t *)(smem + L::F_P);
            bf16_t *sT = (bf16_t *)(smem + L::F_T);
            bf16_t *sTL = (bf16_t *)(smem + L::F_TL);
            bf16_t *sVT = (bf16_t *)(smem + L::F_VT);
            float *sE = (float *)(smem + L::F_E);
            float *sPI = (float *)(smem + L::F_PI);
            float *Tf = (float *)(smem + L::F_KC);

            const int I = w;        // 16-row block owned by this wave in the prep
            const int c0 = l * CPT;
            // Issue every global load of the chunk before any use: rows past the end
            // read the last valid row (always in bounds) and are masked afterwards.
            float rg[16][CPT];
            bf16_t kr[16][CPT], qr[16][CPT], vr[NVT][16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ic = min(16 * I + r, n - 1);
                const int64_t base = ((int64_t)(t0 + ic) * H + h) * DK + c0;
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) {
                    rg[r][cc] = a.raw_gate[base + cc];
                    kr[r][cc] = kb16[base + cc];
                    if (FW) qr[r][cc] = qb16[base + cc];
                }
                if (has_v) {
                    const int64_t vb = ((int64_t)(t0 + ic) * H + h) * DV + col0 + l;
#pragma unroll
                    for (int m = 0; m < NVT; ++m) vr[m][r] = vb16[vb + 64 * m];
                }
            }
            float al[16][CPT], kf[16][CPT], qf[16][CPT];
            float dtb[CPT];
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc) dtb[cc] = a.dt_bias[h * DK + c0 + cc];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const bool valid = 16 * I + r < n;
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) {
                    al[r][cc] = valid ? __expf(gate_log_alpha(rg[r][cc], dtb[cc], Ah, safe, lb)) : 1.f;
                    kf[r][cc] = valid ? (float)kr[r][cc] : 0.f;
                    qf[r][cc] = (FW && valid) ? (float)qr[r][cc] : 0.f;
                }
            }
            // value slice, transposed: sVT[v][row]
#pragma unroll
            for (int m = 0; m < NVT; ++m) {
                const int vv = l + 64 * m;
                bf16x8 lo8, hi8;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const bf16_t x = (has_v && 16 * I + r < n) ? vr[m][r] : (bf16_t)0.f;
                    if (r < 8) lo8[r] = x; else hi8[r - 8] = x;
                }
                *(bf16x8 *)(sVT + vv * PJ + 16 * I) = lo8;
                *(bf16x8 *)(sVT + vv * PJ + 16 * I + 8) = hi8;
            }
            // block decay E_I = prod of the block's alphas
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc) {
                float e = 1.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) e *= al[r][cc];
                sE[I * DK + c0 + cc] = e;
            }
            __syncthreads();
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc) {
                const int c = c0 + cc;
                float pI = 1.f, qS = 1.f, eg = 1.f;
#pragma unroll
                for (int J = 0; J < 4; ++J) {
                    const float e = sE[J * DK + c];
                    if (J < I) pI *= e;
                    if (J > I) qS *= e;
                    eg *= e;
                }
                sPI[I * DK + c] = pI;
                if (I == 0) sEG[c] = eg;
                // forward products: Kr_i = K_i e^{G_i - G_(16I-1)}
                float rr = 1.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    rr *= al[r][cc];
                    const int i = 16 * I + r;
                    sKR[i * PK + c] = (bf16_t)(kf[r][cc] * rr);
                    if (FW) sQR[i * PK + c] = (bf16_t)(qf[r][cc] * rr);
                }
                // backward products: Kc_j = K_j e^{G_(16I+15) - G_j}; Khat_j = Kc_j e^{G_last - G_(16I+15)}
                bf16x8 hh[2], hl[2];
                float cb = 1.f;
#pragma unroll
                for (int r = 15; r >= 0; --r) {
                    const int i = 16 * I + r;
                    const float kc = kf[r][cc] * cb;
                    sKC[i * PK + c] = (bf16_t)kc;
                    const float kh = kc * qS;
                    const bf16_t hb = (bf16_t)kh;
                    hh[r >> 3][r & 7] = hb;
                    hl[r >> 3][r & 7] = (bf16_t)(kh - (float)hb);
                    cb *= al[r][cc];
                }
                *(bf16x8 *)(sKHH + c * PJ + 16 * I) = hh[0];
                *(bf16x8 *)(sKHH + c * PJ + 16 * I + 8) = hh[1];
                *(bf16x8 *)(sKHL + c * PJ + 16 * I) = hl[0];
                *(bf16x8 *)(sKHL + c * PJ + 16 * I + 8) = hl[1];
            }
            __syncthreads();

            // ---- decayed scores: pairs (I,J), J <= I, of 16x16 blocks
            {
                constexpr int PI_[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
                constexpr int PJ_[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
                for (int p = w; p < 10; p += 4) {
                    const int bI = PI_[p], bJ = PJ_[p];
                    f32x4 accA = zero4(), accP = zero4();
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) {
                        const int c = 32 * kb + 8 * g;
                        const bf16x8 aK = *(const bf16x8 *)(sKR + (16 * bI + li) * PK + c);
                        const bf16x8 kc = *(const bf16x8 *)(sKC + (16 * bJ + li) * PK + c);
                        bf16x8 bK;
#pragma unroll
                        for (int s = 0; s < 8; ++s) {
                            float mfac;
                            if (bJ == bI) {
                                mfac = 1.f / sE[bI * DK + c + s];
                            } else {
                                mfac = 1.f;
                                for (int K = bJ + 1; K < bI; ++K) mfac *= sE[K * DK + c + s];
                            }
                            bK[s] = (bf16_t)((float)kc[s] * mfac);
                        }
                        accA = mfma(aK, bK, accA);
                        if (FW) {
                            const bf16x8 aQ = *(const bf16x8 *)(sQR + (16 * bI + li) * PK + c);
                            accP = mfma(aQ, bK, accP);
                        }
                    }
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int i = 16 * bI + 4 * g + s, j = 16 * bJ + li;
                        sA[i * PF + j] = (j < i) ? sBeta[i] * accA[s] : 0.f;
                        if (FW) sP[i * PJ + j] = (bf16_t)((j <= i) ? accP[s] : 0.f);
                    }
                }
            }
            __syncthreads();

            // ---- Kg = Kr e^{G_(16I-1)}, Qbar = Qr e^{G_(16I-1)} in place
            {
                const int i = t >> 2, cq = t & 3, bI = i >> 4;
#pragma unroll
                for (int c = cq * (DK / 4); c < (cq + 1) * (DK / 4); c += 8) {
                    bf16x8 x = *(bf16x8 *)(sKR + i * PK + c);
                    bf16x8 y;
                    if (FW) y = *(bf16x8 *)(sQR + i * PK + c);
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
                        const float f = sPI[bI * DK + c + s];
                        x[s] = (bf16_t)((float)x[s] * f);
                        if (FW) y[s] = (bf16_t)((float)y[s] * f);
                    }
                    *(bf16x8 *)(sKR + i * PK + c) = x;
                    if (FW) *(bf16x8 *)(sQR + i * PK + c) = y;
                }
            }
            invert_unit_lower<PF>(sA, Tf, sX, t);
            for (int e = t; e < 64 * 64; e += NT) {
                const int i = e >> 6, j = e & 63;
                const float x = Tf[i * PF + j];
                const bf16_t hi = (bf16_t)x;
                sT[i * PJ + j] = hi;
                sTL[i * PJ + j] = (bf16_t)(x - (float)hi);
            }
            __syncthreads();

            // ---- chain step for this wave's value tiles.  The prediction K S takes S as
            // bf16 hi + lo: where a key channel barely decays, the rounding of S to bf16
            // is not forgotten between chunks and accumulates to ~1e-3 of the state.  The
            // output product uses the hi part.
            bf16x8 Sb[NVT][NKB], Sl[NVT][NKB];
#pragma unroll
            for (int m = 0; m < NVT; ++m)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    bf16x4 h0, l0, h1, l1;
                    split4(S[m][2 * kb], h0, l0);
                    split4(S[m][2 * kb + 1], h1, l1);
                    Sb[m][kb] = cat(h0, h1);
                    Sl[m][kb] = cat(l0, l1);
                }

            f32x4 Y[NVT][4], Z[NVT][4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
                for (int m = 0; m < NVT; ++m) { Y[m][rt] = zero4(); Z[m][rt] = zero4(); }
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const bf16x8 aK = fragA_perm(sKR, PK, 16 * rt + li, 32 * kb, g);
#pragma unroll
                    for (int m = 0; m < NVT; ++m) {
                        Y[m][rt] = mfma(aK, Sb[m][kb], Y[m][rt]);
                        Y[m][rt] = mfma(aK, Sl[m][kb], Y[m][rt]);
                    }
                    if (FW) {
                        const bf16x8 aQ = fragA_perm(sQR, PK, 16 * rt + li, 32 * kb, g);
#pragma unroll
                        for (int m = 0; m < NVT; ++m) Z[m][rt] = mfma(aQ, Sb[m][kb], Z[m][rt]);
                    }
                }
            }
            // R = beta (V - Y), split hi/lo
            bf16x4 Rh[NVT][4], Rl[NVT][4];
#pragma unroll
            for (int m = 0; m < NVT; ++m) {
                const int vcol = 16 * (w * NVT + m) + li;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const f32x4 vv = f4(*(const bf16x4 *)(sVT + vcol * PJ + 16 * rt + 4 * g));
                    const f32x4 bb = *(const f32x4 *)(sBeta + 16 * rt + 4 * g);
                    split4(bb * (vv - Y[m][rt]), Rh[m][rt], Rl[m][rt]);
                }
            }
            // U = T R (T lower triangular: row tile rt needs k blocks jb <= rt/2)
            bf16x4 Uh[NVT][4], Ul[NVT][4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 Uacc[NVT];
#pragma unroll
                for (int m = 0; m < NVT; ++m) Uacc[m] = zero4();
#pragma unroll
                for (int jb = 0; jb <= (rt >> 1); ++jb) {
                    // T as bf16 hi + lo as well: its rounding, like that of S, is not
                    // forgotten where a key channel barely decays
                    const bf16x8 aT = fragA_perm(sT, PJ, 16 * rt + li, 32 * jb, g);
                    const bf16x8 aTl = fragA_perm(sTL, PJ, 16 * rt + li, 32 * jb, g);
#pragma unroll
                    for (int m = 0; m < NVT; ++m)
                        Uacc[m] = mma3(Uacc[m], aT, aTl, cat(Rh[m][2 * jb], Rh[m][2 * jb + 1]),
                                       cat(Rl[m][2 * jb], Rl[m][2 * jb + 1]), true, true);
                }
#pragma unroll
                for (int m = 0; m < NVT; ++m) split4(Uacc[m], Uh[m][rt], Ul[m][rt]);
            }
            // O = scale (Z + P U)
            if (FW) {
                bf16_t *outp = (bf16_t *)a.out;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
                    for (int jb = 0; jb <= (rt >> 1); ++jb) {
                        const bf16x8 aP = fragA_perm(sP, PJ, 16 * rt + li, 32 * jb, g);
#pragma unroll
                        for (int m = 0; m < NVT; ++m)
                            Z[m][rt] = mfma(aP, cat(Uh[m][2 * jb], Uh[m][2 * jb + 1]), Z[m][rt]);
                    }
#pragma unroll
                    for (int m = 0; m < NVT; ++m) {
                        const int col = col0 + 16 * (w * NVT + m) + li;
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            const int i = 16 * rt + 4 * g + s;
                            if (i < n)
                                outp[((int64_t)(t0 + i) * H + h) * DV + col] = (bf16_t)(a.scale * Z[m][rt][s]);
                        }
                    }
                }
            }
            // S <- Diag(e^{G_last}) S + Khat^T U
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const f32x4 eg = *(const f32x4 *)(sEG + 16 * ct + 4 * g);
#pragma unroll
                for (int m = 0; m < NVT; ++m) S[m][ct] *= eg;
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    const bf16x8 ah = fragA_perm(sKHH, PJ, 16 * ct + li, 32 * jb, g);
                    const bf16x8 alo = fragA_perm(sKHL, PJ, 16 * ct + li, 32 * jb, g);
#pragma unroll
                    for (int m = 0; m < NVT; ++m)
                        S[m][ct] = mma3(S[m][ct], ah, alo, cat(Uh[m][2 * jb], Uh[m][2 * jb + 1]),
                                        cat(Ul[m][2 * jb], Ul[m][2 * jb + 1]), true, true);
                }
            }
            __syncthreads();
        } else {
            // ================= PRECISE: fp32 K, Q, G in LDS; split everything =================
            float *sK = (float *)(smem + L::P_K);
            float *sQ = (float *)(smem + L::P_Q);
            float *sG = (float *)(smem + L::P_G);
            float *sP = (float *)(smem + L::P_P);
            float *sT = (float *)(smem + L::P_T);
            float *sVT = (float *)(smem + L::P_VT);

            if (t < DK) {
                const int c = t;
                const float dtb = a.dt_bias[h * DK + c];
                float G = 0.f;
                for (int i0 = 0; i0 < 64; i0 += 16) {
                    float rg[16], kk[16], qq[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int i = i0 + r;
                        const int64_t base = ((int64_t)(t0 + min(i, n - 1)) * H + h) * DK + c;
                        rg[r] = a.raw_gate[base];
                        kk[r] = i < n ? kf32[base] : 0.f;
                        qq[r] = (FW && i < n) ? qf32[base] : 0.f;
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int i = i0 + r;
                        if (i < n) G += gate_log_alpha(rg[r], dtb, Ah, safe, lb);
                        sG[i * PKF + c] = G;
                        sK[i * PKF + c] = kk[r];
                        if (FW) sQ[i * PKF + c] = qq[r];
                    }
                }
                sEG[c] = __expf(G);
            }
#pragma unroll
            for (int m = 0; m < NVT; ++m) {
                const int vv = l + 64 * m;
                float xv[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = 16 * w + r;
                    xv[r] = has_v ? vf32[((int64_t)(t0 + min(i, n - 1)) * H + h) * DV + col0 + vv] : 0.f;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = 16 * w + r;
                    sVT[vv * PF + i] = (i < n) ? xv[r] : 0.f;
                }
            }
            __syncthreads();

            // ---- decayed scores, elementwise over 4x4 tiles of the lower triangle
            if (t < 136) {
                int bi = 0;
                while ((bi + 1) * (bi + 2) / 2 <= t) ++bi;
                const int bj = t - bi * (bi + 1) / 2;
                float accA[4][4], accP[4][4];
#pragma unroll
                for (int x = 0; x < 4; ++x)
#pragma unroll
                    for (int y = 0; y < 4; ++y) { accA[x][y] = 0.f; accP[x][y] = 0.f; }
                for (int c = 0; c < DK; ++c) {
                    float Ki[4], Qi[4], Gi[4], Kj[4], Gj[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        Ki[x] = sK[(4 * bi + x) * PKF + c];
                        Gi[x] = sG[(4 * bi + x) * PKF + c];
                        Qi[x] = FW ? sQ[(4 * bi + x) * PKF + c] : 0.f;
                        Kj[x] = sK[(4 * bj + x) * PKF + c];
                        Gj[x] = sG[(4 * bj + x) * PKF + c];
                    }
#pragma unroll
                    for (int x = 0; x < 4; ++x)
#pragma unroll
                        for (int y = 0; y < 4; ++y) {
                            const float d = __expf(fminf(Gi[x] - Gj[y], 0.f)) * Kj[y];
                            accA[x][y] += Ki[x] * d;
                            accP[x][y] += Qi[x] * d;
                        }
                }
#pragma unroll
                for (int x = 0; x < 4; ++x)
#pragma unroll
                    for (int y = 0; y < 4; ++y) {
                        const int i = 4 * bi + x, j = 4 * bj + y;
                        sA[i * PF + j] = (j < i) ? sBeta[i] * accA[x][y] : 0.f;
                        if (FW) sP[i * PF + j] = (j <= i) ? accP[x][y] : 0.f;
                    }
            } else if (FW && t < 136 + 120) {
                // zero an upper 4x4 tile of P
                int u = t - 136, bi = 0;
                while (u >= 15 - bi) { u -= 15 - bi; ++bi; }
                const int bj = bi + 1 + u;
#pragma unroll
                for (int x = 0; x < 4; ++x)
#pragma unroll
                    for (int y = 0; y < 4; ++y) sP[(4 * bi + x) * PF + 4 * bj + y] = 0.f;
            }
            __syncthreads();
            invert_unit_lower<PF>(sA, sT, sX, t);

            // ---- chain step, all products split three ways
            bf16x8 Sh[NVT][NKB], Sl[NVT][NKB];
#pragma unroll
            for (int m = 0; m < NVT; ++m)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    bf16x4 h0, l0, h1, l1;
                    split4(S[m][2 * kb], h0, l0);
                    split4(S[m][2 * kb + 1], h1, l1);
                    Sh[m][kb] = cat(h0, h1);
                    Sl[m][kb] = cat(l0, l1);
                }
            f32x4 Y[NVT][4], Z[NVT][4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
                for (int m = 0; m < NVT; ++m) { Y[m][rt] = zero4(); Z[m][rt] = zero4(); }
                const int row = 16 * rt + li;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    float kv[8], gv[8], x[8];
                    load_perm_f32(sK, PKF, row, 32 * kb, g, kv);
                    load_perm_f32(sG, PKF, row, 32 * kb, g, gv);
#pragma unroll
                    for (int s = 0; s < 8; ++s) x[s] = kv[s] * __expf(gv[s]);
                    bf16x8 ah, alo;
                    split8(x, ah, alo);
#pragma unroll
                    for (int m = 0; m < NVT; ++m) Y[m][rt] = mma3(Y[m][rt], ah, alo, Sh[m][kb], Sl[m][kb], true, true);
                    if (FW) {
                        load_perm_f32(sQ, PKF, row, 32 * kb, g, kv);
#pragma unroll
                        for (int s = 0; s < 8; ++s) x[s] = kv[s] * __expf(gv[s]);
                        split8(x, ah, alo);
#pragma unroll
                        for (int m = 0; m < NVT; ++m)
                            Z[m][rt] = mma3(Z[m][rt], ah, alo, Sh[m][kb], Sl[m][kb], true, true);
                    }
                }
            }
            bf16x4 Rh[NVT][4], Rl[NVT][4];
#pragma unroll
            for (int m = 0; m < NVT; ++m) {
                const int vcol = 16 * (w * NVT + m) + li;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const f32x4 vv = *(const f32x4 *)(sVT + vcol * PF + 16 * rt + 4 * g);
                    const f32x4 bb = *(const f32x4 *)(sBeta + 16 * rt + 4 * g);
                    split4(bb * (vv - Y[m][rt]), Rh[m][rt], Rl[m][rt]);
                }
            }
            bf16x4 Uh[NVT][4], Ul[NVT][4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 Uacc[NVT];
#pragma unroll
                for (int m = 0; m < NVT; ++m) Uacc[m] = zero4();
#pragma unroll
                for (int jb = 0; jb <= (rt >> 1); ++jb) {
                    float x[8];
                    load_perm_f32(sT, PF, 16 * rt + li, 32 * jb, g, x);
                    bf16x8 ah, alo;
                    split8(x, ah, alo);
#pragma unroll
                    for (int m = 0; m < NVT; ++m)
                        Uacc[m] = mma3(Uacc[m], ah, alo, cat(Rh[m][2 * jb], Rh[m][2 * jb + 1]),
                                       cat(Rl[m][2 * jb], Rl[m][2 * jb + 1]), true, true);
                }
#pragma unroll
                for (int m = 0; m < NVT; ++m) split4(Uacc[m], Uh[m][rt], Ul[m][rt]);
            }
            if (FW) {
                float *outp = (float *)a.out;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
                    for (int jb = 0; jb <= (rt >> 1); ++jb) {
                        float x[8];
                        load_perm_f32(sP, PF, 16 * rt + li, 32 * jb, g, x);
                        bf16x8 ah, alo;
                        split8(x, ah, alo);
#pragma unroll
                        for (int m = 0; m < NVT; ++m)
                            Z[m][rt] = mma3(Z[m][rt], ah, alo, cat(Uh[m][2 * jb], Uh[m][2 * jb + 1]),
                                            cat(Ul[m][2 * jb], Ul[m][2 * jb + 1]), true, true);
                    }
#pragma unroll
                    for (int m = 0; m < NVT; ++m) {
                        const int col = col0 + 16 * (w * NVT + m) + li;
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            const int i = 16 * rt + 4 * g + s;
                            if (i < n) outp[((int64_t)(t0 + i) * H + h) * DV + col] = a.scale * Z[m][rt][s];
                        }
                    }
                }
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const f32x4 eg = *(const f32x4 *)(sEG + 16 * ct + 4 * g);
#pragma unroll
                for (int m = 0; m < NVT; ++m) S[m][ct] *= eg;
                const int c = 16 * ct + li;
                const float glast = sG[63 * PKF + c];
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    float x[8];
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
                        const int j = 32 * jb + perm_k(g, s);
                        x[s] = sK[j * PKF + c] * __expf(glast - sG[j * PKF + c]);
                    }
                    bf16x8 ah, alo;
                    split8(x, ah, alo);
#pragma unroll
                    for (int m = 0; m < NVT; ++m)
                        S[m][ct] = mma3(S[m][ct], ah, alo, cat(Uh[m][2 * jb], Uh[m][2 * jb + 1]),
                                        cat(Ul[m][2 * jb], Ul[m][2 * jb + 1]), true, true);
                }
            }
            __syncthreads();
        }
    }

    // ---- store the final state slice
#pragma unroll
    for (int m = 0; m < NVT; ++m) {
        const int col = col0 + 16 * (w * NVT + m) + li;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int c = 16 * ct + 4 * g + s;
                if (FW)
                    a.state_pool[a.v_first ? (((int64_t)slot * H + h) * DV + col) * DK + c
                                         : (((int64_t)slot * H + h) * DK + c) * DV + col] = S[m][ct][s];
                else if (isM)
                    a.M[(((int64_t)item * H + h) * DK + c) * DK + col] = S[m][ct][s];
                else
                    a.U[(((int64_t)item * H + h) * DK + c) * DV + col] = S[m][ct][s];
            }
    }
}

template <int DK, int DVS, bool PRECISE, int MODE>
static hipError_t launch_one(const ChainArgs &a, hipStream_t stream) {
    const int n_units = a.n_items * a.H;
    const int groups = (n_units + 7) / 8;
    const dim3 grid(8 * a.n_slices * groups);
    hipLaunchKernelGGL((kda_chain_kernel<DK, DVS, PRECISE, MODE>), grid, dim3(NT), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_chain(const ChainArgs &a, int dk, int dvs, bool precise, int mode, hipStream_t stream) {
    if (mode == MODE_FWD) {
        if (!precise) {
            if (dk == 128 && dvs == 64) return launch_one<128, 64, false, MODE_FWD>(a, stream);
            if (dk == 128 && dvs == 128) return launch_one<128, 128, false, MODE_FWD>(a, stream);
            if (dk == 64 && dvs == 64) return launch_one<64, 64, false, MODE_FWD>(a, stream);
        } else {
            if (dk == 64 && dvs == 64) return launch_one<64, 64, true, MODE_FWD>(a, stream);
        }
    } else {
        if (!precise) {
            if (dk == 128 && dvs == 64) return launch_one<128, 64, false, MODE_SUMMARY>(a, stream);
            if (dk == 128 && dvs == 128) return launch_one<128, 128, false, MODE_SUMMARY>(a, stream);
            if (dk == 64 && dvs == 64) return launch_one<64, 64, false, MODE_SUMMARY>(a, stream);
        } else {
            if (dk == 128 && dvs == 64) return launch_one<128, 64, true, MODE_SUMMARY>(a, stream);
            if (dk == 128 && dvs == 128) return launch_one<128, 128, true, MODE_SUMMARY>(a, stream);
            if (dk == 64 && dvs == 64) return launch_one<64, 64, true, MODE_SUMMARY>(a, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
