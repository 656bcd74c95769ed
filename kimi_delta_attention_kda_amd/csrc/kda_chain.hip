// kda_chain.hip -- chunk-parallel KDA prefill and segment summaries, precise variant, for
// gfx950 (MI355X): fp32 or bf16 q/k/v, either gate form, dk = dv in {64, 128}.
//
// One workgroup (4 waves) owns one (sequence-or-segment, head, column slice) and walks its
// 64-token chunks in order.  For each chunk it
//   1. computes the gate (log alpha = -exp(a_log) softplus(raw + dt_bias), optionally
//      clamped from below), its running sum G from the chunk start, and beta;
//   2. builds the decayed key-key scores A (strictly lower) and query-key scores P (lower)
//      from exponentials of non-positive differences of G only, so no factor e^{-G} is
//      ever formed and any gate, however steep, stays finite: MFMA products of operands
//      decayed towards a row between the two blocks off the diagonal 16-blocks,
//      elementwise inside them;
//   3. inverts the four 16x16 diagonal blocks of the unit lower-triangular I + A (fp32);
//   4. with the fp32 state slice S [dk, 16-column tiles] resident in MFMA accumulators:
//        U  = (I + A)^-1 Diag(beta) (V - (K o e^G) S), by blocked forward substitution
//        O  = scale ((Q o e^G) S + P U)
//        S <- Diag(e^{G_last}) S + (K o e^{G_last - G})^T U
//      with every MFMA operand split into bf16 hi + lo and the products summed three ways
//      (hi*hi + hi*lo + lo*hi), about fp32 accuracy.
// This is the token recurrence S_t = (I - b k k^T) Diag(alpha) S_{t-1} + b k v^T,
// o_t = scale q^T S_t (nx_nofloat_kda.nx source: kda_gate, kda_write, kda_forward)
// rewritten over a chunk; the chunked method's ingredients -- prefix scan of log gates,
// triangular inverse, stable decayed scores -- are those named by "GStar Assignment 2:
// Build Kimi Delta Attention", Learning path (P4, P6, P8, P9).
//
// bf16 inputs are widened exactly to fp32 on load and the output is rounded to bf16 once
// (round to nearest even); the arithmetic is that of the fp32 inputs.  This variant
// serves every call outside the fast kernel's range (kda_fast.hip: bf16 with the safe
// gate): fp32 inputs, and bf16 inputs with the original gate or a bound below -5.3.
// Segment summaries run the same walk on the augmented state X = [M | U] with
// X_0 = [I | 0] and value rows [0 | V] (KDA Context Parallelism, "Theory").
#include <type_traits>

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

constexpr int CH = 64;   // tokens per chunk
constexpr int NT = 256;  // threads per workgroup (4 waves of 64)

template <int DK, int DVS, int MODE>
struct Lds {
    static constexpr bool FW = (MODE == MODE_FWD);
    // dk = 128 forward: the value slice goes from global memory to registers (requested
    // ahead of the chain step) instead of being staged in LDS, which keeps the workgroup
    // within 160 KB
    static constexpr bool VG = FW && DK == 128;
    static constexpr int PF = 64 + 4;    // fp32 pitch, [*][64]
    static constexpr int PKF = DK + 4;   // fp32 pitch, [64][DK]
    static constexpr int K = 0;                                  // K (f32)
    static constexpr int Q = K + 64 * PKF * 4;                   // Q (f32, FWD)
    static constexpr int G = Q + (FW ? 64 * PKF * 4 : 0);        // G [64][DK], then (K e^{G_last-G})^T [DK][64] (f32)
    static constexpr int GB = (64 * PKF > DK * PF ? 64 * PKF : DK * PF) * 4;
    static constexpr int A = G + GB;                             // A (f32)
    static constexpr int P = A + 64 * PF * 4;                    // P (f32, FWD)
    static constexpr int T = P + (FW ? 64 * PF * 4 : 0);         // inverses of the diagonal blocks of I + A (f32)
    static constexpr int VT = T + 64 * PF * 4;                   // V^T slice (f32)
    static constexpr int BETA = VT + (VG ? 0 : DVS * PF * 4);
    static constexpr int EG = BETA + 64 * 4;                     // e^{G_last} [DK]
    static constexpr int GL = EG + DK * 4;                       // G_last [DK]
    static constexpr int X = GL + DK * 4;                        // load-phase part totals [256]
    static constexpr int BYTES = X + 256 * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget of one workgroup");
};

__device__ __forceinline__ float gate_log_alpha(float raw, float dtb, float Ah, int safe, float lb) {
    float la = -Ah * softplus_f(raw + dtb);
    return safe ? fmaxf(la, lb) : la;
}

__device__ __forceinline__ float beta_of(float x, int beta_mode) {
    return beta_mode == 0 ? 1.f / (1.f + __expf(-x)) : x;
}

// one q/k/v element, widened to fp32
template <bool IN16>
__device__ __forceinline__ float ld_in(const void *p, int64_t i) {
    if constexpr (IN16)
        return (float)((const bf16_t *)p)[i];
    else
        return ((const float *)p)[i];
}

template <bool IN16>
__device__ __forceinline__ void st_out(void *p, int64_t i, float x) {
    if constexpr (IN16)
        ((bf16_t *)p)[i] = (bf16_t)x;
    else
        ((float *)p)[i] = x;
}

__device__ __forceinline__ void load_perm_f32(const float *base, int pitch, int row, int k0, int g,
                                              float *x) {
    const float *p = base + row * pitch + k0 + 4 * g;
    f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 16);
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}

// acc += A B with optional hi/lo splits of either operand (lo*lo dropped).
__device__ __forceinline__ f32x4 mma3(f32x4 acc, bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl,
                                      bool split_a, bool split_b) {
    acc = mfma(ah, bh, acc);
    if (split_b) acc = mfma(ah, bl, acc);
    if (split_a) acc = mfma(al, bh, acc);
    return acc;
}

// (I + A_bb)^-1 of one 16x16 diagonal block, by right-looking substitution on the 64
// lanes of a wave: column c = l/4 of the inverse lives on the four lanes of a quad, lane
// quarter q holding rows 4q .. 4q+3 as acc = -x.  Step K takes acc_K from quad lane K/4
// (a DPP quad broadcast) and folds x_K into the rows below K.  The lane's four rows of the
// block arrive in arow up front; the entries on and above the diagonal are zero (the
// diagonal tiles are written with zeros there, the upper tiles are zeroed once), so a step
// updates every row without a mask.
template <int K>
__device__ __forceinline__ void diag_inv_step(float (&acc)[4], const f32x4 (&arow)[4][4]) {
    const float yk = __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, acc[K & 3]), (K >> 2) * 0x55, 0xF, 0xF, false));
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = fmaf(-arow[j][K >> 2][K & 3], yk, acc[j]);
    if constexpr (K < 15) diag_inv_step<K + 1>(acc, arow);
}

// v_mfma_f32_16x16x16_bf16: D[16x16] += A[16x16] B[16x16]; lane (g, li): A slot s =
// A[li][4g+s], B slot s = B[4g+s][li], D slot s = D[4g+s][li] (so an accumulator tile is
// a B operand as it stands).
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a), __builtin_bit_cast(s4, b), c, 0, 0, 0);
}
// acc += A B with both operands split into bf16 hi + lo (lo*lo dropped)
__device__ __forceinline__ f32x4 mma3x16(f32x4 acc, bf16x4 ah, bf16x4 al, bf16x4 bh, bf16x4 bl) {
    acc = mfma16(ah, bh, acc);
    acc = mfma16(ah, bl, acc);
    return mfma16(al, bh, acc);
}

// One unit of the chunk walk: chunks t_begin .. t_end of (item, head h), state column slice
// `slice`.  Forward pass: the state starts from fin (init 0; V_FIRST if fin_vfirst), the identity
// (init 1, a transition chain) or zero (init 2); values are read when v_on; output rows go to
// obase with row 0 at token orow; the final state goes to fin.
template <int DK, int DVS, bool IN16, int MODE>
__device__ __forceinline__ void chain_unit(const ChainArgs &a, char *smem, const int item, const int h,
                                           const int t_begin, const int t_end, const int slice, const int init,
                                           const bool v_on, const bool fin_vfirst, float *fin, void *obase,
                                           const int64_t orow) {
    using L = Lds<DK, DVS, MODE>;
    constexpr bool FW = (MODE == MODE_FWD);
    constexpr int DV = DK;           // equal head dims
    constexpr int NVT = DVS / 64;    // 16-column value tiles per wave
    constexpr int NCT = DK / 16;     // 16-row key tiles of the state
    constexpr int NKB = DK / 32;     // 32-wide k blocks over the key dim
    constexpr int PF = L::PF, PKF = L::PKF;
    const int H = a.H;
    const int hk = h / (H / a.Hk);  // key head of value head h
    const int len = t_end - t_begin;
    const int n_chunks = len > 0 ? (len + CH - 1) / CH : 0;
    // The forward pass on bf16 inputs needs bf16-level results only: the scores and the
    // output's products (Qbar S, P U) take both operands unsplit, Y = Kg S splits only S (the
    // state's own rounding is what accumulates), and the solve and the state update keep
    // every split; fp32 inputs and the summaries keep every three-way split.
    constexpr bool LITE = FW && IN16;

    const int aug0 = slice * DVS;            // first state column of this slice
    const bool isM = (!FW) && aug0 < DK;     // summary: transition-matrix columns
    const int col0 = (FW || isM) ? aug0 : aug0 - DK;
    const bool has_v = FW ? v_on : !isM;

    const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 4, li = l & 15;
    const int safe = a.gate_mode == 1;
    const float lb = a.lb;
    const float Ah = expf(a.a_log[h]);

    // ---- state slice: S[m][ct] holds rows 16ct+4g+s, column col0 + 16(w*NVT+m) + li
    f32x4 S[NVT][NCT];
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
                    val = init == 0 ? fin[fin_vfirst ? col * DK + c : c * DV + col]
                                    : ((init == 1 && c == col) ? 1.f : 0.f);
                else
                    val = (isM && c == col) ? 1.f : 0.f;
                S[m][ct][s] = val;
            }
    }

    float *sBeta = (float *)(smem + L::BETA);
    float *sEG = (float *)(smem + L::EG);
    float *sGL = (float *)(smem + L::GL);
    float *sX = (float *)(smem + L::X);
    float *sA = (float *)(smem + L::A);
    float *sK = (float *)(smem + L::K);
    float *sQ = (float *)(smem + L::Q);
    float *sG = (float *)(smem + L::G);
    float *sP = (float *)(smem + L::P);
    float *sT = (float *)(smem + L::T);
    float *sVT = (float *)(smem + L::VT);

    // Entries that no chunk writes, zeroed once (the first chunk's barriers publish them):
    // the 4x4 tiles above the diagonal inside the diagonal 16-blocks of A, which the block
    // inverses read as zeros, and the strictly upper 4x4 tiles of P.
    for (int e = t; e < 64 * 64; e += NT) {
        const int i = e >> 6, j = e & 63;
        if ((j >> 4) == (i >> 4) && (j >> 2) > (i >> 2)) sA[i * PF + j] = 0.f;
        if (FW && (j >> 2) > (i >> 2)) sP[i * PF + j] = 0.f;
    }

    // Cross-chunk prefetch (every instance but the register-tight dk = 128 forward pass): the
    // inputs of chunk ck + 1 are requested before the state update of chunk ck and land in
    // these registers while it runs.  Same rows and ownership as the load phase below.
    constexpr bool PFX = !(FW && DK == 128);
    constexpr int TPC = NT / DK, RH = 64 / TPC;
    // q/k/v travel as stored (bf16 bits or fp32) and are widened when consumed, so that no
    // conversion waits for its load at the request
    typedef typename std::conditional<IN16, unsigned short, float>::type raw_t;
    auto widen = [](raw_t x) -> float {
        if constexpr (IN16)
            return __builtin_bit_cast(float, (uint32_t)x << 16);
        else
            return x;
    };
    [[maybe_unused]] float nrg[PFX ? RH : 1];
    [[maybe_unused]] raw_t nkk[PFX ? RH : 1], nqq[PFX && FW ? RH : 1];
    [[maybe_unused]] raw_t nxv[PFX && !L::VG ? NVT : 1][16];
    [[maybe_unused]] float nbl = 0.f;
    [[maybe_unused]] auto fetch = [&](int ckf) {
        const int tf = t_begin + ckf * CH, nf = min(CH, t_end - tf);
        const int c = t % DK, part = t / DK;
        if (t < 64) nbl = a.beta_logits[(int64_t)(tf + min(t, nf - 1)) * H + h];
#pragma unroll
        for (int r = 0; r < RH; ++r) {
            const int64_t row = tf + min(RH * part + r, nf - 1);
            nrg[r] = a.raw_gate[(row * H + h) * DK + c];
            const int64_t kbase = (row * a.Hk + hk) * DK + c;
            nkk[r] = ((const raw_t *)a.k)[kbase];
            if constexpr (FW) nqq[r] = ((const raw_t *)a.q)[kbase];
        }
        if constexpr (!L::VG)
#pragma unroll
            for (int m = 0; m < NVT; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    nxv[m][r] = has_v ? ((const raw_t *)a.v)[((int64_t)(tf + min(16 * w + r, nf - 1)) * H + h) * DV +
                                                              col0 + l + 64 * m]
                                      : raw_t(0);
    };
    if constexpr (PFX)
        if (n_chunks > 0) fetch(0);

    for (int ck = 0; ck < n_chunks; ++ck) {
        const int t0 = t_begin + ck * CH;
        const int n = min(CH, t_end - t0);

        // beta of the chunk rows (0 beyond the sequence end)
        if (t < 64) {
            float x;
            if constexpr (PFX)
                x = nbl;
            else
                x = a.beta_logits[(int64_t)(t0 + min(t, n - 1)) * H + h];
            sBeta[t] = (t < n) ? beta_of(x, a.beta_mode) : 0.f;
        }

        // gate, K and Q of the chunk: TPC threads per key channel, each taking RH consecutive
        // rows, so every load of the chunk is issued at once; each part's running sum of
        // log alpha is then offset by the totals of the parts before it (exchanged through
        // a small LDS array).  Adding the non-positive offsets keeps G non-increasing along
        // the chunk.
        {
            // RB rows per batch of loads: all RH at once, or two batches in the dk = 128
            // forward pass, whose registers allow no more
            constexpr int RB = (FW && DK == 128) ? RH / 2 : RH;
            const int c = t % DK, part = t / DK;
            const float dtb = a.dt_bias[h * DK + c];
            float G = 0.f;
#pragma unroll 1
            for (int r0 = 0; r0 < RH; r0 += RB) {
                float rg[RB], kk[RB], qq[RB];
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    if constexpr (PFX) {  // prefetched (RB == RH)
                        rg[r] = nrg[r];
                        kk[r] = widen(nkk[r]);
                        qq[r] = FW ? widen(nqq[r]) : 0.f;
                        continue;
                    }
                    const int i = RH * part + r0 + r;
                    const int64_t row = t0 + min(i, n - 1);
                    rg[r] = a.raw_gate[(row * H + h) * DK + c];
                    // unconditional (rows past the end repeat the last row, zeroed below), so
                    // that no load waits inside a branch for its widening
                    const int64_t kbase = (row * a.Hk + hk) * DK + c;
                    kk[r] = ld_in<IN16>(a.k, kbase);
                    qq[r] = FW ? ld_in<IN16>(a.q, kbase) : 0.f;
                }
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    const int i = RH * part + r0 + r;
                    if (i < n) G += gate_log_alpha(rg[r], dtb, Ah, safe, lb);
                    sG[i * PKF + c] = G;  // this part's own running sum for now
                    sK[i * PKF + c] = i < n ? kk[r] : 0.f;
                    if (FW) sQ[i * PKF + c] = i < n ? qq[r] : 0.f;
                }
            }
            sX[part * DK + c] = G;  // this part's total
            __syncthreads();
            float off = 0.f;
            for (int p = 0; p < part; ++p) off += sX[p * DK + c];
            if (part > 0)
#pragma unroll
                for (int r = 0; r < RH; ++r) sG[(RH * part + r) * PKF + c] += off;
            if (part == TPC - 1) {
                sEG[c] = __expf(off + G);
                sGL[c] = off + G;
            }
        }
        if constexpr (!L::VG) {
#pragma unroll
            for (int m = 0; m < NVT; ++m) {
                const int vv = l + 64 * m;
                float xv[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = 16 * w + r;
                    if constexpr (PFX)
                        xv[r] = widen(nxv[m][r]);
                    else
                        xv[r] = has_v ? ld_in<IN16>(a.v, ((int64_t)(t0 + min(i, n - 1)) * H + h) * DV + col0 + vv) : 0.f;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = 16 * w + r;
                    sVT[vv * PF + i] = (i < n) ? xv[r] : 0.f;
                }
            }
        }
        __syncthreads();

        // ---- decayed scores A (beta folded in) and P.
        //  - Off-diagonal 16x16 blocks (row block I > column block J) as MFMA products:
        //    e^{G_i - G_j} = e^{G_i - G_r} e^{G_r - G_j} with r = 16 I - 1, the row just above
        //    the row block, so A_IJ = (K_I o e^{G_I - G_r}) (K_J o e^{G_r - G_J})^T and both
        //    operands are bounded by |K| (G never increases along the chunk: every log alpha
        //    is <= 0, and adding a non-positive number never rounds upwards).  Wave 0 takes
        //    (1,0); wave 1 (2,1) and (2,0); wave 2 (3,2) and (3,1); wave 3 (3,0): the row
        //    operand is formed once per wave and each column operand once per block.
        //  - Inside the diagonal 16-blocks, elementwise over 4x4 tiles.  Below the diagonal of
        //    4x4 tiles, through the last row r of the column tile (seven exponentials per
        //    channel, both factors <= 1): 24 tiles on waves 0-2, eight lanes per tile with one
        //    channel part each, summed with DPP.  On the diagonal, products of the one-step
        //    factors e^{G_x - G_(x-1)} <= 1 (three exponentials per channel), on wave 3: a quad
        //    of lanes per tile, one channel quarter each.
        {
            // CPS channels per step, read as 8- or 16-byte rows (two in the dk = 128 forward
            // pass, whose registers allow no more)
            constexpr int CPS = (FW && DK == 128) ? 2 : 4;
            typedef float fv __attribute__((ext_vector_type(CPS)));
            auto dpp_add = [](float v, int ctrl_sel) {
                const int x = __builtin_bit_cast(int, v);
                const int y = ctrl_sel == 0 ? __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false)    // lane ^ 1
                            : ctrl_sel == 1 ? __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false)    // lane ^ 2
                                            : __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);  // 7 - lane in 8
                return v + __builtin_bit_cast(float, y);
            };
            if (w < 3) {
                constexpr int CPP = DK / 8;  // channels per part
                const int u = t >> 3, part = t & 7;
                const int db = u / 6, lu = u - 6 * db;
                const int bi4 = lu < 1 ? 1 : (lu < 3 ? 2 : 3), bj4 = lu - bi4 * (bi4 - 1) / 2;
                const int bi = 4 * db + bi4, bj = 4 * db + bj4;
                float accA[4][4], accP[4][4];
#pragma unroll
                for (int x = 0; x < 4; ++x)
#pragma unroll
                    for (int y = 0; y < 4; ++y) { accA[x][y] = 0.f; accP[x][y] = 0.f; }
#pragma unroll 2
                for (int c = part * CPP; c < (part + 1) * CPP; c += CPS) {
                    fv Ki[4], Qi[4], Gi[4], Kj[4], Gj[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        Ki[x] = *(const fv *)(sK + (4 * bi + x) * PKF + c);
                        Gi[x] = *(const fv *)(sG + (4 * bi + x) * PKF + c);
                        Qi[x] = FW ? *(const fv *)(sQ + (4 * bi + x) * PKF + c) : fv{};
                        Kj[x] = *(const fv *)(sK + (4 * bj + x) * PKF + c);
                        Gj[x] = *(const fv *)(sG + (4 * bj + x) * PKF + c);
                    }
#pragma unroll
                    for (int cc = 0; cc < CPS; ++cc) {
                        const float Gr = Gj[3][cc];
                        float kej[4];
#pragma unroll
                        for (int y = 0; y < 3; ++y) kej[y] = __expf(Gr - Gj[y][cc]) * Kj[y][cc];
                        kej[3] = Kj[3][cc];
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            const float ri = __expf(Gi[x][cc] - Gr);
                            const float kx = Ki[x][cc] * ri, qx = Qi[x][cc] * ri;
#pragma unroll
                            for (int y = 0; y < 4; ++y) {
                                accA[x][y] += kx * kej[y];
                                accP[x][y] += qx * kej[y];
                            }
                        }
                    }
                }
#pragma unroll
                for (int x = 0; x < 4; ++x)
#pragma unroll
                    for (int y = 0; y < 4; ++y)
#pragma unroll
                        for (int st = 0; st < 3; ++st) {
                            accA[x][y] = dpp_add(accA[x][y], st);
                            if (FW) accP[x][y] = dpp_add(accP[x][y], st);
                        }
                if (part == 0)
#pragma unroll
                    for (int x = 0; x < 4; ++x)
#pragma unroll
                        for (int y = 0; y < 4; ++y) {
                            const int i = 4 * bi + x, j = 4 * bj + y;
                            sA[i * PF + j] = sBeta[i] * accA[x][y];
                            if (FW) sP[i * PF + j] = accP[x][y];
                        }
            } else {
                const int b = l >> 2, qc = l & 3;  // tile (b, b), channel quarter qc
                float dA[4][4], dP[4][4];
#pragma unroll
                for (int x = 0; x < 4; ++x)
#pragma unroll
                    for (int y = 0; y < 4; ++y) { dA[x][y] = 0.f; dP[x][y] = 0.f; }
                for (int c = qc * (DK / 4); c < (qc + 1) * (DK / 4); c += CPS) {
                    fv K4[4], Q4[4], G4[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        K4[x] = *(const fv *)(sK + (4 * b + x) * PKF + c);
                        G4[x] = *(const fv *)(sG + (4 * b + x) * PKF + c);
                        Q4[x] = FW ? *(const fv *)(sQ + (4 * b + x) * PKF + c) : fv{};
                    }
#pragma unroll
                    for (int cc = 0; cc < CPS; ++cc) {
                        const float a1 = __expf(G4[1][cc] - G4[0][cc]), a2 = __expf(G4[2][cc] - G4[1][cc]),
                                    a3 = __expf(G4[3][cc] - G4[2][cc]);
                        const float D[4][4] = {{1.f, 0.f, 0.f, 0.f},
                                               {a1, 1.f, 0.f, 0.f},
                                               {a2 * a1, a2, 1.f, 0.f},
                                               {a3 * (a2 * a1), a3 * a2, a3, 1.f}};
#pragma unroll
                        for (int x = 0; x < 4; ++x)
#pragma unroll
                            for (int y = 0; y <= x; ++y) {
                                const float d = D[x][y] * K4[y][cc];
                                dA[x][y] += K4[x][cc] * d;
                                dP[x][y] += Q4[x][cc] * d;
                            }
                    }
                }
#pragma unroll
                for (int x = 0; x < 4; ++x)
#pragma unroll
                    for (int y = 0; y <= x; ++y)
#pragma unroll
                        for (int st = 0; st < 2; ++st) {
                            dA[x][y] = dpp_add(dA[x][y], st);
                            if (FW) dP[x][y] = dpp_add(dP[x][y], st);
                        }
                if (qc == 0)
#pragma unroll
                    for (int x = 0; x < 4; ++x)
#pragma unroll
                        for (int y = 0; y < 4; ++y) {
                            const int i = 4 * b + x, j = 4 * b + y;
                            sA[i * PF + j] = (y < x) ? sBeta[i] * dA[x][y] : 0.f;
                            if (FW) sP[i * PF + j] = (y <= x) ? dP[x][y] : 0.f;
                        }
            }
            {
                // off-diagonal 16-blocks: row block RB against one or two column blocks
                const int RB = w == 0 ? 1 : (w == 1 ? 2 : 3), r = 16 * RB - 1;
                const int cb0 = w == 3 ? 0 : RB - 1, cb1 = RB - 2;
                const bool two = (w == 1 || w == 2);
                f32x4 oA[2] = {zero4(), zero4()}, oP[2] = {zero4(), zero4()};
#pragma unroll 1
                for (int kb = 0; kb < NKB; ++kb) {
                    float kx[8], gx[8], gr[8], qx[8];
                    load_perm_f32(sK, PKF, 16 * RB + li, 32 * kb, g, kx);
                    load_perm_f32(sG, PKF, 16 * RB + li, 32 * kb, g, gx);
                    load_perm_f32(sG, PKF, r, 32 * kb, g, gr);
                    if (FW) load_perm_f32(sQ, PKF, 16 * RB + li, 32 * kb, g, qx);
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
                        const float e = __expf(gx[s] - gr[s]);
                        kx[s] *= e;
                        if (FW) qx[s] *= e;
                    }
                    bf16x8 kh, kl, qh, ql;
                    split8(kx, kh, kl);
                    if (FW) split8(qx, qh, ql);
#pragma unroll
                    for (int o = 0; o < 2; ++o) {
                        if (o == 1 && !two) break;
                        const int cb = o == 0 ? cb0 : cb1;
                        float kj[8], gj[8];
                        load_perm_f32(sK, PKF, 16 * cb + li, 32 * kb, g, kj);
                        load_perm_f32(sG, PKF, 16 * cb + li, 32 * kb, g, gj);
#pragma unroll
                        for (int s = 0; s < 8; ++s) kj[s] *= __expf(gr[s] - gj[s]);
                        bf16x8 jh, jl;
                        split8(kj, jh, jl);
                        oA[o] = mma3(oA[o], kh, kl, jh, jl, !LITE, !LITE);
                        if (FW) oP[o] = mma3(oP[o], qh, ql, jh, jl, !LITE, !LITE);
                    }
                }
#pragma unroll
                for (int o = 0; o < 2; ++o) {
                    if (o == 1 && !two) break;
                    const int j = 16 * (o == 0 ? cb0 : cb1) + li;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int i = 16 * RB + 4 * g + s;
                        sA[i * PF + j] = sBeta[i] * oA[o][s];
                        if (FW) sP[i * PF + j] = oP[o][s];
                    }
                }
            }
        }
        __syncthreads();
        // The chain step's operands, formed once per element (the scores above were the last
        // readers of K, Q and G as such): K e^{G} over K, Q e^{G} over Q, and
        // (K e^{G_last - G})^T over G, transposed so that the state update reads its operand
        // rows as 16-byte runs; the transposed writes wait until every thread has read its G.
        // The inverse below neither reads nor writes these arrays, and ends with a barrier.
        {
            constexpr int PER = 64 * DK / NT;
            float kl[PER];
#pragma unroll
            for (int r = 0; r < PER; ++r) {
                const int e = t + r * NT, i = e / DK, c = e - i * DK;
                const float G = sG[i * PKF + c], K = sK[i * PKF + c], eg = __expf(G);
                sK[i * PKF + c] = K * eg;
                if (FW) sQ[i * PKF + c] *= eg;
                kl[r] = K * __expf(sGL[c] - G);
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < PER; ++r) {
                const int e = t + r * NT, i = e / DK, c = e - i * DK;
                sG[c * PF + i] = kl[r];
            }
        }
        {
            // the four diagonal-block inverses of I + A, one per wave, into sT (fp32)
            const int c = l >> 2, q = l & 3;
            float acc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = (4 * q + j == c) ? -1.f : 0.f;
            f32x4 arow[4][4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    arow[j][kb] = *(const f32x4 *)(sA + (16 * w + 4 * q + j) * PF + 16 * w + 4 * kb);
            diag_inv_step<0>(acc, arow);
#pragma unroll
            for (int j = 0; j < 4; ++j) sT[(16 * w + 4 * q + j) * PF + 16 * w + c] = -acc[j];
        }
        __syncthreads();

        // ---- chain step, all products split three ways
        // dk = 128 forward: the value rows of the chunk are requested here, ahead of their use
        // after Y, bf16 pairs sharing a register (rows past the end repeat the last row;
        // their beta is 0)
        typedef unsigned short us2 __attribute__((ext_vector_type(2)));
        [[maybe_unused]] us2 vpk[L::VG && IN16 ? NVT : 1][4][2];
        [[maybe_unused]] float vf[L::VG && !IN16 ? NVT : 1][4][4];
        if constexpr (L::VG) {
#pragma unroll
            for (int m = 0; m < NVT; ++m) {
                const int64_t cbase = (int64_t)h * DV + col0 + 16 * (w * NVT + m) + li;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int64_t idx = (int64_t)(t0 + min(16 * rt + 4 * g + s, n - 1)) * H * DV + cbase;
                        if constexpr (IN16)
                            vpk[m][rt][s >> 1][s & 1] = ((const unsigned short *)a.v)[idx];
                        else
                            vf[m][rt][s] = ((const float *)a.v)[idx];
                    }
            }
        }
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
        {
            // software-pipelined over the (row tile, k block) steps: the operand rows of step
            // st + 1 are requested before the products of step st
            float xk[8], xq[8], nk[8], nq[8];
            load_perm_f32(sK, PKF, li, 0, g, xk);  // K e^{G}
            if (FW) load_perm_f32(sQ, PKF, li, 0, g, xq);  // Q e^{G}
#pragma unroll
            for (int st = 0; st < 4 * NKB; ++st) {
                const int rt = st / NKB, kb = st % NKB;
                if (kb == 0)
#pragma unroll
                    for (int m = 0; m < NVT; ++m) { Y[m][rt] = zero4(); Z[m][rt] = zero4(); }
                if (st + 1 < 4 * NKB) {
                    const int row = 16 * ((st + 1) / NKB) + li, k0 = 32 * ((st + 1) % NKB);
                    load_perm_f32(sK, PKF, row, k0, g, nk);
                    if (FW) load_perm_f32(sQ, PKF, row, k0, g, nq);
                }
                __builtin_amdgcn_sched_barrier(0);  // keep those reads ahead of this step's work
                bf16x8 ah, alo;
                split8(xk, ah, alo);
#pragma unroll
                for (int m = 0; m < NVT; ++m) Y[m][rt] = mma3(Y[m][rt], ah, alo, Sh[m][kb], Sl[m][kb], !LITE, true);
                if (FW) {
                    split8(xq, ah, alo);
#pragma unroll
                    for (int m = 0; m < NVT; ++m)
                        Z[m][rt] = mma3(Z[m][rt], ah, alo, Sh[m][kb], Sl[m][kb], !LITE, !LITE);
                }
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    xk[s] = nk[s];
                    if (FW) xq[s] = nq[s];
                }
            }
        }
        f32x4 R[NVT][4];
#pragma unroll
        for (int m = 0; m < NVT; ++m) {
            const int vcol = 16 * (w * NVT + m) + li;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 vv;
                if constexpr (L::VG && IN16) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const uint32_t p = __builtin_bit_cast(uint32_t, vpk[m][rt][s >> 1]);
                        vv[s] = (s & 1) ? bf_hi(p) : bf_lo(p);
                    }
                } else if constexpr (L::VG) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) vv[s] = vf[m][rt][s];
                } else {
                    vv = *(const f32x4 *)(sVT + vcol * PF + 16 * rt + 4 * g);
                }
                const f32x4 bb = *(const f32x4 *)(sBeta + 16 * rt + 4 * g);
                // a transition chain has no values (its rows were read anyway, unconditionally)
                if constexpr (L::VG)
                    if (!has_v) vv = f32x4{0.f, 0.f, 0.f, 0.f};
                R[m][rt] = bb * (vv - Y[m][rt]);
            }
        }
        // (I + A) U = R by blocks: U_I = D_I (R_I - sum_{J<I} A_IJ U_J) with D_I the
        // diagonal-block inverses; every product split three ways
        bf16x4 Uh[NVT][4], Ul[NVT][4];
#pragma unroll
        for (int bI = 0; bI < 4; ++bI) {
            f32x4 acc[NVT];
#pragma unroll
            for (int m = 0; m < NVT; ++m) acc[m] = R[m][bI];
#pragma unroll
            for (int bJ = 0; bJ < bI; ++bJ) {
                bf16x4 ah, alo;
                split4(-*(const f32x4 *)(sA + (16 * bI + li) * PF + 16 * bJ + 4 * g), ah, alo);
#pragma unroll
                for (int m = 0; m < NVT; ++m) acc[m] = mma3x16(acc[m], ah, alo, Uh[m][bJ], Ul[m][bJ]);
            }
            bf16x4 dh, dl;
            split4(*(const f32x4 *)(sT + (16 * bI + li) * PF + 16 * bI + 4 * g), dh, dl);
#pragma unroll
            for (int m = 0; m < NVT; ++m) {
                bf16x4 xh, xl;
                split4(acc[m], xh, xl);
                split4(mma3x16(zero4(), dh, dl, xh, xl), Uh[m][bI], Ul[m][bI]);
            }
        }
        if (FW) {
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
                                        cat(Ul[m][2 * jb], Ul[m][2 * jb + 1]), !LITE, !LITE);
                }
#pragma unroll
                for (int m = 0; m < NVT; ++m) {
                    const int col = col0 + 16 * (w * NVT + m) + li;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int i = 16 * rt + 4 * g + s;
                        if (i < n) st_out<IN16>(obase, ((t0 - orow + i) * H + h) * DV + col, a.scale * Z[m][rt][s]);
                    }
                }
            }
        }
        if constexpr (PFX)
            if (ck + 1 < n_chunks) fetch(ck + 1);
        {
            // software-pipelined over the key tiles: the operand rows of tile ct + 1 are
            // requested before the products of tile ct
            f32x4 eg[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) eg[ct] = *(const f32x4 *)(sEG + 16 * ct + 4 * g);
            float xc[2][8], xn[2][8];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) load_perm_f32(sG, PF, li, 32 * jb, g, xc[jb]);  // (K e^{G_last - G})^T
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                if (ct + 1 < NCT)
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb) load_perm_f32(sG, PF, 16 * (ct + 1) + li, 32 * jb, g, xn[jb]);
                __builtin_amdgcn_sched_barrier(0);  // keep those reads ahead of this tile's work
#pragma unroll
                for (int m = 0; m < NVT; ++m) S[m][ct] *= eg[ct];
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    bf16x8 ah, alo;
                    split8(xc[jb], ah, alo);
#pragma unroll
                    for (int m = 0; m < NVT; ++m)
                        S[m][ct] = mma3(S[m][ct], ah, alo, cat(Uh[m][2 * jb], Uh[m][2 * jb + 1]),
                                        cat(Ul[m][2 * jb], Ul[m][2 * jb + 1]), true, true);
                }
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int s = 0; s < 8; ++s) xc[jb][s] = xn[jb][s];
            }
        }
        __syncthreads();
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
                    fin[fin_vfirst ? col * DK + c : c * DV + col] = S[m][ct][s];
                else if (isM)
                    a.M[(((int64_t)item * H + h) * DK + c) * DK + col] = S[m][ct][s];
                else
                    a.U[(((int64_t)item * H + h) * DK + c) * DV + col] = S[m][ct][s];
            }
    }
}

template <int DK, int DVS, bool IN16, int MODE>
__global__ __launch_bounds__(NT, 1) void kda_chain_kernel(ChainArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[Lds<DK, DVS, MODE>::BYTES];
    constexpr bool FW = (MODE == MODE_FWD);
    const int H = a.H;
    // ---- work item: XCD-aware order keeps the slices of one (item, head) on one XCD
    const int n_units = a.n_items * H;
    const int lin = blockIdx.x;
    const int xcd = lin & 7, jx = lin >> 3;
    const int slice = jx % a.n_slices;
    const int unit = (jx / a.n_slices) * 8 + xcd;
    if (unit >= n_units) return;
    const int item = unit / H, h = unit - item * H;
    const int t_begin = a.offsets[item], t_end = a.offsets[item + 1];
    if (FW && t_end <= t_begin) return;  // empty sequence: slot untouched, no rows
    float *fin = FW ? a.state_pool + ((int64_t)a.state_indices[item] * H + h) * DK * DK : nullptr;
    chain_unit<DK, DVS, IN16, MODE>(a, smem, item, h, t_begin, t_end, slice, 0, true, a.v_first, fin, a.out, 0);
}

// The forward pass of a load-balanced plan (bf16 inputs): persistent workgroups take the
// planner's queued units (whole sequences, and the transition and contribution chains of
// later pieces) until the queue is drained.
template <int DK>
__global__ __launch_bounds__(NT, 1) void kda_chain_planned_kernel(ChainArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[Lds<DK, DK, MODE_FWD>::BYTES];
    __shared__ int s_next;
    const int H = a.H;
    for (;;) {
        if (threadIdx.x == 0) s_next = atomicAdd((int *)&a.plan->ctr, 1);
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
        const int h = qy & 0xffff, role = qy >> 16;
        const int sb = a.offsets[seq], se = a.offsets[seq + 1];
        const int t_begin = sb + CH * cbeg, t_end = min(se, sb + CH * cend);
        if (t_end <= t_begin) continue;
        // whole sequence: from and to its slot; transition chain of a later piece: from the
        // identity, no values, its outputs the piece's correction rows; contribution chain:
        // from zero
        int init = 0;
        bool v_on = true, vf = a.v_first;
        float *fin = a.state_pool + ((int64_t)a.state_indices[seq] * H + h) * DK * DK;
        void *obase = a.out;
        int64_t orow = 0;
        if (role == ROLE_M) {
            init = 1;
            v_on = false;
            vf = false;
            fin = a.ws_M + ((int64_t)piece * H + h) * DK * DK;
            obase = a.ws_W;
            orow = t_begin - CH * (int64_t)__builtin_amdgcn_readfirstlane(a.ws_piece[piece].w);
        } else if (role == ROLE_U) {
            init = 2;
            vf = false;
            fin = a.ws_U + ((int64_t)piece * H + h) * DK * DK;
        }
        chain_unit<DK, DK, true, MODE_FWD>(a, smem, seq, h, t_begin, t_end, 0, init, v_on, vf, fin, obase, orow);
    }
}

template <int DK, int DVS, bool IN16, int MODE>
static hipError_t launch_one(const ChainArgs &a0, hipStream_t stream) {
    ChainArgs a = a0;
    a.n_slices = (MODE == MODE_FWD ? DK : 2 * DK) / DVS;  // value (or [M | U]) column slices
    const int n_units = a.n_items * a.H;
    const int groups = (n_units + 7) / 8;
    const dim3 grid(8 * a.n_slices * groups);
    hipLaunchKernelGGL((kda_chain_kernel<DK, DVS, IN16, MODE>), grid, dim3(NT), 0, stream, a);
    return hipGetLastError();
}

// Slice width dk: one workgroup per (sequence, head) in the forward pass and two (the
// transition and the contribution columns) for summaries, so that the gate, the scores,
// the inverse and the chain operands of a chunk are formed once per column block of dk.
template <bool IN16, int MODE>
static hipError_t launch_dk(const ChainArgs &a, int dk, hipStream_t stream) {
    if (dk == 128) return launch_one<128, 128, IN16, MODE>(a, stream);
    if (dk == 64) return launch_one<64, 64, IN16, MODE>(a, stream);
    return hipErrorInvalidValue;
}

// The forward pass of a load-balanced plan on bf16 inputs: persistent workgroups (one per
// CU) take the planner's queued units (whole sequences, and the transition and contribution
// chains of later pieces).
hipError_t launch_chain_planned(const ChainArgs &a0, int dk, int n_wg, hipStream_t stream) {
    ChainArgs a = a0;
    a.n_slices = 1;
    if (dk == 128)
        hipLaunchKernelGGL(kda_chain_planned_kernel<128>, dim3(n_wg), dim3(NT), 0, stream, a);
    else if (dk == 64)
        hipLaunchKernelGGL(kda_chain_planned_kernel<64>, dim3(n_wg), dim3(NT), 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_chain(const ChainArgs &a, int dk, bool bf16_in, int mode, hipStream_t stream) {
    if (mode == MODE_FWD)
        return bf16_in ? launch_dk<true, MODE_FWD>(a, dk, stream) : launch_dk<false, MODE_FWD>(a, dk, stream);
    return bf16_in ? launch_dk<true, MODE_SUMMARY>(a, dk, stream) : launch_dk<false, MODE_SUMMARY>(a, dk, stream);
}

}  // namespace kda
