// kda_plan.hip -- load-balanced forward pass: long sequences are cut into pieces that
// run in parallel (bf16, dk = dv in {64, 128}).
//
// A (sequence, head) chain is sequential, so one long sequence would bound the kernel
// while short ones leave their CUs idle.  The context-parallel construction of the "KDA
// Context Parallelism" page (Theory; Incoming and outgoing states) applies inside one
// GPU as well: a piece started from state X has S_t = M_t X + U_t, where M_t is the
// piece's transition up to token t (the chain started from I with no values) and U_t
// its contribution (the chain started from 0).  Hence
//     o_t = scale q_t^T S_t = (scale q_t^T M_t) X + scale q_t^T U_t = W_t X + O_U,t,
// and both chains run without knowing X.  Per forward call:
//   1. plan_kernel (one workgroup) chooses a first-piece length L, cuts every sequence
//      longer than 9L/8 into a first piece of L chunks plus near-equal later pieces of at
//      most L chunks, and lists the units, longest first, in one queue (the two chains of
//      a later piece next to each other);
//   2. kda_fast_kernel drains the queue: whole sequences and first pieces run from the
//      pool slot as usual; a later piece runs its transition chain (W_t rows into the W
//      buffer, final M) and its contribution chain (O_U rows into out, final U);
//   3. piece_scan_kernel walks each split sequence's pieces in order: the incoming
//      state of a piece is X_k, X_{k+1} = M_k X_k + U_k, the last one goes to the slot;
//   4. fixup_kernel adds W_t X_k to the outputs of every later piece.
// L is the smallest length for which the total work (a later piece costs two chains)
// spread over all CUs fits in L chunks and the units longer than L/2 (no two of which
// fit on one CU within L) are no more than the CUs, so the makespan stays near L.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

namespace plan {

constexpr int PT = 1024;   // planner threads
constexpr int PT_ONE = 64; // threads of the one-wave planner (at most 64 entities)
constexpr int NBIN = 1024; // length bins of the longest-first order
constexpr int L_MIN = 4;   // shortest first piece worth a split, in chunks
constexpr int NCACHE = 4096;  // sequences whose chunk counts the planner keeps in LDS
constexpr int ECACHE = 1024;  // entities the planner keeps in LDS

static_assert(NBIN == PT, "one bin per planner thread");

struct PlanArgs {
    const int32_t *cu;
    const int32_t *state_indices;
    int B, H, n_cu;  // n_cu: workgroups of the chunk kernel that run at once
    int cs;          // tokens per chunk
    PlanHeader *hdr;
    int2 *queue;
    int4 *ent;
    int4 *piece;   // (first token, end token, chunks, prefix of later-piece chunks)
    int4 *sseq;    // (sequence, first later piece, number of later pieces, pool slot)
    int *sorted;
    int np_cap, ent_cap;
    int w_cap;     // chunks of later pieces the W rows can hold
};

__device__ __forceinline__ int chunks_of(const int32_t *cu, int b, int cs) {
    const int len = cu[b + 1] - cu[b];
    return len > 0 ? (len + cs - 1) / cs : 0;
}

// Sum / max over the workgroup of NT threads; every thread gets the result.  With one
// wave the lane exchanges suffice: no LDS, no barrier.
template <int NT>
__device__ int64_t block_sum(int64_t v, int64_t *red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if constexpr (NT == 64) return v;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    int64_t s = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) s += red[i];
    return s;
}
template <int NT>
__device__ int block_max(int v, int64_t *red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
    if constexpr (NT == 64) return v;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    int m = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) m = max(m, (int)red[i]);
    return m;
}
// Exclusive prefix sum over the threads of the workgroup; total returned in *tot.
template <int NT>
__device__ int block_excl_scan(int v, int64_t *red, int *tot) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if constexpr (NT == 64) {
        *tot = __shfl(x, 63);
        return x - v;
    }
    __syncthreads();
    if (lane == 63) red[wv] = x;
    __syncthreads();
    int base = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        const int r = (int)red[i];
        if (i < wv) base += r;
        all += r;
    }
    *tot = all;
    return base + x - v;
}

// Three exclusive prefix sums at once (one pair of barriers).
template <int NT>
__device__ void block_excl_scan3(int a, int b, int c, int64_t *red, int *ea, int *eb, int *ec, int *ta,
                                 int *tb, int *tc) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int x = a, y = b, z = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int x1 = __shfl_up(x, o), y1 = __shfl_up(y, o), z1 = __shfl_up(z, o);
        if (lane >= o) {
            x += x1;
            y += y1;
            z += z1;
        }
    }
    if constexpr (NT == 64) {
        *ea = x - a;
        *eb = y - b;
        *ec = z - c;
        *ta = __shfl(x, 63);
        *tb = __shfl(y, 63);
        *tc = __shfl(z, 63);
        return;
    }
    __syncthreads();
    // per-wave totals: (x, y) packed in red, z in zred
    __shared__ int zred[NT / 64];
    if (lane == 63) {
        red[wv] = (int64_t)(((uint64_t)(uint32_t)y << 32) | (uint32_t)x);
        zred[wv] = z;
    }
    __syncthreads();
    int bx = 0, by = 0, bz = 0, ax = 0, ay = 0, az = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        const uint64_t v = (uint64_t)red[i];
        const int vx = (int)(uint32_t)v, vy = (int)(uint32_t)(v >> 32), vz = zred[i];
        if (i < wv) {
            bx += vx;
            by += vy;
            bz += vz;
        }
        ax += vx;
        ay += vy;
        az += vz;
    }
    *ea = bx + x - a;
    *eb = by + y - b;
    *ec = bz + z - c;
    *ta = ax;
    *tb = ay;
    *tc = az;
}

// NT = PT: any plan.  NT = PT_ONE: one wave, for at most 64 entities (sequences plus
// later pieces), whose reductions need no barrier and whose longest-first order is an
// exact rank sort.
template <int NT>
__global__ __launch_bounds__(NT) void plan_kernel(PlanArgs p) {
    constexpr bool ONE = NT == PT_ONE;
    constexpr int NC = ONE ? PT_ONE : NCACHE, EC = ONE ? PT_ONE : ECACHE;
    __shared__ int64_t red[NT / 64];
    __shared__ int hist[ONE ? 1 : NBIN];
    __shared__ int sn[NC];
    __shared__ int4 sent[EC];
    __shared__ int ssort[EC];
    const int t = threadIdx.x;
    const int B = p.B, H = p.H;
    const bool cached = B <= NC;
    // one wave: thread b owns sequence b throughout; its slot is fetched with the lengths
    const int si_own = (ONE && t < B) ? p.state_indices[t] : 0;
    if (cached)
        for (int b = t; b < B; b += NT) sn[b] = chunks_of(p.cu, b, p.cs);
    __syncthreads();
    auto chunks = [&](int b) { return cached ? sn[b] : chunks_of(p.cu, b, p.cs); };

    // ---- chunk totals
    int64_t s_loc = 0;
    int m_loc = 0;
    for (int b = t; b < B; b += NT) {
        const int n = chunks(b);
        s_loc += n;
        m_loc = max(m_loc, n);
    }
    const int64_t S = block_sum<NT>(s_loc, red);
    const int maxn = block_max<NT>(m_loc, red);

    // ---- first-piece length: smallest L >= average load with H (S + E(L)) <= n_cu L,
    // E(L) = chunks moved into later pieces (they run twice), such that the later pieces
    // P(L) and their chunks E(L) fit the workspace (np_cap, w_cap).  All three conditions
    // only get easier as L grows, and L = maxn splits nothing.
    const int64_t L0 = max((int64_t)L_MIN, ((int64_t)H * S + p.n_cu - 1) / p.n_cu);
    int L = 0;
    if (8 * (int64_t)maxn > 9 * L0) {
        int lo = (int)L0, hi = maxn;
        while (lo < hi) {  // uniform: every thread sees the same sums
            const int mid = lo + (hi - lo) / 2;
            int64_t ep = 0;  // chunks moved (high 32 bits) and pieces (low 32 bits)
            for (int b = t; b < B; b += NT) {
                const int n = chunks(b);
                if (8 * (int64_t)n > 9 * (int64_t)mid)
                    ep += ((int64_t)(n - mid) << 32) + (n - mid + mid - 1) / mid;
            }
            const int64_t EP = block_sum<NT>(ep, red);
            const int64_t E = EP >> 32, P = EP & 0xffffffff;
            if ((int64_t)H * (S + E) <= (int64_t)p.n_cu * mid && E <= p.w_cap && P <= p.np_cap) hi = mid;
            else lo = mid + 1;
        }
        L = lo;
        // Units longer than L/2 cannot share a CU within about L: while they outnumber
        // the CUs, lengthen the pieces (fewer, longer units).
        while (L < maxn) {
            int64_t big = 0;
            for (int b = t; b < B; b += NT) {
                const int n = chunks(b);
                if (8 * (int64_t)n > 9 * (int64_t)L) {
                    const int R = n - L, P = (R + L - 1) / L, base = R / P, rem = R % P;
                    big += 1 + 2 * ((2 * (base + 1) > L ? rem : 0) + (2 * base > L ? P - rem : 0));
                } else if (2 * n > L) {
                    big += 1;
                }
            }
            if ((int64_t)H * block_sum<NT>(big, red) <= p.n_cu) break;
            L = max(L + 1, (int)((int64_t)L * 17 / 16));
        }
        if (!(8 * (int64_t)maxn > 9 * (int64_t)L)) L = 0;
    }

    // ---- pieces: each thread owns a contiguous range of sequences, so the later
    // pieces of one sequence get consecutive indices
    const int per = (B + NT - 1) / NT;
    const int b0 = min(B, t * per), b1 = min(B, b0 + per);
    int my_p = 0, my_s = 0, my_e = 0;
    auto split_of = [&](int n) { return L > 0 && 8 * (int64_t)n > 9 * (int64_t)L; };
    for (int b = b0; b < b1; ++b) {
        const int n = chunks(b);
        if (split_of(n)) {
            my_p += (n - L + L - 1) / L;
            my_s += 1;
            my_e += n - L;
        }
    }
    int tot_p, tot_s, tot_e, kb, jb, eb;
    block_excl_scan3<NT>(my_p, my_s, my_e, red, &kb, &jb, &eb, &tot_p, &tot_s, &tot_e);
    if (tot_p > p.np_cap || B + tot_p > p.ent_cap) {  // cannot happen by the sizing; stay safe
        L = 0;
        tot_p = tot_s = tot_e = 0;
    }
    const int n_ent = B + tot_p;
    const bool ecached = n_ent <= EC;
    auto put_ent = [&](int e, int4 v) {
        p.ent[e] = v;
        if (ecached) sent[e] = v;
    };
    auto ent_at = [&](int e) { return ecached ? sent[e] : p.ent[e]; };
    for (int b = b0; b < b1; ++b) {
        const int n = chunks(b);
        if (split_of(n)) {
            const int R = n - L, P = (R + L - 1) / L, base = R / P, rem = R % P;
            p.sseq[jb] = make_int4(b, kb, P, ONE ? si_own : p.state_indices[b]);
            const int cb = p.cu[b], ce = p.cu[b + 1];
            int c = L;
            for (int i = 0; i < P; ++i) {
                const int len = base + (i < rem ? 1 : 0);
                p.piece[kb + i] = make_int4(cb + p.cs * c, min(ce, cb + p.cs * (c + len)), len, eb);
                put_ent(B + kb + i, make_int4(b, c, c + len, kb + i));
                c += len;
                eb += len;
            }
            put_ent(b, make_int4(b, 0, L, -1));
            kb += P;
            jb += 1;
        } else {
            put_ent(b, make_int4(b, 0, n, -1));
        }
    }
    __syncthreads();

    // ---- longest first
    int n_sorted;
    if constexpr (ONE) {
        // exact rank: entity e goes after every longer one and every equally long one
        // with a smaller index (n_ent <= 64, all in LDS)
        const int len = t < n_ent ? sent[t].z - sent[t].y : 0;
        int rank = 0;
        for (int f = 0; f < n_ent; ++f) {
            const int lf = sent[f].z - sent[f].y;
            rank += (lf > len || (lf == len && f < t)) ? 1 : 0;
        }
        n_sorted = __popcll(__ballot(len > 0));
        if (len > 0) ssort[rank] = t;
        __syncthreads();
    } else {
        // counting sort of the entities on 1024 length bins
        int ml = 0;
        for (int e = t; e < n_ent; e += NT) {
            const int4 en = ent_at(e);
            ml = max(ml, en.z - en.y);
        }
        const int maxlen = max(1, block_max<NT>(ml, red));
        hist[t] = 0;
        __syncthreads();
        for (int e = t; e < n_ent; e += NT) {
            const int4 en = ent_at(e);
            const int len = en.z - en.y;
            if (len > 0) atomicAdd(&hist[NBIN - 1 - (int)((int64_t)len * (NBIN - 1) / maxlen)], 1);
        }
        __syncthreads();
        const int start = block_excl_scan<NT>(hist[t], red, &n_sorted);
        __syncthreads();
        hist[t] = start;
        __syncthreads();
        for (int e = t; e < n_ent; e += NT) {
            const int4 en = ent_at(e);
            const int len = en.z - en.y;
            if (len > 0) {
                const int pos = atomicAdd(&hist[NBIN - 1 - (int)((int64_t)len * (NBIN - 1) / maxlen)], 1);
                if (ecached) ssort[pos] = e;
                else p.sorted[pos] = e;
            }
        }
        __syncthreads();
    }
    // ---- one queue for every workgroup: super unit s = (rank, head) takes slots 2s and
    // 2s + 1 (the contribution chain of a later piece, else a skip slot). One queue packs
    // the units over all CUs at once; per-XCD queues, which kept the two chains of a
    // piece on one L2, measured slower (the second chain's re-read of k, q and the gates
    // costs less than the coarser packing).
    const int64_t NS = (int64_t)n_sorted * H;
    for (int64_t s = t; s < NS; s += NT) {
        const int r = (int)(s / H), hh = (int)(s - (int64_t)r * H);
        const int e = ecached ? ssort[r] : p.sorted[r];
        const bool pair = ent_at(e).w >= 0;
        int2 *q = p.queue + 2 * s;
        q[0] = make_int2(e, hh | ((pair ? ROLE_M : ROLE_WHOLE) << 16));
        q[1] = pair ? make_int2(e, hh | (ROLE_U << 16)) : make_int2(0, -1);
    }
    if (t == 0) {
        p.hdr->ctr = 0;
        p.hdr->qlen = (int)(2 * NS);
        p.hdr->n_split = tot_s;
        p.hdr->n_piece = tot_p;
        p.hdr->n_echunk = tot_e;
        p.hdr->L = L;
        p.hdr->n_ent = n_ent;
        p.hdr->n_sorted = n_sorted;
    }
}

struct PieceArgs {
    const PlanHeader *hdr;
    const int4 *piece, *sseq;
    const int32_t *cu;
    const int32_t *state_indices;
    float *state_pool;
    const float *M, *U;
    bf16_t *XT;     // [n_piece][H][dv][dk]: incoming state of each later piece, transposed
    const bf16_t *W;
    bf16_t *out;
    int H;
    int v_first;    // pool slots stored [dv][dk]
    int cs;         // tokens per chunk (a correction task covers one chunk, at most 64)
};

// Incoming states of the later pieces, in order, and the final state into the slot.
// Task = (split sequence, head, 16-column block): X_{k+1} = M_k X_k + U_k on those
// columns with fp32 16x16x4 MFMAs (products and sums in fp32, as the recurrence needs).
// Wave w owns rows RW w .. RW w + RW - 1 (RW = dk/4: TT = dk/64 tiles of 16 rows); lane
// (g, li) holds rows RW w + 16tt + 4g + s of column li, the accumulator layout.  The
// contraction index of MFMA step kk on lane quarter g is KQ g + kk (KQ = dk/4), so a
// lane's A operands are KQ consecutive entries of one row of M_k (16-byte loads) and its
// B operands one column of X_k from LDS, skewed by 16 floats per quarter so the four
// quarters read distinct banks.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
template <int DK>
__device__ __forceinline__ int sx_at(int k, int c) { return 16 * k + c + 16 * (k / (DK / 4)); }

template <int DK>
__global__ __launch_bounds__(256) void piece_scan_kernel(PieceArgs p) {
    constexpr int DV = DK, TT = DK / 64, RW = DK / 4, KQ = DK / 4, NCB = DV / 16;
    __shared__ float sx[16 * DK + 16 * 4];
    const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 4, li = l & 15;
    const int H = p.H;
    const int n_tasks = p.hdr->n_split * H * NCB;
    // The column blocks of one (sequence, head) read the same M_k: keep them on one XCD
    // (workgroups are dealt to the XCDs round-robin), so M_k comes from HBM once.
    for (int lin = blockIdx.x; lin < (n_tasks + 8 * NCB - 1) / (8 * NCB) * (8 * NCB); lin += gridDim.x) {
        const int cb = (lin >> 3) % NCB, jh = (lin / (8 * NCB)) * 8 + (lin & 7);
        if (jh >= p.hdr->n_split * H) continue;  // uniform over the workgroup
        const int h = jh % H, j = jh / H;
        const int4 sq = p.sseq[j];
        const int col = 16 * cb + li;
        float *slot = p.state_pool + ((int64_t)sq.w * H + h) * DK * DV;
        // X_k of this lane: rows RW w + 16tt + 4g + s, column col
        f32x4 x[TT];
        auto slot_at = [&](int r) -> float & { return p.v_first ? slot[col * DK + r] : slot[r * DV + col]; };
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int s = 0; s < 4; ++s) x[tt][s] = slot_at(RW * w + 16 * tt + 4 * g + s);
        for (int i = 0; i < sq.z; ++i) {
            const int64_t kh = (int64_t)(sq.y + i) * H + h;
            // M_k rows and U_k entries are independent of X_k: issue them first
            f32x4 ma[TT][KQ / 4], acc[TT];
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                const float *Mr = p.M + kh * DK * DK + (int64_t)(RW * w + 16 * tt + li) * DK + KQ * g;
#pragma unroll
                for (int q = 0; q < KQ / 4; ++q) ma[tt][q] = *(const f32x4 *)(Mr + 4 * q);
                const float *Ur = p.U + kh * DK * DV + (int64_t)(RW * w + 16 * tt + 4 * g) * DV + col;
#pragma unroll
                for (int s = 0; s < 4; ++s) acc[tt][s] = Ur[s * DV];
            }
            // the correction's MFMA reads X_k^T rows (one column of X_k) as bf16
            bf16_t *xt = p.XT + kh * DV * DK + (int64_t)col * DK + RW * w + 4 * g;
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) *(bf16x4 *)(xt + 16 * tt) = bf4(x[tt]);
            __syncthreads();  // every wave is done reading the previous X from LDS
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int s = 0; s < 4; ++s) sx[sx_at<DK>(RW * w + 16 * tt + 4 * g + s, li)] = x[tt][s];
            __syncthreads();
#pragma unroll
            for (int q = 0; q < KQ / 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float bx = sx[sx_at<DK>(KQ * g + 4 * q + e, li)];
#pragma unroll
                    for (int tt = 0; tt < TT; ++tt) acc[tt] = mfma_f32(ma[tt][q][e], bx, acc[tt]);
                }
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) x[tt] = acc[tt];
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int s = 0; s < 4; ++s) slot_at(RW * w + 16 * tt + 4 * g + s) = x[tt][s];
        __syncthreads();
    }
}

// out_t += W_t X_k for every token of every later piece.  Task = (piece, head, chunk),
// numbered piece-major; a workgroup takes FIX_TASKS consecutive tasks (mostly one piece
// and head), decodes them from the piece table staged once in LDS, and stages X_k^T (bf16,
// written by piece_scan_kernel) in LDS when the piece or head changes.  Wave w owns the
// 16 tokens 16w .. 16w+15 of the chunk and all dv columns, C^T = X^T W^T with 16x16x32
// bf16 MFMAs: each W row is read once.  The column tiles go in pairs whose A rows are
// permuted (fix_col) so that a lane's outputs of the pair are 8 consecutive columns of one
// token: 16-byte read-modify-writes of out, 64 contiguous bytes per token and instruction.
constexpr int FIX_NP = 256;   // pieces staged in LDS (more: read from global memory)
constexpr int FIX_TASKS = 4;  // tasks per group (1, 2 and 4 measured within 10% of each other)

// Column of out (row of X^T) behind A row li of column tile 2q + hf: the lane quarter g of
// the pair's outputs then holds columns 32q + 8g .. 32q + 8g + 7.
__device__ __forceinline__ int fix_col(int q, int hf, int li) { return 32 * q + 8 * (li >> 2) + 4 * hf + (li & 3); }
// Staged X^T row r: a pitch of dk + 8 elements plus 32 elements (four groups of 4 LDS banks)
// per 16 rows, so that the 16 rows of a permuted tile start in distinct bank groups.
template <int DK>
__device__ __forceinline__ int fix_row(int r) { return r * (DK + 8) + 32 * (r >> 4); }

template <int DK>
__global__ __launch_bounds__(256) void fixup_kernel(PieceArgs p) {
    constexpr int DV = DK;
    __shared__ int4 spc[FIX_NP];
    __shared__ __attribute__((aligned(16))) bf16_t sxt[DV * (DK + 8) + 32 * (DV / 16)];
    const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 4, li = l & 15;
    const int H = p.H;
    const int n_piece = p.hdr->n_piece;
    const int64_t n_tasks = (int64_t)p.hdr->n_echunk * H;
    if ((int64_t)blockIdx.x * FIX_TASKS >= n_tasks) return;
    const bool staged = n_piece <= FIX_NP;
    if (staged)
        for (int i = t; i < n_piece; i += 256) spc[i] = p.piece[i];
    __syncthreads();
    auto piece_at = [&](int i) { return staged ? spc[i] : p.piece[i]; };
    // The k-th task of this workgroup: groups of FIX_TASKS consecutive tasks, strided over
    // the grid; -1 past the last (every later k is past it too).
    auto task_of = [&](int64_t k) -> int64_t {
        const int64_t grp = blockIdx.x + (k / FIX_TASKS) * gridDim.x;
        const int64_t task = grp * FIX_TASKS + k % FIX_TASKS;
        return task < min(n_tasks, (grp + 1) * FIX_TASKS) ? task : -1;
    };
    struct Task {
        int key, t0, n, h;
        int64_t rowh;  // this lane's row (token, head); rows past the chunk's end repeat its last
        int64_t roww;  // the same row of the chunk-compact W buffer
    };
    auto decode = [&](int64_t task) {
        int lo = 0, hi = n_piece - 1;  // last piece whose task range starts at or before task
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((int64_t)H * piece_at(mid).w <= task) lo = mid;
            else hi = mid - 1;
        }
        const int4 pc = piece_at(lo);
        const int len = pc.z;
        const int64_t rem = task - (int64_t)H * pc.w;
        Task k;
        k.h = (int)(rem / len);
        const int c = (int)(rem - (int64_t)k.h * len);
        k.key = lo * H + k.h;
        k.t0 = pc.x + p.cs * c;
        k.n = min(p.cs, pc.y - k.t0);
        const int r = min(16 * w + li, k.n - 1);
        k.rowh = (int64_t)(k.t0 + r) * H + k.h;
        k.roww = ((int64_t)(pc.w + c) * p.cs + r) * H + k.h;
        return k;
    };
    bf16x8 bw[DK / 32];
    bf16x8 ov[DV / 32];
    auto load = [&](const Task &k, bf16x8 (&b)[DK / 32], bf16x8 (&o)[DV / 32]) {
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) b[kb] = *(const bf16x8 *)(p.W + k.roww * DK + 32 * kb + 8 * g);
#pragma unroll
        for (int q = 0; q < DV / 32; ++q) o[q] = *(const bf16x8 *)(p.out + k.rowh * DV + 32 * q + 8 * g);
    };
    int cur = -1;
    int64_t tk = task_of(0);  // valid: this workgroup has at least one task
    Task tc = decode(tk);
    load(tc, bw, ov);
    for (int64_t k = 0; tk >= 0; ++k) {
        // the next task's rows are in flight while this one is corrected (tasks cover
        // disjoint rows, so the early reads of out see no store of this workgroup)
        const int64_t tn = task_of(k + 1);
        Task nt = tc;
        bf16x8 bwn[DK / 32];
        bf16x8 ovn[DV / 32];
        if (tn >= 0) {  // uniform over the workgroup
            nt = decode(tn);
            load(nt, bwn, ovn);
        }
        if (tc.key != cur) {  // uniform over the workgroup
            __syncthreads();  // every wave is done with the previous X^T
            const bf16_t *xt = p.XT + (int64_t)tc.key * DV * DK;
#pragma unroll
            for (int i = 0; i < DV * DK / (8 * 256); ++i) {
                const int e = 8 * (t + 256 * i), r = e / DK, cc = e - r * DK;
                *(bf16x8 *)(sxt + fix_row<DK>(r) + cc) = *(const bf16x8 *)(xt + e);
            }
            __syncthreads();
            cur = tc.key;
        }
        // a wave past the end of a short chunk only joins the barriers
        const bool store = 16 * w + li < tc.n;
        bf16_t *o = p.out + ((int64_t)(tc.t0 + 16 * w + li) * H + tc.h) * DV + 8 * g;
#pragma unroll
        for (int q = 0; q < DV / 32; ++q) {
            const bf16x8 oq = ov[q];
            f32x4 acc0 = f4(bf16x4{oq[0], oq[1], oq[2], oq[3]}), acc1 = f4(bf16x4{oq[4], oq[5], oq[6], oq[7]});
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                acc0 = mfma(*(const bf16x8 *)(sxt + fix_row<DK>(fix_col(q, 0, li)) + 32 * kb + 8 * g), bw[kb], acc0);
                acc1 = mfma(*(const bf16x8 *)(sxt + fix_row<DK>(fix_col(q, 1, li)) + 32 * kb + 8 * g), bw[kb], acc1);
            }
            if (store) *(bf16x8 *)(o + 32 * q) = cat(bf4(acc0), bf4(acc1));
        }
        tk = tn;
        tc = nt;
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) bw[kb] = bwn[kb];
#pragma unroll
        for (int q = 0; q < DV / 32; ++q) ov[q] = ovn[q];
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace plan

namespace {
// Offsets of every part for given capacities; W last.
PlanLayout layout_for(int B, int H, int dk, int dv, int np_cap, int64_t w_cap) {
    PlanLayout y;
    y.np_cap = np_cap;
    y.w_cap = (int)w_cap;
    y.ent_cap = B + y.np_cap;
    y.qcap = (int)(2 * (int64_t)y.ent_cap * H);
    size_t o = 0;
    y.hdr = o;
    o = plan::align256(o + sizeof(PlanHeader));
    y.queue = o;
    o = plan::align256(o + (size_t)y.qcap * sizeof(int2));
    y.ent = o;
    o = plan::align256(o + (size_t)y.ent_cap * sizeof(int4));
    y.piece = o;
    o = plan::align256(o + (size_t)y.np_cap * sizeof(int4));
    y.sseq = o;
    o = plan::align256(o + (size_t)y.np_cap * sizeof(int4));
    y.sorted = o;
    o = plan::align256(o + (size_t)y.ent_cap * sizeof(int));
    const size_t st = (size_t)y.np_cap * H * dk * dv * sizeof(float);
    y.M = o;
    o = plan::align256(o + (size_t)y.np_cap * H * dk * dk * sizeof(float));
    y.U = o;
    o = plan::align256(o + st);
    y.XT = o;  // X^T of the later pieces, bf16
    o = plan::align256(o + (size_t)y.np_cap * H * dk * dv * sizeof(bf16_t));
    y.W = o;
    o = plan::align256(o + (size_t)w_cap * 64 * H * dv * sizeof(bf16_t));
    y.total = o;
    return y;
}
}  // namespace

PlanLayout plan_layout(int64_t T, int B, int H, int dk, int dv, int n_slots, size_t max_bytes, bool *ok) {
    // later pieces per head <= total chunks / L <= n_slots / H (L is at least the average
    // load); twice that plus slack.  Chunks of later pieces: at most every chunk.
    const int np_full = 2 * ((n_slots + H - 1) / H) + 2;
    const int64_t w_full = (T + 63) / 64 + B;
    if (ok) *ok = true;
    PlanLayout y = layout_for(B, H, dk, dv, np_full, w_full);
    if (max_bytes == 0 || y.total <= max_bytes) return y;
    // Fit max_bytes: the W rows first, then fewer pieces.
    for (int np = np_full; np >= 0; np = np > 0 ? np / 2 : -1) {
        y = layout_for(B, H, dk, dv, np, 0);
        if (y.total <= max_bytes) {
            const size_t per_chunk = (size_t)64 * H * dv * sizeof(bf16_t);
            const int64_t wc = (int64_t)((max_bytes - y.total) / per_chunk);
            return layout_for(B, H, dk, dv, np, wc < w_full ? wc : w_full);
        }
        if (np == 0) break;
    }
    if (ok) *ok = false;
    return y;
}

hipError_t launch_planned_fwd(ChainArgs a, int dk, char *ws, const PlanLayout &lay, int n_cu,
                              const FwdKernel &fk, hipStream_t stream) {
    if (dk != 64 && dk != 128) return hipErrorInvalidValue;
    plan::PlanArgs pa;
    pa.cu = a.offsets;
    pa.state_indices = a.state_indices;
    pa.B = a.n_items;
    pa.H = a.H;
    pa.n_cu = fk.per_cu * n_cu;
    pa.cs = fk.chunk;
    pa.hdr = (PlanHeader *)(ws + lay.hdr);
    pa.queue = (int2 *)(ws + lay.queue);
    pa.ent = (int4 *)(ws + lay.ent);
    pa.piece = (int4 *)(ws + lay.piece);
    pa.sseq = (int4 *)(ws + lay.sseq);
    pa.sorted = (int *)(ws + lay.sorted);
    pa.np_cap = lay.np_cap;
    pa.ent_cap = lay.ent_cap;
    pa.w_cap = lay.w_cap;
    if (lay.ent_cap <= plan::PT_ONE)
        hipLaunchKernelGGL(plan::plan_kernel<plan::PT_ONE>, dim3(1), dim3(plan::PT_ONE), 0, stream, pa);
    else
        hipLaunchKernelGGL(plan::plan_kernel<plan::PT>, dim3(1), dim3(plan::PT), 0, stream, pa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    a.plan = pa.hdr;
    a.queue = pa.queue;
    a.ent = pa.ent;
    a.ws_M = (float *)(ws + lay.M);
    a.ws_U = (float *)(ws + lay.U);
    a.ws_W = ws + lay.W;
    a.ws_piece = pa.piece;
    e = fk.precise ? launch_chain_planned(a, dk, fk.per_cu * n_cu, stream)
                   : launch_fast_planned(a, dk, fk.per_cu * n_cu, stream);
    if (e != hipSuccess) return e;

    plan::PieceArgs pp;
    pp.hdr = pa.hdr;
    pp.piece = pa.piece;
    pp.sseq = pa.sseq;
    pp.cu = a.offsets;
    pp.state_indices = a.state_indices;
    pp.state_pool = a.state_pool;
    pp.M = a.ws_M;
    pp.U = a.ws_U;
    pp.XT = (bf16_t *)(ws + lay.XT);
    pp.W = (const bf16_t *)a.ws_W;
    pp.out = (bf16_t *)a.out;
    pp.H = a.H;
    pp.v_first = a.v_first;
    pp.cs = fk.chunk;
    if (lay.np_cap == 0) return hipSuccess;  // no room for pieces: nothing was split
    // grids sized from capacities (the counts are known on the device only): every scan
    // task of a full plan at once; surplus workgroups find no task and exit
    const int ncb = dk / 16;  // 16-column blocks of the state
    const int scan_grid = min((lay.np_cap * a.H * ncb + 8 * ncb - 1) / (8 * ncb) * (8 * ncb), 4 * n_cu);
    if (dk == 128)
        hipLaunchKernelGGL(plan::piece_scan_kernel<128>, dim3(scan_grid), dim3(256), 0, stream, pp);
    else
        hipLaunchKernelGGL(plan::piece_scan_kernel<64>, dim3(scan_grid), dim3(256), 0, stream, pp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (dk == 128)
        hipLaunchKernelGGL(plan::fixup_kernel<128>, dim3(4 * n_cu), dim3(256), 0, stream, pp);
    else
        hipLaunchKernelGGL(plan::fixup_kernel<64>, dim3(4 * n_cu), dim3(256), 0, stream, pp);
    return hipGetLastError();
}

}  // namespace kda
