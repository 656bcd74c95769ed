/*
 * kda_oracle.c -- plain, slow fp64 CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or constant with the GPU
 * library; it is compiled on its own with gcc (no -ffast-math, no intrinsics).
 *
 * What it computes, and where each step comes from:
 *
 *   Gate (reading; the kda_chunk API page lists raw_gate as the gate input to
 *   which dt_bias is still to be added, plus a_log and dt_bias, but gives no
 *   formula):
 *       x_c  = raw_gate[t,c] + dt_bias[c]
 *       la_c = -exp(a_log) * softplus(x_c),  softplus(x) = max(x,0)+log1p(exp(-|x|))
 *       gate_mode "safe" (kda_chunk API page, gate_mode parameter): la_c = max(la_c, lb)
 *       alpha_c = exp(la_c)
 *   Beta (kda_chunk API page, beta_mode parameter): "logits" applies the
 *       sigmoid, "probability" uses the value as given.
 *   One token step (nx_nofloat_kda.nx source, header comment and the
 *   kda_gate / kda_write / kda_forward functions):
 *       1. per-key-channel decay   S[i][j] <- alpha_i * S[i][j]
 *       2. prediction              pred = k^T S         (read of the decayed state)
 *       3. delta-rule write        S <- S + k (beta (v - pred))^T
 *       4. read-out                o = scale * q^T S    (of the updated state)
 *     which is S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T.
 *   Segment map (KDA Context Parallelism, "Theory"): F(S) = M S + U with
 *       U = the segment replayed from S = 0, M = the segment replayed from
 *       S = I with every value row set to 0.
 *   Exclusive scan (KDA Context Parallelism, "Incoming and outgoing states" and
 *   "Implementation order"): W = S_init; for each segment in order: record W as
 *   incoming, W = M_i W + U_i, record W as outgoing; final = W.
 *   Composition of two maps (the same page, "Theory" and "A scalar three-segment
 *   example"): F2 after F1 is S -> M2 (M1 S + U1) + U2 = (M2 M1) S + (M2 U1 + U2).
 *
 * All arrays are row-major, contiguous, double precision.
 */
#include <math.h>
#include <pthread.h>
#include <stdatomic.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- gate -- */

static double softplus(double x) {
    /* max(x,0) + log1p(exp(-|x|)): exact form, no large-x switch */
    double ax = x < 0 ? -x : x;
    return (x > 0 ? x : 0.0) + log1p(exp(-ax));
}

/* log-alpha for n tokens x dk channels of one head. */
void kda_ref_log_alpha(int64_t n, int dk, const double *raw, const double *dt_bias,
                       double a_log, int gate_mode, double lb, double *la_out) {
    double A = exp(a_log);
    for (int64_t t = 0; t < n; ++t) {
        for (int c = 0; c < dk; ++c) {
            double la = -A * softplus(raw[t * dk + c] + dt_bias[c]);
            if (gate_mode == 1 && la < lb) la = lb;
            la_out[t * dk + c] = la;
        }
    }
}

void kda_ref_beta(int64_t n, const double *logits, int beta_mode, double *beta_out) {
    for (int64_t t = 0; t < n; ++t)
        beta_out[t] = (beta_mode == 0) ? 1.0 / (1.0 + exp(-logits[t])) : logits[t];
}

/* ---------------------------------------------------------- recurrence -- */

/*
 * Token recurrence with alpha [n,dk] and beta [n] given directly.
 * S [dk,dv] is read as the initial state and overwritten by the final state.
 * q and out may be NULL (no read-out).  pred is scratch of length dv.
 */
void kda_ref_recur(int64_t n, int dk, int dv, const double *q, const double *k,
                   const double *v, const double *alpha, const double *beta,
                   double scale, double *S, double *out) {
    double *pred = (double *)malloc(sizeof(double) * (size_t)dv);
    for (int64_t t = 0; t < n; ++t) {
        const double *kt = k + t * dk, *vt = v + t * dv, *at = alpha + t * dk;
        /* 1. decay each key row by its own channel gate */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[i * dv + j] *= at[i];
        /* 2. pred = k^T S */
        for (int j = 0; j < dv; ++j) {
            double p = 0.0;
            for (int i = 0; i < dk; ++i) p += kt[i] * S[i * dv + j];
            pred[j] = p;
        }
        /* 3. S += k (beta (v - pred))^T */
        for (int j = 0; j < dv; ++j) pred[j] = beta[t] * (vt[j] - pred[j]);
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[i * dv + j] += kt[i] * pred[j];
        /* 4. o = scale * q^T S */
        if (q && out) {
            const double *qt = q + t * dk;
            for (int j = 0; j < dv; ++j) {
                double o = 0.0;
                for (int i = 0; i < dk; ++i) o += qt[i] * S[i * dv + j];
                out[t * dv + j] = scale * o;
            }
        }
    }
    free(pred);
}

/* One (sequence, head) from the raw inputs: gate, beta, recurrence. */
typedef struct {
    int64_t n;                 /* tokens                                   */
    const double *q;           /* [n,dk] or NULL                           */
    const double *k;           /* [n,dk]                                   */
    const double *v;           /* [n,dv]                                   */
    const double *raw_gate;    /* [n,dk]                                   */
    const double *beta_in;     /* [n] logits or probabilities              */
    const double *dt_bias;     /* [dk]                                     */
    double a_log;
    double *S;                 /* [dk,dv] in: initial state, out: final    */
    double *out;               /* [n,dv] or NULL                           */
} kda_ref_item;

typedef struct {
    int dk, dv, gate_mode, beta_mode;
    double lb, scale;
} kda_ref_params;

static void run_item(const kda_ref_item *it, const kda_ref_params *p) {
    double *la = (double *)malloc(sizeof(double) * (size_t)(it->n * p->dk + 1));
    double *beta = (double *)malloc(sizeof(double) * (size_t)(it->n + 1));
    kda_ref_log_alpha(it->n, p->dk, it->raw_gate, it->dt_bias, it->a_log, p->gate_mode, p->lb, la);
    for (int64_t e = 0; e < it->n * p->dk; ++e) la[e] = exp(la[e]); /* alpha */
    kda_ref_beta(it->n, it->beta_in, p->beta_mode, beta);
    kda_ref_recur(it->n, p->dk, p->dv, it->q, it->k, it->v, la, beta, p->scale, it->S, it->out);
    free(la);
    free(beta);
}

typedef struct {
    kda_ref_item *items;
    int n_items;
    const kda_ref_params *p;
    double **M;                /* segment-map mode when non-NULL */
    atomic_int next;
} pool_ctx;

void kda_ref_segment_map(const kda_ref_item *it, int dk, int dv, int gate_mode, double lb,
                         int beta_mode, double *M, double *U);

static void *pool_worker(void *arg) {
    pool_ctx *c = (pool_ctx *)arg;
    for (;;) {
        int i = atomic_fetch_add(&c->next, 1);
        if (i >= c->n_items) break;
        if (c->M)
            kda_ref_segment_map(&c->items[i], c->p->dk, c->p->dv, c->p->gate_mode, c->p->lb,
                                c->p->beta_mode, c->M[i], c->items[i].S);
        else
            run_item(&c->items[i], c->p);
    }
    return NULL;
}

static void run_pool(pool_ctx *c, int nthreads) {
    atomic_init(&c->next, 0);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > c->n_items) nthreads = c->n_items > 0 ? c->n_items : 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, pool_worker, c);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
}

/* Runs every item (independent (sequence, head) pairs) over nthreads threads. */
int kda_ref_forward_items(int n_items, kda_ref_item *items, int dk, int dv, int gate_mode,
                          double lb, int beta_mode, double scale, int nthreads) {
    kda_ref_params p = {dk, dv, gate_mode, beta_mode, lb, scale};
    pool_ctx c;
    c.items = items;
    c.n_items = n_items;
    c.p = &p;
    c.M = NULL;
    run_pool(&c, nthreads);
    return 0;
}

/*
 * Segment maps of every item over nthreads threads: item i writes M into
 * Ms[i] [dk,dk] and U into items[i].S [dk,dv].
 */
int kda_ref_segment_map_items(int n_items, kda_ref_item *items, double **Ms, int dk, int dv,
                              int gate_mode, double lb, int beta_mode, int nthreads) {
    kda_ref_params p = {dk, dv, gate_mode, beta_mode, lb, 1.0};
    pool_ctx c;
    c.items = items;
    c.n_items = n_items;
    c.p = &p;
    c.M = Ms;
    run_pool(&c, nthreads);
    return 0;
}

/* --------------------------------------------------------- segment map -- */

/*
 * F(S) = M S + U for the token segment in one item (item->S and item->out
 * are ignored).  M [dk,dk], U [dk,dv].
 */
void kda_ref_segment_map(const kda_ref_item *it, int dk, int dv, int gate_mode, double lb,
                         int beta_mode, double *M, double *U) {
    double *alpha = (double *)malloc(sizeof(double) * (size_t)(it->n * dk + 1));
    double *beta = (double *)malloc(sizeof(double) * (size_t)(it->n + 1));
    double *zeros = (double *)calloc((size_t)(it->n * dk + 1), sizeof(double));
    kda_ref_log_alpha(it->n, dk, it->raw_gate, it->dt_bias, it->a_log, gate_mode, lb, alpha);
    for (int64_t e = 0; e < it->n * dk; ++e) alpha[e] = exp(alpha[e]);
    kda_ref_beta(it->n, it->beta_in, beta_mode, beta);
    /* U: replay from the zero state with the segment's values */
    memset(U, 0, sizeof(double) * (size_t)dk * dv);
    kda_ref_recur(it->n, dk, dv, NULL, it->k, it->v, alpha, beta, 1.0, U, NULL);
    /* M: replay from the identity with zero values (value width dk) */
    memset(M, 0, sizeof(double) * (size_t)dk * dk);
    for (int i = 0; i < dk; ++i) M[i * dk + i] = 1.0;
    kda_ref_recur(it->n, dk, dk, NULL, it->k, zeros, alpha, beta, 1.0, M, NULL);
    free(alpha);
    free(beta);
    free(zeros);
}

/* ---------------------------------------------------------------- scan -- */

/*
 * Composition of two segment maps, F1 applied first, then F2:
 *   Mo = M2 M1,  Uo = M2 U1 + U2.
 * M1, M2 [dk,dk], U1, U2 [dk,dv] -> Mo [dk,dk], Uo [dk,dv].  The outputs must not
 * alias the inputs.
 */
void kda_ref_compose(int dk, int dv, const double *M2, const double *U2, const double *M1,
                     const double *U1, double *Mo, double *Uo) {
    for (int i = 0; i < dk; ++i) {
        for (int j = 0; j < dk; ++j) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += M2[i * dk + c] * M1[c * dk + j];
            Mo[i * dk + j] = acc;
        }
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += M2[i * dk + c] * U1[c * dv + j];
            Uo[i * dv + j] = acc + U2[i * dv + j];
        }
    }
}

/*
 * Ordered exclusive prefix of affine segment maps.
 * M [n_seg,dk,dk], U [n_seg,dk,dv], S_init [dk,dv]
 * -> incoming, outgoing [n_seg,dk,dv], final_state [dk,dv].
 */
int kda_ref_scan(int n_seg, int dk, int dv, const double *M, const double *U,
                 const double *S_init, double *incoming, double *outgoing, double *final_state) {
    if (n_seg < 1) return 1;
    size_t st = (size_t)dk * dv;
    double *W = (double *)malloc(sizeof(double) * st);
    double *nxt = (double *)malloc(sizeof(double) * st);
    memcpy(W, S_init, sizeof(double) * st);
    for (int s = 0; s < n_seg; ++s) {
        const double *Ms = M + (size_t)s * dk * dk, *Us = U + (size_t)s * st;
        memcpy(incoming + (size_t)s * st, W, sizeof(double) * st);
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int c = 0; c < dk; ++c) acc += Ms[i * dk + c] * W[c * dv + j];
                nxt[i * dv + j] = acc + Us[i * dv + j];
            }
        memcpy(W, nxt, sizeof(double) * st);
        memcpy(outgoing + (size_t)s * st, W, sizeof(double) * st);
    }
    memcpy(final_state, W, sizeof(double) * st);
    free(W);
    free(nxt);
    return 0;
}
