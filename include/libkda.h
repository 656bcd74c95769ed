/*
 * libkda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention prefill library.
 *
 * Every tensor argument is a DEVICE pointer to row-major, contiguous memory
 * owned by the caller.  Calls validate their host-visible arguments, enqueue
 * their kernels on `stream` (a hipStream_t; NULL = the default stream) and
 * return without synchronising.  The chunk kernels keep every intermediate of
 * a chunk in registers and LDS; only the load-balanced forward pass needs a
 * device workspace (kda_chunk_fwd_ws), which kda_chunk_fwd draws from a
 * stream-ordered memory pool owned by the library, one per device.  That pool
 * keeps at most 256 MiB of freed workspace reserved between calls; larger
 * workspaces are returned to the device at the next synchronisation.
 *
 * Per head the method keeps a state S [dk, dv] (key axis = rows) and for each
 * token t applies
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = scale * q_t^T S_t,
 * i.e. decay each key row by its own channel gate, predict k^T S from the
 * decayed state, delta-write k (beta (v - pred))^T, then read the updated
 * state (nx_nofloat_kda.nx source: header comment, kda_gate, kda_write,
 * kda_forward).  The gate is
 *     log alpha = -exp(a_log[h]) * softplus(raw_gate[t,h,:] + dt_bias[h,:]),
 * optionally clamped from below ("safe" mode), and beta = sigmoid(beta_logits)
 * or the logits taken as probabilities (max.nn.state_space.kda_chunk,
 * Parameters: raw_gate, beta_logits, a_log, dt_bias, gate_mode, beta_mode).
 * The prefill is evaluated over 64-token chunks with the same result as the
 * token recurrence (kda_chunk describes the recurrence computed chunk-parallel;
 * its AMD gfx950 pipeline uses 64-token chunks).
 *
 * Errors: a status other than KDA_OK is returned BEFORE anything is launched
 * when a host-checkable argument is wrong (null pointer, extent, dtype, mode,
 * or a combination outside the supported contract).  Data-dependent
 * preconditions (cu_seqlens monotone, state_indices in range and distinct)
 * are not checked by the asynchronous calls; kda_validate_varlen checks them
 * synchronously.  With the environment variable KDA_DEBUG_VALIDATE=1 the
 * calls themselves first synchronise their stream and run the same checks
 * (segment offsets for kda_segment_summary, slot indices for kda_decode),
 * returning KDA_ERR_DATA before any launch on a violation; this is for
 * debugging only, since it stalls the caller.  KDA_ERR_HIP reports a failed
 * kernel launch.
 */
#ifndef LIBKDA_H
#define LIBKDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* a required pointer is NULL                         */
    KDA_ERR_SHAPE = 2,       /* an extent is negative, zero where it must not be,  */
                             /* or inconsistent with another                       */
    KDA_ERR_DTYPE = 3,       /* unknown dtype code                                 */
    KDA_ERR_UNSUPPORTED = 4, /* valid but outside the supported contract           */
    KDA_ERR_ARG = 5,         /* bad mode value or scalar                           */
    KDA_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed         */
    KDA_ERR_DATA = 7,        /* cu_seqlens / offsets / indices invalid (validation) */
    KDA_ERR_SCRATCH = 8      /* kda_chunk_fwd_noalloc: the plan exceeds its scratch  */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

typedef enum { KDA_GATE_ORIGINAL = 0, KDA_GATE_SAFE = 1 } kda_gate_mode;
typedef enum { KDA_BETA_LOGITS = 0, KDA_BETA_PROBABILITY = 1 } kda_beta_mode;
typedef enum { KDA_STATE_K_FIRST = 0, KDA_STATE_V_FIRST = 1 } kda_state_layout;

/*
 * Shapes and modes of one call (max.nn.state_space.kda_chunk, Parameters).
 * num_heads is the value-head count H: of v, the gates, beta, the state pool
 * and out.  q and k have num_key_heads heads Hk (kda_chunk, Parameters: q and
 * k are laid out over the key heads, everything else over the value heads).
 * Hk must divide H; value head h reads key head h / (H / Hk), so each key head
 * serves H / Hk consecutive value heads.  0 means Hk = H, the gfx950 contract
 * of kda_chunk.
 * Supported contract (anything else -> KDA_ERR_UNSUPPORTED), for kda_chunk_fwd,
 * kda_segment_summary and kda_decode alike:
 *   qkv_dtype == out_dtype, bf16 or f32; dk == dv in {64, 128}; either gate mode;
 *   state_layout K_FIRST ([slot][H][dk][dv]) or V_FIRST ([slot][H][dv][dk]).
 * Speed differs by range: bf16 with the SAFE gate and gate_lower_bound >= -5.3 runs
 * the fast chunk kernel (the gfx950 contract of kda_chunk: bf16, safe gate; its
 * 16-token factorisation of the decay needs 16*|bound| < 85); other calls run a
 * slower chunk walk that evaluates every decay factor directly, at fp32 accuracy.
 * Magnitudes on the fast kernel: values and states may be of any finite size (the
 * solve rescales its right-hand side by a power of two into the range of its fp16
 * operands and undoes it exactly); the decayed score blocks beta k_i^T k_j and
 * q_i^T k_j, and the inverses of the 16x16 diagonal blocks of I + A, are held in
 * fp16, which assumes keys and queries of at most unit L2 norm per head (the
 * normalisation KDA applies to q and k).  Larger keys belong on the f32 path.
 */
typedef struct {
    int64_t total_tokens;    /* T: rows of q, k, v, raw_gate, beta_logits, out   */
    int32_t batch;           /* B: sequences (kda_chunk_fwd)                     */
    int32_t num_heads;       /* H                                                */
    int32_t dk;              /* key head dim                                     */
    int32_t dv;              /* value head dim                                   */
    int32_t max_slots;       /* rows of the state pool (kda_chunk_fwd)           */
    int32_t qkv_dtype;       /* kda_dtype of q, k, v                             */
    int32_t out_dtype;       /* kda_dtype of out                                 */
    int32_t gate_mode;       /* kda_gate_mode                                    */
    float gate_lower_bound;  /* SAFE mode: log alpha = max(log alpha, bound)     */
    int32_t beta_mode;       /* kda_beta_mode                                    */
    int32_t state_layout;    /* kda_state_layout                                 */
    float scale;             /* o = scale * q^T S (callers usually pass 1/sqrt(dk)) */
    int32_t num_key_heads;   /* Hk: heads of q and k, dividing num_heads; 0 = H  */
} kda_desc;

/*
 * Chunk-parallel varlen prefill (max.nn.state_space.kda_chunk).
 *   q, k        [T, Hk, dk]  qkv_dtype
 *   v           [T, H, dv]   qkv_dtype
 *   raw_gate    [T, H, dk]   f32, forget-gate pre-activation before dt_bias
 *   beta_logits [T, H]       f32
 *   a_log       [H]          f32
 *   dt_bias     [H, dk]      f32
 *   cu_seqlens  [B+1]        int32, exclusive prefix offsets, cu[0]=0, cu[B]=T
 *   state_pool  [max_slots, H, dk, dv] f32 (K_FIRST; V_FIRST: [max_slots, H, dv, dk]);
 *               the slot state_indices[b]
 *               holds sequence b's incoming state and receives its final state.
 *               No other byte of the pool is read or written.  A sequence of
 *               length 0 leaves its slot untouched.
 *   state_indices [B]        int32, distinct slots
 *   out         [T, H, dv]   out_dtype, every row written; must not alias inputs
 * If the device cannot hold the load-balancing workspace (out of memory), the
 * call runs the same pass without load balancing (as kda_chunk_fwd_ws with no
 * workspace: same contract and results up to rounding, slower when sequence
 * lengths differ widely); any other runtime failure returns KDA_ERR_HIP.
 */
kda_status kda_chunk_fwd(const kda_desc *desc, const void *q, const void *k, const void *v,
                         const float *raw_gate, const float *beta_logits, const float *a_log,
                         const float *dt_bias, const int32_t *cu_seqlens, float *state_pool,
                         const int32_t *state_indices, void *out, void *stream);

/*
 * kda_chunk_fwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same pass, with
 * the load-balancing workspace taken from a fixed 256 MiB device array inside the
 * library instead of an allocation.  The call allocates nothing, on the host or the
 * device; inputs and outputs are the caller's, as for kda_chunk_fwd.
 *   - Each device the library runs on holds its own copy of the array until the
 *     process ends.  Every call on a device shares that device's copy: calls that
 *     may overlap on one device (concurrent streams, other host threads) race and
 *     must be serialised by the caller.  The array keeps the last call's contents;
 *     nothing in it is read before the call has written it.
 *   - When the plan's piece states and correction rows do not all fit, the planner
 *     splits fewer sequences (same results up to rounding, less balancing).
 *     KDA_ERR_SCRATCH, before any launch, when not even an unsplit plan's queue
 *     fits (very many sequences x heads).
 * f32 inputs, which use no workspace, run as in kda_chunk_fwd.  Other arguments
 * and errors as for kda_chunk_fwd.
 */
kda_status kda_chunk_fwd_noalloc(const kda_desc *desc, const void *q, const void *k, const void *v,
                                 const float *raw_gate, const float *beta_logits, const float *a_log,
                                 const float *dt_bias, const int32_t *cu_seqlens, float *state_pool,
                                 const int32_t *state_indices, void *out, void *stream);

/*
 * kda_chunk_fwd with a caller-owned workspace.  For bf16 inputs (dk = dv in
 * {64, 128}, either gate: the fast kernels with the safe gate, the chunk walk
 * otherwise) the forward pass is load-balanced over the GPU's compute units: a
 * sequence
 * much longer than the average load per CU is cut into pieces at chunk
 * boundaries that run in parallel, using the segment maps of KDA Context
 * Parallelism (Theory: a piece started from state X ends in M X + U, and its
 * outputs are q^T M_t X + q^T U_t); the pieces' states are then composed in
 * order and the outputs corrected.  Results equal those of the unsplit pass
 * up to rounding (the correction term is formed with bf16 MFMA operands).
 *   workspace       device memory of at least kda_chunk_fwd_workspace_size()
 *                   bytes, 256-byte aligned, not shared with a call that may
 *                   run concurrently; its contents need no initialisation.
 *                   NULL (or workspace_bytes == 0): no load balancing, one
 *                   workgroup per (sequence, head), no workspace.
 * Other arguments as for kda_chunk_fwd.  KDA_ERR_SHAPE if workspace is given
 * but smaller than required.  For f32 inputs the workspace is not used.
 */
kda_status kda_chunk_fwd_ws(const kda_desc *desc, const void *q, const void *k, const void *v,
                            const float *raw_gate, const float *beta_logits, const float *a_log,
                            const float *dt_bias, const int32_t *cu_seqlens, float *state_pool,
                            const int32_t *state_indices, void *out, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * Workspace bytes kda_chunk_fwd_ws needs for desc on the current device
 * (0 when the load-balanced path does not apply).  It grows with
 * total_tokens * num_heads * dv (bf16 correction rows) plus a few MiB per
 * compute unit for piece states.
 */
kda_status kda_chunk_fwd_workspace_size(const kda_desc *desc, size_t *bytes);

/*
 * Single-token decode (named beside max.nn.state_space.kda_chunk as the path
 * for one-token steps): one step of the recurrence per sequence, in the order
 * of the nx_nofloat_kda.nx source's kda_step (decay, delta-write, read):
 *   S <- Diag(alpha) S;  S <- S + k (beta (v - S^T k))^T;  o = scale * S^T q,
 * on the pool slot state_indices[b] of each sequence b, in fp32.
 *   q, k [B, Hk, dk], v [B, H, dv] (qkv_dtype); raw_gate [B, H, dk] f32;
 *   beta_logits [B, H] f32; a_log [H]; dt_bias [H, dk]; state_pool as for
 *   kda_chunk_fwd (per desc->state_layout); state_indices [B] distinct;
 *   out [B, H, dv] (out_dtype).  desc->total_tokens must equal desc->batch.
 * Any gate mode and bound (no chunk factorisation is involved).  Other pool
 * bytes are untouched.
 */
kda_status kda_decode(const kda_desc *desc, const void *q, const void *k, const void *v,
                      const float *raw_gate, const float *beta_logits, const float *a_log,
                      const float *dt_bias, float *state_pool, const int32_t *state_indices, void *out,
                      void *stream);

/*
 * Affine summaries of token segments (KDA Context Parallelism, "Theory": each
 * segment is the map F_i(S) = M_i S + U_i of its incoming state).  Segment i
 * covers tokens [seg_offsets[i], seg_offsets[i+1]) of one sequence; for each
 * head, U_i is the segment's state when started from S = 0 and M_i the
 * product, later tokens on the left, of (I - beta k k^T) Diag(alpha).
 *   k [T, Hk, dk], v [T, H, dv] (qkv_dtype); raw_gate, beta_logits, a_log,
 *   dt_bias as for kda_chunk_fwd; seg_offsets [n_seg+1] int32 (device),
 *   monotone with seg_offsets[0] >= 0 and seg_offsets[n_seg] <= T;
 *   M [n_seg, H, dk, dk] f32, U [n_seg, H, dk, dv] f32 (written).
 * desc->batch, max_slots, out_dtype and scale are ignored.  n_seg >= 1.
 */
kda_status kda_segment_summary(const kda_desc *desc, const void *k, const void *v,
                               const float *raw_gate, const float *beta_logits,
                               const float *a_log, const float *dt_bias,
                               const int32_t *seg_offsets, int32_t n_seg, float *M, float *U,
                               void *stream);

/*
 * Ordered exclusive prefix of segment maps (KDA Context Parallelism,
 * "Incoming and outgoing states", "Implementation order"): per head,
 *   W = S_init[h]; for i = 0..n_seg-1: incoming[i,h] = W; W = M[i,h] W + U[i,h];
 *   outgoing[i,h] = W;   final_state[h] = W.
 * Composition (M2,U2) o (M1,U1) = (M2 M1, M2 U1 + U2) is applied in segment
 * order with the state multiplied on the left.
 *   M [n_seg, H, dk, dk], U [n_seg, H, dk, dv], S_init [H, dk, dv] (read only);
 *   incoming, outgoing [n_seg, H, dk, dv], final_state [H, dk, dv] (written).
 * f32 throughout; dk in {16, 32, 64, 128}, dv a multiple of 16.
 * n_seg >= 1 (at least one segment; KDA_ERR_SHAPE otherwise).
 */
kda_status kda_affine_exclusive_scan(int32_t n_seg, int32_t num_heads, int32_t dk, int32_t dv,
                                     const float *M, const float *U, const float *S_init,
                                     float *incoming, float *outgoing, float *final_state,
                                     void *stream);

/*
 * The same exclusive prefix, regrouped (KDA Context Parallelism, "Theory": the
 * composition of segment maps is associative, so the ordered prefix may be
 * grouped in any way that keeps the order).  Segments are taken in blocks of
 * `block` consecutive segments:
 *   1. each block's maps, but the last block's, are composed in order into one
 *      map (A_b, B_b) = F_last o ... o F_first (a walk of the augmented state
 *      [A | B] from [I | 0]), all blocks and heads in parallel;
 *   2. W = S_init; W <- A_b W + B_b over the block composites in order gives
 *      every block's incoming state;
 *   3. each block is walked from its incoming state as in the ordered scan,
 *      all blocks in parallel, writing incoming, outgoing and (last block) final.
 * The critical path is about 2 block + n_seg / block map steps instead of n_seg;
 * the work is about three times the ordered scan's.  Results equal those of
 * kda_affine_exclusive_scan up to fp32 rounding of the regrouped products.
 *   block: segments per block; 0 picks the ordered scan below 32 segments (where
 *     its one launch is faster) and about sqrt(n_seg / 2) from 32 on.  It is raised to
 *     at least 1 + ceil(dk / dv), because the block composites (dk x (dk + dv)
 *     per block and head) are kept in `outgoing` until step 3 overwrites it;
 *     a block of n_seg or more is the ordered scan.  kda_affine_scan_block_size
 *     returns the block a call would use.
 *   Arrays, layouts, dtypes and errors as kda_affine_exclusive_scan; the inputs
 *   are read only; `outgoing` is scratch until the call completes.  dk in
 *   {16, 32} runs the ordered scan.  Three kernel launches on `stream`.
 */
kda_status kda_affine_exclusive_scan_blocked(int32_t n_seg, int32_t num_heads, int32_t dk, int32_t dv,
                                             int32_t block, const float *M, const float *U,
                                             const float *S_init, float *incoming, float *outgoing,
                                             float *final_state, void *stream);

/* Block size kda_affine_exclusive_scan_blocked uses for these arguments (n_seg when it
 * runs the ordered scan); -1 for invalid arguments.  Host only, no GPU call. */
int32_t kda_affine_scan_block_size(int32_t n_seg, int32_t dk, int32_t dv, int32_t block);

/*
 * Synchronous debug check of the data-dependent preconditions of
 * kda_chunk_fwd (max.nn.state_space.kda_chunk, Raises: the shape guards that
 * a production build leaves out).  cu_seqlens [batch+1] and state_indices
 * [batch] are DEVICE pointers; returns KDA_ERR_DATA unless cu[0] == 0,
 * cu is non-decreasing, cu[batch] == total_tokens, and the indices are
 * distinct and in [0, max_slots).  Blocks until the copies complete.
 */
kda_status kda_validate_varlen(const int32_t *cu_seqlens, int32_t batch, int64_t total_tokens,
                               const int32_t *state_indices, int32_t max_slots);

/* Static, NUL-terminated description of a status code. */
const char *kda_status_string(kda_status status);

#ifdef __cplusplus
}
#endif

#endif /* LIBKDA_H */
