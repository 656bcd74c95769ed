// kda_launch.h -- host-side launch interface between the C ABI and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

enum { MODE_FWD = 0, MODE_SUMMARY = 1 };

// ---- load-balanced forward pass (kda_plan.hip)
// Roles of a queued unit: the whole sequence or its first piece (state from and to the
// pool slot, V, outputs to out); the transition chain of a later piece (state starts at
// I, no V, outputs W_t = scale q_t^T M_t to the W buffer, final M to the M buffer); the
// contribution chain of a later piece (state starts at 0, V, outputs to out, final U).
enum { ROLE_WHOLE = 0, ROLE_M = 1, ROLE_U = 2 };

struct PlanHeader {
    int ctr;       // queue cursor (atomic), zeroed by the planner
    int qlen;      // queue length, counting skip slots
    int n_split;   // sequences cut into pieces
    int n_piece;   // pieces after the first, over all split sequences
    int n_echunk;  // chunks in those pieces
    int L;         // first-piece length in chunks (0: nothing split)
    int n_ent;
    int n_sorted;
    int pad[28];
};

// Byte offsets of the parts of the forward-pass workspace.
struct PlanLayout {
    size_t hdr, queue, ent, piece, sseq, sorted, M, U, XT, W, total;
    int np_cap;   // capacity for pieces after the first
    int ent_cap;  // capacity for entities (sequences + pieces)
    int qcap;     // capacity of the queue (int2 entries)
    int w_cap;    // capacity of the W rows, in chunks of later pieces
};
// Workspace of the balanced pass.  max_bytes == 0: room for every plan the planner can
// choose (np_cap pieces, W rows for every chunk).  Otherwise the layout fits in
// max_bytes by capping the pieces and the W rows (the planner then splits less), and
// ok is false when not even an unsplit plan fits.
PlanLayout plan_layout(int64_t T, int B, int H, int dk, int dv, int n_slots, size_t max_bytes = 0,
                       bool *ok = nullptr);

struct ChainArgs {
    const void *q;                // [T,Hk,dk] (FWD only)
    const void *k;                // [T,Hk,dk]
    const void *v;                // [T,H,dv]
    const float *raw_gate;        // [T,H,dk]
    const float *beta_logits;     // [T,H]
    const float *a_log;           // [H]
    const float *dt_bias;         // [H,dk]
    const int32_t *offsets;       // cu_seqlens [B+1] (FWD) or segment offsets [n_seg+1]
    float *state_pool;            // FWD
    const int32_t *state_indices; // FWD
    void *out;                    // FWD
    float *M;                     // SUMMARY [n_seg,H,dk,dk]
    float *U;                     // SUMMARY [n_seg,H,dk,dv]
    int n_items;                  // B or n_seg
    int H;                        // value heads
    int Hk;                       // key heads (q, k); value head h reads key head h / (H / Hk)
    int n_slices;                 // value slices per (item, head)
    int gate_mode;
    float lb;
    int beta_mode;
    float scale;
    int v_first;             // pool slots stored [dv][dk] (V_FIRST) instead of [dk][dv]
    // load-balanced forward pass: when plan is set, workgroups take units from the
    // planner's queue instead of one (item, head) each
    const PlanHeader *plan;
    const int2 *queue;       // [qcap]: (entity, head | role << 16), head < 0 in skip slots
    const int4 *ent;         // entity: (sequence, first chunk, end chunk, piece or -1)
    float *ws_M;             // [n_piece][H][dk][dk]
    float *ws_U;             // [n_piece][H][dk][dv]
    void *ws_W;              // [64 w_cap][H][dv] bf16, W rows of the later pieces, chunk-compact
    const int4 *ws_piece;    // (first token, end token, chunks, first W chunk) of each later piece
};

// Precise chunk walk (kda_chain.hip): dk = dv in {64, 128}; the launch sets a.n_slices
// (column slices per item and head) itself.  bf16_in: q/k/v (and out) are bf16, else fp32.
hipError_t launch_chain(const ChainArgs &a, int dk, bool bf16_in, int mode, hipStream_t stream);
// the precise walk's forward pass over the queues of a plan (a.plan set, bf16 inputs), n_wg
// persistent workgroups
hipError_t launch_chain_planned(const ChainArgs &a, int dk, int n_wg, hipStream_t stream);

// bf16 inputs, dk = dv in {64, 128}, safe gate: dv/16-wave kernel, one workgroup per (item, head)
// for the forward pass (n_slices = 1) and two (transition / contribution columns) for
// segment summaries (n_slices = 2).
hipError_t launch_fast(const ChainArgs &a, int dk, int mode, hipStream_t stream);
// forward pass over the queues of a plan (a.plan set), one persistent workgroup per CU
hipError_t launch_fast_planned(const ChainArgs &a, int dk, int n_cu, hipStream_t stream);
// The forward pass at dk = dv = 128 (kda_pipe.hip): producer and chain wave groups one
// chunk apart; grid as for launch_fast (one workgroup per (item, head), or persistent
// over a plan's queue).
hipError_t launch_pipe(const ChainArgs &a, dim3 grid, hipStream_t stream);
// The chunk kernel of the bf16 forward pass: its chunk length, how many of its workgroups
// share a CU (the planner sizes pieces in its chunks, for that many slots), and whether it
// is the precise walk.  LDS admits one workgroup per CU for each of them.
struct FwdKernel {
    int chunk;
    int per_cu;
    bool precise;
};
constexpr FwdKernel FWD64 = {64, 1, false};         // kda_pipe.hip / kda_fast.hip (safe gate)
constexpr FwdKernel FWD64_PRECISE = {64, 1, true};  // kda_chain.hip (other gates)

// Planner, piece-state scan and output correction of the load-balanced forward pass
// (bf16, dk = dv in {64, 128}, either gate; fk names the chunk kernel).  ws is the
// workspace laid out by plan_layout.
hipError_t launch_planned_fwd(ChainArgs a, int dk, char *ws, const PlanLayout &lay, int n_cu,
                              const FwdKernel &fk, hipStream_t stream);

struct DecodeArgs {
    const void *q, *k, *v;        // [B, Hk, dk] / [B, H, dv], one token per sequence
    const float *raw_gate;        // [B, H, dk]
    const float *beta_logits;     // [B, H]
    const float *a_log;           // [H]
    const float *dt_bias;         // [H, dk]
    float *state_pool;            // [slots, H, dk, dv] (or [.., dv, dk] when v_first)
    const int32_t *state_indices; // [B]
    void *out;                    // [B, H, dv]
    int B, H, Hk;                 // value heads H, key heads Hk (dividing H)
    int gate_mode;
    float lb;
    int beta_mode;
    float scale;
    int v_first;
};
// dk = dv in {64, 128}; bf16 or f32 q/k/v/out.
hipError_t launch_decode(const DecodeArgs &a, int dk, bool bf16, hipStream_t stream);

hipError_t launch_affine_scan(int n_seg, int H, int dk, int dv, const float *M, const float *U,
                              const float *S_init, float *incoming, float *outgoing, float *final_state,
                              hipStream_t stream);
// The same prefix regrouped into blocks of blk segments (0: about sqrt(n_seg / 2)): block
// composites, a walk over them, then every block walked from its incoming state; three
// launches, the composites kept in outgoing until the last overwrites it.  dk in {16, 32}
// runs the ordered walk.
int scan_block_size(int n_seg, int dk, int dv, int blk);
hipError_t launch_affine_scan_blocked(int n_seg, int H, int dk, int dv, int blk, const float *M,
                                      const float *U, const float *S_init, float *incoming,
                                      float *outgoing, float *final_state, hipStream_t stream);

}  // namespace kda
