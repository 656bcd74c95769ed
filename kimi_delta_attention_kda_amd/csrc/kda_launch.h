// kda_launch.h -- host-side launch interface between the C ABI and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

enum { MODE_FWD = 0, MODE_SUMMARY = 1 };

struct ChainArgs {
    const void *q;                // [T,H,dk] (FWD only)
    const void *k;                // [T,H,dk]
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
    int H;
    int n_slices;                 // value slices per (item, head)
    int gate_mode;
    float lb;
    int beta_mode;
    float scale;
};

// dvs: value columns per workgroup (64 or 128); precise: fp32 inputs.
hipError_t launch_chain(const ChainArgs &a, int dk, int dvs, bool precise, int mode, hipStream_t stream);

// bf16 inputs, dk = dv = 128, safe gate: 8-wave kernel, one workgroup per (item, head)
// for the forward pass (n_slices = 1) and two (transition / contribution columns) for
// segment summaries (n_slices = 2).
hipError_t launch_fast(const ChainArgs &a, int mode, hipStream_t stream);

hipError_t launch_affine_scan(int n_seg, int H, int dk, int dv, const float *M, const float *U,
                              const float *S_init, float *incoming, float *outgoing, float *final_state,
                              hipStream_t stream);

}  // namespace kda
