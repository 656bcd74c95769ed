// kda_api.hip -- C ABI of libkda: argument validation, launch planning, status codes.
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <cstdlib>
#include <vector>

#include "../../include/libkda.h"
#include "kda_launch.h"

namespace {

bool valid_dtype(int32_t d) { return d == KDA_F32 || d == KDA_BF16; }

// Key heads of q and k (0 in the descriptor: as many as value heads).
int key_heads(const kda_desc *d) { return d->num_key_heads == 0 ? d->num_heads : d->num_key_heads; }
bool key_heads_ok(const kda_desc *d) {
    return d->num_key_heads >= 0 && d->num_heads % key_heads(d) == 0;
}

// Host-visible checks of the descriptor shared by the prefill and the segment summaries.
kda_status check_desc(const kda_desc *d, bool summary) {
    if (!d) return KDA_ERR_NULL;
    if (d->total_tokens < 0 || d->num_heads <= 0 || d->dk <= 0 || d->dv <= 0) return KDA_ERR_SHAPE;
    if (!key_heads_ok(d)) return KDA_ERR_SHAPE;
    if (d->total_tokens > (int64_t)0x7fffffff) return KDA_ERR_SHAPE;  // int32 offsets
    if (!summary && (d->batch < 0 || d->max_slots <= 0)) return KDA_ERR_SHAPE;
    if (!valid_dtype(d->qkv_dtype) || (!summary && !valid_dtype(d->out_dtype))) return KDA_ERR_DTYPE;
    if (d->gate_mode != KDA_GATE_ORIGINAL && d->gate_mode != KDA_GATE_SAFE) return KDA_ERR_ARG;
    if (d->beta_mode != KDA_BETA_LOGITS && d->beta_mode != KDA_BETA_PROBABILITY) return KDA_ERR_ARG;
    if (d->state_layout != KDA_STATE_K_FIRST && d->state_layout != KDA_STATE_V_FIRST) return KDA_ERR_ARG;
    if (d->gate_mode == KDA_GATE_SAFE && !(d->gate_lower_bound <= 0.f)) return KDA_ERR_ARG;
    if (!summary && !(d->scale == d->scale)) return KDA_ERR_ARG;  // NaN scale
    // ---- supported contract
    if (d->dk != d->dv) return KDA_ERR_UNSUPPORTED;
    if (!summary && d->qkv_dtype != d->out_dtype) return KDA_ERR_UNSUPPORTED;
    if (d->dk != 64 && d->dk != 128) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

kda::ChainArgs base_args(const kda_desc *d) {
    kda::ChainArgs a;
    memset(&a, 0, sizeof(a));
    a.H = d->num_heads;
    a.Hk = key_heads(d);
    a.gate_mode = d->gate_mode;
    a.lb = d->gate_lower_bound;
    a.beta_mode = d->beta_mode;
    a.scale = d->scale;
    a.v_first = d->state_layout == KDA_STATE_V_FIRST;
    return a;
}

// The fast kernel (kda_fast.hip) takes bf16 with the safe gate, whose bound keeps the
// reciprocal of a 16-token block decay, e^{16 |bound|}, finite; everything else within
// the contract runs the precise chunk walk.
bool use_fast(const kda_desc *d) {
    return d->qkv_dtype == KDA_BF16 && d->dk == d->dv && (d->dk == 128 || d->dk == 64) &&
           d->gate_mode == KDA_GATE_SAFE && d->gate_lower_bound >= -5.3f;
}

constexpr int MAX_DEV = 64;

// Compute units of the current device (cached per device); -1 on failure.
int current_device_cus(int *dev_out) {
    static std::mutex mu;
    static int cus[MAX_DEV] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) return -1;
    *dev_out = dev;
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return -1;
        cus[dev] = n;
    }
    return cus[dev];
}

// Library-owned stream-ordered pool of device dev, created on first use.  Freed blocks
// up to POOL_KEEP bytes stay reserved for reuse by later calls; anything above that is
// returned to the device at the next synchronisation.  nullptr if unavailable.
constexpr uint64_t POOL_KEEP = 256ull << 20;
hipMemPool_t device_pool(int dev) {
    static std::mutex mu;
    static hipMemPool_t pools[MAX_DEV] = {};
    static bool failed[MAX_DEV] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (!pools[dev] && !failed[dev]) {
        hipMemPoolProps props;
        memset(&props, 0, sizeof(props));
        props.allocType = hipMemAllocationTypePinned;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        if (hipMemPoolCreate(&pool, &props) == hipSuccess) {
            uint64_t thr = POOL_KEEP;
            (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
            pools[dev] = pool;
        } else {
            failed[dev] = true;
            (void)hipGetLastError();
        }
    }
    return pools[dev];
}

// The load-balanced pass serves bf16 inputs (its correction rows and outputs are bf16) with
// either gate: the fast kernels with the safe gate, the precise walk otherwise.
bool planned_applies(const kda_desc *d) {
    return d->qkv_dtype == KDA_BF16 && d->dk == d->dv && (d->dk == 128 || d->dk == 64) && d->batch > 0 &&
           d->total_tokens > 0;
}

// chunk kernel of the bf16 forward pass (dk = dv in {64, 128})
const kda::FwdKernel &fwd_kernel(const kda_desc *d) { return use_fast(d) ? kda::FWD64 : kda::FWD64_PRECISE; }

kda_status workspace_bytes_for(const kda_desc *d, size_t *bytes, kda::PlanLayout *lay, int *n_cu) {
    *bytes = 0;
    if (!planned_applies(d)) return KDA_OK;
    int dev = 0;
    const int cus = current_device_cus(&dev);
    if (cus <= 0) return KDA_ERR_HIP;
    *lay = kda::plan_layout(d->total_tokens, d->batch, d->num_heads, d->dk, d->dv, fwd_kernel(d).per_cu * cus);
    *bytes = lay->total;
    *n_cu = cus;
    return KDA_OK;
}

// Every host-checkable argument of the forward pass.
kda_status check_fwd(const kda_desc *desc, const void *q, const void *k, const void *v,
                     const float *raw_gate, const float *beta_logits, const float *a_log,
                     const float *dt_bias, const int32_t *cu_seqlens, const float *state_pool,
                     const int32_t *state_indices, const void *out) {
    kda_status st = check_desc(desc, false);
    if (st != KDA_OK) return st;
    if (!a_log || !dt_bias || !cu_seqlens || !state_pool || (desc->batch > 0 && !state_indices))
        return KDA_ERR_NULL;
    if (desc->total_tokens > 0 && (!q || !k || !v || !raw_gate || !beta_logits || !out)) return KDA_ERR_NULL;
    return KDA_OK;
}

// Host checks of the data-dependent preconditions (synchronous copies to the host).
// exact: offsets start at 0 and end at total (cu_seqlens); else they lie in [0, total]
// (segment offsets).  Non-decreasing in both cases.
kda_status check_offsets(const int32_t *offsets, int32_t n, int64_t total, bool exact) {
    std::vector<int32_t> cu(n + 1);
    if (hipMemcpy(cu.data(), offsets, sizeof(int32_t) * (n + 1), hipMemcpyDeviceToHost) != hipSuccess)
        return KDA_ERR_HIP;
    if (exact ? (cu[0] != 0 || (int64_t)cu[n] != total) : (cu[0] < 0 || (int64_t)cu[n] > total))
        return KDA_ERR_DATA;
    for (int b = 0; b < n; ++b)
        if (cu[b + 1] < cu[b]) return KDA_ERR_DATA;
    return KDA_OK;
}

kda_status check_indices(const int32_t *indices, int32_t n, int32_t max_slots) {
    if (n == 0) return KDA_OK;
    std::vector<int32_t> idx(n);
    if (hipMemcpy(idx.data(), indices, sizeof(int32_t) * n, hipMemcpyDeviceToHost) != hipSuccess)
        return KDA_ERR_HIP;
    std::vector<char> seen(max_slots, 0);
    for (int b = 0; b < n; ++b) {
        if (idx[b] < 0 || idx[b] >= max_slots || seen[idx[b]]) return KDA_ERR_DATA;
        seen[idx[b]] = 1;
    }
    return KDA_OK;
}

// With KDA_DEBUG_VALIDATE=1 in the environment the asynchronous calls first wait for
// their stream and check the data-dependent preconditions; a violation returns
// KDA_ERR_DATA before anything is launched.  Off by default: the check synchronises.
bool debug_validate() {
    const char *e = getenv("KDA_DEBUG_VALIDATE");
    return e && e[0] == '1' && e[1] == 0;
}

kda_status debug_check(const int32_t *offsets, int32_t n_off, int64_t total, bool exact,
                       const int32_t *indices, int32_t n_idx, int32_t max_slots, void *stream) {
    if (!debug_validate()) return KDA_OK;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return KDA_ERR_HIP;
    if (offsets) {
        const kda_status st = check_offsets(offsets, n_off, total, exact);
        if (st != KDA_OK) return st;
    }
    return indices ? check_indices(indices, n_idx, max_slots) : KDA_OK;
}

// scratch: when set, the workspace is that device memory with the layout *scratch_lay
// (the entry point without allocation), else the caller's workspace of workspace_bytes.
kda_status chunk_fwd_impl(const kda_desc *desc, const void *q, const void *k, const void *v,
                          const float *raw_gate, const float *beta_logits, const float *a_log,
                          const float *dt_bias, const int32_t *cu_seqlens, float *state_pool,
                          const int32_t *state_indices, void *out, void *workspace,
                          size_t workspace_bytes, void *stream, char *scratch = nullptr,
                          const kda::PlanLayout *scratch_lay = nullptr, int scratch_ncu = 0) {
    kda_status st = check_fwd(desc, q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, state_pool,
                              state_indices, out);
    if (st != KDA_OK) return st;
    st = debug_check(cu_seqlens, desc->batch, desc->total_tokens, true, state_indices, desc->batch,
                     desc->max_slots, stream);
    if (st != KDA_OK) return st;
    if (desc->batch == 0 || desc->total_tokens == 0) {
        // no tokens: nothing to read or write (every sequence is empty)
        return KDA_OK;
    }
    kda::ChainArgs a = base_args(desc);
    a.q = q;
    a.k = k;
    a.v = v;
    a.raw_gate = raw_gate;
    a.beta_logits = beta_logits;
    a.a_log = a_log;
    a.dt_bias = dt_bias;
    a.offsets = cu_seqlens;
    a.state_pool = state_pool;
    a.state_indices = state_indices;
    a.out = out;
    a.n_items = desc->batch;
    hipError_t e;
    if (planned_applies(desc) && scratch) {
        a.n_slices = 1;
        e = kda::launch_planned_fwd(a, desc->dk, scratch, *scratch_lay, scratch_ncu, fwd_kernel(desc),
                                    (hipStream_t)stream);
    } else if (planned_applies(desc) && workspace && workspace_bytes > 0) {
        a.n_slices = 1;
        size_t need = 0;
        kda::PlanLayout lay;
        int n_cu = 0;
        st = workspace_bytes_for(desc, &need, &lay, &n_cu);
        if (st != KDA_OK) return st;
        if (workspace_bytes < need) return KDA_ERR_SHAPE;
        e = kda::launch_planned_fwd(a, desc->dk, (char *)workspace, lay, n_cu, fwd_kernel(desc),
                                    (hipStream_t)stream);
    } else if (use_fast(desc)) {
        a.n_slices = 1;
        e = kda::launch_fast(a, desc->dk, kda::MODE_FWD, (hipStream_t)stream);
    } else {
        e = kda::launch_chain(a, desc->dk, desc->qkv_dtype == KDA_BF16, kda::MODE_FWD, (hipStream_t)stream);
    }
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// ---- scratch of the entry point without allocation (kda_chunk_fwd_noalloc)
// The load-balanced pass's workspace in a fixed device array, for callers that cannot
// allocate.  Each device the library runs on holds its own copy until the process ends.
// In host code the array's name is only a stand-in: kernels get the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
constexpr size_t SCRATCH_BYTES = 256ull << 20;
static __device__ __align__(256) char scratch[SCRATCH_BYTES];

char *scratch_ptr(int dev) {
    static std::mutex mu;
    static char *ptrs[MAX_DEV] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        ptrs[dev] = (char *)p;
    }
    return ptrs[dev];
}

}  // namespace

extern "C" {

const char *kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is NULL";
        case KDA_ERR_SHAPE: return "an extent is out of range or inconsistent";
        case KDA_ERR_DTYPE: return "unknown dtype code";
        case KDA_ERR_UNSUPPORTED:
            return "arguments outside the supported contract (out dtype equal to the q/k/v dtype, "
                   "bf16 or f32; dk == dv in {64, 128}; either gate mode)";
        case KDA_ERR_ARG: return "bad mode value or scalar";
        case KDA_ERR_HIP: return "a HIP runtime call or kernel launch failed";
        case KDA_ERR_DATA: return "cu_seqlens or state_indices violate their preconditions";
        case KDA_ERR_SCRATCH:
            return "the call needs more than the 256 MiB device scratch of kda_chunk_fwd_noalloc "
                   "(too many sequences x heads for its plan)";
    }
    return "unknown status";
}

kda_status kda_chunk_fwd(const kda_desc *desc, const void *q, const void *k, const void *v,
                         const float *raw_gate, const float *beta_logits, const float *a_log,
                         const float *dt_bias, const int32_t *cu_seqlens, float *state_pool,
                         const int32_t *state_indices, void *out, void *stream) {
    kda_status st = check_fwd(desc, q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, state_pool,
                              state_indices, out);
    if (st != KDA_OK) return st;  // nothing allocated or launched
    if (planned_applies(desc)) {
        size_t need = 0;
        kda::PlanLayout lay;
        int n_cu = 0;
        int dev = 0;
        if (workspace_bytes_for(desc, &need, &lay, &n_cu) == KDA_OK && need > 0 &&
            current_device_cus(&dev) > 0) {
            hipMemPool_t pool = device_pool(dev);
            void *ws = nullptr;
            const hipError_t ea = pool ? hipMallocFromPoolAsync(&ws, need, pool, (hipStream_t)stream)
                                       : hipErrorOutOfMemory;
            if (ea == hipSuccess) {
                st = chunk_fwd_impl(desc, q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens,
                                    state_pool, state_indices, out, ws, need, stream);
                if (hipFreeAsync(ws, (hipStream_t)stream) != hipSuccess && st == KDA_OK) st = KDA_ERR_HIP;
                return st;
            }
            // Only a workspace the device cannot hold falls back to the unbalanced launch
            // (same results, no workspace); that error is consumed here so the launch
            // check below does not report it.  Any other failure is returned.
            if (ea != hipErrorOutOfMemory) return KDA_ERR_HIP;
            if (pool) (void)hipGetLastError();
        }
    }
    return chunk_fwd_impl(desc, q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, state_pool,
                          state_indices, out, nullptr, 0, stream);
}

kda_status kda_chunk_fwd_noalloc(const kda_desc *desc, const void *q, const void *k, const void *v,
                                 const float *raw_gate, const float *beta_logits, const float *a_log,
                                 const float *dt_bias, const int32_t *cu_seqlens, float *state_pool,
                                 const int32_t *state_indices, void *out, void *stream) {
    kda_status st = check_fwd(desc, q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, state_pool,
                              state_indices, out);
    if (st != KDA_OK) return st;
    if (!planned_applies(desc))  // no workspace on these paths
        return chunk_fwd_impl(desc, q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, state_pool,
                              state_indices, out, nullptr, 0, stream);
    int dev = 0;
    const int cus = current_device_cus(&dev);
    if (cus <= 0) return KDA_ERR_HIP;
    bool fits = false;
    const kda::PlanLayout lay = kda::plan_layout(desc->total_tokens, desc->batch, desc->num_heads, desc->dk,
                                                 desc->dv, fwd_kernel(desc).per_cu * cus, SCRATCH_BYTES, &fits);
    if (!fits) return KDA_ERR_SCRATCH;
    char *ws = scratch_ptr(dev);
    if (!ws) return KDA_ERR_HIP;
    return chunk_fwd_impl(desc, q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, state_pool,
                          state_indices, out, nullptr, 0, stream, ws, &lay, cus);
}

kda_status kda_chunk_fwd_ws(const kda_desc *desc, const void *q, const void *k, const void *v,
                            const float *raw_gate, const float *beta_logits, const float *a_log,
                            const float *dt_bias, const int32_t *cu_seqlens, float *state_pool,
                            const int32_t *state_indices, void *out, void *workspace,
                            size_t workspace_bytes, void *stream) {
    return chunk_fwd_impl(desc, q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, state_pool,
                          state_indices, out, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_workspace_size(const kda_desc *desc, size_t *bytes) {
    if (!bytes) return KDA_ERR_NULL;
    *bytes = 0;
    kda_status st = check_desc(desc, false);
    if (st != KDA_OK) return st;
    kda::PlanLayout lay;
    int n_cu = 0;
    return workspace_bytes_for(desc, bytes, &lay, &n_cu);
}

kda_status kda_decode(const kda_desc *desc, const void *q, const void *k, const void *v,
                      const float *raw_gate, const float *beta_logits, const float *a_log,
                      const float *dt_bias, float *state_pool, const int32_t *state_indices, void *out,
                      void *stream) {
    const kda_desc *d = desc;
    if (!d) return KDA_ERR_NULL;
    if (d->batch < 0 || d->num_heads <= 0 || d->dk <= 0 || d->dv <= 0 || d->max_slots <= 0) return KDA_ERR_SHAPE;
    if (!key_heads_ok(d)) return KDA_ERR_SHAPE;
    if (d->total_tokens != d->batch) return KDA_ERR_SHAPE;  // one token per sequence
    if (!valid_dtype(d->qkv_dtype) || !valid_dtype(d->out_dtype)) return KDA_ERR_DTYPE;
    if (d->gate_mode != KDA_GATE_ORIGINAL && d->gate_mode != KDA_GATE_SAFE) return KDA_ERR_ARG;
    if (d->beta_mode != KDA_BETA_LOGITS && d->beta_mode != KDA_BETA_PROBABILITY) return KDA_ERR_ARG;
    if (d->state_layout != KDA_STATE_K_FIRST && d->state_layout != KDA_STATE_V_FIRST) return KDA_ERR_ARG;
    if (d->gate_mode == KDA_GATE_SAFE && !(d->gate_lower_bound <= 0.f)) return KDA_ERR_ARG;
    if (!(d->scale == d->scale)) return KDA_ERR_ARG;
    // one step needs no chunk factorisation: any gate form, bf16 or f32
    if (d->dk != d->dv || !(d->dk == 64 || d->dk == 128) || d->qkv_dtype != d->out_dtype) return KDA_ERR_UNSUPPORTED;
    if (!a_log || !dt_bias || !state_pool || (desc->batch > 0 && !state_indices)) return KDA_ERR_NULL;
    if (desc->batch > 0 && (!q || !k || !v || !raw_gate || !beta_logits || !out)) return KDA_ERR_NULL;
    if (desc->batch == 0) return KDA_OK;
    const kda_status st = debug_check(nullptr, 0, 0, true, state_indices, desc->batch, desc->max_slots, stream);
    if (st != KDA_OK) return st;
    kda::DecodeArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = k;
    a.v = v;
    a.raw_gate = raw_gate;
    a.beta_logits = beta_logits;
    a.a_log = a_log;
    a.dt_bias = dt_bias;
    a.state_pool = state_pool;
    a.state_indices = state_indices;
    a.out = out;
    a.B = desc->batch;
    a.H = desc->num_heads;
    a.Hk = key_heads(desc);
    a.gate_mode = desc->gate_mode;
    a.lb = desc->gate_lower_bound;
    a.beta_mode = desc->beta_mode;
    a.scale = desc->scale;
    a.v_first = desc->state_layout == KDA_STATE_V_FIRST;
    const hipError_t e = kda::launch_decode(a, desc->dk, desc->qkv_dtype == KDA_BF16, (hipStream_t)stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_segment_summary(const kda_desc *desc, const void *k, const void *v,
                               const float *raw_gate, const float *beta_logits,
                               const float *a_log, const float *dt_bias,
                               const int32_t *seg_offsets, int32_t n_seg, float *M, float *U,
                               void *stream) {
    kda_status st = check_desc(desc, true);
    if (st != KDA_OK) return st;
    if (n_seg < 1) return KDA_ERR_SHAPE;
    if (!a_log || !dt_bias || !seg_offsets || !M || !U) return KDA_ERR_NULL;
    if (desc->total_tokens > 0 && (!k || !v || !raw_gate || !beta_logits)) return KDA_ERR_NULL;
    st = debug_check(seg_offsets, n_seg, desc->total_tokens, false, nullptr, 0, 0, stream);
    if (st != KDA_OK) return st;
    kda::ChainArgs a = base_args(desc);
    a.k = k;
    a.v = v;
    a.raw_gate = raw_gate;
    a.beta_logits = beta_logits;
    a.a_log = a_log;
    a.dt_bias = dt_bias;
    a.offsets = seg_offsets;
    a.M = M;
    a.U = U;
    a.n_items = n_seg;
    hipError_t e;
    if (use_fast(desc)) {
        a.n_slices = 2;
        e = kda::launch_fast(a, desc->dk, kda::MODE_SUMMARY, (hipStream_t)stream);
    } else {
        e = kda::launch_chain(a, desc->dk, desc->qkv_dtype == KDA_BF16, kda::MODE_SUMMARY, (hipStream_t)stream);
    }
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_affine_exclusive_scan(int32_t n_seg, int32_t num_heads, int32_t dk, int32_t dv,
                                     const float *M, const float *U, const float *S_init,
                                     float *incoming, float *outgoing, float *final_state,
                                     void *stream) {
    if (n_seg < 1 || num_heads <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_SHAPE;
    if (!M || !U || !S_init || !incoming || !outgoing || !final_state) return KDA_ERR_NULL;
    if (!(dk == 16 || dk == 32 || dk == 64 || dk == 128) || dv % 16 != 0) return KDA_ERR_UNSUPPORTED;
    hipError_t e = kda::launch_affine_scan(n_seg, num_heads, dk, dv, M, U, S_init, incoming, outgoing,
                                           final_state, (hipStream_t)stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_affine_exclusive_scan_blocked(int32_t n_seg, int32_t num_heads, int32_t dk, int32_t dv,
                                             int32_t block, const float *M, const float *U,
                                             const float *S_init, float *incoming, float *outgoing,
                                             float *final_state, void *stream) {
    if (n_seg < 1 || num_heads <= 0 || dk <= 0 || dv <= 0 || block < 0) return KDA_ERR_SHAPE;
    if (!M || !U || !S_init || !incoming || !outgoing || !final_state) return KDA_ERR_NULL;
    if (!(dk == 16 || dk == 32 || dk == 64 || dk == 128) || dv % 16 != 0) return KDA_ERR_UNSUPPORTED;
    hipError_t e = kda::launch_affine_scan_blocked(n_seg, num_heads, dk, dv, block, M, U, S_init, incoming,
                                                   outgoing, final_state, (hipStream_t)stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int32_t kda_affine_scan_block_size(int32_t n_seg, int32_t dk, int32_t dv, int32_t block) {
    if (n_seg < 1 || dk <= 0 || dv <= 0 || block < 0) return -1;
    if (!(dk == 64 || dk == 128)) return n_seg;
    return kda::scan_block_size(n_seg, dk, dv, block);
}

kda_status kda_validate_varlen(const int32_t *cu_seqlens, int32_t batch, int64_t total_tokens,
                               const int32_t *state_indices, int32_t max_slots) {
    if (batch < 0 || total_tokens < 0 || max_slots <= 0) return KDA_ERR_SHAPE;
    if (!cu_seqlens || (batch > 0 && !state_indices)) return KDA_ERR_NULL;
    const kda_status st = check_offsets(cu_seqlens, batch, total_tokens, true);
    return st != KDA_OK ? st : check_indices(state_indices, batch, max_slots);
}

}  // extern "C"
