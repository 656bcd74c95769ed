"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle, compare."""
from __future__ import annotations

import numpy as np
import torch

import kimi_delta_attention_kda_amd as kda
from kimi_delta_attention_kda_amd import workloads as wl
from oracle import oracle as orc

OUT_TOL_BF16 = 2e-2     # max|o - o_ref| / max|o_ref|, bf16 outputs
OUT_TOL_F32 = 1e-3      # same measure, fp32 outputs
STATE_TOL = 1e-3        # ||S - S_ref||_F / ||S_ref||_F, fp32 states


def gate_name(w):
    return "safe" if w.gate_mode == 1 else "original"


def run_fwd(w, inp, pool=None, workspace="torch"):
    """Runs kda_chunk_fwd on the workload's tensors; returns (out, pool_after)."""
    pool = inp["state_pool"].clone() if pool is None else pool
    out = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["raw_gate"], inp["beta_logits"],
                        inp["a_log"], inp["dt_bias"], inp["cu_seqlens"], pool, inp["state_indices"],
                        gate_mode=gate_name(w), lower_bound=w.lower_bound,
                        beta_mode="logits" if w.beta_mode == 0 else "probability", scale=w.scale,
                        workspace=workspace)
    torch.cuda.synchronize()
    return out, pool


def oracle_items(w, inp, items, nthreads=None):
    """Oracle outputs and final states for (sequence, head) pairs."""
    its = [orc.item_from_inputs(inp, b, h) for (b, h) in items]
    return orc.forward_items(its, w.dk, w.dv, w.gate_mode, w.lower_bound, w.beta_mode, w.scale,
                             nthreads=nthreads)


REPORT = []             # one line per parity check, printed in pytest's terminal summary


def report(line):
    print(line, flush=True)
    REPORT.append(line)


ZERO_ABS = 1e-30        # a vanished reference: the result must be below this in magnitude


def rel_out(o, o_ref):
    """max|o - o_ref| / max|o_ref|.  Where the reference is exactly zero the relative
    measure is undefined: the result passes (0) only if it is zero as well, up to
    ZERO_ABS, and is infinitely wrong otherwise."""
    den = np.max(np.abs(o_ref))
    if den > 0:
        return float(np.max(np.abs(o - o_ref)) / den)
    return 0.0 if np.max(np.abs(o)) <= ZERO_ABS else float("inf")


def rel_fro(S, S_ref):
    """||S - S_ref||_F / ||S_ref||_F, with the same rule as rel_out for a zero reference."""
    den = np.linalg.norm(S_ref)
    if den > 0:
        return float(np.linalg.norm(S - S_ref) / den)
    return 0.0 if np.linalg.norm(S) <= ZERO_ABS else float("inf")


def compare_items(w, inp, out, pool, items, nthreads=None, detail=False, batch_tokens=1 << 21):
    """Returns (worst output error, worst state error) over the given (sequence, head)
    pairs, plus the per-item errors when detail is set.  The oracle runs over batches of
    at most batch_tokens token-heads (bounded host memory).  The final state is compared
    with the oracle's state rounded to fp32, the precision of the pool: a state that has
    decayed below fp32's range is zero there, and the kernel's must then be zero too."""
    worst_o, worst_s = 0.0, 0.0
    per = []
    batch, ntok = [], 0
    todo = list(items)
    for i, (b, h) in enumerate(todo):
        batch.append((b, h))
        ntok += inp["cu"][b + 1] - inp["cu"][b]
        if ntok < batch_tokens and i + 1 < len(todo):
            continue
        ref = oracle_items(w, inp, batch, nthreads)
        for (bb, hh), (o_ref, S_ref) in zip(batch, ref):
            a, e = inp["cu"][bb], inp["cu"][bb + 1]
            o = wl.as_f64(out[a:e, hh])
            S = wl.as_f64(pool[inp["indices"][bb], hh])
            eo = rel_out(o, o_ref) if e > a else 0.0
            es = rel_fro(S, S_ref.astype(np.float32).astype(np.float64))
            worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
            per.append(((bb, hh), eo, es))
        batch, ntok = [], 0
    return (worst_o, worst_s, per) if detail else (worst_o, worst_s)


def untouched_slots_identical(inp, pool_after):
    """Bitwise comparison of every pool slot that no sequence uses."""
    used = set(inp["indices"])
    before = inp["state_pool"]
    n = before.shape[0]
    keep = torch.tensor([s for s in range(n) if s not in used], dtype=torch.long, device=before.device)
    if keep.numel() == 0:
        return True
    a = before.index_select(0, keep).view(torch.int32)
    b = pool_after.index_select(0, keep).view(torch.int32)
    return bool(torch.equal(a, b))
