#!/usr/bin/env python3
"""Throughput of the KDA chunk-parallel prefill (kda_chunk_fwd) on one MI355X.

One step = one kda_chunk_fwd call over the whole varlen batch (gate prep, decayed
scores, triangular inverse, W/U construction, inter-chunk state pass, output), with the
load-balancing workspace: a planner kernel, the chunk kernel (the whole hot path of
every chain), and for sequences cut into pieces a piece-state scan and an output
correction.  Inputs are seeded synthetic tensors already resident in HBM.  Prints one
JSON line; the per-call time is taken with one pair of HIP events on the launch stream
around the whole timed region (all four kernels of every call, divided by the number of
calls).  Events between the calls would add ~7 us of idle GPU time to each call.

Default workload: 8 sequences (lengths uniform in [1024, 8192], 32768 tokens), H=32,
dk=dv=128, bf16 q/k/v/out, fp32 gates and state, safe gate (bound -5), 64-slot pool.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s at H=32 dk=dv=128 bf16, 32K tokens; % MFMA peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILES = {"varlen_32k": os.path.join(ROOT, "profiles", "kda_chunk_fwd_varlen_32k_traffic.json"),
                 "long_131k": os.path.join(ROOT, "profiles", "kda_chunk_fwd_long_131k_traffic.json"),
                 "decode_512": os.path.join(ROOT, "profiles", "kda_decode_kernel_decode_512_traffic.json"),
                 "segments_262k": os.path.join(ROOT, "profiles", "kda_segment_pass_segments_262k_traffic.json")}


def measured_traffic(w):
    """Calibrated HBM bytes per call from the counter summary of this workload, while the
    kernel sources still hash to the measured version; else None."""
    f = TRAFFIC_FILES.get(w.name)
    if not f or not os.path.exists(f):
        return None
    with open(f) as fh:
        tr = json.load(fh)
    if tr.get("kernel_source_sha") == kernel_source_sha() and tr.get("workload") == w.name:
        return tr.get("hbm_bytes_per_call")
    return None


def chunk_kernel(w) -> str:
    """The chunk kernel that kda_chunk_fwd runs for workload w (with its load-balancing
    workspace, as bench.py calls it)."""
    if w.dtype == "bf16" and w.gate_mode == 1 and w.lower_bound >= -5.3:
        return "kda_pipe_kernel" if w.dk == 128 else "kda_fast_kernel"
    return "kda_chain_planned_kernel" if w.dtype == "bf16" else "kda_chain_kernel"


def measured_utilization(w, kernel=None):
    """MFMA- and VALU-busy fractions of the chunk kernel from the counter summary of this
    workload, while the kernel sources still hash to the measured version; else None."""
    f = os.path.join(ROOT, "profiles", f"{kernel or chunk_kernel(w)}_{w.name}_utilization.json")
    if not os.path.exists(f):
        return None
    with open(f) as fh:
        u = json.load(fh)
    if u.get("kernel_source_sha") == kernel_source_sha() and u.get("workload") == w.name:
        return {"mfma_busy": u.get("mfma_busy"), "valu_busy": u.get("valu_busy"), "from": u.get("source")}
    return None


def kernel_source_sha() -> str:
    d = os.path.join(ROOT, "kimi_delta_attention_kda_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):  # the kernel sources (subfolders hold no KDA kernel)
        if os.path.isfile(os.path.join(d, f)):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w) -> int:
    """Compulsory HBM bytes of one call: every input read once, out written once,
    each used pool slot read and written once."""
    e_qkv = 2 if w.dtype == "bf16" else 4
    # per value head: v, out, gate pre-activations, beta; q and k over the key heads
    per_token_head = w.dv * e_qkv + w.dv * e_qkv + w.dk * 4 + 4
    pool = 2 * w.B * w.H * w.dk * w.dv * 4
    return (w.T * (w.H * per_token_head + w.HK * 2 * w.dk * e_qkv) + pool + w.H * (w.dk + 1) * 4
            + (w.B + 1) * 4 + w.B * 4)


def algorithmic_flops(w) -> int:
    """Triangle-aware chunk-form flops: C(3dk + 2dv) + 6 dk dv per token-head (C = 64)."""
    return w.T * w.H * (64 * (3 * w.dk + 2 * w.dv) + 6 * w.dk * w.dv)


def dense_tile_flops(w) -> int:
    return w.T * w.H * (2 * 64 * (3 * w.dk + 2 * w.dv) + 6 * w.dk * w.dv)


def decode_flops(w) -> int:
    """One recurrent step per (sequence, head): decay, predict S^T k, rank-one write and
    read-out S^T q, about 7 dk dv flops."""
    return w.B * w.H * 7 * w.dk * w.dv


def segment_flops(w) -> int:
    """Algorithmic flops of one summary-and-scan pass.  Summaries: the chunk form on the
    augmented state [M | U] of width dk + dv, per token-head C dk (scores, triangle) +
    C (dk + dv) (triangular solve) + 2 dk (dk + dv) (prediction) + 2 dk (dk + dv) (state
    update), C = 64.  Scan: 2 dk^2 dv per map and head."""
    C, W = 64, w.dk + w.dv
    per_th = C * w.dk + C * W + 4 * w.dk * W
    return w.T * w.H * per_th + w.segments * w.H * 2 * w.dk * w.dk * w.dv


def decode_bytes(w) -> int:
    """Compulsory HBM bytes of one decode call: each (sequence, head) reads and writes its
    fp32 state once and reads one token's q, k, v, gate pre-activations and beta logit,
    writing one output row."""
    e = 2 if w.dtype == "bf16" else 4
    per_seq_head = 2 * w.dk * w.dv * 4 + w.dv * e + w.dv * e + w.dk * 4 + 4
    return w.B * (w.H * per_seq_head + w.HK * 2 * w.dk * e) + w.H * (w.dk + 1) * 4 + w.B * 4


def segment_bytes(w) -> int:
    """Compulsory HBM bytes of one summary-and-scan pass: k, v, the gate pre-activations and
    beta read once; M and U written by the summaries and read once by the scan; the scan's
    incoming and outgoing stacks and final state written, the initial state read."""
    e = 2 if w.dtype == "bf16" else 4
    n = w.segments
    inputs = w.T * (w.HK * w.dk * e + w.H * (w.dv * e + w.dk * 4 + 4)) + w.H * (w.dk + 1) * 4 + (n + 1) * 4
    maps = n * w.H * w.dk * (w.dk + w.dv) * 4
    scan = 2 * n * w.H * w.dk * w.dv * 4 + 2 * w.H * w.dk * w.dv * 4
    return inputs + 2 * maps + scan


FP32_PEAK_TFLOPS = 157.3


def roofline_bound(flops, nbytes, peak_tflops):
    """The roofline that caps a launch: HBM when its arithmetic intensity (flop/B) lies
    below the ridge point peak_flops / peak_bandwidth of its arithmetic type, else the
    matrix-core peak."""
    ridge = peak_tflops * 1e12 / (HBM_PEAK_GBS * 1e9)
    return "hbm" if flops / nbytes < ridge else "mfma"


def timed_loop(step, steps):
    """steps back-to-back calls between one pair of HIP events on the launch stream (no
    idle gaps between calls); returns (host ms per call, device ms per call)."""
    import torch
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, ev0.elapsed_time(ev1) / steps


def per_call_protocol(step, restore, reps=20, warm=3):
    """Each call timed alone: warm untimed calls, then reps calls, each bracketed by its
    own pair of HIP events; restore() (putting the touched pool slots back) runs before
    every call, outside the events.  Returns the median and minimum in ms."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        restore()
        step()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        restore()
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    med = ms[reps // 2] if reps % 2 else 0.5 * (ms[reps // 2 - 1] + ms[reps // 2])
    return {"median_ms": round(med, 4), "min_ms": round(ms[0], 4), "reps": reps, "warmup": warm,
            "slots_restored_outside_timing": True}


def cpu_baseline(w, inp, target_s=12.0):
    """The fp64 oracle on a bounded sample of the same workload, all host cores."""
    from oracle import build as obuild
    from oracle import oracle as orc
    obuild.build(force=False)
    nth = orc.default_threads()
    # calibrate on one short item
    b0 = min(range(w.B), key=lambda b: w.lengths[b])
    t = time.perf_counter()
    orc.forward_items([orc.item_from_inputs(inp, b0, 0)], w.dk, w.dv, w.gate_mode, w.lower_bound,
                      w.beta_mode, w.scale, nthreads=1)
    per_tok = (time.perf_counter() - t) / max(1, w.lengths[b0])
    # pick heads so the sample is about target_s of wall time on nth threads
    heads = max(1, min(w.H, int(target_s * nth / (per_tok * w.T))))
    items = [(b, h) for h in range(heads) for b in range(w.B)]
    its = [orc.item_from_inputs(inp, b, h) for (b, h) in items]
    t = time.perf_counter()
    orc.forward_items(its, w.dk, w.dv, w.gate_mode, w.lower_bound, w.beta_mode, w.scale, nthreads=nth)
    dt = time.perf_counter() - t
    token_heads = sum(w.lengths[b] for (b, _) in items)
    return {"value": token_heads / w.H / dt, "unit": "tokens/s", "cores": nth, "kind": "oracle",
            "sample": f"all {w.B} sequences x heads 0..{heads - 1} of {w.H} "
                      f"({token_heads} token-heads, {dt:.1f} s), scaled to all heads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="varlen_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter scale)")
    ap.add_argument("--scan-variants", action="store_true",
                    help="segments workloads: also time the exclusive scan alone, ordered against "
                         "blocked, at 16, 64 and 256 segments")
    ap.add_argument("--mfma-calibration", action="store_true",
                    help="also run a kernel of known MFMA count (MFMA-busy counter scale)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by heads or sequences with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import kimi_delta_attention_kda_amd as kda
    from kimi_delta_attention_kda_amd import workloads as wl

    w = wl.workload(args.workload)
    if w.segments:
        return run_segments(args, w)
    if w.name.startswith("decode"):
        return run_decode(args, w)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] workload={w.name} T={w.T} B={w.B} H={w.H} dk={w.dk} dv={w.dv} dtype={w.dtype}",
          file=sys.stderr, flush=True)
    inp = wl.make_inputs(w, dev)
    torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, inp)
        print(f"[bench] cpu_baseline {cpu['value']:.1f} tokens/s on {cpu['cores']} threads",
              file=sys.stderr, flush=True)

    if args.copy_calibration:
        copy_calibration(dev)
    if args.mfma_calibration:
        mfma_calibration(dev)

    pool = inp["state_pool"]
    gate = "safe" if w.gate_mode == 1 else "original"

    def step(out):
        kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["raw_gate"], inp["beta_logits"], inp["a_log"],
                      inp["dt_bias"], inp["cu_seqlens"], pool, inp["state_indices"], gate_mode=gate,
                      lower_bound=w.lower_bound, scale=w.scale, out=out)

    out = torch.empty((w.T, w.H, w.dv), dtype=inp["q"].dtype, device=dev)
    used = torch.tensor(sorted(set(inp["indices"])), dtype=torch.long, device=dev)
    saved = pool.index_select(0, used)
    protocol = per_call_protocol(lambda: step(out), lambda: pool.index_copy_(0, used, saved))
    for _ in range(args.warmup):
        step(out)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps); per-call median {protocol['median_ms']} ms, "
          f"min {protocol['min_ms']} ms", file=sys.stderr, flush=True)

    ms_step, kern_ms = timed_loop(lambda: step(out), args.steps)
    tokens_s = w.T / (ms_step / 1e3)

    nbytes = algorithmic_bytes(w)
    achieved = nbytes / (kern_ms / 1e3) / 1e9
    traffic = measured_traffic(w)
    fl = algorithmic_flops(w)
    fl_dense = dense_tile_flops(w)
    rec = {
        "metric": METRIC if w.name == "varlen_32k" else
        f"KDA prefill tokens/s, {w.name}: H={w.H} dk=dv={w.dk} {w.dtype}, {w.T} tokens",
        "value": round(tokens_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "total_tokens": w.T, "sequences": w.B, "lengths": list(w.lengths),
                   "heads": w.H, "dk": w.dk, "dv": w.dv, "chunk": 64,
                   "gate": gate, "gate_lower_bound": w.lower_bound, "pool_slots": w.n_slots},
        "roofline": {"bound": roofline_bound(fl, nbytes, BF16_PEAK_TFLOPS), "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": f"kda_chunk_fwd call: plan_kernel + {chunk_kernel(w)} + piece_scan_kernel + fixup_kernel",
                     "kernel_ms": round(kern_ms, 4),
                     "algorithmic_bytes_per_launch": nbytes,
                     "intensity_flop_per_byte": round(fl / nbytes, 1),
                     "hbm_floor_ms": round(nbytes / (HBM_PEAK_GBS * 1e9) * 1e3, 4),
                     "times_hbm_floor": round(kern_ms / (nbytes / (HBM_PEAK_GBS * 1e9) * 1e3), 2)},
        "per_call": protocol,
        "mfma": {"algorithmic_tflops": round(fl / (kern_ms / 1e3) / 1e12, 2),
                 "frac_of_bf16_peak": round(fl / (kern_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                 "dense_tile_frac_of_bf16_peak": round(fl_dense / (kern_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                 "profiled_busy": measured_utilization(w),
                 "flops_per_launch_algorithmic": fl},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def copy_calibration(dev):
    """A plain 1 GiB device copy, three times: the counter runs scale HBM byte counters
    by what they read for it."""
    import torch
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("[bench] copy calibration: 3 x 1 GiB read + 1 GiB write", file=sys.stderr, flush=True)


# the MFMA calibration launch: 2048 workgroups of 4 waves (8 waves per SIMD), 8192
# instructions each
CALIB_WG, CALIB_ITERS = 2048, 8192


def mfma_calibration(dev):
    """A kernel of known MFMA count, three times: the counter runs scale the MFMA-busy
    counter by what it reads for it; its event time gives the sustained MFMA rate."""
    import torch
    import kimi_delta_attention_kda_amd as kda
    out = torch.empty(CALIB_WG * 256, dtype=torch.float32, device=dev)
    kda.calib_mfma(CALIB_WG, 16, out)  # warm-up
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(3):
        kda.calib_mfma(CALIB_WG, CALIB_ITERS, out)
    ev[1].record()
    torch.cuda.synchronize()
    n = CALIB_WG * 4 * CALIB_ITERS
    ms = ev[0].elapsed_time(ev[1]) / 3
    tflops = n * 2 * 16 * 16 * 32 / (ms * 1e-3) / 1e12
    print(f"[bench] mfma calibration: {n} v_mfma_f32_16x16x32_bf16 per launch, 3 launches, "
          f"{ms:.3f} ms per launch, {tflops:.1f} TFLOP/s", file=sys.stderr, flush=True)


def run_decode(args, w):
    """kda_decode of one token per sequence (every sequence of the workload has length 1)."""
    import torch
    import kimi_delta_attention_kda_amd as kda
    from kimi_delta_attention_kda_amd import workloads as wl

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] workload={w.name} B={w.B} H={w.H} dk={w.dk} dv={w.dv} dtype={w.dtype}",
          file=sys.stderr, flush=True)
    inp = wl.make_inputs(w, dev)
    torch.cuda.synchronize()
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import build as obuild
        from oracle import oracle as orc
        obuild.build(force=False)
        nth = orc.default_threads()
        items = [(b, h) for b in range(w.B) for h in range(w.H)]
        its = [orc.item_from_inputs(inp, b, h) for (b, h) in items]
        t = time.perf_counter()
        orc.forward_items(its, w.dk, w.dv, w.gate_mode, w.lower_bound, w.beta_mode, w.scale, nthreads=nth)
        dt = time.perf_counter() - t
        cpu = {"value": w.B / dt, "unit": "tokens/s", "cores": nth, "kind": "oracle",
               "sample": f"the whole call: {w.B} sequences x {w.H} heads, one token each ({dt:.2f} s)"}
    if args.copy_calibration:
        copy_calibration(dev)
    if args.mfma_calibration:
        mfma_calibration(dev)
    gate = "safe" if w.gate_mode == 1 else "original"
    pool = inp["state_pool"]
    out = torch.empty((w.B, w.H, w.dv), dtype=inp["q"].dtype, device=dev)

    def step():
        kda.decode(inp["q"], inp["k"], inp["v"], inp["raw_gate"], inp["beta_logits"], inp["a_log"],
                   inp["dt_bias"], pool, inp["state_indices"], gate_mode=gate, lower_bound=w.lower_bound,
                   scale=w.scale, out=out)

    used = torch.tensor(sorted(set(inp["indices"])), dtype=torch.long, device=dev)
    saved = pool.index_select(0, used)
    protocol = per_call_protocol(step, lambda: pool.index_copy_(0, used, saved))
    for _ in range(args.warmup):
        step()
    ms_step, kern_ms = timed_loop(step, args.steps)
    nbytes = decode_bytes(w)
    achieved = nbytes / (kern_ms / 1e3) / 1e9
    rec = {
        "metric": "KDA decode tokens/s (one token per sequence), H=32 dk=dv=128 bf16, 512 sequences",
        "value": round(w.B / (ms_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "sequences": w.B, "heads": w.H, "dk": w.dk, "dv": w.dv,
                   "gate": gate, "gate_lower_bound": w.lower_bound, "pool_slots": w.n_slots},
        "roofline": {"bound": roofline_bound(decode_flops(w), nbytes, FP32_PEAK_TFLOPS),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(w),
                     "kernel": "kda_decode_kernel", "kernel_ms": round(kern_ms, 4),
                     "algorithmic_bytes_per_launch": nbytes},
        "per_call": protocol,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def scan_variants(dev, H, dk, dv, counts=(16, 64, 256), reps=20):
    """The exclusive scan alone, ordered against blocked (automatic block size), on seeded
    random maps M = I + 0.05 N / sqrt(dk), U ~ N(0, 1) of the workload's head and state
    shapes, for several segment counts: per-call median of HIP-event timings."""
    import torch
    import kimi_delta_attention_kda_amd as kda
    g = torch.Generator(device=dev).manual_seed(11)
    out = []
    for n in counts:
        M = torch.eye(dk, device=dev) + 0.05 * torch.randn(n, H, dk, dk, generator=g, device=dev) / dk ** 0.5
        U = torch.randn(n, H, dk, dv, generator=g, device=dev)
        S = torch.randn(H, dk, dv, generator=g, device=dev)
        inc, outg, fin = torch.empty_like(U), torch.empty_like(U), torch.empty_like(S)
        rec = {"segments": n, "block": kda.affine_scan_block_size(n, dk, dv, 0)}
        for name, blk in (("ordered_ms", None), ("blocked_ms", 0)):
            pc = per_call_protocol(lambda: kda.affine_exclusive_scan(M, U, S, inc, outg, fin, block=blk),
                                   lambda: None, reps=reps)
            rec[name] = pc["median_ms"]
        out.append(rec)
        print(f"[bench] scan alone, {n} segments x {H} heads: ordered {rec['ordered_ms']:.4f} ms, "
              f"blocked (blocks of {rec['block']}) {rec['blocked_ms']:.4f} ms", file=sys.stderr, flush=True)
        del M, U, S, inc, outg, fin
    return out


def run_segments(args, w):
    """kda_segment_summary over the workload's equal segments, then kda_affine_exclusive_scan
    of the maps from the initial state: one step of the per-segment pass of KDA Context
    Parallelism on one GPU's share."""
    import torch
    import kimi_delta_attention_kda_amd as kda
    from kimi_delta_attention_kda_amd import workloads as wl

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] workload={w.name} T={w.T} segments={w.segments} H={w.H} dk={w.dk} dv={w.dv} "
          f"dtype={w.dtype}", file=sys.stderr, flush=True)
    inp = wl.make_inputs(w, dev)
    torch.cuda.synchronize()
    gate = "safe" if w.gate_mode == 1 else "original"
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import build as obuild
        from oracle import oracle as orc
        obuild.build(force=False)
        nth = orc.default_threads()
        offs = inp["seg_offsets"].tolist()
        # head 0, as many segments as fill the host threads once, scaled to every map
        nseg = min(w.segments, nth)
        its = [orc.item_from_inputs(inp, 0, 0, with_q=False, t0=offs[i], t1=offs[i + 1]) for i in range(nseg)]
        t = time.perf_counter()
        orc.segment_maps(its, w.dk, w.dv, w.gate_mode, w.lower_bound, w.beta_mode, nthreads=nth)
        dt = time.perf_counter() - t
        tok = offs[nseg] - offs[0]
        cpu = {"value": tok / w.H / dt, "unit": "tokens/s", "cores": nth, "kind": "oracle",
               "sample": f"segment maps of segments 0..{nseg - 1} for head 0 of {w.H} ({tok} tokens, "
                         f"{dt:.1f} s), scaled to all heads; the scan is not included"}
    if args.copy_calibration:
        copy_calibration(dev)
    if args.mfma_calibration:
        mfma_calibration(dev)
    n = w.segments
    M = torch.empty((n, w.H, w.dk, w.dk), dtype=torch.float32, device=dev)
    U = torch.empty((n, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    inc, outg = torch.empty_like(U), torch.empty_like(U)
    fin = torch.empty_like(inp["S_init"])

    def step():
        kda.segment_summary(inp["k"], inp["v"], inp["raw_gate"], inp["beta_logits"], inp["a_log"],
                            inp["dt_bias"], inp["seg_offsets"], gate_mode=gate, lower_bound=w.lower_bound,
                            M=M, U=U)
        kda.affine_exclusive_scan(M, U, inp["S_init"], inc, outg, fin)

    protocol = per_call_protocol(step, lambda: None)  # no state is mutated in place
    for _ in range(args.warmup):
        step()
    ms_step, kern_ms = timed_loop(step, args.steps)
    nbytes = segment_bytes(w)
    fl = segment_flops(w)
    achieved = nbytes / (kern_ms / 1e3) / 1e9
    peak_tf = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    bound = roofline_bound(fl, nbytes, peak_tf)
    tflops = fl / (kern_ms / 1e3) / 1e12
    rec = {
        "metric": f"KDA segment summaries + exclusive scan tokens/s, {w.name}: {w.segments} segments, "
                  f"H={w.H} dk=dv={w.dk} {w.dtype}, {w.T} tokens",
        "value": round(w.T / (ms_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "total_tokens": w.T, "segments": w.segments, "heads": w.H,
                   "dk": w.dk, "dv": w.dv, "gate": gate},
        "roofline": {"bound": bound,
                     "achieved": round(tflops, 2) if bound == "mfma" else round(achieved, 1),
                     "peak": peak_tf if bound == "mfma" else HBM_PEAK_GBS,
                     "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
                     "frac": round((tflops / peak_tf) if bound == "mfma" else (achieved / HBM_PEAK_GBS), 4),
                     "traffic": measured_traffic(w),
                     "flops_per_launch_algorithmic": fl,
                     "intensity_flop_per_byte": round(fl / nbytes, 1),
                     "hbm_achieved_gbs": round(achieved, 1), "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
                     "kernel": ("kda_fast_kernel" if w.dtype == "bf16" and w.gate_mode == 1 and w.lower_bound >= -5.3
                                else "kda_chain_kernel") + " (summaries) + "
                               + ("kda_affine_scan_mfma" if w.dk in (64, 128) else "kda_affine_scan_kernel"),
                     "kernel_ms": round(kern_ms, 4),
                     "algorithmic_bytes_per_launch": nbytes,
                     "profiled_busy": measured_utilization(
                         w, "kda_fast_kernel" if w.dtype == "bf16" and w.gate_mode == 1 and w.lower_bound >= -5.3
                         else "kda_chain_kernel")},
        "per_call": protocol,
        "scan_variants": scan_variants(dev, w.H, w.dk, w.dv) if args.scan_variants and w.dk in (64, 128) else None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
