"""CPU checks of bench.py's roofline denominators and its one-GPU contract.

The compulsory bytes and algorithmic flops of a call are restated here from their parts
(every input read once, every output written once, each used pool slot read and written
once; the chunk form's triangle-aware flop count), so a slip in bench.py's formulas shows.
"""
import os
import subprocess
import sys

import bench
from kimi_delta_attention_kda_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_compulsory_bytes_varlen_32k():
    w = wl.workload("varlen_32k")
    assert (w.T, w.B, w.H, w.dk, w.dv) == (32768, 8, 32, 128, 128)
    per_token = w.H * (3 * 128 * 2 + 128 * 4 + 4 + 128 * 2)  # q k v bf16, raw f32, beta, out bf16
    assert per_token == 49280
    slots = 8 * 2 * (32 * 128 * 128 * 4)                     # 8 slots of 2 MiB, read and written
    small = 32 * (128 + 1) * 4 + 9 * 4 + 8 * 4                # dt_bias, a_log, cu_seqlens, indices
    assert bench.algorithmic_bytes(w) == 32768 * per_token + slots + small == 1648378052


def test_prefill_algorithmic_flops_varlen_32k():
    w = wl.workload("varlen_32k")
    # per token-head: A, P, W at C dk; U~ and PU at C dv; W S, Qbar S, Khat^T U at 2 dk dv
    per = 3 * 64 * 128 + 2 * 64 * 128 + 3 * 2 * 128 * 128
    assert per == 139264
    assert bench.algorithmic_flops(w) == 32768 * 32 * per
    assert round(bench.algorithmic_flops(w) / 1e9, 1) == 146.0


def test_grouped_key_heads_read_q_and_k_once_per_key_head():
    w = wl.custom([100, 28], H=8, Hk=2, dk=64, dv=64, dtype="bf16", gate_mode=1)
    per_token = 8 * (64 * 2 + 64 * 2 + 64 * 4 + 4) + 2 * (2 * 64 * 2)  # v out raw beta; q k
    slots = 2 * 2 * (8 * 64 * 64 * 4)
    assert bench.algorithmic_bytes(w) == 128 * per_token + slots + 8 * 65 * 4 + 3 * 4 + 2 * 4


def test_segment_pass_compulsory_bytes():
    w = wl.workload("segments_262k")
    assert (w.T, w.H, w.segments, w.dk, w.dv, w.dtype) == (262144, 8, 16, 128, 128, "f32")
    inputs = 262144 * 8 * (128 * 4 + 128 * 4 + 128 * 4 + 4) + 8 * 129 * 4 + 17 * 4  # k v raw beta; gates; offsets
    maps = 16 * 8 * 128 * 256 * 4                 # M and U, written then read by the scan
    scan = 2 * 16 * 8 * 128 * 128 * 4 + 2 * 8 * 128 * 128 * 4   # incoming, outgoing; S_init, final
    assert bench.segment_bytes(w) == inputs + 2 * maps + scan


def test_segment_pass_flops_and_bound():
    """The summaries run the chunk form on the augmented state [M | U] (width dk + dv = 256):
    scores C dk, solve C (dk + dv), prediction and state update 2 dk (dk + dv) each; the
    scan adds 2 dk^2 dv per map.  At ~100 flop/B the fp32 pass lies above the fp32 ridge
    (157.3 TFLOP/s / 8 TB/s ~ 20 flop/B): its roofline is the matrix-core peak."""
    w = wl.workload("segments_262k")
    per = 64 * 128 + 64 * 256 + 2 * 128 * 256 + 2 * 128 * 256
    assert per == 155648
    fl = 262144 * 8 * per + 16 * 8 * 2 * 128 ** 3
    assert bench.segment_flops(w) == fl
    assert bench.roofline_bound(fl, bench.segment_bytes(w), bench.FP32_PEAK_TFLOPS) == "mfma"
    # the bf16 prefill at ~89 flop/B lies below the bf16 ridge (~312 flop/B): HBM
    v = wl.workload("varlen_32k")
    assert bench.roofline_bound(bench.algorithmic_flops(v), bench.algorithmic_bytes(v),
                                bench.BF16_PEAK_TFLOPS) == "hbm"


def test_decode_compulsory_bytes():
    w = wl.workload("decode_512")
    assert (w.B, w.T, w.H, w.dk, w.dv) == (512, 512, 32, 128, 128)
    per = 2 * 128 * 128 * 4 + 3 * 128 * 2 + 128 * 2 + 128 * 4 + 4  # state r+w, q k v, out, raw, beta
    assert bench.decode_bytes(w) == 512 * 32 * per + 32 * 129 * 4 + 512 * 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
