"""GPU parity of the contract variants: single-token decode, the V_FIRST pool layout and
beta given as a probability.

Decode is compared with the fp64 oracle's token recurrence (one token per sequence, on
every (sequence, head)); V_FIRST must reproduce the K_FIRST results bit for bit (only
the addressing of the pool slots differs); probability-mode beta is compared with the
oracle on every (sequence, head).
"""
import pytest
import torch

import kimi_delta_attention_kda_amd as kda
from kimi_delta_attention_kda_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from oracle import build
    build.build(force=False)


def _gate(w):
    return "safe" if w.gate_mode == 1 else "original"


def _beta(w):
    return "logits" if w.beta_mode == 0 else "probability"


def _decode(w, inp, pool, layout="K_FIRST"):
    out = kda.decode(inp["q"], inp["k"], inp["v"], inp["raw_gate"], inp["beta_logits"], inp["a_log"],
                     inp["dt_bias"], pool, inp["state_indices"], gate_mode=_gate(w), lower_bound=w.lower_bound,
                     beta_mode=_beta(w), state_layout=layout, scale=w.scale)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype,dk,gate,beta", [("bf16", 128, 1, 0), ("bf16", 64, 0, 1),
                                                ("f32", 128, 0, 0), ("f32", 64, 1, 1)])
def test_decode_against_oracle(dtype, dk, gate, beta):
    from kda_testlib import compare_items, untouched_slots_identical, OUT_TOL_BF16, OUT_TOL_F32, STATE_TOL
    B, H = 37, 4
    w = wl.custom([1] * B, H=H, dk=dk, dv=dk, dtype=dtype, gate_mode=gate, beta_mode=beta, name="decode",
                  n_slots=2 * B, state_sigma=0.05)
    print(f"[case] decode {dtype} dk={dk} gate={_gate(w)} beta={_beta(w)} B={B} H={H}", flush=True)
    inp = wl.make_inputs(w, "cuda")
    pool = inp["state_pool"].clone()
    out = _decode(w, inp, pool)
    assert untouched_slots_identical(inp, pool)
    # out rows are [B, H, dv]; the helper reads out[cu[b]:cu[b+1], h] -- the same rows
    items = [(b, h) for b in range(B) for h in range(H)]
    eo, es = compare_items(w, inp, out.view(B, H, dk), pool, items)
    print(f"  out_err={eo:.3e} state_err={es:.3e}", flush=True)
    assert eo <= (OUT_TOL_BF16 if dtype == "bf16" else OUT_TOL_F32)
    assert es <= STATE_TOL


def test_decode_v_first_equals_k_first():
    w = wl.custom([1] * 16, H=8, dk=128, dv=128, dtype="bf16", name="decode_vf", n_slots=20)
    print("[case] decode V_FIRST vs K_FIRST", flush=True)
    inp = wl.make_inputs(w, "cuda")
    pk = inp["state_pool"].clone()
    pv = inp["state_pool"].transpose(-1, -2).contiguous()
    ok = _decode(w, inp, pk)
    ov = _decode(w, inp, pv, "V_FIRST")
    assert torch.equal(ok.view(torch.int16), ov.view(torch.int16))
    assert torch.equal(pk.view(torch.int32), pv.transpose(-1, -2).contiguous().view(torch.int32))


@pytest.mark.parametrize("dtype,dk,workspace", [("bf16", 128, "torch"), ("bf16", 128, "none"),
                                                ("bf16", 64, "torch"), ("f32", 64, "torch")])
def test_prefill_v_first_equals_k_first(dtype, dk, workspace):
    """Same arithmetic, only the slot addressing differs: bitwise-equal results.  The
    lengths make the bf16 dk=128 balanced pass split the long sequence into pieces."""
    from kda_testlib import run_fwd
    w = wl.custom([3000, 70, 0, 129, 1], H=2, dk=dk, dv=dk, dtype=dtype, gate_mode=1, name="vfirst")
    print(f"[case] prefill V_FIRST {dtype} dk={dk} workspace={workspace}", flush=True)
    inp = wl.make_inputs(w, "cuda")
    out_k, pool_k = run_fwd(w, inp, workspace=workspace)
    pool_v = inp["state_pool"].transpose(-1, -2).contiguous()
    out_v = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["raw_gate"], inp["beta_logits"], inp["a_log"],
                          inp["dt_bias"], inp["cu_seqlens"], pool_v, inp["state_indices"], gate_mode="safe",
                          lower_bound=w.lower_bound, state_layout="V_FIRST", scale=w.scale, workspace=workspace)
    torch.cuda.synchronize()
    assert torch.equal(out_k.view(torch.int16 if dtype == "bf16" else torch.int32),
                       out_v.view(torch.int16 if dtype == "bf16" else torch.int32))
    assert torch.equal(pool_k.view(torch.int32), pool_v.transpose(-1, -2).contiguous().view(torch.int32))


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_prefill_beta_probability(dtype, dk):
    from kda_testlib import run_fwd, compare_items, OUT_TOL_BF16, OUT_TOL_F32, STATE_TOL
    w = wl.custom([1000, 64, 333], H=2, dk=dk, dv=dk, dtype=dtype, gate_mode=1, beta_mode=1, name="betaprob")
    print(f"[case] prefill beta probability {dtype} dk={dk}", flush=True)
    inp = wl.make_inputs(w, "cuda")
    out, pool = run_fwd(w, inp)
    items = [(b, h) for b in range(w.B) for h in range(w.H)]
    eo, es = compare_items(w, inp, out, pool, items)
    print(f"  out_err={eo:.3e} state_err={es:.3e}", flush=True)
    assert eo <= (OUT_TOL_BF16 if dtype == "bf16" else OUT_TOL_F32)
    assert es <= STATE_TOL
