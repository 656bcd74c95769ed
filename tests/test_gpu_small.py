"""GPU parity at small sizes: every (sequence, head) compared with the fp64 oracle.

Sizes span several 64-token chunks, ragged last chunks and edge lengths
(0, 1, 63, 64, 65), in both arithmetic variants (bf16 safe gate, fp32 any gate).
"""
import numpy as np
import pytest
import torch

from kimi_delta_attention_kda_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from oracle import build
    build.build(force=False)


def _all_items(w):
    return [(b, h) for b in range(w.B) for h in range(w.H)]


@pytest.mark.parametrize("dk", [64, 128])
def test_bf16_varlen_ragged(dk):
    from kda_testlib import compare_items, run_fwd, untouched_slots_identical, OUT_TOL_BF16, STATE_TOL
    w = wl.custom([1, 63, 64, 65, 200, 0, 129], H=2, dk=dk, dv=dk, dtype="bf16", gate_mode=1, seed=3)
    inp = wl.make_inputs(w, "cuda")
    print(f"[case] bf16 varlen dk={dk} lengths={w.lengths}", flush=True)
    out, pool = run_fwd(w, inp)
    eo, es = compare_items(w, inp, out, pool, _all_items(w))
    print(f"  out_err={eo:.3e} state_err={es:.3e}", flush=True)
    assert eo <= OUT_TOL_BF16 and es <= STATE_TOL
    assert untouched_slots_identical(inp, pool)
    # the empty sequence's slot is untouched too
    s_empty = inp["indices"][5]
    assert torch.equal(pool[s_empty].view(torch.int32), inp["state_pool"][s_empty].view(torch.int32))


def test_fp32_tiny_original_gate():
    from kda_testlib import compare_items, run_fwd, OUT_TOL_F32, STATE_TOL
    w = wl.workload("tiny_fp32")
    inp = wl.make_inputs(w, "cuda")
    print(f"[case] tiny_fp32 T={w.T}", flush=True)
    out, pool = run_fwd(w, inp)
    eo, es = compare_items(w, inp, out, pool, _all_items(w))
    print(f"  out_err={eo:.3e} state_err={es:.3e}", flush=True)
    assert eo <= OUT_TOL_F32 and es <= STATE_TOL


def test_fp32_ragged_safe_and_original():
    from kda_testlib import compare_items, run_fwd, OUT_TOL_F32, STATE_TOL
    for gm in (0, 1):
        w = wl.custom([65, 1, 130], H=2, dk=64, dv=64, dtype="f32", gate_mode=gm, seed=5)
        inp = wl.make_inputs(w, "cuda")
        print(f"[case] fp32 ragged gate_mode={gm}", flush=True)
        out, pool = run_fwd(w, inp)
        eo, es = compare_items(w, inp, out, pool, _all_items(w))
        print(f"  out_err={eo:.3e} state_err={es:.3e}", flush=True)
        assert eo <= OUT_TOL_F32 and es <= STATE_TOL


@pytest.mark.parametrize("dtype,dk,gate,lb", [("f32", 128, 0, -5.0), ("f32", 128, 1, -5.0),
                                               ("bf16", 64, 0, -5.0), ("bf16", 128, 0, -5.0),
                                               ("bf16", 128, 1, -8.0)])
def test_precise_walk_ragged(dtype, dk, gate, lb):
    """Calls outside the fast kernel's range -- fp32 inputs, or bf16 with the original gate
    (decays down to about e^-48 per token here) or a safe bound below -5.3 -- run the
    precise chunk walk; ragged lengths around the chunk size, an empty sequence."""
    from kda_testlib import compare_items, run_fwd, untouched_slots_identical
    from kda_testlib import OUT_TOL_BF16, OUT_TOL_F32, STATE_TOL
    w = wl.custom([65, 1, 0, 130, 64], H=2, dk=dk, dv=dk, dtype=dtype, gate_mode=gate, seed=21,
                  lower_bound=lb)
    print(f"[case] precise walk {dtype} dk={dk} gate_mode={gate} bound={lb}", flush=True)
    inp = wl.make_inputs(w, "cuda")
    out, pool = run_fwd(w, inp)
    eo, es = compare_items(w, inp, out, pool, _all_items(w))
    print(f"  out_err={eo:.3e} state_err={es:.3e}", flush=True)
    assert eo <= (OUT_TOL_BF16 if dtype == "bf16" else OUT_TOL_F32) and es <= STATE_TOL
    assert untouched_slots_identical(inp, pool)
