"""The entry point without allocation (kda_chunk_fwd_noalloc): the load-balanced prefill
with its workspace in the library's fixed device scratch, against the same pass with a
caller-provided workspace (kda_chunk_fwd_ws).

Two calls in a row on one device, the second with a smaller input, so that the second
reads a scratch holding the first call's plan: with the same plan the two entry points
must give the same bits.  A call whose plan does not fit the scratch (one long sequence,
many heads) is served with fewer pieces and is held to the oracle's tolerances.
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


def _both(w, inp):
    from kda_testlib import run_fwd
    out_s, pool_s = run_fwd(w, inp, workspace="static")
    out_t, pool_t = run_fwd(w, inp, workspace="torch")
    return out_s, pool_s, out_t, pool_t


@pytest.mark.parametrize("dk,gate", [(128, 1), (64, 1), (128, 0)])
def test_noalloc_matches_the_workspace_entry_point_on_two_calls(dk, gate):
    """gate 1: the safe gate (fast kernels); gate 0: the original gate (the chunk walk over
    the same plan)."""
    from kda_testlib import compare_items, untouched_slots_identical, report, OUT_TOL_BF16, STATE_TOL
    first = wl.custom([5000, 300, 2000, 64, 0, 1500, 700], H=2, dk=dk, dv=dk, dtype="bf16", gate_mode=gate,
                      n_slots=12, seed=31)
    second = wl.custom([1200, 77, 640], H=2, dk=dk, dv=dk, dtype="bf16", gate_mode=gate, n_slots=5, seed=32)
    for w in (first, second):
        print(f"[case] noalloc dk={dk} gate_mode={gate} lengths={w.lengths}", flush=True)
        inp = wl.make_inputs(w, "cuda")
        out_s, pool_s, out_t, pool_t = _both(w, inp)
        assert torch.equal(out_s.view(torch.int16), out_t.view(torch.int16))
        assert torch.equal(pool_s.view(torch.int32), pool_t.view(torch.int32))
        assert untouched_slots_identical(inp, pool_s)
        items = [(b, h) for b in range(w.B) for h in range(w.H)]
        eo, es = compare_items(w, inp, out_s, pool_s, items)
        report(f"no-alloc entry point, dk={dk}, gate_mode={gate}, lengths {w.lengths}: bit-identical to the workspace "
               f"entry point; oracle out_err={eo:.3e} state_err={es:.3e}")
        assert eo <= OUT_TOL_BF16 and es <= STATE_TOL


def test_noalloc_plan_capped_by_the_scratch():
    """One 40,000-token sequence at H = 32: its later pieces' correction rows need more
    than the scratch holds, so the planner cuts fewer pieces; results stay within the
    oracle's tolerances and agree with the workspace entry point up to rounding."""
    from kda_testlib import compare_items, rel_out, rel_fro, report, OUT_TOL_BF16, STATE_TOL
    w = wl.custom([40000, 900], H=32, dk=128, dv=128, dtype="bf16", gate_mode=1, n_slots=3, seed=33)
    print(f"[case] noalloc capped lengths={w.lengths} H={w.H}", flush=True)
    inp = wl.make_inputs(w, "cuda")
    out_s, pool_s, out_t, pool_t = _both(w, inp)
    d_out = rel_out(wl.as_f64(out_s), wl.as_f64(out_t))
    s = inp["indices"][0]
    d_st = rel_fro(wl.as_f64(pool_s[s]), wl.as_f64(pool_t[s]))
    assert d_out <= OUT_TOL_BF16 and d_st <= STATE_TOL
    items = [(0, h) for h in (0, 17, 31)] + [(1, h) for h in range(w.H)]
    eo, es = compare_items(w, inp, out_s, pool_s, items)
    report(f"no-alloc entry point, plan capped by the scratch (40,000 + 900 tokens, H=32): vs workspace "
           f"entry point out {d_out:.3e} state {d_st:.3e}; oracle ({len(items)} pairs) out_err={eo:.3e} "
           f"state_err={es:.3e}")
    assert eo <= OUT_TOL_BF16 and es <= STATE_TOL
