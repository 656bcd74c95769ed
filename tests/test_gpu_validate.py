"""GPU checks of the data-dependent preconditions.

kda_validate_varlen accepts a well-formed batch and returns KDA_ERR_DATA for each kind of
violation (offsets not starting at 0, not ending at T, decreasing; a slot index out of
range or repeated).  With KDA_DEBUG_VALIDATE=1 the asynchronous calls run the same checks
first and refuse bad data before touching the pool.
"""
import ctypes as C
import os

import pytest
import torch

import kimi_delta_attention_kda_amd as kda
from kimi_delta_attention_kda_amd import workloads as wl

pytestmark = pytest.mark.gpu

OK, EDATA = 0, 7


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _validate(cu, T, idx, max_slots):
    cu = torch.tensor(cu, dtype=torch.int32, device="cuda")
    idx = torch.tensor(idx, dtype=torch.int32, device="cuda")
    return kda.lib().kda_validate_varlen(C.c_void_p(cu.data_ptr()), len(idx), T,
                                         C.c_void_p(idx.data_ptr()), max_slots)


def test_validate_varlen_cases():
    print("[case] kda_validate_varlen", flush=True)
    assert _validate([0, 3, 3, 10], 10, [2, 0, 5], 6) == OK
    assert _validate([1, 3, 3, 10], 10, [2, 0, 5], 6) == EDATA   # first offset not 0
    assert _validate([0, 3, 3, 9], 10, [2, 0, 5], 6) == EDATA    # last offset not T
    assert _validate([0, 4, 3, 10], 10, [2, 0, 5], 6) == EDATA   # decreasing
    assert _validate([0, 3, 3, 10], 10, [2, 0, 6], 6) == EDATA   # index out of range
    assert _validate([0, 3, 3, 10], 10, [2, -1, 5], 6) == EDATA  # negative index
    assert _validate([0, 3, 3, 10], 10, [2, 0, 2], 6) == EDATA   # repeated index


def test_debug_validate_refuses_bad_data(monkeypatch):
    from kda_testlib import run_fwd
    w = wl.custom([70, 130], H=2, dk=128, dv=128, dtype="bf16", gate_mode=1, seed=15)
    print("[case] KDA_DEBUG_VALIDATE on chunk_fwd and decode", flush=True)
    inp = wl.make_inputs(w, "cuda")
    monkeypatch.setenv("KDA_DEBUG_VALIDATE", "1")
    # well-formed: runs as usual
    out, pool = run_fwd(w, inp)
    assert not torch.equal(pool.view(torch.int32), inp["state_pool"].view(torch.int32))
    # a repeated slot: refused before any launch, the pool untouched
    bad = dict(inp)
    bad["state_indices"] = torch.full_like(inp["state_indices"], int(inp["indices"][0]))
    for ws in ("torch", "none", "library"):
        p = inp["state_pool"].clone()
        with pytest.raises(ValueError):
            run_fwd(w, bad, pool=p, workspace=ws)
        assert torch.equal(p.view(torch.int32), inp["state_pool"].view(torch.int32))
    # decreasing offsets
    bad = dict(inp)
    bad["cu_seqlens"] = torch.tensor([0, 250, 200], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        run_fwd(w, bad)
    # decode with a repeated slot
    dw = wl.custom([1] * 4, H=2, dk=128, dv=128, dtype="bf16", gate_mode=1, seed=16)
    dinp = wl.make_inputs(dw, "cuda")
    idx = torch.zeros(4, dtype=torch.int32, device="cuda")
    pool_before = dinp["state_pool"].clone()
    with pytest.raises(ValueError):
        kda.decode(dinp["q"], dinp["k"], dinp["v"], dinp["raw_gate"], dinp["beta_logits"], dinp["a_log"],
                   dinp["dt_bias"], dinp["state_pool"], idx, gate_mode="safe", lower_bound=dw.lower_bound)
    torch.cuda.synchronize()
    assert torch.equal(dinp["state_pool"].view(torch.int32), pool_before.view(torch.int32))
    # without the variable, nothing is checked (the call is asynchronous)
    monkeypatch.delenv("KDA_DEBUG_VALIDATE")
    assert os.environ.get("KDA_DEBUG_VALIDATE") is None


def test_debug_validate_segment_offsets(monkeypatch):
    """Segment offsets need only lie in [0, T] and not decrease."""
    w = wl.custom([300], H=2, dk=128, dv=128, dtype="bf16", gate_mode=1, seed=17)
    print("[case] KDA_DEBUG_VALIDATE on segment_summary", flush=True)
    inp = wl.make_inputs(w, "cuda")
    monkeypatch.setenv("KDA_DEBUG_VALIDATE", "1")
    args = (inp["k"], inp["v"], inp["raw_gate"], inp["beta_logits"], inp["a_log"], inp["dt_bias"])
    ok = torch.tensor([10, 100, 290], dtype=torch.int32, device="cuda")   # inside [0, T], not from 0
    M, U = kda.segment_summary(*args, ok)
    torch.cuda.synchronize()
    assert M.shape[0] == 2 and torch.isfinite(M).all() and torch.isfinite(U).all()
    for bad in ([0, 200, 100], [0, 100, 301], [-1, 100, 200]):
        with pytest.raises(ValueError):
            kda.segment_summary(*args, torch.tensor(bad, dtype=torch.int32, device="cuda"))
