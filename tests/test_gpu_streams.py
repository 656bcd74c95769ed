"""The calls run on the caller's stream, and can be captured in a HIP graph.

- On a side stream (default priority), prefill in each workspace mode, decode and the
  segment summaries give the same bits as on the default stream.
- A prefill captured in a graph (torch workspace, and without load balancing) is
  replayed three times with eager work and synchronisations between the replays; every
  replay equals the matching eager call bit for bit (the pool advances one call per
  replay).
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


def _fwd(w, inp, pool, workspace, out=None):
    return kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["raw_gate"], inp["beta_logits"], inp["a_log"],
                         inp["dt_bias"], inp["cu_seqlens"], pool, inp["state_indices"], gate_mode="safe",
                         lower_bound=w.lower_bound, scale=w.scale, workspace=workspace, out=out)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("workspace", ["torch", "library", "none"])
def test_prefill_on_a_side_stream(workspace):
    w = wl.custom([3000, 70, 0, 129, 1], H=2, dk=128, dv=128, dtype="bf16", gate_mode=1, seed=31,
                  name="streams")
    print(f"[case] prefill on a side stream, workspace={workspace}", flush=True)
    inp = wl.make_inputs(w, "cuda")
    pool_d = inp["state_pool"].clone()
    out_d = _fwd(w, inp, pool_d, workspace)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    pool_s = inp["state_pool"].clone()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out_s = _fwd(w, inp, pool_s, workspace)
    s.synchronize()
    assert torch.equal(_bits(out_s), _bits(out_d))
    assert torch.equal(_bits(pool_s), _bits(pool_d))


def test_decode_and_summaries_on_a_side_stream():
    print("[case] decode and segment summaries on a side stream", flush=True)
    dw = wl.custom([1] * 12, H=4, dk=128, dv=128, dtype="bf16", gate_mode=1, name="dstream", n_slots=16)
    d = wl.make_inputs(dw, "cuda")
    sw = wl.custom([3 * 256], H=2, dk=64, dv=64, dtype="bf16", gate_mode=1, name="sstream", n_slots=1,
                   segments=3, raw_mean=-6.0, a_log_hi=0.0)
    g = wl.make_inputs(sw, "cuda")

    def run(pool):
        o = kda.decode(d["q"], d["k"], d["v"], d["raw_gate"], d["beta_logits"], d["a_log"], d["dt_bias"],
                       pool, d["state_indices"], lower_bound=dw.lower_bound)
        M, U = kda.segment_summary(g["k"], g["v"], g["raw_gate"], g["beta_logits"], g["a_log"], g["dt_bias"],
                                   g["seg_offsets"], lower_bound=sw.lower_bound)
        return o, M, U

    pool_d = d["state_pool"].clone()
    ref = run(pool_d)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    pool_s = d["state_pool"].clone()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        got = run(pool_s)
    s.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(_bits(a), _bits(b))
    assert torch.equal(_bits(pool_s), _bits(pool_d))


@pytest.mark.parametrize("workspace", ["torch", "none"])
def test_prefill_graph_replays_match_eager(workspace):
    w = wl.custom([3000, 70, 0, 129, 1], H=2, dk=128, dv=128, dtype="bf16", gate_mode=1, seed=32,
                  name="graph")
    print(f"[case] prefill in a HIP graph, workspace={workspace}", flush=True)
    inp = wl.make_inputs(w, "cuda")
    # eager: three calls in a row on one pool
    pool_e = inp["state_pool"].clone()
    eager = []
    for _ in range(3):
        o = _fwd(w, inp, pool_e, workspace)
        eager.append((o.clone(), pool_e.clone()))
    torch.cuda.synchronize()
    # graph: warm up on a side stream, capture one call, replay three times from the start
    pool_g = inp["state_pool"].clone()
    out_g = torch.empty((w.T, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _fwd(w, inp, pool_g, workspace, out=out_g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _fwd(w, inp, pool_g, workspace, out=out_g)
    pool_g.copy_(inp["state_pool"])
    torch.cuda.synchronize()
    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out_g), _bits(eager[r][0])), r
        assert torch.equal(_bits(pool_g), _bits(eager[r][1])), r
        # eager work between replays
        (inp["raw_gate"] * 1.0).sum().item()
        torch.cuda.synchronize()
