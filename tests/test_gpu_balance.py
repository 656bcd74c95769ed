"""GPU parity of the load-balanced forward pass (bf16, safe gate, dk = dv in {64, 128}).

Long sequences are cut into pieces whose transition and contribution chains run in
parallel; their states are composed in order and the outputs corrected.  These tests
check (1) that the device plans what the host restatement of the rule expects, (2) the
results against the fp64 oracle on every (sequence, head), with many pieces per
sequence, (3) agreement with the unbalanced launch and between the torch and library
workspaces, and (4) that a too-small workspace is refused before any launch.
"""
import ctypes as C

import numpy as np
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


# the forward pass runs 64-token chunks, one workgroup per CU
CHUNK, PER_CU = 64, 1


def _n_slots():
    return PER_CU * torch.cuda.get_device_properties(0).multi_processor_count


def _desc(w, inp):
    return kda.make_desc(w.T, w.B, w.H, w.dk, w.dv, inp["state_pool"].shape[0], torch.bfloat16,
                         torch.bfloat16, "safe" if w.gate_mode == 1 else "original", w.lower_bound, "logits",
                         "K_FIRST", w.scale)


def _run_with_ws(w, inp, nbytes=None):
    """kda_chunk_fwd_ws with a caller workspace; returns (out, pool, header ints)."""
    d = _desc(w, inp)
    need = C.c_size_t(0)
    assert kda.lib().kda_chunk_fwd_workspace_size(C.byref(d), C.byref(need)) == 0
    nb = need.value if nbytes is None else nbytes
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    pool = inp["state_pool"].clone()
    out = torch.empty((w.T, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    st = kda.lib().kda_chunk_fwd_ws(C.byref(d), inp["q"].data_ptr(), inp["k"].data_ptr(),
                                    inp["v"].data_ptr(), inp["raw_gate"].data_ptr(),
                                    inp["beta_logits"].data_ptr(), inp["a_log"].data_ptr(),
                                    inp["dt_bias"].data_ptr(), inp["cu_seqlens"].data_ptr(),
                                    pool.data_ptr(), inp["state_indices"].data_ptr(), out.data_ptr(),
                                    ws.data_ptr(), nb, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    hdr = ws[:128].view(torch.int32).cpu().numpy() if st == 0 else None
    return st, out, pool, hdr


def _header(h):
    # PlanHeader: ctr, qlen, n_split, n_piece, n_echunk, L, n_ent, n_sorted
    return {"ctr": int(h[0]), "qlen": int(h[1]), "n_split": int(h[2]), "n_piece": int(h[3]),
            "n_echunk": int(h[4]), "L": int(h[5]), "n_ent": int(h[6]), "n_sorted": int(h[7])}


def _check_plan(w, hdr):
    from plan_rule import plan
    exp = plan(list(w.lengths), w.H, _n_slots(), CHUNK)
    got = _header(hdr)
    print(f"  plan: expected {exp}, device {got}", flush=True)
    for key in ("L", "n_split", "n_piece", "n_echunk"):
        assert got[key] == exp[key], key
    assert got["n_ent"] == w.B + exp["n_piece"]
    # every (entity of nonzero length, head) is queued once, its later pieces as pairs;
    # the chunk kernel's workgroups drew every slot and one past the end each
    n_nonzero = sum(1 for x in w.lengths if x > 0) + exp["n_piece"]
    assert got["n_sorted"] == n_nonzero
    assert got["qlen"] == 2 * n_nonzero * w.H
    assert got["ctr"] == got["qlen"] + 8 * ((_n_slots() + 7) // 8)


def _compare_all(w, inp, out, pool):
    from kda_testlib import compare_items, OUT_TOL_BF16, STATE_TOL
    items = [(b, h) for b in range(w.B) for h in range(w.H)]
    eo, es = compare_items(w, inp, out, pool, items)
    print(f"  all {len(items)} (sequence, head) pairs: out_err={eo:.3e} state_err={es:.3e}", flush=True)
    assert eo <= OUT_TOL_BF16
    assert es <= STATE_TOL


@pytest.mark.parametrize("lengths,dk", [((4096,), 128), ((3000, 100, 5000, 0, 64, 777), 128),
                                        ((4096,), 64), ((3000, 100, 5000, 0, 64, 777), 64)])
def test_many_pieces_against_oracle(lengths, dk):
    """Few chains on many CUs: every long sequence becomes many pieces."""
    from kda_testlib import untouched_slots_identical
    w = wl.custom(lengths, H=2, dk=dk, dv=dk, name="pieces")
    print(f"[case] pieces lengths={lengths} H=2 dk={dk}", flush=True)
    inp = wl.make_inputs(w, "cuda")
    st, out, pool, hdr = _run_with_ws(w, inp)
    assert st == 0
    _check_plan(w, hdr)
    assert _header(hdr)["n_piece"] >= 4
    assert untouched_slots_identical(inp, pool)
    _compare_all(w, inp, out, pool)


@pytest.mark.parametrize("dk", [128, 64])
def test_original_gate_pieces_against_oracle(dk):
    """bf16 with the original gate runs the precise walk over the same plan: the later
    pieces as transition and contribution chains, then the piece-state scan and the
    correction."""
    from kda_testlib import untouched_slots_identical
    lengths = (3000, 100, 5000, 0, 64, 777)
    w = wl.custom(lengths, H=2, dk=dk, dv=dk, gate_mode=0, name="pieces_original_gate", seed=5)
    print(f"[case] original gate, pieces lengths={lengths} H=2 dk={dk}", flush=True)
    inp = wl.make_inputs(w, "cuda")
    st, out, pool, hdr = _run_with_ws(w, inp)
    assert st == 0
    _check_plan(w, hdr)
    assert _header(hdr)["n_piece"] >= 4
    assert untouched_slots_identical(inp, pool)
    _compare_all(w, inp, out, pool)


@pytest.mark.parametrize("dk", [128, 64])
def test_varlen_32k_plan_and_agreement(dk):
    """The benchmark workload (and its lengths at dk = 64): the three longest sequences are
    split; the balanced pass agrees with the unbalanced one, and the library's pool path
    with the torch one."""
    from kda_testlib import run_fwd, rel_out, rel_fro, untouched_slots_identical
    w = wl.workload("varlen_32k" if dk == 128 else "varlen_32k_dk64")
    print(f"[case] varlen_32k plan dk={dk}, lengths={w.lengths}", flush=True)
    inp = wl.make_inputs(w, "cuda")
    st, out, pool, hdr = _run_with_ws(w, inp)
    assert st == 0
    _check_plan(w, hdr)
    assert _header(hdr)["n_split"] >= 1
    assert untouched_slots_identical(inp, pool)
    out_n, pool_n = run_fwd(w, inp, workspace="none")
    eo = rel_out(out.float().cpu().numpy(), out_n.float().cpu().numpy())
    es = max(rel_fro(pool[s].cpu().numpy().astype(np.float64), pool_n[s].cpu().numpy().astype(np.float64))
             for s in inp["indices"])
    print(f"  balanced vs unbalanced: out {eo:.3e} state {es:.3e}", flush=True)
    assert eo <= 2e-2 and es <= 1e-3
    out_l, pool_l = run_fwd(w, inp, workspace="library")
    assert torch.equal(out.view(torch.int16), out_l.view(torch.int16))
    assert torch.equal(pool.view(torch.int32), pool_l.view(torch.int32))


@pytest.mark.parametrize("dk", [128, 64])
def test_workspace_too_small_is_refused(dk):
    w = wl.custom((4096,), H=2, dk=dk, dv=dk, name="small_ws")
    print(f"[case] too-small workspace dk={dk}", flush=True)
    inp = wl.make_inputs(w, "cuda")
    d = _desc(w, inp)
    need = C.c_size_t(0)
    assert kda.lib().kda_chunk_fwd_workspace_size(C.byref(d), C.byref(need)) == 0
    assert need.value > 0
    st, _, pool, _ = _run_with_ws(w, inp, nbytes=need.value - 1)
    assert st == 2  # KDA_ERR_SHAPE, nothing launched
    assert torch.equal(pool.view(torch.int32), inp["state_pool"].view(torch.int32))


def test_torch_workspace_oom_falls_back(monkeypatch):
    """workspace="torch" whose allocation fails runs the unbalanced launch, bit for bit."""
    from kda_testlib import run_fwd
    w = wl.custom((3000, 700), H=2, dk=128, dv=128, name="oom_ws", seed=21)
    print("[case] torch workspace allocation fails", flush=True)
    inp = wl.make_inputs(w, "cuda")
    real_empty = torch.empty

    def empty(*a, **kw):
        if kw.get("dtype") is torch.uint8:
            raise torch.OutOfMemoryError("simulated workspace allocation failure")
        return real_empty(*a, **kw)

    monkeypatch.setattr(torch, "empty", empty)
    out, pool = run_fwd(w, inp, workspace="torch")
    monkeypatch.undo()
    out_n, pool_n = run_fwd(w, inp, workspace="none")
    assert torch.equal(out.view(torch.int16), out_n.view(torch.int16))
    assert torch.equal(pool.view(torch.int32), pool_n.view(torch.int32))


@pytest.mark.parametrize("dk", [128, 64])
def test_random_mixes_plan_and_agreement(dk):
    """Seeded random batches (1 to 40 sequences of 1 to 20,000 tokens, 1 to 3 heads, some empty):
    the device plan equals the host rule, and the balanced pass agrees with the unbalanced one
    (outputs within the bf16 bound, states within the state bound)."""
    from kda_testlib import run_fwd, rel_out, rel_fro, untouched_slots_identical, OUT_TOL_BF16, STATE_TOL
    rng = np.random.default_rng(100 + dk)
    for trial in range(6):
        B = int(rng.integers(1, 41))
        lengths = rng.integers(1, 20001, size=B)
        lengths[rng.random(B) < 0.1] = 0
        H = int(rng.integers(1, 4))
        w = wl.custom(lengths.tolist(), H=H, dk=dk, dv=dk, seed=200 + trial, name="mix")
        if w.T == 0:
            continue
        print(f"[case] random mix {trial}: dk={dk} B={B} H={H} T={w.T}", flush=True)
        inp = wl.make_inputs(w, "cuda")
        st, out, pool, hdr = _run_with_ws(w, inp)
        assert st == 0
        _check_plan(w, hdr)
        assert untouched_slots_identical(inp, pool)
        out_n, pool_n = run_fwd(w, inp, workspace="none")
        for b in range(w.B):
            a, e = inp["cu"][b], inp["cu"][b + 1]
            s = inp["indices"][b]
            if e > a:
                assert rel_out(wl.as_f64(out[a:e]), wl.as_f64(out_n[a:e])) <= OUT_TOL_BF16
            assert rel_fro(wl.as_f64(pool[s]), wl.as_f64(pool_n[s])) <= STATE_TOL
