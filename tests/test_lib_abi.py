"""CPU-side checks of the C ABI: exported symbols, status strings, and every
host-checkable error path (validation returns before any device work, so these
run without a GPU).  Also: the binding fails loudly when the library is missing."""
import ctypes as C
import os
import re
import subprocess

import pytest
import torch

import kimi_delta_attention_kda_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libkda.h")

OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EARG = 0, 1, 2, 3, 4, 5
FAKE = 0x1000  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kda.LIB_PATH):
        from kimi_delta_attention_kda_amd import build
        build.build()
    return kda.lib()


def _declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kda_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_function_is_exported(L):
    names = _declared_functions()
    assert {"kda_chunk_fwd", "kda_segment_summary", "kda_affine_exclusive_scan",
            "kda_validate_varlen", "kda_status_string"} <= set(names)
    nm = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (kda_\w+)$", nm, flags=re.M))
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)


def test_calibration_library_exports_its_header(L):
    """libkda_calib.so (the MFMA counter calibration kernel) exports what kda_calib.h
    declares and refuses bad arguments before any launch."""
    names = _declared_functions(os.path.join(ROOT, "include", "kda_calib.h"))
    assert names == ["kda_calib_mfma"]
    nm = subprocess.run(["nm", "-D", "--defined-only", kda.CALIB_LIB_PATH], capture_output=True, text=True).stdout
    assert set(names) <= set(re.findall(r" T (kda_\w+)$", nm, flags=re.M))
    C_ = kda.calib_lib()
    assert C_.kda_calib_mfma(0, 1, FAKE, None) == 1
    assert C_.kda_calib_mfma(1, 0, FAKE, None) == 1
    assert C_.kda_calib_mfma(1, 1, None, None) == 1


def test_status_strings(L):
    for code in range(9):
        s = kda.status_string(code)
        assert isinstance(s, str) and s
    assert kda.status_string(0) == "ok"
    assert kda.status_string(99) == "unknown status"
    # the contract the header states for KDA_ERR_UNSUPPORTED: out dtype equal to q/k/v,
    # bf16 or f32, dk == dv in {64, 128}, either gate mode
    unsup = kda.status_string(4)
    for part in ("out dtype equal to the q/k/v dtype", "bf16 or f32", "dk == dv in {64, 128}",
                 "either gate mode"):
        assert part in unsup, (part, unsup)
    hdr = open(os.path.join(ROOT, "include", "libkda.h")).read()
    assert "qkv_dtype == out_dtype, bf16 or f32; dk == dv in {64, 128}; either gate mode" in hdr


def _desc(**kw):
    base = dict(T=128, B=2, H=4, dk=128, dv=128, max_slots=4, qkv_dtype=torch.bfloat16,
                out_dtype=torch.bfloat16, gate_mode="safe", lower_bound=-5.0)
    base.update(kw)
    return kda.make_desc(base["T"], base["B"], base["H"], base["dk"], base["dv"], base["max_slots"],
                         base["qkv_dtype"], base["out_dtype"], base["gate_mode"], base["lower_bound"])


def _fwd(L, d, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, raw=FAKE, beta=FAKE, a_log=FAKE, dtb=FAKE, cu=FAKE, pool=FAKE,
             idx=FAKE, out=FAKE)
    p.update(ptrs)
    return L.kda_chunk_fwd(C.byref(d) if d is not None else None, p["q"], p["k"], p["v"], p["raw"],
                           p["beta"], p["a_log"], p["dtb"], p["cu"], p["pool"], p["idx"], p["out"], None)


def test_chunk_fwd_error_paths(L):
    assert _fwd(L, None) == ENULL
    assert _fwd(L, _desc(), q=None) == ENULL
    assert _fwd(L, _desc(), pool=None) == ENULL
    assert _fwd(L, _desc(), cu=None) == ENULL
    assert _fwd(L, _desc(T=-1)) == ESHAPE
    assert _fwd(L, _desc(H=0)) == ESHAPE
    assert _fwd(L, _desc(max_slots=0)) == ESHAPE
    assert _fwd(L, _desc(qkv_dtype=torch.float16)) == EDTYPE
    assert _fwd(L, _desc(lower_bound=0.5)) == EARG
    assert _fwd(L, _desc(dk=128, dv=64)) == EUNSUP
    assert _fwd(L, _desc(dk=96, dv=96)) == EUNSUP
    assert _fwd(L, _desc(dk=32, dv=32, qkv_dtype=torch.float32, out_dtype=torch.float32)) == EUNSUP
    assert _fwd(L, _desc(out_dtype=torch.float32)) == EUNSUP
    # either gate, any bound <= 0, bf16 or f32 at dk = dv in {64, 128} are in the contract
    # (launching them needs a GPU, so they are exercised by the GPU tests)
    d = _desc(dk=96, dv=96)
    d.state_layout = 1                                              # V_FIRST is in the contract;
    assert _fwd(L, d) == EUNSUP                                     # dk 96 is not
    d = _desc()
    d.state_layout = 2
    assert _fwd(L, d) == EARG
    d = _desc()
    d.gate_mode = 7
    assert _fwd(L, d) == EARG
    d = _desc()
    d.beta_mode = 3
    assert _fwd(L, d) == EARG
    # nothing to do: no sequences / no tokens (returns before any launch)
    assert _fwd(L, _desc(B=0)) == OK
    assert _fwd(L, _desc(T=0)) == OK


def _fwd_ws(L, d, ws=FAKE, nbytes=1 << 40, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, raw=FAKE, beta=FAKE, a_log=FAKE, dtb=FAKE, cu=FAKE, pool=FAKE,
             idx=FAKE, out=FAKE)
    p.update(ptrs)
    return L.kda_chunk_fwd_ws(C.byref(d) if d is not None else None, p["q"], p["k"], p["v"], p["raw"],
                              p["beta"], p["a_log"], p["dtb"], p["cu"], p["pool"], p["idx"], p["out"],
                              ws, nbytes, None)


def test_workspace_variant_error_paths(L):
    # the same validation as kda_chunk_fwd, before the workspace is looked at
    assert _fwd_ws(L, None) == ENULL
    assert _fwd_ws(L, _desc(), out=None) == ENULL
    assert _fwd_ws(L, _desc(T=-1)) == ESHAPE
    assert _fwd_ws(L, _desc(dk=96, dv=96)) == EUNSUP
    assert _fwd_ws(L, _desc(B=0)) == OK
    n = C.c_size_t(7)
    assert L.kda_chunk_fwd_workspace_size(None, C.byref(n)) == ENULL
    assert L.kda_chunk_fwd_workspace_size(C.byref(_desc()), None) == ENULL
    # f32 never uses the load-balanced pass: no workspace, no device query
    assert L.kda_chunk_fwd_workspace_size(C.byref(_desc(qkv_dtype=torch.float32, out_dtype=torch.float32,
                                                         dk=64, dv=64)), C.byref(n)) == OK
    assert n.value == 0
    # bf16 with either gate (the fast kernels, or the precise walk for the original gate)
    # sizes for the current device (HIP error without one)
    for gate in ("safe", "original"):
        for dk in (128, 64):
            st = L.kda_chunk_fwd_workspace_size(C.byref(_desc(dk=dk, dv=dk, gate_mode=gate)), C.byref(n))
            assert st in (OK, 6)
            if st == OK:
                assert n.value >= 128 * 4 * dk * 2


def _fwd_noalloc(L, d, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, raw=FAKE, beta=FAKE, a_log=FAKE, dtb=FAKE, cu=FAKE, pool=FAKE,
             idx=FAKE, out=FAKE)
    p.update(ptrs)
    return L.kda_chunk_fwd_noalloc(C.byref(d) if d is not None else None, p["q"], p["k"], p["v"], p["raw"],
                                   p["beta"], p["a_log"], p["dtb"], p["cu"], p["pool"], p["idx"], p["out"],
                                   None)


def test_noalloc_variant_error_paths(L):
    """The entry point without allocation validates exactly like kda_chunk_fwd, before it
    looks at its scratch; its own status names the scratch limit."""
    assert _fwd_noalloc(L, None) == ENULL
    assert _fwd_noalloc(L, _desc(), out=None) == ENULL
    assert _fwd_noalloc(L, _desc(T=-1)) == ESHAPE
    assert _fwd_noalloc(L, _desc(dk=96, dv=96)) == EUNSUP
    assert _fwd_noalloc(L, _desc(qkv_dtype=torch.float16)) == EDTYPE
    assert _fwd_noalloc(L, _desc(lower_bound=0.5)) == EARG
    assert _fwd_noalloc(L, _desc(B=0)) == OK
    assert _fwd_noalloc(L, _desc(T=0)) == OK
    assert "256 MiB" in kda.status_string(8) and "kda_chunk_fwd_noalloc" in kda.status_string(8)


def _dec(L, d, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, raw=FAKE, beta=FAKE, a_log=FAKE, dtb=FAKE, pool=FAKE, idx=FAKE, out=FAKE)
    p.update(ptrs)
    return L.kda_decode(C.byref(d) if d is not None else None, p["q"], p["k"], p["v"], p["raw"], p["beta"],
                        p["a_log"], p["dtb"], p["pool"], p["idx"], p["out"], None)


def test_decode_error_paths(L):
    assert _dec(L, None) == ENULL
    assert _dec(L, _desc(T=8, B=4)) == ESHAPE                     # one token per sequence
    assert _dec(L, _desc(T=4, B=4), q=None) == ENULL
    assert _dec(L, _desc(T=4, B=4), pool=None) == ENULL
    assert _dec(L, _desc(T=4, B=4, dk=96, dv=96)) == EUNSUP
    assert _dec(L, _desc(T=4, B=4, dk=128, dv=64)) == EUNSUP
    assert _dec(L, _desc(T=4, B=4, qkv_dtype=torch.float16)) == EDTYPE
    assert _dec(L, _desc(T=4, B=4, lower_bound=0.5)) == EARG
    assert _dec(L, _desc(T=0, B=0)) == OK                         # nothing to do, nothing launched


def test_summary_and_scan_error_paths(L):
    d = _desc()
    args = [FAKE] * 7
    assert L.kda_segment_summary(C.byref(d), *args, 0, FAKE, FAKE, None) == ESHAPE    # n_seg >= 1
    assert L.kda_segment_summary(C.byref(d), *args, 2, None, FAKE, None) == ENULL
    d32 = _desc(qkv_dtype=torch.float32, dk=96, dv=96)
    assert L.kda_segment_summary(C.byref(d32), *args, 2, FAKE, FAKE, None) == EUNSUP
    sargs = [FAKE] * 6
    assert L.kda_affine_exclusive_scan(0, 2, 16, 16, *sargs, None) == ESHAPE           # n_seg >= 1
    assert L.kda_affine_exclusive_scan(2, 2, 48, 16, *sargs, None) == EUNSUP
    assert L.kda_affine_exclusive_scan(2, 2, 16, 8, *sargs, None) == EUNSUP
    assert L.kda_affine_exclusive_scan(2, 2, 16, 16, None, *sargs[1:], None) == ENULL
    blk = L.kda_affine_exclusive_scan_blocked
    assert blk(0, 2, 64, 64, 0, *sargs, None) == ESHAPE                                 # n_seg >= 1
    assert blk(4, 2, 64, 64, -1, *sargs, None) == ESHAPE                                # block >= 0
    assert blk(4, 2, 48, 64, 0, *sargs, None) == EUNSUP
    assert blk(4, 2, 64, 8, 0, *sargs, None) == EUNSUP
    assert blk(4, 2, 64, 64, 0, *sargs[:5], None, None) == ENULL


def test_scan_block_size_rule(L):
    """Automatic: the ordered scan below 32 segments, else blocks of about sqrt(n_seg / 2)
    segments (critical path ~ 2 block + n_seg / block map steps).  Any block is raised to
    at least 1 + ceil(dk / dv) so that the block composites fit in the outgoing stack, and
    is n_seg (the ordered scan) when one block holds everything or dk is 16 or 32."""
    bs = L.kda_affine_scan_block_size
    assert [bs(n, 128, 128, 0) for n in (1, 2, 3, 16, 31, 32, 64, 200)] == [1, 2, 3, 16, 31, 4, 6, 10]
    assert bs(16, 128, 128, 5) == 5 and bs(16, 128, 128, 1) == 2   # raised to 1 + dk/dv
    assert bs(16, 128, 64, 1) == 3 and bs(16, 64, 128, 1) == 2
    assert bs(16, 128, 128, 16) == 16 and bs(16, 128, 128, 40) == 16
    assert bs(16, 32, 32, 4) == 16                                  # ordered walk at dk 32
    assert bs(0, 128, 128, 0) == -1 and bs(4, 128, 128, -2) == -1
    # the composites of all blocks but the last fit in the outgoing stack
    for n in range(1, 80):
        for dk, dv in ((128, 128), (128, 64), (64, 128), (64, 64)):
            b = bs(n, dk, dv, 0)
            nb = -(-n // b)
            assert (nb - 1) * dk * (dk + dv) <= n * dk * dv
    assert L.kda_validate_varlen(FAKE, -1, 0, FAKE, 4) == ESHAPE
    assert L.kda_validate_varlen(None, 2, 0, FAKE, 4) == ENULL


def test_python_binding_checks_before_the_library():
    T, H, dk = 8, 2, 64
    q = torch.zeros(T, H, dk, dtype=torch.bfloat16)
    raw = torch.zeros(T, H, dk)
    with pytest.raises(ValueError):   # k has the wrong extent
        kda.chunk_fwd(q, torch.zeros(T, H, 32, dtype=torch.bfloat16), q, raw, torch.zeros(T, H),
                      torch.zeros(H), torch.zeros(H, dk), torch.tensor([0, T], dtype=torch.int32),
                      torch.zeros(1, H, dk, dk), torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError):   # wrong dtype of the gate
        kda.chunk_fwd(q, q, q, raw.double(), torch.zeros(T, H), torch.zeros(H), torch.zeros(H, dk),
                      torch.tensor([0, T], dtype=torch.int32), torch.zeros(1, H, dk, dk),
                      torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError):   # at least one segment
        kda.context_parallel(torch.zeros(0, 16, 16), torch.zeros(0, 16, 16), torch.zeros(16, 16))
    q3 = torch.zeros(T, 3, dk, dtype=torch.bfloat16)
    v4 = torch.zeros(T, 4, dk, dtype=torch.bfloat16)
    with pytest.raises(ValueError):   # 3 key heads do not divide 4 value heads
        kda.chunk_fwd(q3, q3, v4, torch.zeros(T, 4, dk), torch.zeros(T, 4), torch.zeros(4),
                      torch.zeros(4, dk), torch.tensor([0, T], dtype=torch.int32),
                      torch.zeros(1, 4, dk, dk), torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError):
        kda.decode(q3, q3, v4, torch.zeros(T, 4, dk), torch.zeros(T, 4), torch.zeros(4),
                   torch.zeros(4, dk), torch.zeros(T, 4, dk, dk), torch.zeros(T, dtype=torch.int32))
    with pytest.raises(ValueError):
        kda.segment_summary(q3, v4, torch.zeros(T, 4, dk), torch.zeros(T, 4), torch.zeros(4),
                            torch.zeros(4, dk), torch.tensor([0, T], dtype=torch.int32))


def test_python_binding_checks_output_buffers():
    """Caller-provided outputs must have the exact shape, dtype and contiguity the C ABI
    writes (it cannot see extents), and every tensor must be on a GPU; each is refused with
    ValueError before the library is called (these tensors live on the CPU)."""
    T, H, dk, B = 8, 2, 64, 1
    bf = dict(dtype=torch.bfloat16)
    q = torch.zeros(T, H, dk, **bf)
    args = (q, q, q, torch.zeros(T, H, dk), torch.zeros(T, H), torch.zeros(H), torch.zeros(H, dk),
            torch.tensor([0, T], dtype=torch.int32), torch.zeros(1, H, dk, dk), torch.zeros(B, dtype=torch.int32))
    for bad, what in ((torch.zeros(T - 1, H, dk, **bf), "shape"), (torch.zeros(T, H, dk + 1, **bf), "shape"),
                      (torch.zeros(T, H, dk), "dtype"), (torch.zeros(T, dk, H, **bf).transpose(1, 2), "contiguous")):
        with pytest.raises(ValueError, match="out"):
            kda.chunk_fwd(*args, out=bad)
    with pytest.raises(ValueError, match="GPU"):   # well-formed, but on the CPU
        kda.chunk_fwd(*args, out=torch.zeros(T, H, dk, **bf))
    dargs = (q[:B], q[:B], q[:B], torch.zeros(B, H, dk), torch.zeros(B, H), torch.zeros(H), torch.zeros(H, dk),
             torch.zeros(1, H, dk, dk), torch.zeros(B, dtype=torch.int32))
    with pytest.raises(ValueError, match="out"):
        kda.decode(*dargs, out=torch.zeros(B + 1, H, dk, **bf))
    sargs = (q, q, torch.zeros(T, H, dk), torch.zeros(T, H), torch.zeros(H), torch.zeros(H, dk),
             torch.tensor([0, 4, T], dtype=torch.int32))
    with pytest.raises(ValueError, match="M"):
        kda.segment_summary(*sargs, M=torch.zeros(1, H, dk, dk))
    with pytest.raises(ValueError, match="U"):
        kda.segment_summary(*sargs, U=torch.zeros(2, H, dk, dk, dtype=torch.float64))
    M, U, S0 = torch.zeros(3, H, dk, dk), torch.zeros(3, H, dk, dk), torch.zeros(H, dk, dk)
    with pytest.raises(ValueError, match="incoming"):
        kda.affine_exclusive_scan(M, U, S0, incoming=torch.zeros(2, H, dk, dk))
    with pytest.raises(ValueError, match="outgoing"):
        kda.affine_exclusive_scan(M, U, S0, outgoing=torch.zeros(3, H, dk, dk).transpose(2, 3))
    with pytest.raises(ValueError, match="final_state"):
        kda.affine_exclusive_scan(M, U, S0, final_state=torch.zeros(H, dk, dk - 1))
    with pytest.raises(ValueError, match="GPU"):
        kda.affine_exclusive_scan(M, U, S0)
    with pytest.raises(ValueError, match="state_indices"):
        kda.validate_varlen(torch.tensor([0, T], dtype=torch.int32), torch.zeros(2, dtype=torch.int32), T, 4)


def test_key_heads_must_divide_value_heads(L):
    for hk in (3, -1, 5):
        d = _desc()
        d.num_key_heads = hk
        assert _fwd(L, d) == ESHAPE
        assert _fwd_ws(L, d) == ESHAPE
        assert L.kda_segment_summary(C.byref(d), *([FAKE] * 7), 2, FAKE, FAKE, None) == ESHAPE
    d = _desc(T=4, B=4)
    d.num_key_heads = 3
    assert _dec(L, d) == ESHAPE
    # 0 means as many key heads as value heads; 1, 2 and 4 divide H = 4 (nothing to launch: B = 0)
    for hk in (0, 1, 2, 4):
        d = _desc(B=0)
        d.num_key_heads = hk
        assert _fwd(L, d) == OK


def test_descriptor_layout_matches_the_header(tmp_path):
    """The binding's ctypes descriptor has the size and field offsets the C compiler gives
    kda_desc in include/libkda.h."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    names = [f[0] for f in kda.KdaDesc._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"libkda.h\"\nint main(void) {\n"
                   + '  printf("%zu\\n", sizeof(kda_desc));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(kda_desc, {n}));\n' for n in names)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(root, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == C.sizeof(kda.KdaDesc)
    assert got[1:] == [getattr(kda.KdaDesc, n).offset for n in names]


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(kda, "_lib", None)
    monkeypatch.setattr(kda, "LIB_PATH", "/nonexistent/libkda.so")
    with pytest.raises(RuntimeError):
        kda.lib()
