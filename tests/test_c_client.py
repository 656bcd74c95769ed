"""The C ABI from a plain C program: tests/c_client/kda_client.c includes only
include/libkda.h and the HIP runtime API, is compiled by gcc and links libkda.so.

CPU: the host-checkable error paths.  GPU: a ragged bf16 prefill through the C program
gives the same bits as the Python binding.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import kimi_delta_attention_kda_amd as kda
from kimi_delta_attention_kda_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "kimi_delta_attention_kda_amd")


def _client(tmp_path):
    if shutil.which("gcc") is None or not os.path.exists(os.path.join(LIBDIR, "libkda.so")):
        pytest.skip("needs gcc and the built library")
    exe = str(tmp_path / "kda_client")
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", os.path.join(ROOT, "tests", "c_client", "kda_client.c"),
           "-L", LIBDIR, "-lkda", "-L", "/opt/rocm/lib", "-lamdhip64",
           f"-Wl,-rpath,{LIBDIR}", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def test_c_client_error_paths(tmp_path):
    exe = _client(tmp_path)
    r = subprocess.run([exe, "errors"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "errors ok"


@pytest.mark.gpu
def test_c_client_prefill_matches_binding(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = _client(tmp_path)
    w = wl.custom([300, 1, 0, 129], H=2, dk=128, dv=128, dtype="bf16", gate_mode=1, seed=41, name="cclient")
    print("[case] C client prefill bf16 dk=128", flush=True)
    inp = wl.make_inputs(w, "cuda")
    for name, key in (("q", "q"), ("k", "k"), ("v", "v"), ("raw", "raw_gate"), ("beta", "beta_logits"),
                      ("alog", "a_log"), ("dtb", "dt_bias"), ("cu", "cu_seqlens"), ("pool", "state_pool"),
                      ("idx", "state_indices")):
        t = inp[key].contiguous().cpu()
        (tmp_path / f"{name}.bin").write_bytes(t.view(torch.uint8).numpy().tobytes() if t.numel() else b"")
    args = [exe, "fwd", str(tmp_path), str(w.T), str(w.B), str(w.H), str(w.dk), str(w.dv),
            str(inp["state_pool"].shape[0]), "1", "1", repr(float(w.lower_bound)), repr(float(w.scale))]
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out_c = np.frombuffer((tmp_path / "out.bin").read_bytes(), dtype=np.uint16)
    pool_c = np.frombuffer((tmp_path / "pool_out.bin").read_bytes(), dtype=np.uint32)
    pool = inp["state_pool"].clone()
    out = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["raw_gate"], inp["beta_logits"], inp["a_log"],
                        inp["dt_bias"], inp["cu_seqlens"], pool, inp["state_indices"], gate_mode="safe",
                        lower_bound=w.lower_bound, scale=w.scale, workspace="library")
    torch.cuda.synchronize()
    assert np.array_equal(out_c, out.cpu().view(torch.int16).numpy().view(np.uint16).ravel())
    assert np.array_equal(pool_c, pool.cpu().view(torch.int32).numpy().view(np.uint32).ravel())
