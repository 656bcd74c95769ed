"""Kimi Delta Attention (KDA) prefill on MI355X (gfx950): Python binding of libkda.

Argument marshalling only: every step of the computation runs in the HIP kernels of
libkda.so (built in-tree by kimi_delta_attention_kda_amd/build.py).  PyTorch supplies
device memory and the current stream.  If the library is missing, importing works but
every call raises RuntimeError; there is no CPU fallback.

Entry points (names as in the C ABI, include/libkda.h):
  chunk_fwd(...)          varlen chunk-parallel prefill, mutates the state pool in place
  segment_summary(...)    per-segment affine maps (M_i, U_i)
  affine_exclusive_scan(M, U, S_init[, block]) -> (incoming, outgoing, final), ordered or blocked
  context_parallel(transition_matrices, local_contributions, initial_state) -> dict
  validate_varlen(...)    synchronous debug check of cu_seqlens / state_indices
"""
from __future__ import annotations

import ctypes as C
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

F32, BF16 = 0, 1
_DT = {torch.float32: F32, torch.bfloat16: BF16}
_GATE = {"original": 0, "safe": 1}
_BETA = {"logits": 0, "probability": 1}
_LAYOUT = {"K_FIRST": 0, "V_FIRST": 1}


class KdaDesc(C.Structure):
    _fields_ = [("total_tokens", C.c_int64), ("batch", C.c_int32), ("num_heads", C.c_int32),
                ("dk", C.c_int32), ("dv", C.c_int32), ("max_slots", C.c_int32),
                ("qkv_dtype", C.c_int32), ("out_dtype", C.c_int32), ("gate_mode", C.c_int32),
                ("gate_lower_bound", C.c_float), ("beta_mode", C.c_int32),
                ("state_layout", C.c_int32), ("scale", C.c_float), ("num_key_heads", C.c_int32)]


_lib = None


def lib():
    """Loads libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libkda.so not built ({LIB_PATH}); run kimi_delta_attention_kda_amd/build.py")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        dp = C.POINTER(KdaDesc)
        L.kda_chunk_fwd.argtypes = [dp] + [vp] * 12
        L.kda_chunk_fwd_ws.argtypes = [dp] + [vp] * 12 + [C.c_size_t, vp]
        L.kda_chunk_fwd_noalloc.argtypes = [dp] + [vp] * 12
        L.kda_chunk_fwd_workspace_size.argtypes = [dp, C.POINTER(C.c_size_t)]
        L.kda_decode.argtypes = [dp] + [vp] * 11
        L.kda_segment_summary.argtypes = [dp] + [vp] * 7 + [i32, vp, vp, vp]
        L.kda_affine_exclusive_scan.argtypes = [i32, i32, i32, i32] + [vp] * 7
        L.kda_affine_exclusive_scan_blocked.argtypes = [i32, i32, i32, i32, i32] + [vp] * 7
        L.kda_affine_scan_block_size.argtypes = [i32, i32, i32, i32]
        L.kda_affine_scan_block_size.restype = i32
        L.kda_validate_varlen.argtypes = [vp, i32, i64, vp, i32]
        L.kda_status_string.argtypes = [C.c_int]
        L.kda_status_string.restype = C.c_char_p
        for f in ("kda_chunk_fwd", "kda_chunk_fwd_ws", "kda_chunk_fwd_noalloc", "kda_chunk_fwd_workspace_size", "kda_decode",
                  "kda_segment_summary", "kda_affine_exclusive_scan", "kda_affine_exclusive_scan_blocked",
                  "kda_validate_varlen"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


CALIB_LIB_PATH = os.path.join(_HERE, "libkda_calib.so")
_calib = None


def calib_lib():
    """Loads libkda_calib.so (include/kda_calib.h): a kernel of known MFMA count that scales
    the profiler's MFMA-busy counter.  Measurement only, no part of the KDA computation."""
    global _calib
    if _calib is None:
        if not os.path.exists(CALIB_LIB_PATH):
            raise RuntimeError(f"libkda_calib.so not built ({CALIB_LIB_PATH}); run kimi_delta_attention_kda_amd/build.py")
        L = C.CDLL(CALIB_LIB_PATH)
        L.kda_calib_mfma.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_void_p]
        L.kda_calib_mfma.restype = C.c_int
        _calib = L
    return _calib


def calib_mfma(n_workgroups: int, iters: int, out: torch.Tensor) -> None:
    """Launches the calibration kernel on the current stream: n_workgroups * 4 * iters
    v_mfma_f32_16x16x32_bf16 instructions; out: fp32, n_workgroups * 256 elements."""
    if out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous() \
            or out.numel() < n_workgroups * 256:
        raise ValueError("out must be a contiguous fp32 device tensor of n_workgroups * 256 elements")
    code = calib_lib().kda_calib_mfma(n_workgroups, iters, _ptr(out), _stream())
    if code != 0:
        raise RuntimeError(f"kda_calib_mfma failed ({code})")


def status_string(code: int) -> str:
    return lib().kda_status_string(code).decode()


def _check(code: int):
    if code != 0:
        raise ValueError(f"libkda: {status_string(code)} (status {code})")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _need(t, name, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")


def _need_out(t, name, shape, dtype, device):
    """A caller-provided output buffer: exact shape, dtype, device, contiguous (the C ABI
    cannot see extents, so a short or strided buffer would be written out of bounds)."""
    _need(t, name, dtype, device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _on_gpu(device):
    if device.type != "cuda":
        raise ValueError(f"libkda runs on a GPU; the tensors are on {device}")


def make_desc(T, B, H, dk, dv, max_slots, qkv_dtype, out_dtype, gate_mode="safe", lower_bound=-5.0,
              beta_mode="logits", state_layout="K_FIRST", scale=None, Hk=None) -> KdaDesc:
    """Hk: key heads of q and k (None: as many as the value heads H)."""
    if gate_mode not in _GATE or beta_mode not in _BETA or state_layout not in _LAYOUT:
        raise ValueError("unknown gate_mode / beta_mode / state_layout")
    return KdaDesc(int(T), int(B), int(H), int(dk), int(dv), int(max_slots),
                   _DT.get(qkv_dtype, -1), _DT.get(out_dtype, -1), _GATE[gate_mode],
                   float(lower_bound), _BETA[beta_mode], _LAYOUT[state_layout],
                   float(1.0 / math.sqrt(dk) if scale is None else scale), int(H if Hk is None else Hk))


def _heads(q_or_k, v):
    """(H, Hk): value heads from v, key heads from q/k; Hk must divide H."""
    H, Hk = v.shape[1], q_or_k.shape[1]
    if Hk <= 0 or H % Hk != 0:
        raise ValueError("the key heads of q and k must divide the value heads of v")
    return H, Hk


def chunk_fwd(q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, state_pool, state_indices,
              *, output_dtype=None, gate_mode="safe", lower_bound=-5.0, beta_mode="logits",
              state_layout="K_FIRST", scale=None, out=None, workspace="torch"):
    """Chunk-parallel varlen KDA prefill; mutates state_pool[state_indices] in place.

    Shapes follow max.nn.state_space.kda_chunk: q,k [T,Hk,dk]; v [T,H,dv]; raw_gate
    [T,H,dk] f32; beta_logits [T,H] f32; a_log [H] f32; dt_bias [H,dk] f32; cu_seqlens
    [B+1] int32; state_pool [slots,H,dk,dv] f32; state_indices [B] int32.  Returns out
    [T,H,dv] in output_dtype (default: q's dtype).  Hk (key heads) divides H (value
    heads); value head h reads key head h // (H // Hk).

    workspace: "torch" (load-balanced pass, workspace from torch's allocator on the
    current stream; the unbalanced launch if that allocation fails), "library" (kda_chunk_fwd: the library's own stream-ordered pool),
    "static" (kda_chunk_fwd_noalloc: the library's fixed device scratch, no allocation
    at all; calls on one device must not overlap) or "none" (no load balancing).
    """
    if workspace not in ("torch", "library", "static", "none"):
        raise ValueError("workspace must be 'torch', 'library', 'static' or 'none'")
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("ranks and extents of the inputs disagree")
    T, _, dk = q.shape
    H, Hk = _heads(q, v)
    dv = v.shape[-1]
    dev = q.device
    B = cu_seqlens.numel() - 1
    for t_, n_ in ((q, "q"), (k, "k"), (v, "v")):
        _need(t_, n_, q.dtype, dev)
    for t_, n_ in ((raw_gate, "raw_gate"), (beta_logits, "beta_logits"), (a_log, "a_log"),
                   (dt_bias, "dt_bias"), (state_pool, "state_pool")):
        _need(t_, n_, torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    _need(state_indices, "state_indices", torch.int32, dev)
    slot_shape = (H, dk, dv) if state_layout == "K_FIRST" else (H, dv, dk)
    if k.shape != (T, Hk, dk) or v.shape[:2] != (T, H) or raw_gate.shape != (T, H, dk) \
            or beta_logits.shape != (T, H) or a_log.shape != (H,) or dt_bias.shape != (H, dk) \
            or state_pool.dim() != 4 or state_pool.shape[1:] != slot_shape \
            or state_indices.shape != (B,):
        raise ValueError("ranks and extents of the inputs disagree")
    odt = output_dtype or q.dtype
    if out is None:
        _on_gpu(dev)
        out = torch.empty((T, H, dv), dtype=odt, device=dev)
    else:
        _need_out(out, "out", (T, H, dv), odt, dev)
    _on_gpu(dev)
    d = make_desc(T, B, H, dk, dv, state_pool.shape[0], q.dtype, odt, gate_mode, lower_bound,
                  beta_mode, state_layout, scale, Hk)
    args = (C.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(raw_gate), _ptr(beta_logits), _ptr(a_log),
            _ptr(dt_bias), _ptr(cu_seqlens), _ptr(state_pool), _ptr(state_indices), _ptr(out))
    if workspace == "library":
        _check(lib().kda_chunk_fwd(*args, _stream()))
        return out
    if workspace == "static":
        _check(lib().kda_chunk_fwd_noalloc(*args, _stream()))
        return out
    ws, nbytes = None, 0
    if workspace == "torch":
        need = C.c_size_t(0)
        _check(lib().kda_chunk_fwd_workspace_size(C.byref(d), C.byref(need)))
        if need.value > 0:
            try:
                ws = torch.empty(need.value, dtype=torch.uint8, device=dev)
                nbytes = need.value
            except torch.OutOfMemoryError:
                # as kda_chunk_fwd does when its pool cannot serve the workspace: the
                # unbalanced launch, which needs none
                ws, nbytes = None, 0
    _check(lib().kda_chunk_fwd_ws(*args, _ptr(ws), nbytes, _stream()))
    return out


def decode(q, k, v, raw_gate, beta_logits, a_log, dt_bias, state_pool, state_indices, *,
           output_dtype=None, gate_mode="safe", lower_bound=-5.0, beta_mode="logits",
           state_layout="K_FIRST", scale=None, out=None):
    """One recurrent step per sequence on its pool slot (single-token decode).

    q, k [B,Hk,dk]; v [B,H,dv]; raw_gate [B,H,dk] f32; beta_logits [B,H] f32; a_log [H];
    dt_bias [H,dk]; state_pool [slots,H,dk,dv] (V_FIRST: [slots,H,dv,dk]) f32, mutated at
    state_indices [B] int32.  Returns out [B,H,dv] in output_dtype (default: q's dtype).
    """
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("ranks and extents of the inputs disagree")
    B, _, dk = q.shape
    H, Hk = _heads(q, v)
    dv = v.shape[-1]
    dev = q.device
    for t_, n_ in ((q, "q"), (k, "k"), (v, "v")):
        _need(t_, n_, q.dtype, dev)
    for t_, n_ in ((raw_gate, "raw_gate"), (beta_logits, "beta_logits"), (a_log, "a_log"),
                   (dt_bias, "dt_bias"), (state_pool, "state_pool")):
        _need(t_, n_, torch.float32, dev)
    _need(state_indices, "state_indices", torch.int32, dev)
    slot_shape = (H, dk, dv) if state_layout == "K_FIRST" else (H, dv, dk)
    if k.shape != (B, Hk, dk) or v.shape[:2] != (B, H) or raw_gate.shape != (B, H, dk) \
            or beta_logits.shape != (B, H) or a_log.shape != (H,) or dt_bias.shape != (H, dk) \
            or state_pool.dim() != 4 or state_pool.shape[1:] != slot_shape or state_indices.shape != (B,):
        raise ValueError("ranks and extents of the inputs disagree")
    odt = output_dtype or q.dtype
    if out is None:
        _on_gpu(dev)
        out = torch.empty((B, H, dv), dtype=odt, device=dev)
    else:
        _need_out(out, "out", (B, H, dv), odt, dev)
    _on_gpu(dev)
    d = make_desc(B, B, H, dk, dv, state_pool.shape[0], q.dtype, odt, gate_mode, lower_bound,
                  beta_mode, state_layout, scale, Hk)
    _check(lib().kda_decode(C.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(raw_gate), _ptr(beta_logits),
                            _ptr(a_log), _ptr(dt_bias), _ptr(state_pool), _ptr(state_indices), _ptr(out),
                            _stream()))
    return out


def segment_summary(k, v, raw_gate, beta_logits, a_log, dt_bias, seg_offsets, *, gate_mode="safe",
                    lower_bound=-5.0, beta_mode="logits", M=None, U=None):
    """Affine map F_i(S) = M_i S + U_i of every segment [seg_offsets[i], seg_offsets[i+1]).

    k [T,Hk,dk] and v [T,H,dv] (bf16 or f32); raw_gate [T,H,dk], beta_logits [T,H], a_log [H],
    dt_bias [H,dk] f32.  Returns M [n_seg,H,dk,dk] f32 and U [n_seg,H,dk,dv] f32."""
    if k.dim() != 3 or v.dim() != 3:
        raise ValueError("ranks and extents of the inputs disagree")
    T, _, dk = k.shape
    H, Hk = _heads(k, v)
    dv = v.shape[-1]
    dev = k.device
    n_seg = seg_offsets.numel() - 1
    _need(k, "k", None, dev)
    _need(v, "v", k.dtype, dev)
    for t_, n_ in ((raw_gate, "raw_gate"), (beta_logits, "beta_logits"), (a_log, "a_log"),
                   (dt_bias, "dt_bias")):
        _need(t_, n_, torch.float32, dev)
    _need(seg_offsets, "seg_offsets", torch.int32, dev)
    if v.shape[0] != T or raw_gate.shape != (T, H, dk) or beta_logits.shape != (T, H) \
            or a_log.shape != (H,) or dt_bias.shape != (H, dk):
        raise ValueError("ranks and extents of the inputs disagree")
    n_alloc = max(n_seg, 0)
    if M is None:
        M = torch.empty((n_alloc, H, dk, dk), dtype=torch.float32, device=dev)
    else:
        _need_out(M, "M", (n_alloc, H, dk, dk), torch.float32, dev)
    if U is None:
        U = torch.empty((n_alloc, H, dk, dv), dtype=torch.float32, device=dev)
    else:
        _need_out(U, "U", (n_alloc, H, dk, dv), torch.float32, dev)
    _on_gpu(dev)
    d = make_desc(T, 1, H, dk, dv, 1, k.dtype, k.dtype, gate_mode, lower_bound, beta_mode, Hk=Hk)
    _check(lib().kda_segment_summary(C.byref(d), _ptr(k), _ptr(v), _ptr(raw_gate), _ptr(beta_logits),
                                     _ptr(a_log), _ptr(dt_bias), _ptr(seg_offsets), int(n_seg),
                                     _ptr(M), _ptr(U), _stream()))
    return M, U


def affine_scan_block_size(n_seg, dk, dv, block=0):
    """Segments per block that the blocked scan uses for these arguments (n_seg: the
    ordered scan).  Host only."""
    b = lib().kda_affine_scan_block_size(int(n_seg), int(dk), int(dv), int(block))
    if b < 0:
        raise ValueError("invalid scan arguments")
    return b


def affine_exclusive_scan(M, U, S_init, incoming=None, outgoing=None, final_state=None, block=None):
    """M [n,H,dk,dk], U [n,H,dk,dv], S_init [H,dk,dv] (f32, device) -> (incoming, outgoing, final).

    block None: the ordered scan (kda_affine_exclusive_scan).  block >= 0: the same
    prefix regrouped into blocks of that many segments (0: automatic), three launches
    (kda_affine_exclusive_scan_blocked)."""
    if M.dim() != 4 or U.dim() != 4 or S_init.dim() != 3:
        raise ValueError("expected M [n,H,dk,dk], U [n,H,dk,dv], S_init [H,dk,dv]")
    n, H, dk, _ = M.shape
    dv = U.shape[-1]
    dev = M.device
    for t_, n_ in ((M, "M"), (U, "U"), (S_init, "S_init")):
        _need(t_, n_, torch.float32, dev)
    if M.shape != (n, H, dk, dk) or U.shape != (n, H, dk, dv) or S_init.shape != (H, dk, dv):
        raise ValueError("ranks and extents of the inputs disagree")
    for t_, n_, shp in ((incoming, "incoming", U.shape), (outgoing, "outgoing", U.shape),
                        (final_state, "final_state", S_init.shape)):
        if t_ is not None:
            _need_out(t_, n_, shp, torch.float32, dev)
    _on_gpu(dev)
    incoming = torch.empty_like(U) if incoming is None else incoming
    outgoing = torch.empty_like(U) if outgoing is None else outgoing
    final_state = torch.empty_like(S_init) if final_state is None else final_state
    if block is None:
        _check(lib().kda_affine_exclusive_scan(int(n), int(H), int(dk), int(dv), _ptr(M), _ptr(U),
                                               _ptr(S_init), _ptr(incoming), _ptr(outgoing),
                                               _ptr(final_state), _stream()))
    else:
        if int(block) < 0:
            raise ValueError("block must be >= 0")
        _check(lib().kda_affine_exclusive_scan_blocked(int(n), int(H), int(dk), int(dv), int(block), _ptr(M),
                                                       _ptr(U), _ptr(S_init), _ptr(incoming), _ptr(outgoing),
                                                       _ptr(final_state), _stream()))
    return incoming, outgoing, final_state


def context_parallel(transition_matrices, local_contributions, initial_state):
    """Incoming, outgoing and final states of segments combined in order.

    Follows KDA Context Parallelism (Requirements): returns a dict with exactly the keys
    incoming_states, outgoing_states, final_state; stacks lead with the segment axis;
    dtype and device are preserved; inputs are not modified.  Accepts the single-state
    shapes (segments, w, w), (segments, w, v), (w, v) or a head axis after the segment
    axis.  fp32 on the GPU only."""
    M, U, S = transition_matrices, local_contributions, initial_state
    squeeze = M.dim() == 3
    if squeeze:
        M, U, S = M.unsqueeze(1), U.unsqueeze(1), S.unsqueeze(0)
    if M.shape[0] < 1:
        raise ValueError("at least one segment is required")
    if M.dtype != torch.float32 or M.device.type != "cuda":
        raise ValueError("context_parallel runs on the GPU in float32")
    inc, out, fin = affine_exclusive_scan(M.contiguous(), U.contiguous(), S.contiguous())
    if squeeze:
        inc, out, fin = inc.squeeze(1), out.squeeze(1), fin.squeeze(0)
    return {"incoming_states": inc, "outgoing_states": out, "final_state": fin}


def validate_varlen(cu_seqlens, state_indices, total_tokens, max_slots):
    """Synchronous check of cu_seqlens / state_indices; raises ValueError when invalid."""
    B = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", torch.int32, cu_seqlens.device)
    _need(state_indices, "state_indices", torch.int32, cu_seqlens.device)
    if cu_seqlens.dim() != 1 or tuple(state_indices.shape) != (B,):
        raise ValueError("cu_seqlens must be [B+1] and state_indices [B]")
    _on_gpu(cu_seqlens.device)
    _check(lib().kda_validate_varlen(_ptr(cu_seqlens), int(B), int(total_tokens), _ptr(state_indices),
                                     int(max_slots)))
