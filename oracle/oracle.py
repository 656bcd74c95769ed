"""Python side of the fp64 CPU oracle for KDA (TEST INFRASTRUCTURE ONLY).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It wraps oracle/kda_oracle.c (compiled by oracle/build.py with
gcc) through ctypes and holds no GPU code.  See kda_oracle.c for the
definition of every quantity and the passages it follows.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


class _Item(C.Structure):
    _fields_ = [("n", C.c_int64), ("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p),
                ("raw_gate", C.c_void_p), ("beta_in", C.c_void_p), ("dt_bias", C.c_void_p),
                ("a_log", C.c_double), ("S", C.c_void_p), ("out", C.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path):
            path = _build.build()
        L = C.CDLL(path)
        dp = C.c_void_p
        L.kda_ref_log_alpha.argtypes = [C.c_int64, C.c_int, dp, dp, C.c_double, C.c_int, C.c_double, dp]
        L.kda_ref_beta.argtypes = [C.c_int64, dp, C.c_int, dp]
        L.kda_ref_recur.argtypes = [C.c_int64, C.c_int, C.c_int, dp, dp, dp, dp, dp, C.c_double, dp, dp]
        L.kda_ref_forward_items.argtypes = [C.c_int, C.POINTER(_Item), C.c_int, C.c_int, C.c_int,
                                            C.c_double, C.c_int, C.c_double, C.c_int]
        L.kda_ref_segment_map_items.argtypes = [C.c_int, C.POINTER(_Item), C.POINTER(C.c_void_p),
                                                C.c_int, C.c_int, C.c_int, C.c_double, C.c_int, C.c_int]
        L.kda_ref_scan.argtypes = [C.c_int, C.c_int, C.c_int, dp, dp, dp, dp, dp, dp]
        L.kda_ref_scan.restype = C.c_int
        L.kda_ref_compose.argtypes = [C.c_int, C.c_int, dp, dp, dp, dp, dp, dp]
        _lib = L
    return _lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


# ----------------------------------------------------------------- pieces --

def log_alpha(raw, dt_bias, a_log, gate_mode=0, lb=-5.0):
    """log-alpha [n,dk] of one head from raw_gate [n,dk], dt_bias [dk], a_log."""
    raw = _f64(raw)
    n, dk = raw.shape
    out = np.empty_like(raw)
    lib().kda_ref_log_alpha(n, dk, _p(raw), _p(_f64(dt_bias)), float(a_log), int(gate_mode),
                            float(lb), _p(out))
    return out


def beta(logits, beta_mode=0):
    x = _f64(logits)
    out = np.empty_like(x)
    lib().kda_ref_beta(x.size, _p(x), int(beta_mode), _p(out))
    return out


def recur(k, v, alpha, beta_, S0, q=None, scale=1.0):
    """Token recurrence with alpha [n,dk] and beta [n] given; returns (out|None, S)."""
    k, v, alpha, beta_ = _f64(k), _f64(v), _f64(alpha), _f64(beta_)
    n, dk = k.shape
    dv = v.shape[1]
    S = _f64(S0).copy()
    qq = None if q is None else _f64(q)
    out = None if q is None else np.zeros((n, dv))
    lib().kda_ref_recur(n, dk, dv, _p(qq), _p(k), _p(v), _p(alpha), _p(beta_), float(scale),
                        _p(S), _p(out))
    return out, S


# ------------------------------------------------------------ whole items --

def forward_items(items, dk, dv, gate_mode, lb, beta_mode, scale, nthreads=None):
    """items: list of dicts with n-token fp64 arrays q,k,v,raw_gate,beta_in,
    dt_bias, a_log, S0.  Returns list of (out [n,dv], S_final [dk,dv])."""
    keep = []
    arr = (_Item * len(items))()
    res = []
    for i, it in enumerate(items):
        q = None if it.get("q") is None else _f64(it["q"])
        k, v = _f64(it["k"]), _f64(it["v"])
        raw, bi, dtb = _f64(it["raw_gate"]), _f64(it["beta_in"]), _f64(it["dt_bias"])
        S = _f64(it["S0"]).copy()
        n = k.shape[0]
        out = np.zeros((n, dv)) if q is not None else None
        keep += [q, k, v, raw, bi, dtb, S, out]
        arr[i] = _Item(n, _p(q), _p(k), _p(v), _p(raw), _p(bi), _p(dtb), float(it["a_log"]),
                       _p(S), _p(out))
        res.append((out, S))
    lib().kda_ref_forward_items(len(items), arr, dk, dv, int(gate_mode), float(lb),
                                int(beta_mode), float(scale), nthreads or default_threads())
    return res


def segment_maps(items, dk, dv, gate_mode, lb, beta_mode, nthreads=None):
    """Per item (token segment of one head): returns list of (M [dk,dk], U [dk,dv])."""
    keep = []
    arr = (_Item * len(items))()
    Mp = (C.c_void_p * len(items))()
    res = []
    for i, it in enumerate(items):
        k, v = _f64(it["k"]), _f64(it["v"])
        raw, bi, dtb = _f64(it["raw_gate"]), _f64(it["beta_in"]), _f64(it["dt_bias"])
        U = np.zeros((dk, dv))
        M = np.zeros((dk, dk))
        keep += [k, v, raw, bi, dtb, U, M]
        arr[i] = _Item(k.shape[0], None, _p(k), _p(v), _p(raw), _p(bi), _p(dtb),
                       float(it["a_log"]), _p(U), None)
        Mp[i] = _p(M)
        res.append((M, U))
    lib().kda_ref_segment_map_items(len(items), arr, Mp, dk, dv, int(gate_mode), float(lb),
                                    int(beta_mode), nthreads or default_threads())
    return res


def scan(M, U, S_init):
    """Ordered exclusive prefix of affine maps for one head.

    M [n,dk,dk], U [n,dk,dv], S_init [dk,dv] -> dict with exactly the keys
    incoming_states, outgoing_states, final_state."""
    M, U, S_init = _f64(M), _f64(U), _f64(S_init)
    n, dk, dv = U.shape
    inc = np.zeros((n, dk, dv))
    outg = np.zeros((n, dk, dv))
    fin = np.zeros((dk, dv))
    rc = lib().kda_ref_scan(n, dk, dv, _p(M), _p(U), _p(S_init), _p(inc), _p(outg), _p(fin))
    if rc != 0:
        raise ValueError("at least one segment is required")
    return {"incoming_states": inc, "outgoing_states": outg, "final_state": fin}


def compose(M2, U2, M1, U1):
    """The map "F1, then F2" of two affine maps F(S) = M S + U of one head:
    (M2 M1, M2 U1 + U2).  M [dk,dk], U [dk,dv] -> (M, U)."""
    M2, U2, M1, U1 = _f64(M2), _f64(U2), _f64(M1), _f64(U1)
    dk, dv = U1.shape
    if M1.shape != (dk, dk) or M2.shape != (dk, dk) or U2.shape != (dk, dv):
        raise ValueError("maps of different shapes")
    Mo, Uo = np.zeros((dk, dk)), np.zeros((dk, dv))
    lib().kda_ref_compose(dk, dv, _p(M2), _p(U2), _p(M1), _p(U1), _p(Mo), _p(Uo))
    return Mo, Uo


# ----------------------------------------------------------- from inputs --

def item_from_inputs(inp: dict, b: int, h: int, with_q=True, t0=None, t1=None, S0=None):
    """Slices sequence b, value head h of a workload's inputs (torch tensors) into
    fp64 numpy arrays for the oracle.  t0/t1 bound the token range (absolute).

    q and k have Hk key heads, everything else H value heads (max.nn.state_space.kda_chunk,
    Parameters); Hk divides H and value head h reads key head h // (H // Hk), so that each
    key head serves a run of consecutive value heads (the reading taken where the page
    leaves the grouping open)."""
    cu = inp["cu"]
    a, e = cu[b], cu[b + 1]
    if t0 is not None:
        a = t0
    if t1 is not None:
        e = t1

    H, Hk = inp["v"].shape[1], inp["k"].shape[1]
    assert H % Hk == 0
    hk = h // (H // Hk)

    def sl(name, head=h):
        return inp[name][a:e, head].detach().to("cpu", dtype=__import__("torch").float64).numpy()

    if S0 is None:
        slot = inp["indices"][b]
        S0 = inp["state_pool"][slot, h].detach().to("cpu").double().numpy()
    return dict(q=sl("q", hk) if with_q else None, k=sl("k", hk), v=sl("v"), raw_gate=sl("raw_gate"),
                beta_in=sl("beta_logits"),
                dt_bias=inp["dt_bias"][h].detach().cpu().double().numpy(),
                a_log=float(inp["a_log"][h].item()), S0=S0)
