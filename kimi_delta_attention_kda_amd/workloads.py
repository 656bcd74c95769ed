"""Seeded synthetic inputs for the KDA prefill path.

This module only draws random numbers and shapes them.  It holds none of the
method's arithmetic (no gate, no recurrence, no chunking), so both the GPU
library's tests/benchmark and the CPU oracle can take their inputs from here.

Value recipe (shared by every workload):
  q, k ~ N(0,1), then L2-normalised per (token, head) in fp32, then cast;
  v ~ N(0,1) then cast; raw_gate ~ N(0,1) fp32; dt_bias ~ N(0, 0.1^2) [H,dk];
  a_log ~ U(0, ln 16) [H]; beta_logits ~ N(0, sigma_b^2) fp32 [T,H];
  used pool slots ~ N(0, s0^2); unused pool slots hold random fp32 bit
  patterns (canaries that must survive a call bit-identically).
Casts to bfloat16 round to nearest even.

Each named workload fixes shapes, dtypes, gate mode and sequence-length mix:
  tiny_fp32        1 x 512 tokens, H=2, dk=dv=64, fp32, original gate, zero state
  varlen_32k       8 sequences, lengths in [1024, 8192] summing to 32768,
                   H=32, dk=dv=128, bf16 q/k/v/out, safe gate (lower bound -5),
                   64-slot pool, distinct random slots, states ~ N(0, 0.01^2)
  varlen_32k_dk64  the same lengths and draws with dk=dv=64
  long_131k        1 x 131072 tokens, as varlen_32k, one zero slot
  segments_262k    1 x 262144 tokens as 16 segments of 16384, H=8, fp32,
                   original gate, initial state ~ N(0, 0.01^2)
  short_varlen_512 512 sequences, lengths U{16..2048}, bf16, safe gate,
                   beta_logits ~ N(0, 2^2), 1024-slot pool
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    lengths: tuple            # tokens per sequence
    H: int
    dk: int
    dv: int
    dtype: str                # "f32" or "bf16" for q/k/v/out
    gate_mode: int            # 0 original, 1 safe
    lower_bound: float = -5.0
    beta_mode: int = 0        # 0 logits, 1 probability
    beta_sigma: float = 1.0
    n_slots: int = 1
    state_sigma: float = 0.0  # used-slot init std (0 = zeros)
    canary_unused: bool = True
    seed: int = 0
    segments: int = 0         # >0: segment-summary workload, equal segments
    raw_mean: float = 0.0     # raw_gate ~ N(raw_mean, 1)
    beta_mean: float = 0.0    # beta_logits ~ N(beta_mean, beta_sigma^2)
    a_log_hi: float = math.log(16.0)  # a_log ~ U(0, a_log_hi)
    Hk: int = 0               # key heads of q and k (0: as many as value heads H)

    @property
    def T(self) -> int:
        return int(sum(self.lengths))

    @property
    def HK(self) -> int:
        return self.Hk or self.H

    @property
    def B(self) -> int:
        return len(self.lengths)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dk)


def _varlen_32k_lengths(rng: np.random.Generator, B=8, total=32768, lo=1024, hi=8192):
    while True:
        x = rng.uniform(lo, hi, size=B)
        L = np.floor(x * total / x.sum()).astype(np.int64)
        L[np.argmax(L)] += total - int(L.sum())
        if L.min() >= lo and L.max() <= hi:
            return tuple(int(v) for v in L)


def workload(name: str, seed: int = 0) -> Workload:
    rng = np.random.default_rng(seed)
    if name == "tiny_fp32":
        return Workload(name, (512,), 2, 64, 64, "f32", 0, n_slots=1, seed=seed)
    if name == "varlen_32k":
        return Workload(name, _varlen_32k_lengths(rng), 32, 128, 128, "bf16", 1,
                        n_slots=64, state_sigma=0.01, seed=seed)
    if name == "varlen_32k_original":  # the 32K lengths with the original (unclamped) gate
        return Workload(name, _varlen_32k_lengths(rng), 32, 128, 128, "bf16", 0,
                        n_slots=64, state_sigma=0.01, seed=seed)
    if name == "varlen_32k_dk64":
        return Workload(name, _varlen_32k_lengths(rng), 32, 64, 64, "bf16", 1,
                        n_slots=64, state_sigma=0.01, seed=seed)
    if name == "long_131k":
        return Workload(name, (131072,), 32, 128, 128, "bf16", 1, n_slots=1, seed=seed)
    if name == "segments_262k":
        return Workload(name, (262144,), 8, 128, 128, "f32", 0, n_slots=1,
                        state_sigma=0.01, segments=16, seed=seed)
    if name == "short_varlen_512":
        L = tuple(int(v) for v in rng.integers(16, 2049, size=512))
        return Workload(name, L, 32, 128, 128, "bf16", 1, beta_sigma=2.0,
                        n_slots=1024, state_sigma=0.01, seed=seed)
    if name == "decode_512":  # one token for each of 512 sequences (single-token decode)
        return Workload(name, (1,) * 512, 32, 128, 128, "bf16", 1, n_slots=1024, state_sigma=0.01,
                        seed=seed)
    raise KeyError(name)


NAMES = ("tiny_fp32", "varlen_32k", "varlen_32k_original", "varlen_32k_dk64", "long_131k", "segments_262k", "short_varlen_512", "decode_512")


def custom(lengths, H=2, dk=64, dv=64, dtype="bf16", gate_mode=1, n_slots=None,
           state_sigma=0.01, beta_sigma=1.0, seed=0, name="custom", **kw) -> Workload:
    """A workload with explicit shapes (tests: ragged tails, edge lengths)."""
    lengths = tuple(int(x) for x in lengths)
    if n_slots is None:
        n_slots = len(lengths) + 3
    return Workload(name, lengths, H, dk, dv, dtype, gate_mode, n_slots=n_slots,
                    state_sigma=state_sigma, beta_sigma=beta_sigma, seed=seed, **kw)


def slow_gate_segments(segments=4, seg_len=2048, H=2, dk=128, seed=0) -> Workload:
    """Segment workload whose maps stay O(1): log-alpha ~ -1e-5 (a_log = 0,
    raw_gate ~ N(-11.5, 1)) and beta ~ 1e-3 (beta_logits ~ N(-7, 1))."""
    return Workload("slow_gate_segments", (segments * seg_len,), H, dk, dk, "f32", 0, n_slots=1,
                    state_sigma=0.01, segments=segments, raw_mean=-11.5, beta_mean=-7.0,
                    a_log_hi=0.0, seed=seed)


def torch_dtype(d: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[d]


def make_inputs(w: Workload, device="cpu") -> dict:
    """Draws every tensor of workload `w` on `device` (deterministic per device).

    Returns a dict of torch tensors in the library's layouts:
      q, k [T,Hk,dk]; v [T,H,dv] (dtype per workload); raw_gate [T,H,dk] f32;
      beta_logits [T,H] f32; a_log [H] f32; dt_bias [H,dk] f32;
      cu_seqlens [B+1] int32; state_pool [n_slots,H,dk,dv] f32;
      state_indices [B] int32; plus host copies of lengths/indices.
    """
    rng = np.random.default_rng(w.seed + 1)
    T, H, dk, dv = w.T, w.H, w.dk, w.dv
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    dt = torch_dtype(w.dtype)

    def normal(*shape, std=1.0):
        return torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * std

    def unit_rows(x):
        return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)

    q = unit_rows(normal(T, w.HK, dk)).to(dt)
    k = unit_rows(normal(T, w.HK, dk)).to(dt)
    v = normal(T, H, dv).to(dt)
    raw_gate = normal(T, H, dk) + w.raw_mean
    beta_logits = normal(T, H, std=w.beta_sigma) + w.beta_mean
    if w.beta_mode == 1:  # beta given directly as a probability: uniform in (0, 1)
        beta_logits = torch.rand(T, H, generator=g, device=device, dtype=torch.float32)
    a_log = torch.rand(H, generator=g, device=device, dtype=torch.float32) * w.a_log_hi
    dt_bias = normal(H, dk, std=0.1)

    cu = np.zeros(w.B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(w.lengths)
    cu_seqlens = torch.tensor(cu, dtype=torch.int32, device=device)

    if w.segments:
        idx = np.zeros(w.B, dtype=np.int64)
    else:
        idx = rng.permutation(w.n_slots)[: w.B]
    state_indices = torch.tensor(idx, dtype=torch.int32, device=device)

    pool_shape = (w.n_slots, H, dk, dv)
    if w.canary_unused:
        bits = torch.randint(-(2 ** 31), 2 ** 31 - 1, pool_shape, generator=g, device=device,
                             dtype=torch.int64).to(torch.int32)
        pool = bits.view(torch.float32)
    else:
        pool = torch.zeros(pool_shape, device=device, dtype=torch.float32)
    used = torch.tensor(idx, dtype=torch.int64, device=device)
    if w.state_sigma > 0:
        pool[used] = normal(w.B, H, dk, dv, std=w.state_sigma)
    else:
        pool[used] = 0.0

    out = dict(q=q, k=k, v=v, raw_gate=raw_gate, beta_logits=beta_logits, a_log=a_log,
               dt_bias=dt_bias, cu_seqlens=cu_seqlens, state_pool=pool,
               state_indices=state_indices, lengths=list(w.lengths), cu=cu.tolist(),
               indices=idx.tolist())
    if w.segments:
        seg = T // w.segments
        out["seg_offsets"] = torch.arange(0, T + 1, seg, dtype=torch.int32, device=device)
        out["S_init"] = normal(H, dk, dv, std=w.state_sigma if w.state_sigma > 0 else 0.01)
    return out


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 host copy (bf16 and fp32 are exactly representable)."""
    return t.detach().to("cpu", torch.float64).numpy()
