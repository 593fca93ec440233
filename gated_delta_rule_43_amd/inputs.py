"""Seeded synthetic inputs for the KDA operator.

This module draws random tensors and nothing else: it holds none of the
operator's arithmetic, so both the HIP path and the fp64 oracle can take
their inputs from it without sharing any computation.

Distributions (one recipe for every workload):
  q, k  ~ N(0, 1), then L2-normalised per (token, head) over the key channels
  v     ~ N(0, 1)
  beta  = sigmoid(N(0, 1)), one scalar per (token, head)
  g     = -g_lb * sigmoid(N(0, 1)) per (token, head, key channel), g = log(alpha),
          g_lb = 0.25 by default (the lower-bounded decay parameterisation of
          "Kimi K3: Open Frontier Intelligence and Implementation Framework",
          section "Hybrid Attention Mechanism")
  S_0   ~ N(0, sigma^2) in fp32 when the workload has an initial state

All values are drawn in fp32 with numpy's PCG64 generator and then rounded
to the input dtype (round-to-nearest-even for bf16).  Draw order:
lengths (varlen only), q, k, v, beta logits, g logits, S_0.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "draw_fixed", "draw_varlen", "draw_decode_step",
           "draw_decode_state", "varlen_lengths", "to_dtype"]


@dataclass(frozen=True)
class Workload:
    """A named synthetic workload.  kind is 'fixed', 'varlen' or 'decode'."""
    name: str
    kind: str
    H: int
    K: int
    V: int
    chunk: int
    dtype: str                      # 'f32' or 'bf16' for q, k, v, g, beta
    seed: int
    B: int = 0                      # fixed: batch
    T: int = 0                      # fixed: tokens per sequence
    N: int = 0                      # varlen / decode: number of sequences
    len_min: int = 0                # varlen: log-uniform length range
    len_max: int = 0
    steps: int = 0                  # decode: consecutive steps
    s0_std: Optional[float] = None  # None: S_0 = 0 (no initial state passed)
    notes: str = field(default="", compare=False)


WORKLOADS = {
    w.name: w for w in [
        Workload("single_f32_T64_d32", "fixed", H=1, K=32, V=32, chunk=16, dtype="f32",
                 seed=0, B=1, T=64,
                 notes="single-sequence fp32 forward, B=1 H=1 T=64 d_k=d_v=32 chunk=16"),
        Workload("prefill_bf16_B1_H8_T4096", "fixed", H=8, K=128, V=128, chunk=64,
                 dtype="bf16", seed=1, B=1, T=4096,
                 notes="prefill, bf16 inputs, fp32 state/accumulation, B=1 H=8 T=4096"),
        Workload("batched_bf16_B4_H32_T8192", "fixed", H=32, K=128, V=128, chunk=64,
                 dtype="bf16", seed=2, B=4, T=8192, s0_std=0.1,
                 notes="batched prefill, B=4 H=32 T=8192, S_0 ~ N(0, 0.01), S_T returned"),
        Workload("varlen_bf16_N64_H16", "varlen", H=16, K=128, V=128, chunk=64,
                 dtype="bf16", seed=3, N=64, len_min=16, len_max=32768,
                 notes="64 packed sequences, lengths log-uniform in [16, 32768]"),
        Workload("decode_bf16_N256_H32", "decode", H=32, K=128, V=128, chunk=64,
                 dtype="bf16", seed=4, N=256, steps=1000, s0_std=0.1,
                 notes="one token per sequence per step, 256 sequences x 32 heads, "
                       "persistent fp32 state, 1000 consecutive steps"),
    ]
}


def to_dtype(x32: np.ndarray, dtype: str) -> torch.Tensor:
    """fp32 numpy array -> CPU tensor of the input dtype (RNE for bf16)."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    if dtype == "f32":
        return t
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError(f"unknown dtype {dtype!r}")


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-30)).astype(np.float32)


def _draw_token_tensors(rng: np.random.Generator, tokens: int, H: int, K: int, V: int,
                        dtype: str, g_lb: float, g_mode: str):
    q = _unit_rows(rng.standard_normal((tokens, H, K), dtype=np.float32))
    q = to_dtype(q, dtype)
    k = _unit_rows(rng.standard_normal((tokens, H, K), dtype=np.float32))
    k = to_dtype(k, dtype)
    v = to_dtype(rng.standard_normal((tokens, H, V), dtype=np.float32), dtype)
    beta = to_dtype(_sigmoid(rng.standard_normal((tokens, H), dtype=np.float32)), dtype)
    glog = rng.standard_normal((tokens, H, K), dtype=np.float32)
    if g_mode == "default":
        g32 = (-g_lb * _sigmoid(glog)).astype(np.float32)
    elif g_mode == "zero":           # alpha = 1: no decay at all
        g32 = np.zeros_like(glog)
    elif g_mode == "bound":          # every step at the lower bound
        g32 = np.full_like(glog, -g_lb)
    elif g_mode == "uniform":        # uniform in [-g_lb, 0]
        g32 = (-g_lb * rng.random(glog.shape, dtype=np.float32)).astype(np.float32)
    else:
        raise ValueError(f"unknown g_mode {g_mode!r}")
    g = to_dtype(g32, dtype)
    return q, k, v, g, beta


def draw_fixed(seed: int, B: int, T: int, H: int, K: int, V: int, dtype: str,
               s0_std: Optional[float] = None, g_lb: float = 0.25,
               g_mode: str = "default") -> dict:
    """Fixed-length batch: q, k, g [B, T, H, K]; v [B, T, H, V]; beta [B, T, H];
    s0 [B, H, K, V] fp32 or None."""
    rng = np.random.default_rng(seed)
    q, k, v, g, beta = _draw_token_tensors(rng, B * T, H, K, V, dtype, g_lb, g_mode)
    s0 = None
    if s0_std is not None:
        s0 = torch.from_numpy(
            (rng.standard_normal((B, H, K, V), dtype=np.float32) * np.float32(s0_std)))
    return dict(q=q.view(B, T, H, K), k=k.view(B, T, H, K), v=v.view(B, T, H, V),
                g=g.view(B, T, H, K), beta=beta.view(B, T, H), s0=s0)


def varlen_lengths(rng: np.random.Generator, N: int, lo: int, hi: int) -> np.ndarray:
    """N lengths log-uniform in [lo, hi], rounded and clamped to [lo, hi]."""
    u = rng.uniform(math.log(lo), math.log(hi), size=N)
    return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int64)


def draw_varlen(seed: int, H: int, K: int, V: int, dtype: str, N: int = 0,
                len_min: int = 16, len_max: int = 32768, lengths=None,
                s0_std: Optional[float] = None, g_lb: float = 0.25,
                g_mode: str = "default") -> dict:
    """Packed sequences: tokens = sum(lengths); q, k, g [tokens, H, K];
    v [tokens, H, V]; beta [tokens, H]; cu_seqlens int32 [N+1]."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = varlen_lengths(rng, N, len_min, len_max)
    lengths = np.asarray(lengths, dtype=np.int64)
    N = len(lengths)
    cu = np.zeros(N + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    total = int(cu[-1])
    q, k, v, g, beta = _draw_token_tensors(rng, total, H, K, V, dtype, g_lb, g_mode)
    s0 = None
    if s0_std is not None:
        s0 = torch.from_numpy(
            (rng.standard_normal((N, H, K, V), dtype=np.float32) * np.float32(s0_std)))
    return dict(q=q, k=k, v=v, g=g, beta=beta, s0=s0,
                cu_seqlens=torch.from_numpy(cu.astype(np.int32)), lengths=lengths)


def _draw_raw_token_tensors(rng: np.random.Generator, tokens: int, H: int, K: int, V: int,
                            dtype: str):
    """Raw projections for the input prologue: q, k ~ N(0, 1) per element times a
    per-(token, head) scale exp(U(-2, 2)) (so row norms vary over e^+-2 sqrt(K));
    v ~ N(0, 1); gate logits ~ N(0, 1) per (token, head, channel); beta logits
    ~ N(0, 1) per (token, head)."""
    def rows(n):
        x = rng.standard_normal((tokens, H, n), dtype=np.float32)
        return x * np.exp(rng.uniform(-2.0, 2.0, size=(tokens, H, 1))).astype(np.float32)
    q = to_dtype(rows(K), dtype)
    k = to_dtype(rows(K), dtype)
    v = to_dtype(rng.standard_normal((tokens, H, V), dtype=np.float32), dtype)
    x = to_dtype(rng.standard_normal((tokens, H, K), dtype=np.float32), dtype)
    b = to_dtype(rng.standard_normal((tokens, H), dtype=np.float32), dtype)
    return q, k, v, x, b


def draw_raw_fixed(seed: int, B: int, T: int, H: int, K: int, V: int, dtype: str,
                   s0_std: Optional[float] = None) -> dict:
    """Raw prologue inputs, fixed-length batch: q, k [B, T, H, K] (unnormalised),
    g [B, T, H, K] gate logits, v [B, T, H, V], beta [B, T, H] logits; s0 or None."""
    rng = np.random.default_rng(seed)
    q, k, v, x, b = _draw_raw_token_tensors(rng, B * T, H, K, V, dtype)
    s0 = None
    if s0_std is not None:
        s0 = torch.from_numpy(
            (rng.standard_normal((B, H, K, V), dtype=np.float32) * np.float32(s0_std)))
    return dict(q=q.view(B, T, H, K), k=k.view(B, T, H, K), v=v.view(B, T, H, V),
                g=x.view(B, T, H, K), beta=b.view(B, T, H), s0=s0)


def draw_raw_varlen(seed: int, H: int, K: int, V: int, dtype: str, lengths,
                    s0_std: Optional[float] = None) -> dict:
    """Raw prologue inputs for packed sequences of the given lengths."""
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    N = len(lengths)
    cu = np.zeros(N + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    q, k, v, x, b = _draw_raw_token_tensors(rng, int(cu[-1]), H, K, V, dtype)
    s0 = None
    if s0_std is not None:
        s0 = torch.from_numpy(
            (rng.standard_normal((N, H, K, V), dtype=np.float32) * np.float32(s0_std)))
    return dict(q=q, k=k, v=v, g=x, beta=b, s0=s0,
                cu_seqlens=torch.from_numpy(cu.astype(np.int32)), lengths=lengths)


def draw_decode_state(seed: int, N: int, H: int, K: int, V: int, s0_std: float) -> torch.Tensor:
    """Initial persistent decode state [N, H, K, V] fp32 ~ N(0, s0_std^2)."""
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.standard_normal((N, H, K, V), dtype=np.float32)
                            * np.float32(s0_std))


def draw_decode_step(seed: int, step: int, N: int, H: int, K: int, V: int, dtype: str,
                     g_lb: float = 0.25, g_mode: str = "default") -> dict:
    """Fresh inputs for decode step `step` (one token per sequence), drawn from the
    generator seeded with [seed, step]: q, k, g [N, H, K]; v [N, H, V]; beta [N, H]."""
    rng = np.random.default_rng([seed, step])
    q, k, v, g, beta = _draw_token_tensors(rng, N, H, K, V, dtype, g_lb, g_mode)
    return dict(q=q, k=k, v=v, g=g, beta=beta)
