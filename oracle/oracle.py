"""Python front end of the fp64 KDA oracle (kda_oracle.c).

TEST INFRASTRUCTURE ONLY.  Imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product path.  It shares no code
with the HIP library: it reads the exact input values the GPU receives
(bf16 or fp32, upcast element by element to fp64) and runs the sequential
recurrence of "Kimi K3: Open Frontier Intelligence and Implementation
Framework", section "Hybrid Attention Mechanism" (the delta rule with a
channel-wise forget gate; the exact form is written out in kda_oracle.c).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile kda_oracle.c with gcc (fp64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                        "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str):
    """Open a compiled oracle library and declare its entry point."""
    lib = ctypes.CDLL(path)
    p = ctypes.POINTER(ctypes.c_double)
    lib.kda_oracle_recurrence.argtypes = [p, p, p, p, p, p, p, p,
                                          ctypes.POINTER(ctypes.c_int64),
                                          ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    lib.kda_oracle_recurrence.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = load_library(_LIB)
    return _lib


def host_threads() -> int:
    """Threads the oracle uses by default: the host cores this process may run on."""
    return len(os.sched_getaffinity(0))


def as_f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (fp32 or bf16) or array to contiguous fp64."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrence(q, k, v, g, beta, cu_seqlens, s0=None, nthreads: int | None = None):
    """Packed sequences.  q, k, g [tokens, H, K]; v [tokens, H, V]; beta [tokens, H];
    cu_seqlens [N + 1]; s0 [N, H, K, V] or None.  Returns (o [tokens, H, V],
    sT [N, H, K, V]) in fp64."""
    q, k, v, g, beta, s0 = (as_f64(x) for x in (q, k, v, g, beta, s0))
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    tokens, H, K = q.shape
    V = v.shape[-1]
    N = len(cu) - 1
    assert k.shape == (tokens, H, K) and g.shape == (tokens, H, K)
    assert v.shape == (tokens, H, V) and beta.shape == (tokens, H)
    assert cu[-1] == tokens
    if s0 is not None:
        assert s0.shape == (N, H, K, V)
    o = np.zeros((tokens, H, V), dtype=np.float64)
    sT = np.zeros((N, H, K, V), dtype=np.float64)
    rc = _load().kda_oracle_recurrence(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(o), _ptr(sT),
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), N, H, K, V,
        int(nthreads or host_threads()))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_recurrence failed with code {rc}")
    return o, sT


def fixed(q, k, v, g, beta, s0=None, nthreads: int | None = None):
    """Fixed-length batch [B, T, H, *]: the packed recurrence with cu = {0, T, .., B*T}.
    Returns (o [B, T, H, V], sT [B, H, K, V])."""
    q = as_f64(q)
    B, T, H, K = q.shape
    V = v.shape[-1]
    cu = np.arange(B + 1, dtype=np.int64) * T
    o, sT = recurrence(q.reshape(B * T, H, K), as_f64(k).reshape(B * T, H, K),
                       as_f64(v).reshape(B * T, H, V), as_f64(g).reshape(B * T, H, K),
                       as_f64(beta).reshape(B * T, H), cu, s0, nthreads)
    return o.reshape(B, T, H, V), sT


def prologue(q, k, g, beta, normalize_qk: bool = False, gate_lower_bound=None,
             beta_logits: bool = False, norm_eps: float = 0.0):
    """The input prologue, in fp64: maps raw projections to what the recurrence
    reads.  "Kimi K3: Open Frontier Intelligence and Implementation Framework",
    section "Hybrid Attention Mechanism", calls KDA's gate channel-wise and its
    decay lower-bounded; the parameterisation taken here is
        g    = -g_lb * sigmoid(x)             (gate logits x, g_lb = gate_lower_bound)
        beta = sigmoid(b)                     (beta logits b)
        q, k = x / sqrt(sum_c x_c^2 + eps)    (per token and head; 0 if the sum is 0)
    with sigmoid(x) = 1 / (1 + exp(-x)).  Each map applies only when selected;
    the others pass their input through.  Returns fp64 (q, k, g, beta)."""
    q, k, g, beta = (as_f64(x) for x in (q, k, g, beta))
    if normalize_qk:
        def unit(x):
            s = np.sum(x * x, axis=-1, keepdims=True) + norm_eps
            safe = np.where(s > 0.0, s, 1.0)
            return np.where(s > 0.0, x / np.sqrt(safe), 0.0)
        q, k = unit(q), unit(k)
    with np.errstate(over="ignore"):
        if gate_lower_bound is not None:
            g = -float(gate_lower_bound) / (1.0 + np.exp(-g))
        if beta_logits:
            beta = 1.0 / (1.0 + np.exp(-beta))
    return q, k, g, beta


def backward(q, k, v, g, beta, cu_seqlens, s0, do, dsT):
    """Gradients of the recurrence, in fp64: for the scalar loss
        L = sum(do * o) + sum(dsT * sT)
    returns (dq, dk, dv, dg, dbeta, ds0) with the shapes of q, k, v, g, beta and
    of the states [N, H, K, V].  The recurrence is the one of
    kda_oracle.c (section "Hybrid Attention Mechanism" of "Kimi K3: Open
    Frontier Intelligence and Implementation Framework": the delta rule with a
    channel-wise forget gate), written here as a plain token loop in torch fp64
    on the CPU, one sequence at a time with its heads as a batch, and
    differentiated by torch.autograd (no chunking, no hand-derived gradient).
    s0 and dsT may be None (zeros).  Memory grows with tokens * H * K * V:
    meant for test-sized inputs."""
    import torch
    q, k, v, g, beta, do = (as_f64(x) for x in (q, k, v, g, beta, do))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    tokens, H, K = q.shape
    V = v.shape[-1]
    N = len(cu) - 1
    s0 = np.zeros((N, H, K, V)) if s0 is None else as_f64(s0)
    dsT = np.zeros((N, H, K, V)) if dsT is None else as_f64(dsT)
    outs = [np.zeros_like(x) for x in (q, k, v, g, beta)] + [np.zeros((N, H, K, V))]
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        ts = [torch.tensor(x[a:b], dtype=torch.float64, requires_grad=True)
              for x in (q, k, v, g, beta)]
        S0 = torch.tensor(s0[n], dtype=torch.float64, requires_grad=True)
        tq, tk, tv, tg, tb = ts
        S = S0
        loss = torch.zeros((), dtype=torch.float64)
        dO = torch.tensor(do[a:b], dtype=torch.float64)
        for t in range(b - a):
            S = torch.exp(tg[t])[:, :, None] * S                        # Diag(alpha_t) S
            e = tv[t] - torch.einsum("hkv,hk->hv", S, tk[t])            # v_t - S^T k_t
            S = S + tb[t][:, None, None] * tk[t][:, :, None] * e[:, None, :]
            o = torch.einsum("hkv,hk->hv", S, tq[t])                    # S_t^T q_t
            loss = loss + (o * dO[t]).sum()
        loss = loss + (S * torch.tensor(dsT[n], dtype=torch.float64)).sum()
        loss.backward()
        for i, x in enumerate(ts):
            if x.grad is not None:          # None for an empty sequence
                outs[i][a:b] = x.grad.numpy()
        outs[5][n] = S0.grad.numpy()
    return tuple(outs)


def decode_step(q, k, v, g, beta, state, nthreads: int | None = None):
    """One token per sequence: q, k, g [N, H, K]; v [N, H, V]; beta [N, H];
    state [N, H, K, V] fp64.  Returns (o [N, H, V], new state)."""
    q = as_f64(q)
    N, H, K = q.shape
    cu = np.arange(N + 1, dtype=np.int64)
    return recurrence(q, k, v, g, beta, cu, state, nthreads)
