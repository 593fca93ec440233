"""Thin Python binding of libkda.so (include/kda.h).

Argument marshalling only: dtype/shape checks, output allocation with torch
and the current HIP stream.  Every step of the computation runs in the HIP
kernels behind the C ABI; there is no fallback of any kind, and every call
raises if the library is not built or the tensors are not on the GPU.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = ["chunk_fwd", "varlen_fwd", "varlen_fwd_noalloc", "decode_step", "varlen_fwd_paged", "decode_step_paged",
           "decode_multi_paged", "Prologue", "chunk_bwd", "varlen_bwd", "bwd_workspace_bytes",
           "workspace_bytes",
           "two_pass_workspace_bytes", "library", "kda_varlen", "kda_chunk",
           "KdaError", "LIB_PATH", "F32", "BF16"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")
F32, BF16 = 0, 1
PROLOGUE_NORM_QK, PROLOGUE_GATE_LOGIT, PROLOGUE_BETA_LOGIT = 1, 2, 4
_lib = None


@dataclass(frozen=True)
class Prologue:
    """Input prologue of the *_prologue entry points (kda.h): the kernels take raw
    projections and apply, while loading,
      normalize_qk:     q, k <- x (sum x^2 + norm_eps)^-1/2 per (token, head);
      gate_lower_bound: g holds logits x and g = -gate_lower_bound * sigmoid(x)
                        (None: g is the decay itself);
      beta_logits:      beta holds logits b and beta = sigmoid(b)."""
    normalize_qk: bool = False
    gate_lower_bound: Optional[float] = None
    beta_logits: bool = False
    norm_eps: float = 0.0

    def flags(self) -> int:
        return ((PROLOGUE_NORM_QK if self.normalize_qk else 0)
                | (PROLOGUE_GATE_LOGIT if self.gate_lower_bound is not None else 0)
                | (PROLOGUE_BETA_LOGIT if self.beta_logits else 0))

    def args(self):
        glb = 0.0 if self.gate_lower_bound is None else float(self.gate_lower_bound)
        return (ctypes.c_uint(self.flags()), ctypes.c_float(glb), ctypes.c_float(self.norm_eps))


class KdaError(RuntimeError):
    """A nonzero kda_status_t from the library."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


def library():
    """Load libkda.so (once) and declare the ABI."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run gated_delta_rule_43_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp,
                                  i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.kda_chunk_fwd.restype = i32
    lib.kda_varlen_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.kda_varlen_fwd.restype = i32
    lib.kda_varlen_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           i32, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.kda_varlen_fwd_noalloc.restype = i32
    lib.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.kda_decode_step.restype = i32
    lib.kda_varlen_fwd_paged.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp,
                                         i32, i32, i32, vp, vp,
                                         i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.kda_varlen_fwd_paged.restype = i32
    lib.kda_decode_step_paged.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                          i32, i32, i32, i32, i32, i32, vp]
    lib.kda_decode_step_paged.restype = i32
    lib.kda_decode_multi_paged.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                           i32, i32, i32, i32, i32, i32, i32, vp]
    lib.kda_decode_multi_paged.restype = i32
    # the *_prologue variants: the same arguments, then (flags, gate_lower_bound,
    # norm_eps) before the stream
    u32, f32 = ctypes.c_uint, ctypes.c_float
    for name in ("kda_chunk_fwd", "kda_varlen_fwd", "kda_varlen_fwd_paged", "kda_decode_step",
                 "kda_decode_step_paged", "kda_decode_multi_paged"):
        fn = getattr(lib, name + "_prologue")
        fn.argtypes = getattr(lib, name).argtypes[:-1] + [u32, f32, f32, vp]
        fn.restype = i32
    lib.kda_chunk_bwd.argtypes = [vp] * 14 + [i32] * 7 + [vp, sz, vp]
    lib.kda_chunk_bwd.restype = i32
    lib.kda_varlen_bwd.argtypes = [vp] * 15 + [i32] * 7 + [vp, sz, vp]
    lib.kda_varlen_bwd.restype = i32
    lib.kda_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.kda_bwd_workspace_bytes.restype = sz
    lib.kda_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.kda_workspace_bytes.restype = sz
    lib.kda_two_pass_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.kda_two_pass_workspace_bytes.restype = sz
    lib.kda_status_str.argtypes = [i32]
    lib.kda_status_str.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = i32
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        msg = library().kda_status_str(status).decode()
        if status in (1, 2, 3, 4, 5, 7):
            raise ValueError(f"{fn}: {msg}")
        raise KdaError(fn, status, msg)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported dtype {t}; expected torch.float32 or torch.bfloat16")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_gpu(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("KDA tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("KDA tensors must be contiguous")


def _default_chunk(K: int) -> int:
    return 16 if K == 32 else 64


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _call(name, prologue, *args):
    """Call entry point `name`, or its _prologue variant when a prologue is given;
    args end with the stream."""
    lib = library()
    if prologue is None:
        st = getattr(lib, name)(*args)
    else:
        name = name + "_prologue"
        st = getattr(lib, name)(*args[:-1], *prologue.args(), args[-1])
    _check(name, st)


def workspace_bytes(N: int, total_T: int, H: int, K: int, V: int, chunk: int) -> int:
    """Workspace bytes of the recommended implementation (0: single pass)."""
    return int(library().kda_workspace_bytes(N, total_T, H, K, V, chunk))


def two_pass_workspace_bytes(N: int, total_T: int, H: int, K: int, V: int, chunk: int) -> int:
    """Workspace bytes that select the two-pass path (0: not supported)."""
    return int(library().kda_two_pass_workspace_bytes(N, total_T, H, K, V, chunk))


def _workspace(dev, N, total, H, K, V, chunk, two_pass, workspace):
    """Workspace for one call: none when two_pass is False (single-pass kernels);
    the two-pass size when two_pass is True (ValueError if unsupported) or when
    two_pass is None and the library recommends it; the caller's uint8 tensor
    if given, else a fresh one."""
    if two_pass is False:
        return None, 0
    if two_pass:
        nbytes = two_pass_workspace_bytes(N, total, H, K, V, chunk)
        if nbytes == 0:
            raise ValueError(f"the two-pass path does not support N={N}, (K, V, chunk)="
                             f"({K}, {V}, {chunk})")
    else:
        nbytes = workspace_bytes(N, total, H, K, V, chunk)
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
        if workspace.numel() < nbytes:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, {nbytes} needed")
        return workspace, workspace.numel()
    return torch.empty(nbytes, dtype=torch.uint8, device=dev), nbytes


def chunk_fwd(q, k, v, g, beta, initial_state=None, output_final_state=True, chunk=None,
              out_dtype=torch.float32, final_state=None, out=None, two_pass=None,
              workspace=None, prologue=None):
    """Chunked KDA forward over a fixed-length batch.

    q, k, g: [B, T, H, K]; v: [B, T, H, V]; beta: [B, T, H]; all float32 or all bfloat16.
    initial_state: [B, H, K, V] float32 or None (zeros).
    Returns (o [B, T, H, V] of out_dtype, final state [B, H, K, V] float32 or None).
    final_state may be passed to receive S_T in place (it may be initial_state itself);
    out may be passed to receive o.
    two_pass: None takes the library's recommendation (the two-pass bf16 kernels
    when kda_workspace_bytes is nonzero: few (sequence, head) units, long
    sequences); True forces the two-pass path, False the single-pass kernels.
    workspace: optional preallocated uint8 tensor.
    prologue: a Prologue (raw q/k, gate and beta logits), or None.
    """
    _need_gpu(q, k, v, g, beta, initial_state, final_state, out)
    B, T, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    if any(x.dtype != dt for x in (k, v, g, beta)):
        raise ValueError("q, k, v, g and beta must share one dtype")
    if k.shape != q.shape or g.shape != q.shape or v.shape != (B, T, H, V) or beta.shape != (B, T, H):
        raise ValueError("shape mismatch among q, k, v, g, beta")
    for s in (initial_state, final_state):
        if s is not None and (s.dtype != torch.float32 or s.shape != (B, H, K, V)):
            raise ValueError("states must be float32 [B, H, K, V]")
    chunk = chunk or _default_chunk(K)
    dev = q.device
    o = out if out is not None else torch.empty((B, T, H, V), dtype=out_dtype, device=dev)
    if o.shape != (B, T, H, V):
        raise ValueError("out must be [B, T, H, V]")
    sT = final_state
    if sT is None and output_final_state:
        sT = torch.empty((B, H, K, V), dtype=torch.float32, device=dev)
    ws, nws = _workspace(dev, B, B * T, H, K, V, chunk, two_pass, workspace)
    _call("kda_chunk_fwd", prologue, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
          _ptr(initial_state), _ptr(o), _ptr(sT), B, T, H, K, V, chunk, _dtype_code(dt),
          _dtype_code(o.dtype), _ptr(ws), nws, _stream(dev))
    return o, sT


def varlen_fwd(q, k, v, g, beta, cu_seqlens, initial_state=None, output_final_state=True,
               chunk=None, out_dtype=torch.float32, final_state=None, out=None, two_pass=None,
               workspace=None, prologue=None):
    """Chunked KDA forward over packed sequences.

    q, k, g: [total_T, H, K]; v: [total_T, H, V]; beta: [total_T, H];
    cu_seqlens: int32 [N + 1] on the GPU.  initial_state: [N, H, K, V] float32 or None.
    Returns (o [total_T, H, V], final states [N, H, K, V] or None).
    two_pass, workspace, prologue: as for chunk_fwd.
    """
    _need_gpu(q, k, v, g, beta, cu_seqlens, initial_state, final_state, out)
    total, H, K = q.shape
    V = v.shape[-1]
    N = cu_seqlens.numel() - 1
    dt = q.dtype
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if any(x.dtype != dt for x in (k, v, g, beta)):
        raise ValueError("q, k, v, g and beta must share one dtype")
    if k.shape != q.shape or g.shape != q.shape or v.shape != (total, H, V) or beta.shape != (total, H):
        raise ValueError("shape mismatch among q, k, v, g, beta")
    for s in (initial_state, final_state):
        if s is not None and (s.dtype != torch.float32 or s.shape != (N, H, K, V)):
            raise ValueError("states must be float32 [N, H, K, V]")
    chunk = chunk or _default_chunk(K)
    dev = q.device
    o = out if out is not None else torch.empty((total, H, V), dtype=out_dtype, device=dev)
    if o.shape != (total, H, V):
        raise ValueError("out must be [total_T, H, V]")
    sT = final_state
    if sT is None and output_final_state:
        sT = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    ws, nws = _workspace(dev, N, total, H, K, V, chunk, two_pass, workspace)
    _call("kda_varlen_fwd", prologue, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
          _ptr(initial_state), _ptr(o), _ptr(sT), _ptr(cu_seqlens), N, total, H, K, V, chunk,
          _dtype_code(dt), _dtype_code(o.dtype), _ptr(ws), nws, _stream(dev))
    return o, sT


def varlen_fwd_noalloc(q, k, v, g, beta, cu_seqlens, initial_state=None, final_state=None,
                       out=None, chunk=None):
    """kda_varlen_fwd_noalloc: the two-pass packed forward with the library's
    static scratch instead of a workspace (no device allocation in the library;
    the outputs are the caller's when `out` / `final_state` are given, else
    allocated here by torch).  bf16 inputs, K = V = 128, at most 126 sequences
    and a two-pass workspace within the 80 MiB scratch.  Returns
    (o [total_T, H, V] float32, final states [N, H, K, V] or None)."""
    _need_gpu(q, k, v, g, beta, cu_seqlens, initial_state, final_state, out)
    total, H, K = q.shape
    V = v.shape[-1]
    N = cu_seqlens.numel() - 1
    dt = q.dtype
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if any(x.dtype != dt for x in (k, v, g, beta)):
        raise ValueError("q, k, v, g and beta must share one dtype")
    if k.shape != q.shape or g.shape != q.shape or v.shape != (total, H, V) or beta.shape != (total, H):
        raise ValueError("shape mismatch among q, k, v, g, beta")
    for s in (initial_state, final_state):
        if s is not None and (s.dtype != torch.float32 or s.shape != (N, H, K, V)):
            raise ValueError("states must be float32 [N, H, K, V]")
    chunk = chunk or _default_chunk(K)
    o = out if out is not None else torch.empty((total, H, V), dtype=torch.float32, device=q.device)
    if o.shape != (total, H, V):
        raise ValueError("out must be [total_T, H, V]")
    _call("kda_varlen_fwd_noalloc", None, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
          _ptr(initial_state), _ptr(o), _ptr(final_state), _ptr(cu_seqlens), N, total, H, K, V,
          chunk, _dtype_code(dt), _dtype_code(o.dtype), _stream(q.device))
    return o, final_state


def decode_step(q, k, v, g, beta, state, out_dtype=torch.float32, out=None, prologue=None):
    """One recurrent step: q, k, g [N, H, K]; v [N, H, V]; beta [N, H];
    state [N, H, K, V] float32, updated in place.  Returns o [N, H, V].
    prologue: as for chunk_fwd."""
    _need_gpu(q, k, v, g, beta, state, out)
    N, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    if any(x.dtype != dt for x in (k, v, g, beta)):
        raise ValueError("q, k, v, g and beta must share one dtype")
    if k.shape != q.shape or g.shape != q.shape or v.shape != (N, H, V) or beta.shape != (N, H):
        raise ValueError("shape mismatch among q, k, v, g, beta")
    if state.dtype != torch.float32 or state.shape != (N, H, K, V):
        raise ValueError("state must be float32 [N, H, K, V]")
    o = out if out is not None else torch.empty((N, H, V), dtype=out_dtype, device=q.device)
    _call("kda_decode_step", prologue, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
          _ptr(state), _ptr(o), N, H, K, V, _dtype_code(dt), _dtype_code(o.dtype),
          _stream(q.device))
    return o


def _slots(t, N, name):
    if t is None:
        return None
    if t.dtype != torch.int32 or t.shape != (N,):
        raise ValueError(f"{name} must be int32 [N]")
    return t


def _pool_check(pool, H, K, V):
    if pool.dtype != torch.float32 or pool.dim() != 4 or tuple(pool.shape[1:]) != (H, K, V):
        raise ValueError("pool must be float32 [slots, H, K, V]")
    return pool.shape[0]


def varlen_fwd_paged(q, k, v, g, beta, cu_seqlens, pool, s0_slot=None, sT_slot=None,
                     start_pos=None, block_table=None, snap_tokens=512, page_tokens=6144,
                     chunk=None, out_dtype=torch.float32, out=None, two_pass=None,
                     workspace=None, prologue=None):
    """kda_varlen_fwd_paged: packed sequences whose states live in a pool.

    pool: float32 [slots, H, K, V]; s0_slot, sT_slot, start_pos: int32 [N] or None;
    block_table: int32 [N, blocks] (physical page of each page_tokens block) or None
    for no snapshots.  Returns o [total_T, H, V]; states and snapshots land in pool.
    prologue: as for chunk_fwd.
    """
    _need_gpu(q, k, v, g, beta, cu_seqlens, pool, s0_slot, sT_slot, start_pos, block_table, out)
    total, H, K = q.shape
    V = v.shape[-1]
    N = cu_seqlens.numel() - 1
    dt = q.dtype
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if any(x.dtype != dt for x in (k, v, g, beta)):
        raise ValueError("q, k, v, g and beta must share one dtype")
    if k.shape != q.shape or g.shape != q.shape or v.shape != (total, H, V) or beta.shape != (total, H):
        raise ValueError("shape mismatch among q, k, v, g, beta")
    slots = _pool_check(pool, H, K, V)
    for t, name in ((s0_slot, "s0_slot"), (sT_slot, "sT_slot"), (start_pos, "start_pos")):
        _slots(t, N, name)
    stride = 0
    if block_table is not None:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != N:
            raise ValueError("block_table must be int32 [N, blocks]")
        stride = block_table.shape[1]
    chunk = chunk or _default_chunk(K)
    dev = q.device
    o = out if out is not None else torch.empty((total, H, V), dtype=out_dtype, device=dev)
    if o.shape != (total, H, V):
        raise ValueError("out must be [total_T, H, V]")
    ws, nws = _workspace(dev, N, total, H, K, V, chunk, two_pass, workspace)
    _call("kda_varlen_fwd_paged", prologue,
          _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(pool), slots, _ptr(s0_slot),
          _ptr(sT_slot), _ptr(start_pos), _ptr(block_table), stride, snap_tokens, page_tokens,
          _ptr(o), _ptr(cu_seqlens), N, total, H, K, V, chunk, _dtype_code(dt),
          _dtype_code(o.dtype), _ptr(ws), nws, _stream(dev))
    return o


def decode_step_paged(q, k, v, g, beta, pool, slot_in, slot_out, out_dtype=torch.float32,
                      out=None, prologue=None):
    """kda_decode_step_paged: one step for N sequences whose states live in a pool
    (float32 [slots, H, K, V]); sequence n reads slot_in[n] and writes slot_out[n]
    (int32 [N] each).  Returns o [N, H, V].  prologue: as for chunk_fwd."""
    _need_gpu(q, k, v, g, beta, pool, slot_in, slot_out, out)
    N, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    if any(x.dtype != dt for x in (k, v, g, beta)):
        raise ValueError("q, k, v, g and beta must share one dtype")
    if k.shape != q.shape or g.shape != q.shape or v.shape != (N, H, V) or beta.shape != (N, H):
        raise ValueError("shape mismatch among q, k, v, g, beta")
    slots = _pool_check(pool, H, K, V)
    _slots(slot_in, N, "slot_in")
    _slots(slot_out, N, "slot_out")
    o = out if out is not None else torch.empty((N, H, V), dtype=out_dtype, device=q.device)
    _call("kda_decode_step_paged", prologue, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
          _ptr(pool), slots, _ptr(slot_in), _ptr(slot_out), _ptr(o), N, H, K, V,
          _dtype_code(dt), _dtype_code(o.dtype), _stream(q.device))
    return o


def decode_multi_paged(q, k, v, g, beta, pool, slot_in, slot_out, out_dtype=torch.float32,
                       out=None, prologue=None):
    """kda_decode_multi_paged: T tokens per sequence in one pass (draft verification).
    q, k, g [N, T, H, K]; v [N, T, H, V]; beta [N, T, H]; pool float32 [slots, H, K, V];
    slot_in int32 [N]; slot_out int32 [N, T] (state after token j, -1: not kept).
    Returns o [N, T, H, V].  prologue: as for chunk_fwd."""
    _need_gpu(q, k, v, g, beta, pool, slot_in, slot_out, out)
    N, T, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    if any(x.dtype != dt for x in (k, v, g, beta)):
        raise ValueError("q, k, v, g and beta must share one dtype")
    if k.shape != q.shape or g.shape != q.shape or v.shape != (N, T, H, V) or beta.shape != (N, T, H):
        raise ValueError("shape mismatch among q, k, v, g, beta")
    slots = _pool_check(pool, H, K, V)
    _slots(slot_in, N, "slot_in")
    if slot_out.dtype != torch.int32 or slot_out.shape != (N, T):
        raise ValueError("slot_out must be int32 [N, T]")
    o = out if out is not None else torch.empty((N, T, H, V), dtype=out_dtype, device=q.device)
    _call("kda_decode_multi_paged", prologue, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
          _ptr(beta), _ptr(pool), slots, _ptr(slot_in), _ptr(slot_out), _ptr(o), N, T, H, K, V,
          _dtype_code(dt), _dtype_code(o.dtype), _stream(q.device))
    return o


def bwd_workspace_bytes(N: int, total_T: int, H: int, K: int, V: int, chunk: int) -> int:
    """Workspace bytes of a backward call (kda_bwd_workspace_bytes)."""
    return int(library().kda_bwd_workspace_bytes(N, total_T, H, K, V, chunk))


def _bwd_common(q, k, v, g, beta, do, N, total, initial_state, dsT, need_ds0, chunk, workspace):
    _need_gpu(q, k, v, g, beta, do, initial_state, dsT, workspace)
    H, K = q.shape[-2], q.shape[-1]
    V = v.shape[-1]
    dt = q.dtype
    if any(x.dtype != dt for x in (k, v, g, beta)):
        raise ValueError("q, k, v, g and beta must share one dtype")
    if do.dtype != torch.float32 or do.shape != v.shape:
        raise ValueError("do must be float32 with the shape of v")
    for s in (initial_state, dsT):
        if s is not None and (s.dtype != torch.float32 or s.shape != (N, H, K, V)):
            raise ValueError("states and their gradients must be float32 [N, H, K, V]")
    chunk = chunk or _default_chunk(K)
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    grads = (torch.empty(q.shape, **f32), torch.empty(k.shape, **f32), torch.empty(v.shape, **f32),
             torch.empty(g.shape, **f32), torch.empty(beta.shape, **f32))
    ds0 = torch.empty((N, H, K, V), **f32) if need_ds0 else None
    nbytes = bwd_workspace_bytes(N, total, H, K, V, chunk)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.numel() < nbytes:
        raise ValueError(f"workspace must be a uint8 tensor of at least {nbytes} bytes")
    return H, K, V, chunk, dt, grads, ds0, workspace


def chunk_bwd(q, k, v, g, beta, do, initial_state=None, dsT=None, chunk=None, need_ds0=True,
              workspace=None):
    """Gradients of sum(do * o) + sum(dsT * S_T) for the chunk_fwd call with the same
    inputs: returns (dq, dk, dv, dg, dbeta, ds0 or None), all float32.
    q, k, g: [B, T, H, K]; v, do: [B, T, H, V]; beta: [B, T, H]; states [B, H, K, V]."""
    B, T = q.shape[0], q.shape[1]
    H, K, V, chunk, dt, grads, ds0, ws = _bwd_common(q, k, v, g, beta, do, B, B * T,
                                                     initial_state, dsT, need_ds0, chunk,
                                                     workspace)
    _call("kda_chunk_bwd", None, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
          _ptr(initial_state), _ptr(do), _ptr(dsT), *(_ptr(x) for x in grads), _ptr(ds0),
          B, T, H, K, V, chunk, _dtype_code(dt), _ptr(ws), ws.numel(), _stream(q.device))
    return (*grads, ds0)


def varlen_bwd(q, k, v, g, beta, do, cu_seqlens, initial_state=None, dsT=None, chunk=None,
               need_ds0=True, workspace=None):
    """Gradients for the varlen_fwd call with the same inputs (packed sequences):
    returns (dq, dk, dv, dg, dbeta, ds0 or None), all float32."""
    _need_gpu(cu_seqlens)
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    N, total = cu_seqlens.numel() - 1, q.shape[0]
    H, K, V, chunk, dt, grads, ds0, ws = _bwd_common(q, k, v, g, beta, do, N, total,
                                                     initial_state, dsT, need_ds0, chunk,
                                                     workspace)
    _call("kda_varlen_bwd", None, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
          _ptr(initial_state), _ptr(do), _ptr(dsT), *(_ptr(x) for x in grads), _ptr(ds0),
          _ptr(cu_seqlens), N, total, H, K, V, chunk, _dtype_code(dt), _ptr(ws), ws.numel(),
          _stream(q.device))
    return (*grads, ds0)


class _KdaVarlen(torch.autograd.Function):
    """varlen_fwd with its gradients from varlen_bwd (both the library's
    kernels); outputs that the loss does not use contribute no gradient."""

    @staticmethod
    def forward(ctx, q, k, v, g, beta, cu_seqlens, initial_state, two_pass):
        o, sT = varlen_fwd(q, k, v, g, beta, cu_seqlens, initial_state, two_pass=two_pass)
        ctx.save_for_backward(q, k, v, g, beta, cu_seqlens, initial_state)
        ctx.set_materialize_grads(False)
        return o, sT

    @staticmethod
    def backward(ctx, do, dsT):
        q, k, v, g, beta, cu, s0 = ctx.saved_tensors
        if do is None:
            do = torch.zeros(v.shape, dtype=torch.float32, device=v.device)
        do = do.float().contiguous()
        dsT = dsT.float().contiguous() if dsT is not None else None
        dq, dk, dv, dg, db, ds0 = varlen_bwd(q, k, v, g, beta, do, cu, initial_state=s0,
                                             dsT=dsT, need_ds0=ctx.needs_input_grad[6])
        return (dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), dg.to(g.dtype),
                db.to(beta.dtype), None, ds0, None)


def kda_varlen(q, k, v, g, beta, cu_seqlens, initial_state=None, two_pass=None):
    """Differentiable packed KDA: (o [total_T, H, V] float32, S_T [N, H, K, V]
    float32), with gradients for q, k, v, g, beta (in their own dtype) and
    initial_state through torch autograd.  Arguments as for varlen_fwd; the
    gradients are those of varlen_bwd (fp32 arithmetic), so the decay
    precondition of the backward applies."""
    return _KdaVarlen.apply(q, k, v, g, beta, cu_seqlens, initial_state, two_pass)


def kda_chunk(q, k, v, g, beta, initial_state=None, two_pass=None):
    """kda_varlen over a fixed-length batch: q, k, g [B, T, H, K], v [B, T, H, V],
    beta [B, T, H]; returns (o [B, T, H, V], S_T [B, H, K, V])."""
    B, T, H = q.shape[0], q.shape[1], q.shape[2]
    cu = torch.arange(B + 1, dtype=torch.int32, device=q.device) * T
    flat = [x.reshape(B * T, *x.shape[2:]) for x in (q, k, v, g, beta)]
    o, sT = kda_varlen(*flat, cu, initial_state, two_pass)
    return o.view(B, T, H, v.shape[-1]), sT
