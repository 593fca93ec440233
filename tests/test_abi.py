"""The C-ABI library loads on the host, exports every declared symbol and
rejects bad arguments before touching the GPU (no compute calls here)."""

import ctypes
import os
import re

import pytest

from gated_delta_rule_43_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        from gated_delta_rule_43_amd import build
        build.build()
    return kda.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("kda_chunk_fwd", "kda_varlen_fwd", "kda_decode_step", "kda_varlen_fwd_paged",
              "kda_decode_step_paged", "kda_decode_multi_paged", "kda_workspace_bytes",
              "kda_two_pass_workspace_bytes", "kda_status_str", "kda_version",
              "kda_chunk_fwd_prologue", "kda_varlen_fwd_prologue",
              "kda_varlen_fwd_paged_prologue", "kda_decode_step_prologue",
              "kda_decode_step_paged_prologue", "kda_decode_multi_paged_prologue",
              "kda_chunk_bwd", "kda_varlen_bwd", "kda_bwd_workspace_bytes",
              "kda_varlen_fwd_noalloc"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    for code in range(8):
        s = lib.kda_status_str(code).decode()
        assert s.startswith("KDA_")
    assert lib.kda_status_str(7).decode().startswith("KDA_ERR_VALUE")
    assert lib.kda_status_str(99).decode() == "KDA_ERR_UNKNOWN"
    assert lib.kda_version() == 105


def two_pass_size(N, total, H):
    # one 131584-byte record per (chunk, head) for the packed-sequence chunk bound
    return -(-(total + 63 * N) // 64) * H * 131584


def test_workspace_sizes(lib):
    rec, two = lib.kda_workspace_bytes, lib.kda_two_pass_workspace_bytes
    # recommended: two-pass for few units and long sequences only
    assert rec(1, 4096, 8, 128, 128, 64) == two_pass_size(1, 4096, 8)
    assert rec(1, 4096, 24, 128, 128, 64) == two_pass_size(1, 4096, 24)
    assert rec(1, 4096, 25, 128, 128, 64) == 0
    assert rec(1, 1024, 32, 128, 128, 64) == two_pass_size(1, 1024, 32)
    assert rec(1, 1024, 33, 128, 128, 64) == 0
    assert rec(1, 1025, 32, 128, 128, 64) == 0
    assert rec(4, 32768, 32, 128, 128, 64) == 0
    assert rec(1, 256, 8, 128, 128, 64) == two_pass_size(1, 256, 8)
    assert rec(1, 255, 8, 128, 128, 64) == 0
    # supported whenever (K, V, chunk) = (128, 128, 64) and N < 127
    assert two(4, 32768, 32, 128, 128, 64) == two_pass_size(4, 32768, 32)
    assert two(2, 0, 3, 128, 128, 64) == two_pass_size(2, 0, 3)
    assert two(126, 1000, 1, 128, 128, 64) > 0
    assert two(127, 1000, 1, 128, 128, 64) == 0
    assert two(1, 64, 1, 32, 32, 16) == 0
    assert two(0, 0, 1, 128, 128, 64) == 0


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def chunk(lib, *, B=1, T=64, H=1, K=128, V=128, C=64, ind=1, outd=0, null=None, wsp=None, ws=0):
    ptrs = [FAKE] * 8
    if null is not None:
        ptrs[null] = None
    return lib.kda_chunk_fwd(*ptrs, B, T, H, K, V, C, ind, outd, wsp, ws, None)


def test_chunk_argument_errors(lib):
    assert chunk(lib, K=64, V=64) == 4                       # unsupported shape
    assert chunk(lib, K=128, V=128, C=16) == 4
    assert chunk(lib, K=32, V=32, C=64) == 4
    assert chunk(lib, ind=7) == 3                            # unknown dtype
    assert chunk(lib, outd=-1) == 3
    assert chunk(lib, B=-1) == 2
    assert chunk(lib, T=-5) == 2
    assert chunk(lib, H=0) == 2
    assert chunk(lib, T=1 << 22, H=64) == 2                   # > 2^31 elements
    for i in (0, 1, 2, 3, 4, 6):                              # q, k, v, g, beta, o
        assert chunk(lib, null=i) == 1
    need = two_pass_size(1, 64, 1)
    assert chunk(lib, wsp=None, ws=need) == 1                 # workspace size but no pointer
    assert chunk(lib, wsp=FAKE, ws=need - 1) == 5             # workspace too small
    assert chunk(lib, wsp=FAKE, ws=1, K=32, V=32, C=16, B=-1) == 2  # shape checked first


def test_varlen_argument_errors(lib):
    f = lib.kda_varlen_fwd
    assert f(*[FAKE] * 8, None, 2, 10, 1, 128, 128, 64, 1, 0, None, 0, None) == 1  # no cu
    assert f(*[FAKE] * 9, -1, 10, 1, 128, 128, 64, 1, 0, None, 0, None) == 2
    assert f(*[FAKE] * 9, 2, -10, 1, 128, 128, 64, 1, 0, None, 0, None) == 2
    assert f(*[FAKE] * 9, 2, 10, 1, 96, 128, 64, 1, 0, None, 0, None) == 4
    assert f(*[FAKE] * 9, 2, 10, 1, 128, 128, 64, 5, 0, None, 0, None) == 3


def test_noalloc_argument_errors(lib):
    """kda_varlen_fwd_noalloc rejects, before any HIP call, what its static
    scratch cannot serve: other than bf16 / (128, 128, 64) / N < 127, or a
    two-pass workspace above KDA_NOALLOC_SCRATCH_BYTES (80 MiB)."""
    f = lib.kda_varlen_fwd_noalloc
    assert f(*[FAKE] * 8, None, 2, 10, 1, 128, 128, 64, 1, 0, None) == 1       # no cu_seqlens
    assert f(*[FAKE] * 9, 0, 0, 1, 128, 128, 64, 1, 0, None) == 0              # nothing to do
    assert f(*[FAKE] * 9, 2, 10, 1, 128, 128, 64, 0, 0, None) == 4             # fp32 inputs
    assert f(*[FAKE] * 9, 2, 10, 1, 32, 32, 16, 1, 0, None) == 4               # d = 32
    assert f(*[FAKE] * 9, 127, 1000, 1, 128, 128, 64, 1, 0, None) == 4         # N > 126
    limit = 80 << 20
    assert two_pass_size(1, 4096, 8) <= limit < two_pass_size(1, 4096 * 2, 8)
    assert f(*[FAKE] * 9, 1, 8192, 8, 128, 128, 64, 1, 0, None) == 5          # above the scratch
    assert f(*[FAKE] * 9, 2, 10, 1, 128, 128, 64, 1, 9, None) == 3             # bad out dtype
    for i in (0, 1, 2, 3, 4, 6):
        ptrs = [FAKE] * 9
        ptrs[i] = None
        assert f(*ptrs, 1, 10, 1, 128, 128, 64, 1, 0, None) == 1


def test_decode_argument_errors(lib):
    f = lib.kda_decode_step
    assert f(*[FAKE] * 7, 4, 2, 64, 64, 1, 0, None) == 4
    assert f(*[FAKE] * 7, -1, 2, 128, 128, 1, 0, None) == 2
    assert f(*[FAKE] * 7, 4, 0, 128, 128, 1, 0, None) == 2
    assert f(*[FAKE] * 7, 4, 2, 128, 128, 2, 0, None) == 3
    for i in range(7):
        ptrs = [FAKE] * 7
        ptrs[i] = None
        assert f(*ptrs, 4, 2, 128, 128, 1, 0, None) == 1


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 32)
    with pytest.raises(ValueError):
        kda.chunk_fwd(x, x, x, x, torch.zeros(1, 4, 1))


def paged_fwd(lib, *, pool=FAKE, slots=4, table=None, stride=0, snap=512, page=6144, N=2, T=10,
              H=1, K=128, V=128, C=64, cu=FAKE, null=None):
    ptrs = [FAKE] * 5
    if null is not None:
        ptrs[null] = None
    return lib.kda_varlen_fwd_paged(*ptrs, pool, slots, None, None, None, table, stride, snap,
                                    page, FAKE, cu, N, T, H, K, V, C, 1, 0, None, 0, None)


def test_paged_fwd_argument_errors(lib):
    assert paged_fwd(lib, pool=None) == 1                     # no pool
    assert paged_fwd(lib, slots=0) == 2                       # empty pool
    assert paged_fwd(lib, cu=None) == 1
    assert paged_fwd(lib, K=96) == 4
    for i in range(5):
        assert paged_fwd(lib, null=i) == 1
    # snapshot schedule: only checked when a block table is given
    assert paged_fwd(lib, table=FAKE, stride=0) == 2
    assert paged_fwd(lib, table=FAKE, stride=4, snap=100) == 2     # not a multiple of chunk
    assert paged_fwd(lib, table=FAKE, stride=4, snap=0) == 2
    assert paged_fwd(lib, table=FAKE, stride=4, page=1000) == 2    # not a multiple of snap
    assert paged_fwd(lib, table=FAKE, stride=4, page=0) == 2


def test_paged_decode_argument_errors(lib):
    f = lib.kda_decode_step_paged

    def call(null=None, slots=8, N=4, K=128):
        ptrs = [FAKE] * 10   # q, k, v, g, beta, pool, (slots), slot_in, slot_out, o
        if null is not None:
            ptrs[null] = None
        return f(*ptrs[:6], slots, *ptrs[6:9], N, 2, K, K, 1, 0, None)

    assert call(K=64) == 4
    assert call(slots=0) == 2
    assert call(N=-1) == 2
    for i in range(9):
        assert call(null=i) == 1


def test_multi_decode_argument_errors(lib):
    f = lib.kda_decode_multi_paged

    def call(null=None, slots=8, N=4, T=3, K=128):
        ptrs = [FAKE] * 9   # q, k, v, g, beta, pool, slot_in, slot_out, o
        if null is not None:
            ptrs[null] = None
        return f(*ptrs[:6], slots, *ptrs[6:9], N, T, 2, K, K, 1, 0, None)

    assert call(K=64) == 4
    assert call(slots=0) == 2
    assert call(T=-1) == 2
    assert call(N=-1) == 2
    assert call(T=0, null=0) == 0       # nothing to do: no pointer is needed
    for i in range(9):
        assert call(null=i) == 1


def pro_args(flags, glb=0.25, eps=0.0):
    return ctypes.c_uint(flags), ctypes.c_float(glb), ctypes.c_float(eps)


def chunk_pro(lib, flags, glb=0.25, eps=0.0, *, C=64, K=128, ind=1, B=1, ws=0):
    # ws = 1: an undersized workspace, the check that follows the prologue's
    # (so a call whose prologue is accepted still fails, with KDA_ERR_WORKSPACE)
    return lib.kda_chunk_fwd_prologue(*[FAKE] * 8, B, 64, 1, K, K, C, ind, 0,
                                      FAKE if ws else None, ws, *pro_args(flags, glb, eps), None)


def test_prologue_argument_errors(lib):
    nan, inf = float("nan"), float("inf")
    assert chunk_pro(lib, 8) == 7                             # unknown flag bit
    assert chunk_pro(lib, 1 << 31) == 7
    assert chunk_pro(lib, 1, eps=-1e-6) == 7                  # negative eps
    assert chunk_pro(lib, 1, eps=nan) == 7
    assert chunk_pro(lib, 0, eps=inf) == 7
    assert chunk_pro(lib, 2, glb=-0.1) == 7                   # negative gate bound
    assert chunk_pro(lib, 2, glb=nan) == 7
    # bf16 inputs: a bound past the fp16 decay factors' range (g_lb * chunk > 16)
    # is accepted (the call runs the exact-decay kernel); the undersized
    # workspace checked after the prologue is what fails here
    assert chunk_pro(lib, 2, glb=0.26, ws=1) == 5
    assert chunk_pro(lib, 2, glb=2.0, ws=1) == 5
    assert chunk_pro(lib, 2, glb=2.0, ind=0, ws=1) == 5       # fp32 inputs: any finite bound
    assert chunk_pro(lib, 5, glb=100.0, ws=1) == 5            # bound unused without the gate map
    assert chunk_pro(lib, 7, glb=0.25, eps=1e-6, ws=1) == 5   # the largest bf16 bound at chunk 64
    assert chunk_pro(lib, 7, B=-1) == 2                       # shapes are checked first
    v = lib.kda_varlen_fwd_prologue
    assert v(*[FAKE] * 9, 2, 10, 1, 128, 128, 64, 1, 0, None, 0, *pro_args(16), None) == 7
    vp = lib.kda_varlen_fwd_paged_prologue
    assert vp(*[FAKE] * 6, 4, None, None, None, None, 0, 512, 6144, FAKE, FAKE, 2, 10, 1,
              128, 128, 64, 1, 0, None, 0, *pro_args(2, glb=-0.5), None) == 7
    assert vp(*[FAKE] * 6, 4, None, None, None, None, 0, 512, 6144, FAKE, FAKE, 2, 10, 1,
              128, 128, 64, 1, 0, FAKE, 1, *pro_args(2, glb=0.5), None) == 5
    d = lib.kda_decode_step_prologue
    assert d(*[FAKE] * 7, 4, 2, 128, 128, 1, 0, *pro_args(2, glb=-1.0), None) == 7
    assert d(*[FAKE] * 7, 4, 2, 128, 128, 1, 0, *pro_args(64), None) == 7
    dp = lib.kda_decode_step_paged_prologue
    assert dp(*[FAKE] * 6, 8, FAKE, FAKE, FAKE, 4, 2, 128, 128, 1, 0,
              *pro_args(1, eps=-1.0), None) == 7
    dm = lib.kda_decode_multi_paged_prologue
    assert dm(*[FAKE] * 6, 8, FAKE, FAKE, FAKE, 4, 3, 2, 128, 128, 1, 0,
              *pro_args(9), None) == 7
    # decode has no chunk: a large gate bound is accepted (N = 0: nothing to launch)
    assert d(*[FAKE] * 7, 0, 2, 128, 128, 1, 0, *pro_args(2, glb=5.0), None) == 0


def test_binding_prologue_flags():
    assert kda.Prologue().flags() == 0
    assert kda.Prologue(normalize_qk=True).flags() == 1
    assert kda.Prologue(gate_lower_bound=0.25).flags() == 2
    assert kda.Prologue(beta_logits=True).flags() == 4
    assert kda.Prologue(True, 0.25, True, 1e-6).flags() == 7


def test_backward_argument_errors(lib):
    need = lib.kda_bwd_workspace_bytes(1, 64, 1, 128, 128, 64)
    # bytes per (chunk, head): the record (Kp, Km, Qp, E, Gk, P, T, beta, F, exp(G_m), MM, NN,
    # NB, MM and MM^T as MFMA fragments), start state and end-state gradient, U and dY,
    # per-16-column partial sums
    rec = lambda C, K: 4 * (4 * C * K + 3 * C * C + C + 2 * K + 5 * K * K)
    extra = lambda C, K: 4 * (2 * K * K + 2 * C * K + (K // 16) * (C + K))
    assert need == 1 * 1 * (rec(64, 128) + extra(64, 128))
    assert lib.kda_bwd_workspace_bytes(1, 64, 1, 64, 64, 64) == 0        # unsupported
    assert lib.kda_bwd_workspace_bytes(3, 100, 2, 32, 32, 16) == \
        ((100 + 15 * 3) // 16) * 2 * (rec(16, 32) + extra(16, 32))
    f = lib.kda_chunk_bwd

    def call(B=1, T=64, H=1, K=128, C=64, ind=1, null=None, ws=FAKE, nws=None):
        ptrs = [FAKE] * 14
        if null is not None:
            ptrs[null] = None
        return f(*ptrs, B, T, H, K, K, C, ind, ws, need if nws is None else nws, None)

    assert call(K=64, C=64) == 4
    assert call(ind=3) == 3
    assert call(B=-1) == 2
    assert call(H=0) == 2
    for i in (0, 1, 2, 3, 4, 6, 8, 9, 10, 11, 12):       # inputs, do, the five gradients
        assert call(null=i) == 1
    assert call(ws=None) == 1                              # workspace required
    assert call(nws=need - 1) == 5
    v = lib.kda_varlen_bwd
    assert v(*[FAKE] * 14, None, 2, 10, 1, 128, 128, 64, 1, FAKE, 1 << 30, None) == 1  # no cu
    assert v(*[FAKE] * 15, 2, 10, 1, 128, 128, 64, 1, FAKE, 10, None) == 5
