"""kda_varlen_fwd_noalloc (the two-pass packed forward on the library's static
scratch, for callers that cannot allocate) against kda_varlen_fwd with a
caller-allocated two-pass workspace: the same kernels on the same inputs give
the same bits.  Two calls in a row, the second smaller than the first, so that
the second runs over scratch the first left behind; both are also checked
against the fp64 oracle."""

import numpy as np
import pytest
import torch

from gated_delta_rule_43_amd import inputs, kda
from oracle import oracle
from tests.parity import TOL, rel_err, report, to_gpu

pytestmark = pytest.mark.gpu


def _case(seed, lengths, H):
    d = inputs.draw_varlen(seed, H=H, K=128, V=128, dtype="bf16", lengths=lengths, s0_std=0.1)
    x = to_gpu(d)
    N, total = len(lengths), int(np.sum(lengths))
    assert kda.two_pass_workspace_bytes(N, total, H, 128, 128, 64) <= 80 << 20
    o_ref, s_ref = kda.varlen_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"],
                                  x["s0"], two_pass=True)
    sT = torch.full_like(s_ref, float("nan"))
    o = torch.full_like(o_ref, float("nan"))
    kda.varlen_fwd_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"], x["s0"],
                           final_state=sT, out=o)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(sT, s_ref)
    ob, sb = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"],
                               d["cu_seqlens"].numpy(), oracle.as_f64(d["s0"]))
    eo, es = rel_err(o, ob), rel_err(sT, sb)
    report(f"noalloc N={N} H={H} total={total}", o=eo, sT=es)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_noalloc_matches_workspace_path_twice():
    print("[case] noalloc: two calls, the second smaller", flush=True)
    _case(120, [700, 64, 1, 333, 0, 1500], 4)
    _case(121, [65, 200, 3], 2)
