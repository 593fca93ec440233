"""Seeded combinational sweep of the forward entry points against the oracle.

The other GPU tests vary one property at a time (length, head count, path,
output type, prologue map); here each case draws all of them together from
its own seed, so that combinations no single test names are still compared
element by element with the sequential fp64 recurrence: implementation
(two-pass, single-pass or the library's choice for bf16 d = 128; the fp32 and
d = 32 kernels), packed lengths mixing chunk-edge values and zeros with
random ones, head count, initial state or none, fp32 or bf16 output, and the
input prologue with a random subset of its maps.  Bounds as everywhere:
max|err| / RMS(ref) <= 1e-4 (fp32 inputs) or 2e-2 (bf16 inputs), a bf16
output allowed its own rounding on top.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_43_amd import inputs, kda
from oracle import oracle
from tests.parity import TOL, rel_err, rel_err_rounded, report, to_gpu

pytestmark = pytest.mark.gpu

G_LB = 0.25  # decay bound of the draws and of the gate map (the bf16 kernels' at chunk 64)
CASES = 40


def _case(seed):
    rng = np.random.default_rng(9000 + seed)
    kind = rng.choice(["bf16-128", "bf16-128", "bf16-128", "bf16-128", "bf16-32", "f32-32",
                       "f32-128"])
    dtype, K = kind.split("-")
    K = int(K)
    C = 64 if K == 128 else 16
    N = int(rng.integers(1, 10))
    edge = [0, 1, C - 1, C, C + 1, 2 * C + 3, 5 * C]
    lengths = [int(rng.choice(edge)) if rng.random() < 0.4 else int(rng.integers(0, 600 if K == 128 else 200))
               for _ in range(N)]
    if dtype == "f32" and K == 128:
        lengths = [min(x, 200) for x in lengths]
    H = int(rng.choice([1, 2, 3, 5]))
    two_pass = None
    if kind == "bf16-128":
        two_pass = [None, True, False][int(rng.integers(0, 3))]
    s0 = bool(rng.random() < 0.6)
    out_bf16 = bool(rng.random() < 0.3)
    flags = int(rng.integers(1, 8)) if rng.random() < 0.4 else 0
    return dict(dtype=dtype, K=K, lengths=lengths, H=H, two_pass=two_pass, s0=s0,
                out_bf16=out_bf16, flags=flags)


@pytest.mark.parametrize("seed", range(CASES))
def test_forward_sweep(seed):
    c = _case(seed)
    print(f"[case] sweep seed={seed} {c}", flush=True)
    dtype, K, H = c["dtype"], c["K"], c["H"]
    s0_std = 0.1 if c["s0"] else None
    p = None
    if c["flags"]:
        f = c["flags"]
        raw = inputs.draw_raw_varlen(500 + seed, H, K, K, dtype, c["lengths"], s0_std=s0_std)
        plain = inputs.draw_varlen(700 + seed, H, K, K, dtype, lengths=c["lengths"], g_lb=G_LB)
        d = dict(raw)
        if not f & 1:
            d["q"], d["k"] = plain["q"], plain["k"]
        if not f & 2:
            d["g"] = plain["g"]
        if not f & 4:
            d["beta"] = plain["beta"]
        p = kda.Prologue(normalize_qk=bool(f & 1), gate_lower_bound=G_LB if f & 2 else None,
                         beta_logits=bool(f & 4), norm_eps=1e-6 if f & 1 else 0.0)
        q, k, g, b = oracle.prologue(d["q"], d["k"], d["g"], d["beta"],
                                     normalize_qk=p.normalize_qk,
                                     gate_lower_bound=p.gate_lower_bound,
                                     beta_logits=p.beta_logits, norm_eps=p.norm_eps)
        ref_in = (q, k, oracle.as_f64(d["v"]), g, b)
    else:
        d = inputs.draw_varlen(500 + seed, H, K, K, dtype, lengths=c["lengths"], s0_std=s0_std,
                               g_lb=G_LB)
        ref_in = tuple(d[x] for x in ("q", "k", "v", "g", "beta"))
    cu = d["cu_seqlens"].numpy().astype(np.int64)
    s0_ref = oracle.as_f64(d["s0"]) if d["s0"] is not None else None
    o_ref, s_ref = oracle.recurrence(*ref_in, cu, s0_ref)
    x = to_gpu(d)
    out_dtype = torch.bfloat16 if c["out_bf16"] else torch.float32
    o, sT = kda.varlen_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"], x["s0"],
                           out_dtype=out_dtype, two_pass=c["two_pass"], prologue=p)
    torch.cuda.synchronize()
    eo = rel_err_rounded(o, o_ref, 2.0 ** -8) if c["out_bf16"] else rel_err(o, o_ref)
    es = rel_err(sT, s_ref)
    report(f"sweep_{seed}", o=eo, sT=es)
    assert eo <= TOL[dtype] and es <= TOL[dtype]
