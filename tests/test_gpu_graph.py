"""The entry points under HIP graph capture.

The library allocates nothing, issues no memset or copy and launches only its
own kernels on the caller's stream, so a caller may capture its calls into a
graph (torch.cuda.graph records them on its capture stream) and replay them:
a serving loop's decode steps, or a prefill with a preallocated workspace or
the allocation-free entry point.  Each graph is replayed several times, with
eager work, input changes and synchronisations between the replays, and every
replay must give the same bits as the same calls made eagerly on the same
inputs (the kernels are deterministic).
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_43_amd import inputs, kda
from tests.parity import to_gpu

pytestmark = pytest.mark.gpu


def _eager_work():
    # unrelated device work and a host synchronisation between replays
    x = torch.randn(1 << 20, device="cuda")
    (x * x).sum().item()
    torch.cuda.synchronize()


def test_graph_decode_steps():
    N, H, K, steps = 32, 8, 128, 4
    print(f"[case] graph: {steps} decode steps N={N} H={H} K={K}", flush=True)
    s_init = inputs.draw_decode_state(31, N, H, K, K, 0.1).cuda()
    xs = [to_gpu(inputs.draw_decode_step(32, t, N, H, K, K, "bf16")) for t in range(steps)]
    # eager reference (also loads the library and sets kernel attributes
    # before any capture)
    s_ref = s_init.clone()
    o_ref = [kda.decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], s_ref) for x in xs]
    torch.cuda.synchronize()
    state = s_init.clone()
    outs = [torch.empty(N, H, K, device="cuda") for _ in range(steps)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for x, o in zip(xs, outs):
            kda.decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state, out=o)
    for rep in range(3):
        state.copy_(s_init)
        for o in outs:
            o.fill_(float("nan"))
        _eager_work()
        g.replay()
        torch.cuda.synchronize()
        for t in range(steps):
            assert torch.equal(outs[t], o_ref[t]), (rep, t)
        assert torch.equal(state, s_ref), rep


def test_graph_prefill_paths():
    B, T, H = 1, 1000, 4
    lengths = [400, 0, 65, 300, 1]
    print(f"[case] graph: two-pass and single-pass chunk_fwd B={B} T={T} H={H}, "
          f"noalloc varlen {lengths}", flush=True)
    draws = [inputs.draw_fixed(40 + r, B, T, H, 128, 128, "bf16", s0_std=0.1) for r in range(3)]
    vdraws = [inputs.draw_varlen(50 + r, H, 128, 128, "bf16", lengths=lengths, s0_std=0.1)
              for r in range(3)]
    x = to_gpu(draws[0])
    y = to_gpu(vdraws[0])
    ws = torch.empty(kda.two_pass_workspace_bytes(B, B * T, H, 128, 128, 64), dtype=torch.uint8,
                     device="cuda")
    N = len(lengths)
    o2, s2 = torch.empty(B, T, H, 128, device="cuda"), torch.empty(B, H, 128, 128, device="cuda")
    o1, s1 = torch.empty_like(o2), torch.empty_like(s2)
    on, sn = torch.empty(sum(lengths), H, 128, device="cuda"), torch.empty(N, H, 128, 128, device="cuda")

    def calls():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], final_state=s2, out=o2,
                      two_pass=True, workspace=ws)
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], final_state=s1, out=o1,
                      two_pass=False)
        kda.varlen_fwd_noalloc(y["q"], y["k"], y["v"], y["g"], y["beta"], y["cu_seqlens"],
                               y["s0"], final_state=sn, out=on)

    calls()  # eager first: library loaded, kernel attributes and the scratch address set
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(3):
        # new inputs into the captured buffers, the eager reference on them
        for key in ("q", "k", "v", "g", "beta", "s0"):
            x[key].copy_(draws[rep][key].cuda())
            y[key].copy_(vdraws[rep][key].cuda())
        calls()
        torch.cuda.synchronize()
        ref = [t.clone() for t in (o2, s2, o1, s1, on, sn)]
        for t in (o2, s2, o1, s1, on, sn):
            t.fill_(float("nan"))
        _eager_work()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip((o2, s2, o1, s1, on, sn), ref)):
            assert torch.equal(t, r), (rep, i)
        # the outputs are those of the current inputs, not of the captured ones
        if rep > 0:
            assert not torch.equal(o2, first_o2)
        else:
            first_o2 = o2.clone()
