"""Seeded generators: determinism and the stated distributions."""

import numpy as np
import torch

from gated_delta_rule_43_amd import inputs


def test_fixed_is_deterministic_and_shaped():
    a = inputs.draw_fixed(7, B=2, T=33, H=3, K=16, V=8, dtype="bf16", s0_std=0.1)
    b = inputs.draw_fixed(7, B=2, T=33, H=3, K=16, V=8, dtype="bf16", s0_std=0.1)
    c = inputs.draw_fixed(8, B=2, T=33, H=3, K=16, V=8, dtype="bf16", s0_std=0.1)
    for key in ("q", "k", "v", "g", "beta", "s0"):
        assert torch.equal(a[key], b[key])
        assert not torch.equal(a[key], c[key])
    assert a["q"].shape == (2, 33, 3, 16) and a["v"].shape == (2, 33, 3, 8)
    assert a["beta"].shape == (2, 33, 3) and a["s0"].shape == (2, 3, 16, 8)
    assert a["q"].dtype == torch.bfloat16 and a["s0"].dtype == torch.float32


def test_distributions():
    d = inputs.draw_fixed(3, B=1, T=512, H=4, K=128, V=128, dtype="f32")
    for key in ("q", "k"):
        n = d[key].double().norm(dim=-1)
        assert torch.allclose(n, torch.ones_like(n), atol=1e-5)
    assert float(d["g"].max()) <= 0.0 and float(d["g"].min()) >= -0.25
    assert float(d["beta"].min()) > 0.0 and float(d["beta"].max()) < 1.0
    assert abs(float(d["v"].std()) - 1.0) < 0.02
    b = inputs.draw_fixed(3, B=1, T=512, H=4, K=128, V=128, dtype="bf16")
    # bf16 values are the fp32 values rounded once
    assert torch.equal(b["v"], d["v"].to(torch.bfloat16))


def test_stress_gate_modes():
    z = inputs.draw_fixed(1, 1, 8, 1, 4, 4, "f32", g_mode="zero")
    assert float(z["g"].abs().max()) == 0.0
    bnd = inputs.draw_fixed(1, 1, 8, 1, 4, 4, "f32", g_lb=2.0, g_mode="bound")
    assert torch.all(bnd["g"] == -2.0)


def test_varlen_lengths_and_offsets():
    d = inputs.draw_varlen(3, H=2, K=8, V=8, dtype="bf16", N=64, len_min=16, len_max=32768)
    L = d["lengths"]
    assert len(L) == 64 and L.min() >= 16 and L.max() <= 32768
    cu = d["cu_seqlens"].numpy()
    assert cu[0] == 0 and np.all(np.diff(cu) == L) and cu[-1] == d["q"].shape[0]
    assert d["cu_seqlens"].dtype == torch.int32


def test_decode_steps_are_fresh_and_reproducible():
    a = inputs.draw_decode_step(4, 0, N=8, H=2, K=16, V=16, dtype="bf16")
    b = inputs.draw_decode_step(4, 1, N=8, H=2, K=16, V=16, dtype="bf16")
    c = inputs.draw_decode_step(4, 0, N=8, H=2, K=16, V=16, dtype="bf16")
    assert not torch.equal(a["q"], b["q"]) and torch.equal(a["q"], c["q"])
    s = inputs.draw_decode_state(4, 8, 2, 16, 16, 0.1)
    assert s.shape == (8, 2, 16, 16) and abs(float(s.std()) - 0.1) < 0.01
