"""Pins of the oracle's input prologue (oracle.prologue) to values fixed by
mathematics, and a check that each pin has teeth.

Reading under test ("Kimi K3: Open Frontier Intelligence and Implementation
Framework", section "Hybrid Attention Mechanism": a channel-wise gate with a
lower-bounded decay; the parameterisation taken here): g = -g_lb sigmoid(x)
from gate logits x, beta = sigmoid(b) from beta logits b, and q, k scaled to
unit L2 norm per (token, head) as x (sum x^2 + eps)^-1/2.

The pins use values whose results are known in closed form: sigmoid(0) = 1/2,
sigmoid(+-ln 3) = 3/4 and 1/4, the limits at +-inf, the 3-4-5 triangle, and
end-to-end cases in which the recurrence itself reduces to a closed form
(beta = 0: pure decay of the initial state).
"""

import inspect
import math

import numpy as np
import pytest

from oracle import oracle

LN3 = math.log(3.0)
LOGITS = np.array([0.0, LN3, -LN3, -np.inf, np.inf])


def _ones(shape):
    return np.ones(shape)


def pin_gate_values(pf):
    """g = -g_lb sigmoid(x) at logits with exact sigmoids."""
    x = LOGITS.reshape(1, 1, 5)
    _, _, g, _ = pf(_ones((1, 1, 5)), _ones((1, 1, 5)), x, _ones((1, 1)), gate_lower_bound=0.5)
    np.testing.assert_allclose(g.ravel(), [-0.25, -0.375, -0.125, 0.0, -0.5], rtol=0, atol=1e-15)


def pin_beta_values(pf):
    """beta = sigmoid(b) at logits with exact sigmoids."""
    b = LOGITS.reshape(5, 1)
    _, _, _, beta = pf(_ones((5, 1, 2)), _ones((5, 1, 2)), _ones((5, 1, 2)), b, beta_logits=True)
    np.testing.assert_allclose(beta.ravel(), [0.5, 0.75, 0.25, 0.0, 1.0], rtol=0, atol=1e-15)


def pin_norm_hand_values(pf):
    """3-4-5 rows, per (token, head): two heads of different norms, a zero row,
    and the eps term (3, 4) / sqrt(25 + 11) = (1/2, 2/3)."""
    q = np.array([[[3.0, 4.0], [0.0, 0.5]], [[0.0, 0.0], [-6.0, 8.0]]])   # [T=2, H=2, K=2]
    k = np.array([[[0.0, 5.0], [12.0, 5.0]], [[1.0, 0.0], [0.0, 0.0]]])
    qn, kn, _, _ = pf(q, k, _ones((2, 2, 2)), _ones((2, 2)), normalize_qk=True)
    np.testing.assert_allclose(qn, [[[0.6, 0.8], [0.0, 1.0]], [[0.0, 0.0], [-0.6, 0.8]]],
                               rtol=0, atol=1e-15)
    np.testing.assert_allclose(kn, [[[0.0, 1.0], [12 / 13, 5 / 13]], [[1.0, 0.0], [0.0, 0.0]]],
                               rtol=0, atol=1e-15)
    qe, _, _, _ = pf(q[:1, :1], k[:1, :1], _ones((1, 1, 2)), _ones((1, 1)), normalize_qk=True,
                     norm_eps=11.0)
    np.testing.assert_allclose(qe.ravel(), [0.5, 2 / 3], rtol=0, atol=1e-15)


def pin_identity_when_off(pf):
    """With no map selected the inputs pass through unchanged."""
    rng = np.random.default_rng(5)
    xs = [rng.standard_normal(s) for s in ((3, 2, 4), (3, 2, 4), (3, 2, 4), (3, 2))]
    for a, b in zip(pf(*xs), xs):
        assert np.array_equal(a, b)


def pin_end_to_end_pure_decay(pf):
    """beta logits -inf give beta = 0, so the state only decays: with gate logits
    ln 3 and g_lb = 0.4 every step has g = -0.3 on every channel, and with raw
    queries c_t e_{pi(t)} (c_t a power of two) the normalised query is e_{pi(t)},
    so o_t = exp(-0.3 t) S_0[pi(t), :] and S_T = exp(-0.3 T) S_0."""
    T, H, K, V = 6, 2, 4, 3
    rng = np.random.default_rng(11)
    s0 = rng.standard_normal((1, H, K, V))
    pi = np.array([[2, 0], [1, 3], [3, 3], [0, 1], [2, 2], [1, 0]])
    q = np.zeros((T, H, K))
    for t in range(T):
        for h in range(H):
            q[t, h, pi[t, h]] = 2.0 ** (t - h - 2)
    k = rng.standard_normal((T, H, K)) * 3.0
    v = rng.standard_normal((T, H, V))
    x = np.full((T, H, K), LN3)
    b = np.full((T, H), -np.inf)
    qn, kn, g, beta = pf(q, k, x, b, normalize_qk=True, gate_lower_bound=0.4, beta_logits=True)
    o, sT = oracle.recurrence(qn, kn, v, g, beta, [0, T], s0=s0, nthreads=1)
    for t in range(T):
        for h in range(H):
            np.testing.assert_allclose(o[t, h], math.exp(-0.3 * (t + 1)) * s0[0, h, pi[t, h]],
                                       rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(sT, math.exp(-0.3 * T) * s0, rtol=1e-13, atol=0)


def pin_scale_invariance(pf):
    """Raw q and k rows scaled by powers of two (exact in binary) give the same
    result through the prologue and the recurrence."""
    T, H, K, V = 9, 2, 8, 4
    rng = np.random.default_rng(12)
    q, k = rng.standard_normal((T, H, K)), rng.standard_normal((T, H, K))
    v, x, b = rng.standard_normal((T, H, V)), rng.standard_normal((T, H, K)), rng.standard_normal((T, H))
    c = 2.0 ** rng.integers(-6, 7, size=(T, H, 1))
    d = 2.0 ** rng.integers(-6, 7, size=(T, H, 1))
    kw = dict(normalize_qk=True, gate_lower_bound=0.25, beta_logits=True)
    r1 = oracle.recurrence(*pf(q, k, x, b, **kw)[:2], v, *pf(q, k, x, b, **kw)[2:], [0, T],
                           nthreads=1)
    a = pf(q * c, k * d, x, b, **kw)
    r2 = oracle.recurrence(a[0], a[1], v, a[2], a[3], [0, T], nthreads=1)
    np.testing.assert_allclose(r2[0], r1[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(r2[1], r1[1], rtol=0, atol=1e-14)


PINS = [pin_gate_values, pin_beta_values, pin_norm_hand_values, pin_identity_when_off,
        pin_end_to_end_pure_decay, pin_scale_invariance]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_prologue_pin(pin):
    pin(oracle.prologue)


# (name, original fragment of oracle.prologue, replacement): plausible slips
MUTANTS = [
    ("gate_sigmoid_sign", "g = -float(gate_lower_bound) / (1.0 + np.exp(-g))",
     "g = -float(gate_lower_bound) / (1.0 + np.exp(g))"),
    ("gate_bound_dropped", "g = -float(gate_lower_bound) / (1.0 + np.exp(-g))",
     "g = -1.0 / (1.0 + np.exp(-g))"),
    ("gate_not_negated", "g = -float(gate_lower_bound) / (1.0 + np.exp(-g))",
     "g = float(gate_lower_bound) / (1.0 + np.exp(-g))"),
    ("beta_sigmoid_sign", "beta = 1.0 / (1.0 + np.exp(-beta))", "beta = 1.0 / (1.0 + np.exp(beta))"),
    ("beta_map_skipped", "beta = 1.0 / (1.0 + np.exp(-beta))", "beta = beta"),
    ("norm_over_heads", "s = np.sum(x * x, axis=-1, keepdims=True) + norm_eps",
     "s = np.sum(x * x, axis=-2, keepdims=True) + norm_eps"),
    ("norm_eps_dropped", "s = np.sum(x * x, axis=-1, keepdims=True) + norm_eps",
     "s = np.sum(x * x, axis=-1, keepdims=True)"),
    ("norm_not_sqrt", "return np.where(s > 0.0, x / np.sqrt(safe), 0.0)",
     "return np.where(s > 0.0, x / safe, 0.0)"),
    ("k_not_normalised", "q, k = unit(q), unit(k)", "q, k = unit(q), k"),
]


def _mutant(old, new):
    src = inspect.getsource(oracle.prologue)
    assert src.count(old) == 1, old
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["prologue"]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_prologue_mutant_fails_a_pin(name, old, new):
    pf = _mutant(old, new)
    failed = []
    for pin in PINS:
        try:
            pin(pf)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every prologue pin"
