"""Pins of the oracle's gradients (oracle.backward) to facts fixed by
mathematics, independent of the autograd they use, and a check that each pin
has teeth.

The loss is L = sum(do * o) + sum(dsT * S_T) for the recurrence of "Kimi K3:
Open Frontier Intelligence and Implementation Framework", section "Hybrid
Attention Mechanism" (delta rule with a channel-wise forget gate).  Pins:
  * central finite differences of the separately written C forward oracle
    (kda_oracle.c) on every input element of a small packed batch;
  * the closed form at beta = 0, where the state only decays: with
    G_t = sum_{s<=t} g_s,  o_u = S_0^T (e^{G_u} * q_u), so
      dq_t = e^{G_t} * (S_0 do_t),   dk = dv = 0,
      ds0  = sum_t (e^{G_t} * q_t) do_t^T + Diag(e^{G_T}) dsT,
      dg_s[c] = sum_{u>=s} e^{G_u[c]} q_u[c] (S_0[c,:] . do_u) + e^{G_T[c]} (S_0[c,:] . dsT[c,:]),
      dbeta_t = e_t . ( sum_{u>=t} do_u (q_u . (e^{G_u - G_t} * k_t)) + dsT^T (e^{G_T - G_t} * k_t) )
    with e_t = v_t - S_0^T (e^{G_t} * k_t) (a write at t, then pure decay);
  * linearity of the gradients in (do, dsT).
"""

import inspect

import numpy as np
import pytest

from oracle import oracle


def _case(seed, lengths, H, K, V, beta_zero=False):
    rng = np.random.default_rng(seed)
    n = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    d = dict(q=unit(rng.standard_normal((n, H, K))), k=unit(rng.standard_normal((n, H, K))),
             v=rng.standard_normal((n, H, V)),
             g=-0.5 / (1 + np.exp(-rng.standard_normal((n, H, K)))),
             beta=np.zeros((n, H)) if beta_zero else 1 / (1 + np.exp(-rng.standard_normal((n, H)))),
             s0=0.5 * rng.standard_normal((len(lengths), H, K, V)))
    do = rng.standard_normal((n, H, V))
    dsT = rng.standard_normal((len(lengths), H, K, V))
    return d, cu, do, dsT


def _loss(d, cu, do, dsT):
    o, sT = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["s0"], nthreads=1)
    return float(np.sum(o * do) + np.sum(sT * dsT))


NAMES = ("q", "k", "v", "g", "beta", "s0")


def pin_finite_differences(bwd):
    d, cu, do, dsT = _case(1, [3, 0, 5], H=2, K=3, V=2)
    grads = bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["s0"], do, dsT)
    h = 1e-5
    for name, gr in zip(NAMES, grads):
        x = d[name]
        fd = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            keep = x[i]
            x[i] = keep + h
            lp = _loss(d, cu, do, dsT)
            x[i] = keep - h
            lm = _loss(d, cu, do, dsT)
            x[i] = keep
            fd[i] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(gr, fd, rtol=0, atol=2e-8 * (1 + np.max(np.abs(fd))),
                                   err_msg=f"d{name}")


def pin_beta_zero_closed_form(bwd):
    T, H, K, V = 7, 2, 4, 3
    d, cu, do, dsT = _case(2, [T], H=H, K=K, V=V, beta_zero=True)
    dq, dk, dv, dg, dbeta, ds0 = bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["s0"],
                                    do, dsT)
    for h in range(H):
        S0, q, k, v, dO, dST = d["s0"][0, h], d["q"][:, h], d["k"][:, h], d["v"][:, h], do[:, h], dsT[0, h]
        G = np.cumsum(d["g"][:, h], axis=0)
        eGT = np.exp(G[-1])
        ref_ds0 = np.diag(eGT) @ dST
        for t in range(T):
            ref_ds0 += np.outer(np.exp(G[t]) * q[t], dO[t])
            np.testing.assert_allclose(dq[t, h], np.exp(G[t]) * (S0 @ dO[t]), rtol=1e-12, atol=1e-14)
            e = v[t] - S0.T @ (np.exp(G[t]) * k[t])
            acc = dST.T @ (np.exp(G[-1] - G[t]) * k[t])
            for u in range(t, T):
                acc = acc + dO[u] * (q[u] @ (np.exp(G[u] - G[t]) * k[t]))
            np.testing.assert_allclose(dbeta[t, h], e @ acc, rtol=1e-12, atol=1e-13)
            ref_dg = eGT * np.sum(S0 * dST, axis=1)
            for u in range(t, T):
                ref_dg = ref_dg + np.exp(G[u]) * q[u] * (S0 @ dO[u])
            np.testing.assert_allclose(dg[t, h], ref_dg, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ds0[0, h], ref_ds0, rtol=1e-12, atol=1e-14)
    assert np.max(np.abs(dk)) < 1e-15 and np.max(np.abs(dv)) < 1e-15


def pin_linear_in_output_gradients(bwd):
    d, cu, do, dsT = _case(3, [4, 6], H=1, K=3, V=2)
    rng = np.random.default_rng(4)
    do2, dsT2 = rng.standard_normal(do.shape), rng.standard_normal(dsT.shape)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["s0"])
    a = bwd(*args, do, dsT)
    b = bwd(*args, do2, dsT2)
    c = bwd(*args, do + 3 * do2, dsT + 3 * dsT2)
    for x, y, z in zip(a, b, c):
        np.testing.assert_allclose(z, x + 3 * y, rtol=1e-12, atol=1e-12)


PINS = [pin_finite_differences, pin_beta_zero_closed_form, pin_linear_in_output_gradients]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_backward_pin(pin):
    pin(oracle.backward)


def test_backward_empty_sequence_passes_the_state_gradient_through():
    d, cu, do, dsT = _case(5, [0, 2], H=1, K=3, V=2)
    grads = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["s0"], do, dsT)
    np.testing.assert_array_equal(grads[5][0], dsT[0])


# (name, fragment of oracle.backward, replacement): plausible slips in the loop
MUTANTS = [
    ("state_loss_dropped", "loss = loss + (S * torch.tensor(dsT[n], dtype=torch.float64)).sum()",
     "loss = loss + 0.0 * S.sum()"),
    ("error_sign", "e = tv[t] - torch.einsum(\"hkv,hk->hv\", S, tk[t])",
     "e = tv[t] + torch.einsum(\"hkv,hk->hv\", S, tk[t])"),
    ("beta_dropped", "S = S + tb[t][:, None, None] * tk[t][:, :, None] * e[:, None, :]",
     "S = S + tk[t][:, :, None] * e[:, None, :]"),
    ("output_reads_key", "o = torch.einsum(\"hkv,hk->hv\", S, tq[t])",
     "o = torch.einsum(\"hkv,hk->hv\", S, tk[t])"),
    ("decay_dropped", "S = torch.exp(tg[t])[:, :, None] * S                        # Diag(alpha_t) S",
     "S = S"),
    ("gate_not_exponentiated", "S = torch.exp(tg[t])[:, :, None] * S",
     "S = (1.0 + tg[t])[:, :, None] * S"),
]


def _mutant(old, new):
    src = inspect.getsource(oracle.backward)
    assert src.count(old) == 1, old
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["backward"]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_backward_mutant_fails_a_pin(name, old, new):
    bwd = _mutant(old, new)
    failed = []
    for pin in PINS:
        try:
            pin(bwd)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every backward pin"
