"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

Reading under test ("Kimi K3: Open Frontier Intelligence and Implementation
Framework", section "Hybrid Attention Mechanism": the delta rule with a
channel-wise forget gate):

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t

Each pin is chosen so that a plausible slip in the oracle fails at least one:
  * decay dropped or applied to columns instead of rows -> decay-only closed form,
    decay-only golden file (K != V)
  * decay applied after the delta write instead of before -> hand golden file, q = k invariant
  * output read from S_{t-1} instead of S_t, or S q instead of S^T q -> retrieval pin,
    hand golden file (asymmetric S_0)
  * wrong sign / missing beta in the correction -> q = k invariant, hand golden file,
    exact-rational brute force
  * sequences or heads mixed up, initial state ignored -> varlen and state-passing pins
"""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle


def _read_golden(path):
    out = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            out[key] = [float(x) for x in vals]
    return out


def _golden_inputs(d):
    K, V, T = int(d["K"][0]), int(d["V"][0]), int(d["T"][0])
    q = np.array(d["q"]).reshape(T, 1, K)
    k = np.array(d["k"]).reshape(T, 1, K)
    v = np.array(d["v"]).reshape(T, 1, V)
    g = np.log(np.array(d["alpha"])).reshape(T, 1, K)
    beta = np.array(d["beta"]).reshape(T, 1)
    s0 = np.array(d["S0"]).reshape(1, 1, K, V)
    return K, V, T, q, k, v, g, beta, s0


def test_hand_example_two_steps(golden_dir):
    d = _read_golden(os.path.join(golden_dir, "hand_k2v2_t2.txt"))
    K, V, T, q, k, v, g, beta, s0 = _golden_inputs(d)
    o, sT = oracle.recurrence(q, k, v, g, beta, [0, T], s0)
    np.testing.assert_allclose(o.reshape(-1), d["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(sT.reshape(-1), d["S2"], rtol=0, atol=1e-14)
    o1, s1 = oracle.recurrence(q[:1], k[:1], v[:1], g[:1], beta[:1], [0, 1], s0)
    np.testing.assert_allclose(s1.reshape(-1), d["S1"], rtol=0, atol=1e-14)


def test_decay_only_golden(golden_dir):
    d = _read_golden(os.path.join(golden_dir, "decay_only_k3v2_t3.txt"))
    K, V, T, q, k, v, g, beta, s0 = _golden_inputs(d)
    o, sT = oracle.recurrence(q, k, v, g, beta, [0, T], s0)
    np.testing.assert_allclose(o.reshape(-1), d["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(sT.reshape(-1), d["S3"], rtol=0, atol=1e-14)


def _rand_unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def test_decay_only_closed_form():
    """beta = 0: S_T = Diag(exp(sum_t g_t)) S_0 and o_t = S_0^T (exp(G_t) * q_t)."""
    rng = np.random.default_rng(11)
    T, H, K, V = 9, 2, 5, 3
    q = rng.standard_normal((T, H, K))
    k = _rand_unit(rng, (T, H, K))
    v = rng.standard_normal((T, H, V))
    g = -rng.random((T, H, K))
    beta = np.zeros((T, H))
    s0 = rng.standard_normal((1, H, K, V))
    o, sT = oracle.recurrence(q, k, v, g, beta, [0, T], s0)
    G = np.cumsum(g, axis=0)                                   # [T, H, K]
    for h in range(H):
        np.testing.assert_allclose(sT[0, h], np.exp(G[-1, h])[:, None] * s0[0, h],
                                   rtol=1e-13, atol=1e-14)
        for t in range(T):
            np.testing.assert_allclose(o[t, h], s0[0, h].T @ (np.exp(G[t, h]) * q[t, h]),
                                       rtol=1e-13, atol=1e-14)


def test_no_decay_is_textbook_delta_rule_and_retrieves_written_value():
    """alpha = 1, beta = 1, |k| = 1: after writing (k_t, v_t), reading k_t returns v_t
    exactly, whatever the earlier state (the delta rule overwrites the value at k_t)."""
    rng = np.random.default_rng(12)
    T, H, K, V = 12, 3, 6, 4
    k = _rand_unit(rng, (T, H, K))
    q = k.copy()
    v = rng.standard_normal((T, H, V))
    g = np.zeros((T, H, K))
    beta = np.ones((T, H))
    s0 = rng.standard_normal((1, H, K, V))
    o, _ = oracle.recurrence(q, k, v, g, beta, [0, T], s0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def test_orthonormal_keys_retrieval():
    """alpha = 1, beta = 1, S_0 = 0 and orthonormal keys (T <= K): S_t = sum_{s<=t} k_s v_s^T,
    so querying with an earlier key k_s returns v_s, and an unwritten direction returns 0."""
    rng = np.random.default_rng(13)
    K, V, T = 8, 5, 7
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    keys = Qm.T[:T]                                            # orthonormal rows
    k = keys[:, None, :]
    v = rng.standard_normal((T, 1, V))
    pick = np.array([rng.integers(0, t + 1) for t in range(T)])
    q = keys[pick][:, None, :].copy()
    q[3, 0] = Qm.T[K - 1]                                      # never written
    g = np.zeros((T, 1, K))
    beta = np.ones((T, 1))
    o, sT = oracle.recurrence(q, k, v, g, beta, [0, T])
    for t in range(T):
        want = np.zeros(V) if t == 3 else v[pick[t], 0]
        np.testing.assert_allclose(o[t, 0], want, rtol=0, atol=1e-13)
    np.testing.assert_allclose(sT[0, 0], keys.T @ v[:, 0], rtol=0, atol=1e-13)


def _frac_vec(rng, n, lo, hi, den):
    return [Fraction(int(rng.integers(lo, hi + 1)), den) for _ in range(n)]


def test_bruteforce_exact_rationals():
    """T <= 8 in exact rational arithmetic with explicit transition matrices
    M_t = (I - beta_t k_t k_t^T) Diag(alpha_t):
        S_t = M_t ... M_1 S_0 + sum_{s<=t} (M_t ... M_{s+1}) beta_s k_s v_s^T,  o_t = S_t^T q_t.
    The oracle (fed g = log alpha) must agree to fp64 rounding."""
    rng = np.random.default_rng(14)
    K, V, T = 3, 2, 8
    ks = [_frac_vec(rng, K, -4, 4, 4) for _ in range(T)]
    vs = [_frac_vec(rng, V, -6, 6, 3) for _ in range(T)]
    qs = [_frac_vec(rng, K, -5, 5, 5) for _ in range(T)]
    al = [[Fraction(int(rng.integers(1, 9)), 8) for _ in range(K)] for _ in range(T)]
    be = [Fraction(int(rng.integers(0, 5)), 4) for _ in range(T)]
    S0 = [_frac_vec(rng, V, -3, 3, 2) for _ in range(K)]

    def matmul(A, B):
        return [[sum(A[i][l] * B[l][j] for l in range(len(B))) for j in range(len(B[0]))]
                for i in range(len(A))]

    def transition(t):
        return [[((1 if i == j else 0) - be[t] * ks[t][i] * ks[t][j]) * al[t][j]
                 for j in range(K)] for i in range(K)]

    Ms = [transition(t) for t in range(T)]
    for t in range(T):
        # product M_t ... M_1 applied to S_0
        P = S0
        for s in range(t + 1):
            P = matmul(Ms[s], P)
        S = [row[:] for row in P]
        for s in range(t + 1):
            W = [[be[s] * ks[s][i] * vs[s][j] for j in range(V)] for i in range(K)]
            for r in range(s + 1, t + 1):
                W = matmul(Ms[r], W)
            S = [[S[i][j] + W[i][j] for j in range(V)] for i in range(K)]
        o_exact = [sum(S[i][j] * qs[t][i] for i in range(K)) for j in range(V)]

        f = lambda a: np.array([[float(x) for x in r] for r in a]) if isinstance(a[0], list) \
            else np.array([float(x) for x in a])
        q = np.stack([f(x) for x in qs[:t + 1]])[:, None, :]
        k = np.stack([f(x) for x in ks[:t + 1]])[:, None, :]
        v = np.stack([f(x) for x in vs[:t + 1]])[:, None, :]
        g = np.log(np.stack([f(x) for x in al[:t + 1]]))[:, None, :]
        beta = np.array([float(x) for x in be[:t + 1]])[:, None]
        o, sT = oracle.recurrence(q, k, v, g, beta, [0, t + 1], f(S0)[None, None])
        np.testing.assert_allclose(sT[0, 0], f(S), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(o[t, 0], f(o_exact), rtol=1e-12, atol=1e-12)


def _random_problem(seed, T, H, K, V, N=1, glb=0.25):
    rng = np.random.default_rng(seed)
    tok = T * N
    q = _rand_unit(rng, (tok, H, K))
    k = _rand_unit(rng, (tok, H, K))
    v = rng.standard_normal((tok, H, V))
    g = -glb / (1 + np.exp(-rng.standard_normal((tok, H, K))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((tok, H))))
    s0 = 0.1 * rng.standard_normal((N, H, K, V))
    return q, k, v, g, beta, s0


def test_state_passing_resume():
    """run(T1 + T2, S_0) == run(T2, S_T of run(T1, S_0)): the state is the whole checkpoint."""
    q, k, v, g, beta, s0 = _random_problem(21, 50, 2, 6, 5)
    o, sT = oracle.recurrence(q, k, v, g, beta, [0, 50], s0)
    o1, s1 = oracle.recurrence(q[:23], k[:23], v[:23], g[:23], beta[:23], [0, 23], s0)
    o2, s2 = oracle.recurrence(q[23:], k[23:], v[23:], g[23:], beta[23:], [0, 27], s1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s2, sT, rtol=1e-13, atol=1e-14)


def test_linear_in_values_and_state_and_column_separable():
    q, k, v, g, beta, s0 = _random_problem(22, 30, 1, 6, 5)
    rng = np.random.default_rng(5)
    v2 = rng.standard_normal(v.shape)
    s02 = rng.standard_normal(s0.shape)
    c = -1.75
    oa, sa = oracle.recurrence(q, k, v, g, beta, [0, 30], s0)
    ob, sb = oracle.recurrence(q, k, v2, g, beta, [0, 30], s02)
    oc, sc = oracle.recurrence(q, k, v + c * v2, g, beta, [0, 30], s0 + c * s02)
    np.testing.assert_allclose(oc, oa + c * ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sc, sa + c * sb, rtol=1e-12, atol=1e-12)
    perm = np.array([3, 0, 4, 1, 2])
    op, sp = oracle.recurrence(q, k, v[..., perm], g, beta, [0, 30], s0[..., perm])
    np.testing.assert_allclose(op, oa[..., perm], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sp, sa[..., perm], rtol=1e-13, atol=1e-14)


def test_varlen_equals_independent_runs_with_empty_sequence():
    lengths = [5, 0, 17, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    H, K, V = 3, 4, 6
    q, k, v, g, beta, _ = _random_problem(23, int(cu[-1]), H, K, V)
    s0 = np.random.default_rng(6).standard_normal((len(lengths), H, K, V))
    o, sT = oracle.recurrence(q, k, v, g, beta, cu, s0, nthreads=3)
    for n in range(len(lengths)):
        a, b = cu[n], cu[n + 1]
        on, sn = oracle.recurrence(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], [0, b - a],
                                   s0[n:n + 1], nthreads=1)
        np.testing.assert_array_equal(o[a:b], on)
        np.testing.assert_array_equal(sT[n], sn[0])
    np.testing.assert_array_equal(sT[1], s0[1])              # empty sequence keeps S_0


def _step_states(q, k, v, g, beta, s0):
    T = q.shape[0]
    states = [s0]
    outs = []
    for t in range(T):
        o, s = oracle.recurrence(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1],
                                 beta[t:t + 1], [0, 1], states[-1])
        states.append(s)
        outs.append(o[0])
    return np.array(outs), states


def test_q_equals_k_delta_invariant():
    """q_t = k_t, |k_t| = 1: o_t = (1 - beta_t) (Diag(alpha_t) S_{t-1})^T k_t + beta_t v_t."""
    q, k, v, g, beta, s0 = _random_problem(24, 20, 2, 7, 3)
    q = k.copy()
    outs, states = _step_states(q, k, v, g, beta, s0)
    for t in range(20):
        for h in range(2):
            Y = np.exp(g[t, h])[:, None] * states[t][0, h]
            want = (1 - beta[t, h]) * (Y.T @ k[t, h]) + beta[t, h] * v[t, h]
            np.testing.assert_allclose(outs[t][h], want, rtol=1e-12, atol=1e-13)


def test_state_norm_bound():
    """|k| <= 1, 0 <= beta <= 1, 0 < alpha <= 1: ||S_t||_2 <= ||S_{t-1}||_2 + beta_t ||v_t||."""
    q, k, v, g, beta, s0 = _random_problem(25, 40, 1, 5, 4, glb=2.0)
    _, states = _step_states(q, k, v, g, beta, 3.0 * s0)
    for t in range(40):
        lhs = np.linalg.norm(states[t + 1][0, 0], 2)
        rhs = np.linalg.norm(states[t][0, 0], 2) + beta[t, 0] * np.linalg.norm(v[t, 0])
        assert lhs <= rhs * (1 + 1e-12)


def test_decode_steps_equal_prefill():
    q, k, v, g, beta, s0 = _random_problem(26, 6, 2, 4, 4, N=3)
    # sequences of 6 tokens each, packed; decode runs them step by step across the batch
    cu = np.arange(4) * 6
    o, sT = oracle.recurrence(q, k, v, g, beta, cu, s0)
    state = s0.copy()
    for t in range(6):
        idx = cu[:-1] + t
        od, state = oracle.decode_step(q[idx], k[idx], v[idx], g[idx], beta[idx], state)
        np.testing.assert_allclose(od, o[idx], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(state, sT, rtol=1e-13, atol=1e-14)


def test_rejects_bad_offsets():
    q, k, v, g, beta, _ = _random_problem(27, 4, 1, 2, 2)
    with pytest.raises(RuntimeError):
        oracle.recurrence(q, k, v, g, beta, np.array([0, 3, 2, 4]))
