"""Pins for the oracle's backward pass (oracle.kda_bwd), independent of its code.

The backward is the gradient of a scalar loss L = <do, o> + <dS_T, S_final> through the
forward recurrence, so it is fixed by the forward alone:
* central finite differences of oracle.kda_fwd (a different program: the forward only) for
  every input element, on tiny packed problems with an initial state, zero write strengths
  and zero decay included;
* exact Euler identities: (o, S_final) is linear in (v, S_init) jointly and o is linear in q
  with S_final independent of q, so <dv, v> + <dS_init, S_init> = L and <dq, q> = <do, o>;
* a closed form without writes (beta = 0): S_t = Diag(e^{G_t}) S_init, from which dq, dg,
  dbeta and dS_init are written out directly as sums over later tokens;
* splitting a chain anywhere: the backward of the second part hands dS at the cut to the
  backward of the first part as its final-state gradient; packed sequences equal separate
  calls.
A dropped term, a wrong sign, a transposed operand or the decay applied on the wrong side
of the read-out fails one of them.
"""

import numpy as np
import pytest

import oracle


def case(seed, T, H, K, V, *, g_scale=0.3, unit=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, V))
    g = -g_scale * rng.random((T, H, K)) * 2.0
    beta = rng.random((T, H))
    return q, k, v, g, beta


def loss(inputs, do, dsT, cu, scale, s0):
    q, k, v, g, beta = inputs
    o, S = oracle.kda_fwd(q, k, v, g, beta, scale=scale, initial_state=s0, cu_seqlens=cu)
    return float(np.sum(o * do) + np.sum(S * dsT))


@pytest.mark.parametrize("variant", ["plain", "beta0_tokens", "no_decay", "raw_keys"])
def test_bwd_matches_central_differences(variant):
    """Every gradient element of a 2-sequence packed problem (lengths 4 and 5, K=3, V=2, an
    initial state, scale 0.7) against (L(x+h) - L(x-h)) / 2h, h = 1e-6."""
    T, H, K, V = 9, 1, 3, 2
    cu = np.array([0, 4, 9])
    q, k, v, g, beta = case(11, T, H, K, V, unit=variant != "raw_keys")
    if variant == "beta0_tokens":
        beta[[1, 6]] = 0.0
    if variant == "no_decay":
        g[:] = 0.0
    rng = np.random.default_rng(12)
    s0 = rng.standard_normal((2, H, K, V))
    do = rng.standard_normal((T, H, V))
    dsT = rng.standard_normal((2, H, K, V))
    scale = 0.7
    dq, dk, dv, dg, db, ds0 = oracle.kda_bwd(q, k, v, g, beta, do, scale=scale, initial_state=s0,
                                             dfinal_state=dsT, cu_seqlens=cu)
    inputs = [q, k, v, g, beta]
    grads = [dq, dk, dv, dg, db]
    h = 1e-6
    for which, (x, gx) in enumerate(zip(inputs + [s0], grads + [ds0])):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xs = [a.copy() for a in inputs]
            st = s0.copy()
            target = xs[which] if which < 5 else st
            target[idx] += h
            lp = loss(xs, do, dsT, cu, scale, st)
            target[idx] -= 2 * h
            lm = loss(xs, do, dsT, cu, scale, st)
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(gx, fd, rtol=1e-6, atol=1e-7,
                                   err_msg=["dq", "dk", "dv", "dg", "dbeta", "ds0"][which])


def test_bwd_euler_identities():
    """Linearity in (v, S_init) and in q, exactly (up to float64 rounding)."""
    T, H, K, V = 50, 2, 16, 12
    cu = np.array([0, 7, 7, 50])
    q, k, v, g, beta = case(21, T, H, K, V)
    rng = np.random.default_rng(22)
    s0 = rng.standard_normal((3, H, K, V))
    do = rng.standard_normal((T, H, V))
    dsT = rng.standard_normal((3, H, K, V))
    o, S = oracle.kda_fwd(q, k, v, g, beta, initial_state=s0, cu_seqlens=cu)
    dq, dk, dv, dg, db, ds0 = oracle.kda_bwd(q, k, v, g, beta, do, initial_state=s0,
                                             dfinal_state=dsT, cu_seqlens=cu)
    L = np.sum(o * do) + np.sum(S * dsT)
    assert abs(np.sum(dv * v) + np.sum(ds0 * s0) - L) <= 1e-12 * (1 + abs(L))
    Lo = np.sum(o * do)
    assert abs(np.sum(dq * q) - Lo) <= 1e-12 * (1 + abs(Lo))
    # the empty sequence hands its final-state gradient straight back
    np.testing.assert_array_equal(ds0[1], dsT[1])


def test_bwd_pure_decay_closed_form():
    """beta = 0: S_t = Diag(e^{G_t}) S_init with G_t the running sum of g, o_t = S_t^T q_t
    scale. Then, with Z_t = dL/dS_t from the read-outs at t' >= t and the final state,
    dq_t = scale S_t do_t, dS_init = Diag(e^{G_1}) Z_1 ... written out as explicit sums."""
    T, H, K, V = 12, 1, 5, 4
    q, k, v, g, _ = case(31, T, H, K, V)
    beta = np.zeros((T, H))
    rng = np.random.default_rng(32)
    s0 = rng.standard_normal((1, H, K, V))
    do = rng.standard_normal((T, H, V))
    dsT = rng.standard_normal((1, H, K, V))
    scale = 1.3
    dq, dk, dv, dg, db, ds0 = oracle.kda_bwd(q, k, v, g, beta, do, scale=scale, initial_state=s0,
                                             dfinal_state=dsT)
    S0 = s0[0, 0]
    G = np.cumsum(g[:, 0], axis=0)                     # G_t, [T, K]
    S = [np.exp(G[t])[:, None] * S0 for t in range(T)]
    # dL/dS_t counting every read-out t' >= t and the final state, carried back by the decay
    Z = []
    for t in range(T):
        z = np.exp(G[T - 1] - G[t])[:, None] * dsT[0, 0]
        for tp in range(t, T):
            z = z + np.exp(G[tp] - G[t])[:, None] * scale * np.outer(q[tp, 0], do[tp, 0])
        Z.append(z)
    for t in range(T):
        np.testing.assert_allclose(dq[t, 0], scale * S[t] @ do[t, 0], rtol=1e-12, atol=1e-13)
        # L depends on g_t through G_{t'} for t' >= t: dL/dg_t = sum_{t' >= t} dL/dG_{t'}
        dG = [scale * q[tp, 0] * (S[tp] @ do[tp, 0]) for tp in range(T)]
        dG[T - 1] = dG[T - 1] + np.sum(S[T - 1] * dsT[0, 0], axis=1)
        np.testing.assert_allclose(dg[t, 0], np.sum(dG[t:], axis=0), rtol=1e-11, atol=1e-12)
        # dbeta_t = (Z_t^T k_t) . (v_t - S'_t^T k_t) with S'_t = S_t (no write)
        np.testing.assert_allclose(db[t, 0], (Z[t].T @ k[t, 0]) @ (v[t, 0] - S[t].T @ k[t, 0]),
                                   rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ds0[0, 0], np.exp(G[0])[:, None] * Z[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(dk, 0.0)
    np.testing.assert_array_equal(dv, 0.0)


@pytest.mark.parametrize("m", [1, 17, 31])
def test_bwd_split_chain(m):
    """Backward over [0, T) == backward over [m, T) from S_m, then over [0, m) with the
    handed-back dS_m as the final-state gradient."""
    T, H, K, V = 40, 2, 8, 6
    q, k, v, g, beta = case(41, T, H, K, V)
    rng = np.random.default_rng(42)
    s0 = rng.standard_normal((1, H, K, V))
    do = rng.standard_normal((T, H, V))
    dsT = rng.standard_normal((1, H, K, V))
    full = oracle.kda_bwd(q, k, v, g, beta, do, initial_state=s0, dfinal_state=dsT)
    _, Sm = oracle.kda_fwd(q[:m], k[:m], v[:m], g[:m], beta[:m], initial_state=s0)
    b2 = oracle.kda_bwd(q[m:], k[m:], v[m:], g[m:], beta[m:], do[m:], initial_state=Sm,
                        dfinal_state=dsT)
    b1 = oracle.kda_bwd(q[:m], k[:m], v[:m], g[:m], beta[:m], do[:m], initial_state=s0,
                        dfinal_state=b2[5])
    for i in range(5):
        np.testing.assert_allclose(full[i], np.concatenate([b1[i], b2[i]]), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(full[5], b1[5], rtol=1e-10, atol=1e-12)


def test_bwd_packed_equals_separate():
    T, H, K, V = 30, 2, 6, 5
    cu = np.array([0, 0, 11, 30])
    q, k, v, g, beta = case(51, T, H, K, V)
    rng = np.random.default_rng(52)
    s0 = rng.standard_normal((3, H, K, V))
    do = rng.standard_normal((T, H, V))
    dsT = rng.standard_normal((3, H, K, V))
    packed = oracle.kda_bwd(q, k, v, g, beta, do, initial_state=s0, dfinal_state=dsT, cu_seqlens=cu)
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        sep = oracle.kda_bwd(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], do[a:b],
                             initial_state=s0[n:n + 1], dfinal_state=dsT[n:n + 1])
        for i in range(5):
            np.testing.assert_array_equal(packed[i][a:b], sep[i])
        np.testing.assert_array_equal(packed[5][n], sep[5][0])
