"""Pins for the float64 oracle, independent of the oracle's own code.

Each test checks the oracle against something the pages or the mathematics fix: a
hand-derived closed form, exact rational arithmetic on the defining matrix equation,
reductions to the textbook delta rule, exact-overwrite and pure-decay identities, the
spectral behaviour the KV-cache page (section 5) describes for unnormalised keys,
linearity, split/resume and packed-vs-separate equalities. Together they catch a dropped
term, a wrong sign, decay on the wrong axis, a read-out before the write, a transposed
operand or a chunk/sequence boundary slip.
"""

import itertools
import math
import random
from fractions import Fraction as F

import numpy as np
import pytest

import oracle


def rnd_unit(rng, T, d):
    x = rng.standard_normal((T, d))
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rnd_case(seed, T, H, K, V, g_scale=0.1):
    rng = np.random.default_rng(seed)
    q = rnd_unit(rng, T * H, K).reshape(T, H, K)
    k = rnd_unit(rng, T * H, K).reshape(T, H, K)
    v = rng.standard_normal((T, H, V))
    g = -g_scale * rng.random((T, H, K)) * 3.0
    beta = rng.random((T, H))
    return q, k, v, g, beta


# ----------------------------------------------------------------- hand-derived example

def test_hand_derived_two_tokens():
    """K=2, V=3, two tokens, worked by hand in exact fractions (rows of S = key channels).

    t=1 (zero state): k=(4/5,3/5), v=(1,2,-1), beta=1, q=(1,0)
        S1 = k v^T = [[4/5, 8/5, -4/5], [3/5, 6/5, -3/5]],  o1 = S1^T q = (4/5, 8/5, -4/5)
    t=2: alpha=(1/2,1/4), k=(3/5,4/5), v=(0,1,2), beta=1/2, q=(0,1)
        Diag(alpha) S1 = [[2/5, 4/5, -2/5], [3/20, 3/10, -3/20]]
        p = (Diag(alpha) S1)^T k = (9/25, 18/25, -9/25)
        u = beta (v - p) = (-9/50, 7/50, 59/50)
        S2 = Diag(alpha) S1 + k u^T = [[73/250, 221/250, 77/250], [3/500, 103/250, 397/500]]
        (the same as (I - beta k k^T) Diag(alpha) S1 + beta k v^T, also done by hand)
        o2 = S2^T q = (3/500, 103/250, 397/500)
    """
    q = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    k = np.array([[[0.8, 0.6]], [[0.6, 0.8]]])
    v = np.array([[[1.0, 2.0, -1.0]], [[0.0, 1.0, 2.0]]])
    g = np.array([[[math.log(0.3), math.log(0.7)]], [[math.log(0.5), math.log(0.25)]]])
    beta = np.array([[1.0], [0.5]])
    o, S = oracle.kda_fwd(q, k, v, g, beta)
    np.testing.assert_allclose(o[0, 0], [0.8, 1.6, -0.8], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(o[1, 0], [3 / 500, 103 / 250, 397 / 500], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(S[0, 0], [[73 / 250, 221 / 250, 77 / 250],
                                         [3 / 500, 103 / 250, 397 / 500]], rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------ exact rational brute force

_UNIT2 = [(F(3, 5), F(4, 5)), (F(5, 13), F(12, 13)), (F(8, 17), F(15, 17)), (F(7, 25), F(24, 25))]
_UNIT3 = [(F(1, 3), F(2, 3), F(2, 3)), (F(2, 7), F(3, 7), F(6, 7)), (F(2, 3), F(1, 3), F(2, 3))]


def _rand_unit_rational(r, d):
    base = list(r.choice(_UNIT2 if d == 2 else _UNIT3))
    r.shuffle(base)
    return [x * r.choice((1, -1)) for x in base]


def _matrix_form_exact(ks, vs, qs, alphas, betas, S0):
    """S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t,
    with explicit d x d matrices in exact rational arithmetic."""
    K = len(ks[0])
    V = len(vs[0])
    S = [row[:] for row in S0]
    outs = []
    for k, v, q, a, b in zip(ks, vs, qs, alphas, betas):
        P = [[(F(1) if i == j else F(0)) - b * k[i] * k[j] for j in range(K)] for i in range(K)]
        D = [[a[i] * S[i][j] for j in range(V)] for i in range(K)]
        S = [[sum(P[i][m] * D[m][j] for m in range(K)) + b * k[i] * v[j] for j in range(V)]
             for i in range(K)]
        outs.append([sum(S[i][j] * q[i] for i in range(K)) for j in range(V)])
    return outs, S


@pytest.mark.parametrize("seed", range(6))
def test_exact_rational_matrix_form(seed):
    r = random.Random(seed)
    K = r.choice((2, 3))
    V = r.choice((2, 3))
    T = r.randint(1, 6)
    fr = [F(1, 2), F(2, 3), F(3, 4), F(1), F(1, 5), F(7, 8)]
    ks = [_rand_unit_rational(r, K) for _ in range(T)]
    qs = [_rand_unit_rational(r, K) for _ in range(T)]
    vs = [[F(r.randint(-5, 5), r.randint(1, 4)) for _ in range(V)] for _ in range(T)]
    alphas = [[r.choice(fr) for _ in range(K)] for _ in range(T)]
    betas = [r.choice([F(0), F(1, 4), F(1, 2), F(1), F(3, 5)]) for _ in range(T)]
    S0 = [[F(r.randint(-3, 3), r.randint(1, 3)) for _ in range(V)] for _ in range(K)]
    outs, S = _matrix_form_exact(ks, vs, qs, alphas, betas, S0)

    f = lambda x: np.array(x, dtype=np.float64)  # noqa: E731
    o, Sf = oracle.kda_fwd(f(qs)[:, None], f(ks)[:, None], f(vs)[:, None],
                           np.log(f(alphas))[:, None], f(betas)[:, None],
                           initial_state=f(S0)[None, None])
    np.testing.assert_allclose(o[:, 0], f(outs), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Sf[0, 0], f(S), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------------ closed forms

def test_single_token_closed_form():
    """From a zero state: S_1 = beta k v^T and o_1 = scale * beta (q.k) v."""
    q, k, v, g, beta = rnd_case(1, 1, 3, 7, 5)
    o, S = oracle.kda_fwd(q, k, v, g, beta, scale=0.37)
    for h in range(3):
        np.testing.assert_allclose(S[0, h], beta[0, h] * np.outer(k[0, h], v[0, h]), rtol=1e-14)
        np.testing.assert_allclose(o[0, h], 0.37 * beta[0, h] * (q[0, h] @ k[0, h]) * v[0, h],
                                   rtol=1e-13, atol=1e-15)


def test_pure_decay_when_beta_zero():
    """beta = 0: S_t = Diag(exp(sum_{tau<=t} g_tau)) S_0 (rows = key channels), o_t = S_t^T q_t."""
    T, H, K, V = 20, 2, 6, 4
    q, k, v, g, _ = rnd_case(2, T, H, K, V, g_scale=0.5)
    beta = np.zeros((T, H))
    S0 = np.random.default_rng(3).standard_normal((1, H, K, V))
    o, S = oracle.kda_fwd(q, k, v, g, beta, initial_state=S0)
    G = np.cumsum(g, axis=0)
    for t in range(T):
        for h in range(H):
            St = np.exp(G[t, h])[:, None] * S0[0, h]
            np.testing.assert_allclose(o[t, h], St.T @ q[t, h], rtol=1e-12, atol=1e-14)
    for h in range(H):
        np.testing.assert_allclose(S[0, h], np.exp(G[-1, h])[:, None] * S0[0, h], rtol=1e-12)


def test_exact_overwrite_unit_key_beta_one():
    """beta=1, |k|=1, q=k: o_t = v_t for any prior state and any decay, because
    k^T (I - k k^T) = 0."""
    T, H, K, V = 30, 2, 8, 5
    q, k, v, g, _ = rnd_case(4, T, H, K, V, g_scale=1.0)
    beta = np.ones((T, H))
    S0 = np.random.default_rng(5).standard_normal((1, H, K, V)) * 3
    o, _ = oracle.kda_fwd(k, k, v, g, beta, initial_state=S0)
    np.testing.assert_allclose(o, v, atol=1e-13)


def test_orthonormal_keys_store_and_recall():
    """alpha=1, beta=1, orthonormal keys, zero state: S_d = sum_i k_i v_i^T, and reading
    with k_i returns v_i."""
    K, V = 6, 4
    rng = np.random.default_rng(6)
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    keys = Qm.T  # rows orthonormal
    v = rng.standard_normal((K, 1, V))
    o, S = oracle.kda_fwd(keys[:, None], keys[:, None], v, np.zeros((K, 1, K)),
                          np.ones((K, 1)))
    np.testing.assert_allclose(S[0, 0], keys.T @ v[:, 0], atol=1e-13)
    np.testing.assert_allclose(keys @ S[0, 0], v[:, 0], atol=1e-13)


def test_unnormalised_key_blows_up_state():
    """The KV-cache page (section 5) warns that with |k| != 1 the erase term
    (I - beta k k^T) leaves the unit disc and the state explodes. Its eigenvalues are
    1 (d-1 times) and 1 - beta |k|^2, so with v = 0, alpha = 1 and one repeated key:
    S_T = S_0 + ((1 - beta |k|^2)^T - 1) khat khat^T S_0."""
    K, V, T = 5, 3, 12
    rng = np.random.default_rng(7)
    khat = rnd_unit(rng, 1, K)[0]
    kvec = math.sqrt(10.2) * khat
    b = 0.9
    lam = 1 - b * 10.2  # -8.18
    S0 = rng.standard_normal((1, 1, K, V))
    _, S = oracle.kda_fwd(np.tile(khat, (T, 1, 1)), np.tile(kvec, (T, 1, 1)),
                          np.zeros((T, 1, V)), np.zeros((T, 1, K)), np.full((T, 1), b),
                          initial_state=S0)
    expect = S0[0, 0] + (lam ** T - 1) * np.outer(khat, khat) @ S0[0, 0]
    np.testing.assert_allclose(S[0, 0], expect, rtol=1e-9)
    assert np.linalg.norm(S[0, 0], 2) > 1e9 * np.linalg.norm(S0[0, 0], 2) / 1e3


def test_state_norm_bound_with_unit_keys():
    """With |k|=1, beta in [0,1] and alpha <= 1, ||(I - beta k k^T) Diag(alpha)||_2 <= 1, so
    ||S_t||_2 <= ||S_{t-1}||_2 + beta_t |v_t|."""
    T, H, K, V = 40, 1, 8, 8
    q, k, v, g, beta = rnd_case(8, T, H, K, V)
    S = np.random.default_rng(9).standard_normal((1, 1, K, V))
    for t in range(T):
        _, S1 = oracle.kda_decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1],
                                       beta[t:t + 1], S)
        assert np.linalg.norm(S1[0, 0], 2) <= np.linalg.norm(S[0, 0], 2) + \
            beta[t, 0] * np.linalg.norm(v[t, 0]) + 1e-12
        S = S1


# --------------------------------------------------------------------------- reductions

def test_reduces_to_delta_rule_sgd_when_no_decay():
    """alpha = 1 (g = 0): DeltaNet, i.e. one gradient step of size beta on
    0.5 |S^T k - v|^2 per token: S <- S - beta k (S^T k - v)^T."""
    T, H, K, V = 25, 2, 7, 3
    q, k, v, _, beta = rnd_case(10, T, H, K, V)
    g = np.zeros((T, H, K))
    o, S = oracle.kda_fwd(q, k, v, g, beta)
    for h in range(H):
        Sh = np.zeros((K, V))
        for t in range(T):
            grad = np.outer(k[t, h], Sh.T @ k[t, h] - v[t, h])
            Sh = Sh - beta[t, h] * grad
            np.testing.assert_allclose(o[t, h], Sh.T @ q[t, h], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(S[0, h], Sh, rtol=1e-11, atol=1e-13)


def test_scalar_gate_is_gated_delta_rule():
    """alpha equal across channels (Gated DeltaNet): the scalar decay commutes with the
    erase, S_t = alpha_t [S - beta k (S^T k)^T] + beta k v^T."""
    T, K, V = 25, 6, 4
    q, k, v, _, beta = rnd_case(11, T, 1, K, V)
    a = np.random.default_rng(12).uniform(0.5, 1.0, T)
    g = np.repeat(np.log(a)[:, None, None], K, axis=2)
    o, S = oracle.kda_fwd(q, k, v, g, beta)
    Sh = np.zeros((K, V))
    for t in range(T):
        kt, bt = k[t, 0], beta[t, 0]
        Sh = a[t] * (Sh - bt * np.outer(kt, Sh.T @ kt)) + bt * np.outer(kt, v[t, 0])
        np.testing.assert_allclose(o[t, 0], Sh.T @ q[t, 0], rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------------------- structure

def test_linear_in_values_and_initial_state():
    T, H, K, V = 33, 2, 5, 4
    q, k, v1, g, beta = rnd_case(13, T, H, K, V)
    rng = np.random.default_rng(14)
    v2 = rng.standard_normal(v1.shape)
    s1 = rng.standard_normal((1, H, K, V))
    s2 = rng.standard_normal((1, H, K, V))
    a, b = 0.7, -1.3
    o1, S1 = oracle.kda_fwd(q, k, v1, g, beta, initial_state=s1)
    o2, S2 = oracle.kda_fwd(q, k, v2, g, beta, initial_state=s2)
    o3, S3 = oracle.kda_fwd(q, k, a * v1 + b * v2, g, beta, initial_state=a * s1 + b * s2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, atol=1e-12)
    np.testing.assert_allclose(S3, a * S1 + b * S2, atol=1e-12)


@pytest.mark.parametrize("m", [1, 16, 17, 40])
def test_split_resume_equals_single_run(m):
    T, H, K, V = 57, 2, 6, 5
    q, k, v, g, beta = rnd_case(15, T, H, K, V)
    o, S = oracle.kda_fwd(q, k, v, g, beta)
    oa, Sa = oracle.kda_fwd(q[:m], k[:m], v[:m], g[:m], beta[:m])
    ob, Sb = oracle.kda_fwd(q[m:], k[m:], v[m:], g[m:], beta[m:], initial_state=Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(Sb, S, rtol=1e-12, atol=1e-14)


def test_prefill_then_decode_equals_prefill():
    T, P, H, K, V = 30, 20, 3, 4, 6
    q, k, v, g, beta = rnd_case(16, T, H, K, V)
    o, S = oracle.kda_fwd(q, k, v, g, beta)
    _, St = oracle.kda_fwd(q[:P], k[:P], v[:P], g[:P], beta[:P])
    for t in range(P, T):
        ot, St = oracle.kda_decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1],
                                        beta[t:t + 1], St)
        np.testing.assert_allclose(ot[0], o[t], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(St, S, rtol=1e-12, atol=1e-14)


def test_packed_equals_separate_runs_including_empty():
    H, K, V = 2, 4, 3
    lens = [5, 0, 17, 1, 0, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta = rnd_case(17, int(cu[-1]), H, K, V)
    S0 = np.random.default_rng(18).standard_normal((len(lens), H, K, V))
    o, S = oracle.kda_fwd(q, k, v, g, beta, initial_state=S0, cu_seqlens=cu)
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        on, Sn = oracle.kda_fwd(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b],
                                initial_state=S0[n:n + 1])
        np.testing.assert_allclose(o[a:b], on, rtol=1e-14)
        np.testing.assert_allclose(S[n], Sn[0], rtol=1e-14)
        if a == b:
            np.testing.assert_array_equal(S[n], S0[n])


def test_batched_layout_is_sequences():
    B, T, H, K, V = 3, 11, 2, 4, 5
    q, k, v, g, beta = rnd_case(19, B * T, H, K, V)
    rs = lambda x: x.reshape(B, T, *x.shape[1:])  # noqa: E731
    o, S = oracle.kda_fwd(rs(q), rs(k), rs(v), rs(g), rs(beta))
    o2, S2 = oracle.kda_fwd(q, k, v, g, beta, cu_seqlens=np.arange(B + 1) * T)
    np.testing.assert_array_equal(o.reshape(B * T, H, V), o2)
    np.testing.assert_array_equal(S, S2)


def test_heads_are_independent_and_scale_is_linear():
    T, H, K, V = 21, 3, 5, 5
    q, k, v, g, beta = rnd_case(20, T, H, K, V)
    o, S = oracle.kda_fwd(q, k, v, g, beta, scale=2.5)
    o1, S1 = oracle.kda_fwd(q, k, v, g, beta, scale=1.0)
    np.testing.assert_allclose(o, 2.5 * o1, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(S, S1)
    oh, Sh = oracle.kda_fwd(q[:, 1:2], k[:, 1:2], v[:, 1:2], g[:, 1:2], beta[:, 1:2], scale=2.5)
    np.testing.assert_array_equal(o[:, 1:2], oh)
    np.testing.assert_array_equal(S[:, 1:2], Sh)


# ------------------------------------------------------------------------ chunked form

@pytest.mark.parametrize("T,chunk", [(48, 16), (45, 16), (64, 64), (130, 64), (7, 16)])
def test_chunked_form_equals_recurrence(T, chunk):
    H, K, V = 2, 8, 6
    q, k, v, g, beta = rnd_case(21 + T, T, H, K, V, g_scale=0.5)
    S0 = np.random.default_rng(22).standard_normal((1, H, K, V))
    o, S = oracle.kda_fwd(q, k, v, g, beta, initial_state=S0, scale=0.5)
    oc, Sc = oracle.chunked_fwd(q, k, v, g, beta, chunk=chunk, initial_state=S0, scale=0.5)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Sc, S, rtol=1e-10, atol=1e-12)


def test_chunked_form_packed_and_strong_decay():
    H, K, V = 1, 4, 3
    lens = [70, 0, 33]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, _, beta = rnd_case(23, int(cu[-1]), H, K, V)
    g = np.full((int(cu[-1]), H, K), -3.0)  # |G| reaches 192 over a 64-token chunk
    o, S = oracle.kda_fwd(q, k, v, g, beta, cu_seqlens=cu)
    oc, Sc = oracle.chunked_fwd(q, k, v, g, beta, chunk=64, cu_seqlens=cu)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Sc, S, rtol=1e-10, atol=1e-12)


def test_oracle_rejects_bad_cu_seqlens():
    q, k, v, g, beta = rnd_case(24, 4, 1, 2, 2)
    with pytest.raises(ValueError):
        oracle.kda_fwd(q, k, v, g, beta, cu_seqlens=[0, 3])
    with pytest.raises(RuntimeError):
        oracle.kda_fwd(q, k, v, g, beta, cu_seqlens=[0, 3, 2, 4])


def test_threads_do_not_change_results():
    q, k, v, g, beta = rnd_case(25, 40, 6, 5, 5)
    o1, S1 = oracle.kda_fwd(q, k, v, g, beta, threads=1)
    o4, S4 = oracle.kda_fwd(q, k, v, g, beta, threads=4)
    np.testing.assert_array_equal(o1, o4)
    np.testing.assert_array_equal(S1, S4)


def test_all_pairs_signs_of_hand_example_are_distinct():
    """Guard for the hand example: the wrong orders (decay after the erase, or reading
    before the write) give different numbers, so the test above can tell them apart."""
    k1, k2 = np.array([0.8, 0.6]), np.array([0.6, 0.8])
    S1 = np.outer(k1, [1.0, 2.0, -1.0])
    a = np.array([0.5, 0.25])
    P = np.eye(2) - 0.5 * np.outer(k2, k2)
    right = P @ (a[:, None] * S1) + 0.5 * np.outer(k2, [0, 1, 2])
    wrong_order = a[:, None] * (P @ S1) + 0.5 * np.outer(k2, [0, 1, 2])
    read_before = (a[:, None] * S1)[1]
    assert not np.allclose(right, wrong_order)
    assert not np.allclose(right[1], read_before)
    for i, j in itertools.product(range(2), range(3)):
        assert right[i, j] != 0
