"""Pins for the oracle's layer fusions (oracle/fused.py), independent of its own code.

Each check rests on a closed form, a hand-worked example or an invariance, chosen so that a
plausible slip fails one of them: the gate's rate indexed by channel instead of head, its
bias transposed, a sign or an argument of softplus flipped, exp(A_log) replaced by A_log,
normalisation over the wrong axis, eps added outside the square root, the sigmoid gate
dropped or applied before the norm, or the fused gate acting on the state's value columns.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import fused

LN2 = 0.6931471805599453


# ------------------------------------------------------------------------------- gate

def test_softplus_closed_forms():
    assert fused.softplus(0.0) == pytest.approx(LN2, rel=1e-15)
    assert fused.softplus(40.0) == 40.0                       # log1p(e^-40) is below half an ulp
    # log(1 + e^-40) = e^-40 - e^-80/2 + ...
    assert fused.softplus(-40.0) == pytest.approx(4.248354255291589e-18, rel=1e-14)
    z = np.linspace(-30.0, 30.0, 121)
    np.testing.assert_allclose(fused.softplus(z) - fused.softplus(-z), z, rtol=0, atol=1e-13)


def _params(seed, H, K):
    rng = np.random.default_rng(seed)
    return rng.uniform(math.log(0.01), math.log(0.5), H), rng.normal(-2.0, 0.5, (H, K))


def test_gate_at_zero_shift_is_minus_rate_ln2():
    """x = -dt_bias makes every softplus argument zero: g[t, h, c] = -exp(A_log[h]) ln 2.
    H != K, and distinct rates per head, so a transposed bias or a rate read per channel
    fails."""
    H, K, T = 3, 5, 4
    A_log, b = _params(1, H, K)
    x = np.broadcast_to(-b, (T, H, K))
    g = fused.kda_gate(x, A_log, b)
    for h in range(H):
        np.testing.assert_allclose(g[:, h, :], -math.exp(A_log[h]) * LN2, rtol=1e-15)


def test_gate_unit_rate_is_log_sigmoid_complement():
    """With A_log = 0 the gate is exp(g) = 1 / (1 + e^(x + b))."""
    H, K, T = 2, 7, 6
    _, b = _params(2, H, K)
    x = np.random.default_rng(3).standard_normal((T, H, K)) * 3.0
    g = fused.kda_gate(x, np.zeros(H), b)
    np.testing.assert_allclose(np.exp(g), 1.0 / (1.0 + np.exp(x + b)), rtol=1e-14)


def test_gate_rate_is_exponential_in_A_log():
    """Adding ln 2 to A_log doubles g (the rate is exp(A_log), not A_log)."""
    H, K = 4, 3
    A_log, b = _params(4, H, K)
    x = np.random.default_rng(5).standard_normal((9, H, K))
    np.testing.assert_allclose(fused.kda_gate(x, A_log + LN2, b), 2.0 * fused.kda_gate(x, A_log, b),
                               rtol=1e-14)


def test_gate_sign_monotone_and_asymptote():
    H, K = 2, 4
    A_log, b = _params(6, H, K)
    xs = np.linspace(-20.0, 20.0, 81)
    x = np.broadcast_to(xs[:, None, None], (81, H, K))
    g = fused.kda_gate(x, A_log, b)
    assert np.all(g < 0)
    assert np.all(np.diff(g, axis=0) < 0)                     # decreasing in the pre-activation
    # far right: softplus(z) -> z, so g -> -exp(A_log) (x + b)
    xr = np.full((1, H, K), 40.0)
    np.testing.assert_allclose(fused.kda_gate(xr, A_log, b)[0],
                               -np.exp(A_log)[:, None] * (40.0 + b), rtol=1e-15)


# ---------------------------------------------------------------------------- l2norm

def test_l2norm_examples_and_invariances():
    np.testing.assert_allclose(fused.l2norm(np.array([3.0, 4.0, 0.0])), [0.6, 0.8, 0.0], rtol=1e-15)
    x = np.random.default_rng(7).standard_normal((5, 3, 8))   # [T, H, K], K != H
    y = fused.l2norm(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=1e-15)
    np.testing.assert_allclose(fused.l2norm(x * 7.5), y, rtol=1e-15)
    np.testing.assert_allclose(np.sum(y * x, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
    z = x.copy()
    z[2, 1] = 0.0
    yz = fused.l2norm(z)
    assert np.all(yz[2, 1] == 0.0) and np.all(np.isfinite(yz))


# --------------------------------------------------------------------- gated RMSNorm

def test_gated_rmsnorm_worked_example():
    """o = (3, 4): mean square 12.5. weight (1, 2); gate pre-activations (ln 3, 0) give
    sigmoid (3/4, 1/2).
    eps = 0:    y = (3, 4) / sqrt(12.5) * (1, 2) * (3/4, 1/2) = (0.63639610..., 1.13137084...)
    eps = 12.5: y = (3, 4) / sqrt(25)   * (1, 2) * (3/4, 1/2) = (0.45, 0.8)"""
    o = np.array([3.0, 4.0])
    w = np.array([1.0, 2.0])
    z = np.array([math.log(3.0), 0.0])
    np.testing.assert_allclose(fused.gated_rmsnorm(o, z, w, 0.0),
                               [0.6363961030678928, 1.1313708498984762], rtol=1e-15)
    np.testing.assert_allclose(fused.gated_rmsnorm(o, z, w, 12.5), [0.45, 0.8], rtol=1e-15)


def test_gated_rmsnorm_rows_over_values():
    """Unit weight and a saturated gate: every (token, head) row over the value axis has
    mean square exactly 1 (eps = 0); positive scaling of o changes nothing, negation flips
    the sign; zero rows stay zero."""
    rng = np.random.default_rng(8)
    o = rng.standard_normal((6, 3, 10))                       # [T, H, V], V != H
    z = np.full_like(o, 60.0)
    y = fused.gated_rmsnorm(o, z, np.ones(10), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-14)
    zr = rng.standard_normal(o.shape)
    w = rng.normal(1.0, 0.1, 10)
    y1 = fused.gated_rmsnorm(o, zr, w, 0.0)
    np.testing.assert_allclose(fused.gated_rmsnorm(3.25 * o, zr, w, 0.0), y1, rtol=1e-14)
    np.testing.assert_allclose(fused.gated_rmsnorm(-o, zr, w, 0.0), -y1, rtol=1e-14)
    o0 = o.copy()
    o0[1, 2] = 0.0
    for eps in (0.0, 1e-6):
        y0 = fused.gated_rmsnorm(o0, zr, w, eps)
        assert np.all(y0[1, 2] == 0.0) and np.all(np.isfinite(y0))


def test_gated_rmsnorm_gate_after_norm():
    """The sigmoid gate multiplies the normalised output: halving one element's gate
    halves that element only (a gate applied before the norm would move every element of
    the row)."""
    rng = np.random.default_rng(9)
    o = rng.standard_normal(16)
    z = np.full(16, 60.0)
    y = fused.gated_rmsnorm(o, z, np.ones(16), 0.0)
    z2 = z.copy()
    z2[5] = 0.0                                               # sigmoid 1 -> 1/2
    y2 = fused.gated_rmsnorm(o, z2, np.ones(16), 0.0)
    np.testing.assert_allclose(y2[5], 0.5 * y[5], rtol=1e-14)
    np.testing.assert_allclose(np.delete(y2, 5), np.delete(y, 5), rtol=1e-15)


# ----------------------------------------------------------------------- composition

def _fused_case(seed, T, H, K, V):
    rng = np.random.default_rng(seed)
    A_log, b = _params(seed + 100, H, K)
    return dict(q=rng.standard_normal((T, H, K)), k=rng.standard_normal((T, H, K)),
                v=rng.standard_normal((T, H, V)), x=rng.standard_normal((T, H, K)),
                A_log=A_log, dt_bias=b, beta=rng.random((T, H)),
                z=rng.standard_normal((T, H, V)), w=rng.normal(1.0, 0.1, V))


def test_fused_fwd_ignores_qk_scale():
    """normalize_qk: positive per-(token, head) rescaling of raw q and k changes nothing."""
    c = _fused_case(10, 40, 2, 6, 5)
    o1, S1 = oracle.kda_fused_fwd(c["q"], c["k"], c["v"], c["x"], c["A_log"], c["dt_bias"],
                                  c["beta"])
    rng = np.random.default_rng(11)
    sq = rng.uniform(0.1, 10.0, (40, 2, 1))
    sk = rng.uniform(0.1, 10.0, (40, 2, 1))
    o2, S2 = oracle.kda_fused_fwd(c["q"] * sq, c["k"] * sk, c["v"], c["x"], c["A_log"],
                                  c["dt_bias"], c["beta"])
    np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(S2, S1, rtol=1e-11, atol=1e-13)


def test_fused_gate_decays_key_rows_in_closed_form():
    """beta = 0: the state only decays, row c (key channel c) by prod_t (1 + e^(x_t + b_c))
    ^ -exp(A_log): a closed form through the gate's sigmoid, with H, K and V all distinct."""
    T, H, K, V = 7, 2, 3, 4
    c = _fused_case(12, T, H, K, V)
    rng = np.random.default_rng(13)
    S0 = rng.standard_normal((1, H, K, V))
    _, S = oracle.kda_fused_fwd(c["q"], c["k"], c["v"], c["x"], c["A_log"], c["dt_bias"],
                                np.zeros((T, H)), initial_state=S0)
    for h in range(H):
        base = 1.0 + np.exp(c["x"][:, h, :] + c["dt_bias"][h])           # [T, K]
        decay = np.prod(base ** (-math.exp(c["A_log"][h])), axis=0)      # [K]
        np.testing.assert_allclose(S[0, h], S0[0, h] * decay[:, None], rtol=1e-13)


def test_fused_output_norm_ignores_value_scale():
    """With o_norm (eps = 0) and a zero initial state, o is linear in v, so scaling v by a
    positive constant leaves y unchanged while the state scales."""
    c = _fused_case(14, 30, 2, 4, 6)
    kw = dict(o_gate=c["z"], o_weight=c["w"], o_eps=0.0)
    y1, S1 = oracle.kda_fused_fwd(c["q"], c["k"], c["v"], c["x"], c["A_log"], c["dt_bias"],
                                  c["beta"], **kw)
    y2, S2 = oracle.kda_fused_fwd(c["q"], c["k"], 4.0 * c["v"], c["x"], c["A_log"],
                                  c["dt_bias"], c["beta"], **kw)
    np.testing.assert_allclose(y2, y1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S2, 4.0 * S1, rtol=1e-12, atol=1e-14)
    assert np.max(np.abs(np.mean(y1 ** 2 / (c["w"] * fused.sigmoid(c["z"])) ** 2, -1) - 1)) < 1e-12


def test_fused_prefill_then_decode_equals_prefill():
    """A fused prefill followed by fused decode steps (y and state) equals one fused
    prefill over the concatenated tokens."""
    T, P, H, K, V = 12, 9, 2, 4, 4
    c = _fused_case(15, T, H, K, V)
    kw = dict(o_weight=c["w"], o_eps=1e-6)
    y_all, S_all = oracle.kda_fused_fwd(c["q"], c["k"], c["v"], c["x"], c["A_log"],
                                        c["dt_bias"], c["beta"], o_gate=c["z"], **kw)
    sl = slice(0, P)
    y_p, S = oracle.kda_fused_fwd(c["q"][sl], c["k"][sl], c["v"][sl], c["x"][sl], c["A_log"],
                                  c["dt_bias"], c["beta"][sl], o_gate=c["z"][sl], **kw)
    np.testing.assert_allclose(y_p, y_all[:P], rtol=1e-12, atol=1e-14)
    for t in range(P, T):
        y_t, S = oracle.kda_fused_decode_step(c["q"][t:t + 1], c["k"][t:t + 1], c["v"][t:t + 1],
                                              c["x"][t:t + 1], c["A_log"], c["dt_bias"],
                                              c["beta"][t:t + 1], S, o_gate=c["z"][t:t + 1], **kw)
        np.testing.assert_allclose(y_t[0], y_all[t], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(S, S_all, rtol=1e-11, atol=1e-13)


# -------------------------------------------------------------------- short convolution

def test_short_conv_impulse_response_by_hand():
    """Taps (1, 2, 3, 4), the last one on the current token: an impulse at t = 1 in channel 0
    comes out as 4, 3, 2, 1 at t = 1..4; channel 1 sees nothing (depthwise)."""
    x = np.zeros((7, 2))
    x[1, 0] = 1.0
    w = np.array([[1.0, 2.0, 3.0, 4.0], [0.5, -1.0, 2.0, 1.0]])
    y, f = oracle.short_conv(x, w, activation=None)
    np.testing.assert_array_equal(y[:, 0], [0.0, 4.0, 3.0, 2.0, 1.0, 0.0, 0.0])
    np.testing.assert_array_equal(y[:, 1], 0.0)
    np.testing.assert_array_equal(f[0], x[4:7])


def test_short_conv_step_response_and_bias():
    """A constant input c with a zero state ramps through the partial tap sums, then holds
    c * sum(w) + bias: c = 2, taps (1, 2, 3, 4), bias 0.5 -> 8.5, 14.5, 18.5, 20.5, 20.5."""
    x = np.full((5, 1), 2.0)
    y, _ = oracle.short_conv(x, np.array([[1.0, 2.0, 3.0, 4.0]]), np.array([0.5]), activation=None)
    np.testing.assert_array_equal(y[:, 0], [8.5, 14.5, 18.5, 20.5, 20.5])


def test_silu_closed_forms():
    assert fused.silu(0.0) == 0.0
    assert fused.silu(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    z = np.linspace(-20.0, 20.0, 81)
    np.testing.assert_allclose(fused.silu(-z), fused.silu(z) - z, rtol=0, atol=1e-13)
    # the activation acts on the biased sum: zero input gives silu(bias)
    y, _ = oracle.short_conv(np.zeros((3, 2)), np.ones((2, 4)), np.array([1.5, -2.0]))
    np.testing.assert_allclose(y, np.broadcast_to(fused.silu(np.array([1.5, -2.0])), (3, 2)),
                               rtol=1e-15)


def test_short_conv_is_causal_and_carries_its_state():
    """Outputs never depend on later tokens; running a sequence in two parts with the conv
    state carried equals one run (outputs and final state), for every split point."""
    rng = np.random.default_rng(20)
    T, C, W = 11, 5, 4
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    b = rng.standard_normal(C)
    s0 = rng.standard_normal((1, W - 1, C))
    y, f = oracle.short_conv(x, w, b, initial_state=s0)
    x2 = x.copy()
    x2[6:] += 10.0
    y2, _ = oracle.short_conv(x2, w, b, initial_state=s0)
    np.testing.assert_array_equal(y2[:6], y[:6])
    for m in range(T + 1):
        ya, fa = oracle.short_conv(x[:m], w, b, initial_state=s0)
        yb, fb = oracle.short_conv(x[m:], w, b, initial_state=fa)
        np.testing.assert_allclose(np.concatenate([ya, yb]), y, rtol=1e-14, atol=1e-14)
        np.testing.assert_array_equal(fb, f)


def test_short_conv_packed_equals_separate():
    """Packed sequences never see each other's tokens; a zero-length sequence returns its
    state unchanged and a one-token sequence shifts it by one."""
    rng = np.random.default_rng(21)
    lens = [5, 0, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    C, W = 3, 4
    x = rng.standard_normal((int(cu[-1]), C))
    w = rng.standard_normal((C, W))
    s0 = rng.standard_normal((len(lens), W - 1, C))
    y, f = oracle.short_conv(x, w, initial_state=s0, cu_seqlens=cu)
    for n in range(len(lens)):
        yn, fn = oracle.short_conv(x[cu[n]:cu[n + 1]], w, initial_state=s0[n:n + 1])
        np.testing.assert_array_equal(y[cu[n]:cu[n + 1]], yn)
        np.testing.assert_array_equal(f[n], fn[0])
    np.testing.assert_array_equal(f[1], s0[1])
    np.testing.assert_array_equal(f[2], np.concatenate([s0[2][1:], x[cu[2]:cu[3]]]))
