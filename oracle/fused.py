"""The KDA layer's input- and output-side fusions around the core, in float64.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it. It shares no code with the HIP
path.

What the fused entry points compute, step by step (each function below is one step):

1. ``kda_gate``   the channel-wise forget gate from its pre-activation. The loading page
                  (section 3) names the gate's parameters: ``A_log`` (the decay rate, one per
                  head) and ``dt_bias`` (a time-step bias, one per head and key channel),
                  applied to the output of the gate's low-rank projection. The functional
                  form, g = -exp(A_log_h) * softplus(x + dt_bias_{h,c}), is the reading
                  adopted here; it is the law the synthetic workloads draw their gates from.
                  g <= 0, so the gate exp(g) lies in (0, 1].
2. ``l2norm``     q and k divided by their Euclidean norm per (token, head): the KV-cache
                  page (section 3's ``normalize_kq`` and section 5) makes this mandatory for
                  a bounded delta-rule erase term. No epsilon; a zero vector stays zero.
3. the core recurrence (``oracle.kda_fwd``) on the normalised q, k and the gate's g.
4. ``gated_rmsnorm``  ``o_norm``: the loading page (section 3) says the output passes a gated
                  RMSNorm whose activation is fixed to sigmoid (sigmoid beats no gate and
                  Swish in the ablation). Reading adopted: per (token, head), over the
                  value dimension, y = o / sqrt(mean(o^2) + eps) * weight * sigmoid(z),
                  with z the output gate's pre-activation, weight a per-channel gain and
                  eps the config's rms_norm_eps (1e-6 in the loading page's config).

5. ``short_conv``  the short causal convolution in front of the core: the loading page
                  (section 3) gives the KDA layer a short convolution of kernel size 4, and
                  (section 6) a decode cache holding conv_states beside the recurrent states.
                  Reading adopted: a depthwise (per-channel) causal convolution over the
                  tokens of each sequence, y_t[c] = act(bias[c] + sum_j w[c, j] x_{t-W+1+j}[c]),
                  whose inputs before a sequence's first token come from its conv state (the
                  W - 1 previous inputs, oldest first; zeros without one); the final conv
                  state is the sequence's last W - 1 inputs. act is the identity or SiLU
                  (the pages name none).

Every function is pinned in tests/test_oracle_fused_pins.py (closed forms, identities and
invariances, not a retyping of these formulas).
"""

from __future__ import annotations

import numpy as np

from . import kda_fwd


def softplus(z):
    """log(1 + e^z), evaluated without overflow."""
    return np.logaddexp(0.0, np.asarray(z, dtype=np.float64))


def kda_gate(x, A_log, dt_bias):
    """Log-decay g[t, h, c] = -exp(A_log[h]) * softplus(x[t, h, c] + dt_bias[h, c]).

    x: [..., H, K] pre-activation; A_log: [H]; dt_bias: [H, K]. Returns float64 like x.
    """
    x = np.asarray(x, dtype=np.float64)
    A_log = np.asarray(A_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    H, K = x.shape[-2], x.shape[-1]
    if A_log.shape != (H,) or dt_bias.shape != (H, K):
        raise ValueError(f"A_log must be [{H}] and dt_bias [{H}, {K}]")
    rate = np.exp(A_log)[:, None]                   # [H, 1]
    return -rate * softplus(x + dt_bias)            # broadcasts over the leading dims


def l2norm(x):
    """x / ||x||_2 over the last axis; rows of zeros stay zero."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return np.exp(-np.logaddexp(0.0, -z))


def gated_rmsnorm(o, z, weight, eps):
    """y = o / sqrt(mean(o^2 over the last axis) + eps) * weight * sigmoid(z).

    o, z: [..., V]; weight: [V]; eps >= 0.
    """
    o = np.asarray(o, dtype=np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    inv = 1.0 / np.sqrt(ms + float(eps)) if eps > 0 else np.divide(
        1.0, np.sqrt(ms), out=np.zeros_like(ms), where=ms > 0)
    return o * inv * np.asarray(weight, dtype=np.float64) * sigmoid(z)


def kda_fused_fwd(q, k, v, x, A_log, dt_bias, beta, *, normalize_qk=True, o_gate=None,
                  o_weight=None, o_eps=1e-6, scale=1.0, initial_state=None, cu_seqlens=None,
                  threads=0):
    """The fused prefill: gate, optional q/k normalisation, the recurrence, optional o_norm.

    Layouts as ``oracle.kda_fwd`` (token-major [T, H, D], or batched [B, T, H, D]); x has
    q's shape; o_gate (if given) has v's shape, o_weight is [V]. Returns (y or o, final
    state), float64.
    """
    g = kda_gate(x, A_log, dt_bias)
    if normalize_qk:
        q, k = l2norm(q), l2norm(k)
    o, S = kda_fwd(q, k, v, g, beta, scale=scale, initial_state=initial_state,
                   cu_seqlens=cu_seqlens, threads=threads)
    if o_gate is not None:
        o = gated_rmsnorm(o, o_gate, o_weight, o_eps)
    return o, S


def kda_fused_decode_step(q, k, v, x, A_log, dt_bias, beta, state, *, normalize_qk=True,
                          o_gate=None, o_weight=None, o_eps=1e-6, scale=1.0):
    """One fused decode step for N sequences: inputs [N, H, D], state [N, H, K, V] (not
    modified). Returns (y or o [N, H, V], new state)."""
    q = np.asarray(q, dtype=np.float64)
    N = q.shape[0]
    cu = np.arange(N + 1)
    # N one-token sequences packed along the token axis
    o, S = kda_fused_fwd(q, np.asarray(k, np.float64), np.asarray(v, np.float64),
                         np.asarray(x, np.float64), A_log, dt_bias,
                         np.asarray(beta, np.float64), normalize_qk=normalize_qk,
                         o_gate=None if o_gate is None else np.asarray(o_gate, np.float64),
                         o_weight=o_weight, o_eps=o_eps, scale=scale,
                         initial_state=np.asarray(state, np.float64), cu_seqlens=cu)
    return o, S


def silu(z):
    """z * sigmoid(z)."""
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


def short_conv(x, weight, bias=None, *, initial_state=None, cu_seqlens=None,
               activation="silu"):
    """Depthwise causal convolution per sequence, with a conv state.

    x: [T, C] (packed sequences, ``cu_seqlens`` [N + 1]; default one sequence), weight: [C, W]
    (weight[c, W - 1] multiplies the current token), bias: [C] or None, initial_state:
    [N, W - 1, C] (the previous inputs, oldest first) or None (zeros). activation: "silu" or
    None. Returns (y [T, C], final_state [N, W - 1, C]), float64.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    T, C = x.shape
    W = w.shape[1]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    b = np.zeros(C) if bias is None else np.asarray(bias, dtype=np.float64)
    s0 = np.zeros((N, W - 1, C)) if initial_state is None else np.asarray(initial_state,
                                                                            dtype=np.float64)
    y = np.zeros((T, C))
    final = np.zeros((N, W - 1, C))
    for n in range(N):
        seq = x[cu[n]:cu[n + 1]]
        hist = np.concatenate([s0[n], seq])          # [W - 1 + L, C]: history, then the tokens
        for t in range(len(seq)):
            acc = b.copy()
            for j in range(W):                        # tap j sees input t - (W - 1) + j
                acc = acc + w[:, j] * hist[t + j]
            y[cu[n] + t] = acc
        final[n] = hist[len(hist) - (W - 1):]
    if activation == "silu":
        y = silu(y)
    elif activation is not None:
        raise ValueError(f"unknown activation {activation!r}")
    return y, final
