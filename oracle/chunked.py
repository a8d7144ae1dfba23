"""Chunkwise form of the KDA recurrence in float64 numpy (test infrastructure only).

The KV-cache page ("Starting from the KV-cache explosion: what KimiLinear's linear
attention solves", section 6) names the chunked parallel form with a WY representation
as what turns the recurrence into GPU-friendly matrix products, with chunk sizes of 64 to
128 (section 3: chunk_size 64). This module writes that form out plainly, one chunk at a
time, so that the algebra the GPU kernel implements is itself checked against the
token-by-token oracle (tests/test_oracle_pins.py). Derivation, per chunk of L tokens with
state S entering it and G_i = sum_{t<=i} g_t (per key channel, from the chunk start):

* Unrolling S_t = Diag(e^{g_t}) S_{t-1} + k_t u_t^T with the delta-rule correction
  u_t = beta_t (v_t - S_{t-1}^T Diag(e^{g_t}) k_t) gives, for every token i of the chunk,
  u_i = beta_i v_i - beta_i (k_i * e^{G_i})^T S - sum_{j<i} A_ij u_j with
  A_ij = beta_i sum_c k_i[c] k_j[c] e^{G_i[c] - G_j[c]}  (j < i).
* So (I + A) U = Diag(beta) V - Diag(beta) (K * e^G) S, i.e. with T = (I + A)^{-1}:
  U = T Diag(beta) V - T Diag(beta) (K * e^G) S = U~ - W S.
* Outputs: O = scale [(Q * e^G) S + M U] with M_ij = sum_c q_i[c] k_j[c] e^{G_i[c]-G_j[c]}
  for j <= i.
* Next state: S' = Diag(e^{G_L}) S + (K * e^{G_L - G})^T U.
"""

from __future__ import annotations

import numpy as np


def _chunk(q, k, v, g, beta, S, scale):
    L = q.shape[0]
    G = np.cumsum(g, axis=0)                                   # [L, K]
    diff = G[:, None, :] - G[None, :, :]                       # G_i - G_j, [L, L, K]
    lower = np.tril(np.ones((L, L), dtype=bool))               # j <= i
    strict = np.tril(np.ones((L, L), dtype=bool), -1)          # j < i
    dec = np.where(lower[:, :, None], np.exp(np.where(lower[:, :, None], diff, 0.0)), 0.0)
    kk = np.einsum("ic,jc,ijc->ij", k, k, dec)
    A = np.where(strict, beta[:, None] * kk, 0.0)
    M = np.where(lower, np.einsum("ic,jc,ijc->ij", q, k, dec), 0.0)
    T = np.linalg.inv(np.eye(L) + A)
    eG = np.exp(G)
    W = T @ (beta[:, None] * k * eG)
    Ut = T @ (beta[:, None] * v)
    U = Ut - W @ S
    O = scale * ((q * eG) @ S + M @ U)
    S_next = np.exp(G[-1])[:, None] * S + (k * np.exp(G[-1][None, :] - G)).T @ U
    return O, S_next


def chunked_fwd(q, k, v, g, beta, *, chunk: int, scale: float = 1.0, initial_state=None,
                cu_seqlens=None):
    """Same contract as ``oracle.kda_fwd`` (unbatched [T, H, D] inputs), computed chunk by
    chunk; the last chunk of each sequence may be shorter than ``chunk``."""
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g))
    beta = np.asarray(beta, dtype=np.float64)
    Tt, H, K = q.shape
    V = v.shape[-1]
    cu = np.array([0, Tt]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    o = np.zeros((Tt, H, V))
    S_out = np.zeros((N, H, K, V))
    for n in range(N):
        for h in range(H):
            S = np.zeros((K, V)) if initial_state is None else \
                np.array(initial_state[n, h], dtype=np.float64)
            for t0 in range(int(cu[n]), int(cu[n + 1]), chunk):
                t1 = min(t0 + chunk, int(cu[n + 1]))
                sl = slice(t0, t1)
                o[sl, h], S = _chunk(q[sl, h], k[sl, h], v[sl, h], g[sl, h], beta[sl, h], S,
                                     scale)
            S_out[n, h] = S
    return o, S_out
