"""Seeded synthetic inputs for the KDA core (gated delta rule with per-channel decay).

This package only draws random inputs and converts between storage dtypes. It holds
none of the method's arithmetic: the recurrence, its chunked form and everything the
kernels compute live elsewhere. Both the CPU oracle's tests and the GPU path's tests and
benchmark draw their inputs from here, so the two sides always see identical values.

Every (sequence n, head h) slab of every tensor has its own numpy PCG64 stream, keyed by
``SeedSequence([ROOT_SEED, workload_id, tensor_id, n, h])``, so any slab can be
regenerated alone (the oracle checks sampled slabs of workloads far too large to
recompute whole).

Distributions (the workloads of the KDA pages: head_dim 128, chunk 64, retention-biased
forget gate, write gate centred on 0.5; q and k L2-normalised, as the pages require for a
stable delta-rule erase term):

* q, k ~ N(0, 1) per token and head, L2-normalised per token in float64 (no epsilon),
  then rounded to the storage dtype (bf16 round-to-nearest-even from the float64 value,
  or float32).
* v ~ N(0, 1), rounded to the storage dtype.
* beta = sigmoid(N(beta_mu, 1)) per token and head, float32.
* log-decay g = -exp(a_h) * softplus(x + b_{h,c}), with a_h ~ U(ln 0.01, ln 0.5) per head,
  b_{h,c} ~ N(b_mu, 0.5) per head and key channel (drawn once per workload, like model
  parameters), and x ~ N(0, 1) per token and channel; float32, always < 0.
* optional initial states: M ~ N(0,1)^{K x V} in float64 divided by its largest singular
  value, stored as float32.
* packed lengths: round(LogNormal(ln 8192, 1.4)), clipped to [1024, 65536].

Fused-layer inputs (``fused_slab``, ``make_fused_inputs``): the raw values that the layer
feeds the fused entry points, drawn from streams of their own. q, k ~ N(0, 1) are NOT
normalised; the gate's pre-activation x ~ N(0, 1) and the output gate's pre-activation
z ~ N(0, 1) are rounded to the storage dtype like q, k, v; A_log = a_h and dt_bias = b_{h,c}
are the gate parameters above, stored as float32; the output norm's gain is
1 + N(0, 0.1^2) per value channel (float32) and its epsilon 1e-6. v and beta are the same
as in the core workloads.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

ROOT_SEED = 20260

# tensor ids inside the seed key
_T_Q, _T_K, _T_V, _T_BETA, _T_X, _T_S0 = 0, 1, 2, 3, 4, 6
_P_A, _P_B, _P_LEN = 10, 11, 12
_T_QR, _T_KR, _T_XG, _T_Z, _P_W = 20, 21, 22, 23, 13
_P_CW, _P_CB, _T_CS = 14, 15, 24
_T_DO, _T_DST = 25, 26    # upstream gradients of the backward pass: dL/do, dL/dS_final
NORM_EPS = 1e-6


@dataclass(frozen=True)
class Workload:
    """Shape and distribution recipe of one synthetic workload.

    Fixed-length workloads have ``B`` sequences of ``T`` tokens. Decode workloads have
    ``B`` sequences of ``prefill_T + decode_steps`` tokens: the first ``prefill_T`` tokens
    build the state, the rest are fed one decode step at a time. Packed workloads have
    ``n_seqs`` sequences whose lengths come from :func:`seq_lengths`.
    """

    name: str
    wid: int
    H: int
    K: int
    V: int
    chunk: int
    dtype: str  # storage dtype of q, k, v: "bf16" or "f32"
    beta_mu: float = 0.0
    b_mu: float = -2.0
    B: int = 1
    T: int = 0
    prefill_T: int = 0
    decode_steps: int = 0
    n_seqs: int = 0
    len_median: int = 8192
    len_sigma: float = 1.4
    len_min: int = 1024
    len_max: int = 65536
    spectral_init: bool = False

    @property
    def packed(self) -> bool:
        return self.n_seqs > 0

    @property
    def decode(self) -> bool:
        return self.decode_steps > 0

    @property
    def tokens_per_seq(self) -> int:
        return self.prefill_T + self.decode_steps if self.decode else self.T

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # fp32 everywhere, tiny: the fp32 parity case
    "tiny_f32": Workload("tiny_f32", 0, H=2, K=16, V=16, chunk=16, dtype="f32", B=1, T=256),
    # bf16 q/k/v, fp32 gates/state, one 4K sequence, 16 heads
    "prefill_4k_h16": Workload("prefill_4k_h16", 1, H=16, K=128, V=128, chunk=64,
                               dtype="bf16", B=1, T=4096),
    # long context, retention-biased decay and beta centred higher
    "prefill_128k_h32": Workload("prefill_128k_h32", 2, H=32, K=128, V=128, chunk=64,
                                 dtype="bf16", beta_mu=0.5, b_mu=-4.0, B=1, T=131072),
    # 256 sequences x 32 heads: 2048-token prefill, then 1000 decode steps
    "decode_256x32": Workload("decode_256x32", 3, H=32, K=128, V=128, chunk=64,
                              dtype="bf16", B=256, prefill_T=2048, decode_steps=1000),
    # 64 packed sequences, ~1M tokens, per-sequence spectral-norm-1 initial states
    "varlen_64seq_h16": Workload("varlen_64seq_h16", 4, H=16, K=128, V=128, chunk=64,
                                 dtype="bf16", n_seqs=64, spectral_init=True),
}


# ----------------------------------------------------------------------------- dtypes

def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (round to nearest, ties to even) directly from
    the float64 value; returns the 16-bit patterns as uint16. Finite, normal-range inputs
    only (all generated values are)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    u = x.view(np.uint64)
    # bf16 keeps 7 of float64's 52 stored mantissa bits: drop 45 with RNE
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = (u + np.uint64(0x0FFFFFFFFFFF) + lsb) & ~np.uint64(0x1FFFFFFFFFFF)
    f = r.view(np.float64).astype(np.float32)  # exact: 8 significant bits
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def stored_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a stored q/k/v array (uint16 bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f64_to_bf16_bits(x64)
    if dtype == "f32":
        return x64.astype(np.float32)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, *key])))


# ------------------------------------------------------------------------- parameters

def gate_params(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    """Per-head a_h ~ U(ln 0.01, ln 0.5) and per-(head, channel) b ~ N(b_mu, 0.5)."""
    a = _rng(w.wid, _P_A).uniform(math.log(0.01), math.log(0.5), size=w.H)
    b = _rng(w.wid, _P_B).normal(w.b_mu, 0.5, size=(w.H, w.K))
    return a, b


def seq_lengths(w: Workload) -> np.ndarray:
    """Sequence lengths of a workload (int64)."""
    if not w.packed:
        return np.full(w.B, w.tokens_per_seq, dtype=np.int64)
    raw = _rng(w.wid, _P_LEN).lognormal(math.log(w.len_median), w.len_sigma, size=w.n_seqs)
    return np.clip(np.rint(raw), w.len_min, w.len_max).astype(np.int64)


def initial_state(w: Workload, n: int, h: int) -> np.ndarray:
    """float32 [K, V] state with spectral norm 1 (to float32 rounding)."""
    m = _rng(w.wid, _T_S0, n, h).standard_normal((w.K, w.V))
    s = np.linalg.svd(m, compute_uv=False)[0]
    return (m / s).astype(np.float32)


# ------------------------------------------------------------------------------ slabs

def slab(w: Workload, n: int, h: int, L: int | None = None,
         params: tuple[np.ndarray, np.ndarray] | None = None) -> dict:
    """All per-token inputs of sequence ``n``, head ``h`` (``L`` tokens, default the
    workload's length for that sequence). q, k, v are stored arrays (uint16 bf16 bits or
    float32) of shape [L, K] / [L, V]; g is float32 [L, K]; beta float32 [L]."""
    if L is None:
        L = int(seq_lengths(w)[n]) if w.packed else w.tokens_per_seq
    a, b = params if params is not None else gate_params(w)
    out = {}
    for name, tid in (("q", _T_Q), ("k", _T_K)):
        x = _rng(w.wid, tid, n, h).standard_normal((L, w.K))
        x /= np.sqrt(np.einsum("td,td->t", x, x))[:, None]
        out[name] = _store(x, w.dtype)
    out["v"] = _store(_rng(w.wid, _T_V, n, h).standard_normal((L, w.V)), w.dtype)
    z = _rng(w.wid, _T_BETA, n, h).standard_normal(L) + w.beta_mu
    out["beta"] = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    x = _rng(w.wid, _T_X, n, h).standard_normal((L, w.K)) + b[h][None, :]
    out["g"] = (-math.exp(a[h]) * np.logaddexp(0.0, x)).astype(np.float32)
    return out


def norm_weight(w: Workload) -> np.ndarray:
    """float32 [V] gain of the output norm."""
    return (1.0 + 0.1 * _rng(w.wid, _P_W).standard_normal(w.V)).astype(np.float32)


def conv_params(w: Workload, C: int, which: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """float32 taps [C, 4] and bias [C] of one short convolution (``which`` tells the
    layer's convolutions apart)."""
    weight = _rng(w.wid, _P_CW, which).uniform(-0.5, 0.5, size=(C, 4)).astype(np.float32)
    bias = _rng(w.wid, _P_CB, which).uniform(-0.5, 0.5, size=C).astype(np.float32)
    return weight, bias


def conv_state(w: Workload, N: int, C: int, which: int = 0) -> np.ndarray:
    """Initial conv states [N, 3, C] in the storage dtype (the 3 inputs before each sequence)."""
    return _store(_rng(w.wid, _T_CS, which).standard_normal((N, 3, C)), w.dtype)


def grad_out(w: Workload, n: int, h: int, L: int | None = None) -> np.ndarray:
    """float32 [L, V] upstream gradient dL/do of sequence ``n``, head ``h``: N(0, 1), like
    the gradient a loss hands back through the layer."""
    if L is None:
        L = int(seq_lengths(w)[n]) if w.packed else w.tokens_per_seq
    return _rng(w.wid, _T_DO, n, h).standard_normal((L, w.V)).astype(np.float32)


def grad_state(w: Workload, N: int) -> np.ndarray:
    """float32 [N, H, K, V] upstream gradient dL/dS_final, N(0, 1)."""
    return _rng(w.wid, _T_DST).standard_normal((N, w.H, w.K, w.V)).astype(np.float32)


def fused_slab(w: Workload, n: int, h: int, L: int | None = None) -> dict:
    """Raw fused-layer inputs of sequence ``n``, head ``h``: q, k, x [L, K] and v, z [L, V]
    as stored arrays (unnormalised q and k), beta float32 [L]."""
    if L is None:
        L = int(seq_lengths(w)[n]) if w.packed else w.tokens_per_seq
    out = {}
    for name, tid, D in (("q", _T_QR, w.K), ("k", _T_KR, w.K), ("x", _T_XG, w.K),
                         ("z", _T_Z, w.V), ("v", _T_V, w.V)):
        out[name] = _store(_rng(w.wid, tid, n, h).standard_normal((L, D)), w.dtype)
    z = _rng(w.wid, _T_BETA, n, h).standard_normal(L) + w.beta_mu
    out["beta"] = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    return out


def _workers(workers: int | None) -> int:
    if workers:
        return workers
    return max(1, min(16, os.cpu_count() or 1))


def make_inputs(w: Workload, seqs=None, workers: int | None = None, fused: bool = False) -> dict:
    """Assemble whole token-major tensors for a workload (or for the sequences ``seqs``,
    whose slabs are identical to those of the full workload).

    Returns numpy arrays: q, k [T_total, H, K]; v [T_total, H, V]; g [T_total, H, K];
    beta [T_total, H]; ``cu_seqlens`` int64 [N+1]; ``lengths``; ``initial_state``
    float32 [N, H, K, V] or None. For decode workloads the tensors cover the
    ``prefill_T``-token prefill, and ``dec_q``... ``dec_beta`` hold the decode tokens as
    [steps, N, H, D] (step-major, one token per sequence and head per step).

    ``fused=True``: the fused layer's raw inputs instead (``fused_slab``): q, k, x
    [T_total, H, K]; v, z [T_total, H, V]; beta; plus ``A_log`` float32 [H], ``dt_bias``
    float32 [H, K], ``norm_weight`` float32 [V] and ``norm_eps``.
    """
    all_len = seq_lengths(w)
    seqs = list(range(len(all_len))) if seqs is None else list(seqs)
    lengths = all_len[seqs]
    pre = lengths.copy()
    if w.decode:
        pre[:] = w.prefill_T
    cu = np.zeros(len(seqs) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(pre)
    Tt = int(cu[-1])
    kdt = np.uint16 if w.dtype == "bf16" else np.float32
    H, K, V = w.H, w.K, w.V
    if fused:  # name -> (width, dtype)
        spec = {"q": (K, kdt), "k": (K, kdt), "v": (V, kdt), "x": (K, kdt), "z": (V, kdt),
                "beta": (0, np.float32)}
    else:
        spec = {"q": (K, kdt), "k": (K, kdt), "v": (V, kdt), "g": (K, np.float32),
                "beta": (0, np.float32)}
    shp = lambda lead, D: lead + ((D,) if D else ())  # noqa: E731
    res = {name: np.empty(shp((Tt, H), D), dt) for name, (D, dt) in spec.items()}
    res.update({"cu_seqlens": cu, "lengths": pre, "seqs": np.asarray(seqs),
                "initial_state": None})
    S = w.decode_steps
    N = len(seqs)
    if S:
        res.update({"dec_" + name: np.empty(shp((S, N, H), D), dt)
                    for name, (D, dt) in spec.items()})
    if w.spectral_init:
        res["initial_state"] = np.empty((N, H, K, V), np.float32)
    params = gate_params(w)
    if fused:
        res["A_log"] = params[0].astype(np.float32)
        res["dt_bias"] = params[1].astype(np.float32)
        res["norm_weight"] = norm_weight(w)
        res["norm_eps"] = NORM_EPS

    def job(i_n_h):
        i, n, h = i_n_h
        s = (fused_slab(w, n, h, int(lengths[i])) if fused
             else slab(w, n, h, int(lengths[i]), params))
        t0, t1 = int(cu[i]), int(cu[i + 1])
        P = t1 - t0
        for key in spec:
            res[key][t0:t1, h] = s[key][:P]
            if S:
                res["dec_" + key][:, i, h] = s[key][P:P + S]
        if w.spectral_init:
            res["initial_state"][i, h] = initial_state(w, n, h)

    jobs = [(i, n, h) for i, n in enumerate(seqs) for h in range(H)]
    with ThreadPoolExecutor(_workers(workers)) as ex:
        list(ex.map(job, jobs))
    return res
