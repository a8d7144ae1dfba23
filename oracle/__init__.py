"""KDA oracle: a plain, slow, float64 CPU implementation of the KDA core.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. The product path (the HIP
library and its binding) never imports, links or calls it, and shares no code with it.

Functions
---------
``kda_fwd``          token-by-token recurrence (C, float64, OpenMP over (sequence, head)):
                     the definition of what the chunked GPU prefill and the GPU decode step
                     compute. Pinned by tests/test_oracle_pins.py against closed forms,
                     exact rational arithmetic, invariants and reductions.
``kda_bwd``          the gradients of a loss through ``kda_fwd`` (C, float64): reverse-mode
                     differentiation of the recurrence, token by token. Pinned by
                     tests/test_oracle_bwd_pins.py against central finite differences of
                     ``kda_fwd``, exact Euler identities, a closed form without writes and
                     split/packed equalities.
``kda_decode_step``  one token per (sequence, head) on a persistent state: ``kda_fwd`` with
                     one-token sequences.
``chunked_fwd``      (oracle/chunked.py) the chunkwise form of the same recurrence in
                     float64 numpy, pinned by equality with ``kda_fwd``.
``fused``            (oracle/fused.py) the layer's fusions around the core: the forget gate
                     from its pre-activation, q/k L2 normalisation, the gated RMSNorm of the
                     output, and their composition with ``kda_fwd`` (``kda_fused_fwd``,
                     ``kda_fused_decode_step``); the short causal convolution with its conv
                     state (``short_conv``). Pinned by tests/test_oracle_fused_pins.py.

Nothing here is "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import build, lib_path  # noqa: F401
from .chunked import chunked_fwd  # noqa: F401

_lib = None


def _load():
    global _lib
    if _lib is None:
        p = lib_path()
        if not os.path.exists(p):
            build()
        lib = ctypes.CDLL(p)
        dp = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.kda_oracle_fwd.restype = ctypes.c_int
        lib.kda_oracle_fwd.argtypes = [ctypes.c_int64, i64p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, dp, dp, dp, dp, dp, ctypes.c_double,
                                       dp, dp, dp, ctypes.c_int]
        lib.kda_oracle_bwd.restype = ctypes.c_int
        lib.kda_oracle_bwd.argtypes = [ctypes.c_int64, i64p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, dp, dp, dp, dp, dp, ctypes.c_double,
                                       dp, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def _f64(a, shape=None):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def kda_fwd(q, k, v, g, beta, *, scale: float = 1.0, initial_state=None, cu_seqlens=None,
            threads: int = 0):
    """float64 recurrence over packed sequences.

    q, k, g: [T, H, K]; v: [T, H, V]; beta: [T, H]; cu_seqlens: int [N+1] (default: one
    sequence of T tokens); initial_state: [N, H, K, V] or None (zeros).
    A leading batch dimension [B, T, ...] is accepted and means B sequences of T tokens.
    Returns (o [.., H, V] float64, final_state [N, H, K, V] float64).
    """
    q = np.asarray(q)
    batched = q.ndim == 4
    if batched:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens requires unbatched [T, H, D] inputs")
        B, T = q.shape[:2]
        cu_seqlens = np.arange(B + 1, dtype=np.int64) * T
        q, k, v, g = (np.asarray(x).reshape(B * T, *np.asarray(x).shape[2:]) for x in (q, k, v, g))
        beta = np.asarray(beta).reshape(B * T, -1)
    Tt, H, K = q.shape
    V = np.asarray(v).shape[-1]
    if cu_seqlens is None:
        cu_seqlens = np.array([0, Tt], dtype=np.int64)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = len(cu) - 1
    if cu[-1] != Tt:
        raise ValueError("cu_seqlens[-1] must equal the number of tokens")
    q = _f64(q, (Tt, H, K))
    k = _f64(k, (Tt, H, K))
    g = _f64(g, (Tt, H, K))
    v = _f64(v, (Tt, H, V))
    beta = _f64(beta, (Tt, H))
    s0 = None if initial_state is None else _f64(initial_state, (N, H, K, V))
    o = np.zeros((Tt, H, V), dtype=np.float64)
    s_out = np.zeros((N, H, K, V), dtype=np.float64)
    rc = _load().kda_oracle_fwd(N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, K, V,
                                _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                                _ptr(s0), _ptr(o), _ptr(s_out), int(threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_fwd failed with code {rc}")
    if batched:
        o = o.reshape(B, T, H, V)
    return o, s_out


def kda_bwd(q, k, v, g, beta, do, *, scale: float = 1.0, initial_state=None, dfinal_state=None,
            cu_seqlens=None, threads: int = 0):
    """float64 gradients through ``kda_fwd`` of a loss with gradients ``do`` = dL/do (shape
    of o) and ``dfinal_state`` = dL/dS_final ([N, H, K, V] or None: zero).

    Layouts as ``kda_fwd`` (a leading batch dimension [B, T, ...] means B sequences).
    Returns (dq, dk, dv, dg, dbeta, dinitial_state), float64, shaped like q, k, v, g, beta
    and [N, H, K, V].
    """
    q = np.asarray(q)
    batched = q.ndim == 4
    if batched:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens requires unbatched [T, H, D] inputs")
        B, T = q.shape[:2]
        cu_seqlens = np.arange(B + 1, dtype=np.int64) * T
        q, k, v, g, do = (np.asarray(x).reshape(B * T, *np.asarray(x).shape[2:])
                          for x in (q, k, v, g, do))
        beta = np.asarray(beta).reshape(B * T, -1)
    Tt, H, K = q.shape
    V = np.asarray(v).shape[-1]
    if cu_seqlens is None:
        cu_seqlens = np.array([0, Tt], dtype=np.int64)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = len(cu) - 1
    if cu[-1] != Tt:
        raise ValueError("cu_seqlens[-1] must equal the number of tokens")
    q = _f64(q, (Tt, H, K))
    k = _f64(k, (Tt, H, K))
    g = _f64(g, (Tt, H, K))
    v = _f64(v, (Tt, H, V))
    do = _f64(do, (Tt, H, V))
    beta = _f64(beta, (Tt, H))
    s0 = None if initial_state is None else _f64(initial_state, (N, H, K, V))
    dsT = None if dfinal_state is None else _f64(dfinal_state, (N, H, K, V))
    dq = np.zeros((Tt, H, K))
    dk = np.zeros((Tt, H, K))
    dg = np.zeros((Tt, H, K))
    dv = np.zeros((Tt, H, V))
    db = np.zeros((Tt, H))
    ds0 = np.zeros((N, H, K, V))
    rc = _load().kda_oracle_bwd(N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, K, V,
                                _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                                _ptr(s0), _ptr(do), _ptr(dsT), _ptr(dq), _ptr(dk), _ptr(dv),
                                _ptr(dg), _ptr(db), _ptr(ds0), int(threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_bwd failed with code {rc}")
    if batched:
        dq, dk, dg = (x.reshape(B, T, H, K) for x in (dq, dk, dg))
        dv = dv.reshape(B, T, H, V)
        db = db.reshape(B, T, H)
    return dq, dk, dv, dg, db, ds0


def kda_decode_step(q, k, v, g, beta, state, *, scale: float = 1.0, threads: int = 0):
    """One token per (sequence, head): q, k, g [N, H, K]; v [N, H, V]; beta [N, H];
    state [N, H, K, V]. Returns (o [N, H, V], new_state [N, H, K, V]), float64."""
    q = np.asarray(q)
    N = q.shape[0]
    cu = np.arange(N + 1, dtype=np.int64)
    return kda_fwd(q, k, v, g, beta, scale=scale, initial_state=state, cu_seqlens=cu,
                   threads=threads)


from . import fused  # noqa: E402,F401  (needs kda_fwd above)
from .fused import kda_fused_decode_step, kda_fused_fwd, short_conv  # noqa: E402,F401
