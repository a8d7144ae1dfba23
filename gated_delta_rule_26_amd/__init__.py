"""MI355X (gfx950) KDA core: Kimi Delta Attention's gated delta rule with per-channel decay.

A thin binding over the C ABI of ``include/kda.h`` (``libkda.so``, built in-tree by
``gated_delta_rule_26_amd/build.py``). The functions carry the C names and only marshal
arguments: shapes and pointers are taken from torch tensors on the HIP device, outputs are
allocated with torch, and every step of the computation runs in the library's HIP kernels
on the caller's current torch stream. There is no CPU or PyTorch fallback: if the library
is missing, loading fails loudly.
"""

from __future__ import annotations

import ctypes
import os

__all__ = ["KdaError", "kda_chunk_fwd", "kda_decode_step", "kda_chunk_fwd_fused",
           "kda_decode_step_fused", "kda_recurrent_fwd", "kda_short_conv_fwd", "kda_short_conv_update",
           "kda_chunk_bwd", "kda_chunk_bwd_noalloc", "check_cu_seqlens", "chunk_fwd_workspace_bytes", "chunk_bwd_workspace_bytes", "load_library", "KDA_F32", "KDA_BF16"]

KDA_F32, KDA_BF16 = 0, 1
_STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARGUMENT", 2: "KDA_ERR_UNSUPPORTED",
           3: "KDA_ERR_WORKSPACE_TOO_SMALL", 4: "KDA_ERR_HIP"}

_LIB = None
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

# Debugging aid: with KDA_CHECK_CU_SEQLENS=1 in the environment, every call that takes packed
# offsets first checks them on the host (a copy that synchronises the stream). Without it the
# offsets are a precondition: the kernels clamp them to [0, T], so malformed offsets give
# wrong results but no access outside the caller's arrays.
CHECK_CU_SEQLENS = os.environ.get("KDA_CHECK_CU_SEQLENS", "0") not in ("", "0")


class _Fusion(ctypes.Structure):
    """Mirror of the C struct kda_fusion (include/kda.h)."""
    _fields_ = [("gate_x", ctypes.c_void_p), ("A_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p), ("normalize_qk", ctypes.c_int32),
                ("o_gate", ctypes.c_void_p), ("o_weight", ctypes.c_void_p),
                ("o_eps", ctypes.c_float)]


class KdaError(RuntimeError):
    """A non-OK kda_status, with the library's detail message."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libkda.so (once) and declare the C signatures. Raises if it is not built."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libkda.so not found at {p}: build it with "
                           "`python gated_delta_rule_26_amd/build.py`")
    # torch first: its HIP runtime must be the one the process uses (libkda resolves against
    # the already loaded runtime), or torch and the library would disagree on devices/streams
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    i32, f32, vp, sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [i32]
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_version.restype = i32
    lib.kda_version.argtypes = []
    lib.kda_chunk_fwd_workspace_bytes.restype = sz
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [i32] * 8
    lib.kda_chunk_fwd.restype = i32
    lib.kda_chunk_fwd.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, f32,
                                  vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.kda_chunk_bwd_workspace_bytes.restype = sz
    lib.kda_chunk_bwd_workspace_bytes.argtypes = [i32] * 8
    lib.kda_chunk_bwd.restype = i32
    lib.kda_chunk_bwd.argtypes = [i32, i32, i32, i32, i32, i32, i32, f32,
                                  vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                  vp, i32, vp, sz, vp]
    lib.kda_chunk_bwd_noalloc.restype = i32
    lib.kda_chunk_bwd_noalloc.argtypes = [i32, i32, i32, i32, i32, i32, i32, f32,
                                          vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                          vp, i32, vp]
    lib.kda_probe_copy.restype = i32
    lib.kda_probe_copy.argtypes = [vp, vp, sz, vp]
    lib.kda_probe_read.restype = i32
    lib.kda_probe_read.argtypes = [vp, sz, vp]
    lib.kda_probe_rmw.restype = i32
    lib.kda_probe_rmw.argtypes = [vp, sz, f32, vp]
    lib.kda_probe_mfma_f16.restype = i32
    lib.kda_probe_mfma_f16.argtypes = [i32, i32, i32, vp, vp]
    lib.kda_probe_mfma_bf16.restype = i32
    lib.kda_probe_mfma_bf16.argtypes = [i32, i32, i32, vp, vp]
    lib.kda_probe_mfma_f16_flops.restype = ctypes.c_double
    lib.kda_probe_mfma_f16_flops.argtypes = [i32, i32]
    lib.kda_decode_step.restype = i32
    lib.kda_decode_step.argtypes = [i32, i32, i32, i32, i32, i32, f32,
                                    vp, vp, vp, vp, vp, vp, vp, vp]
    fp = ctypes.POINTER(_Fusion)
    lib.kda_chunk_fwd_fused.restype = i32
    lib.kda_chunk_fwd_fused.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, f32,
                                        vp, vp, vp, fp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.kda_decode_step_fused.restype = i32
    lib.kda_decode_step_fused.argtypes = [i32, i32, i32, i32, i32, i32, f32,
                                          vp, vp, vp, fp, vp, vp, vp, vp]
    lib.kda_recurrent_fwd.restype = i32
    lib.kda_recurrent_fwd.argtypes = [i32, i32, i32, i32, i32, i32, i32, f32,
                                      vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kda_short_conv_fwd.restype = i32
    lib.kda_short_conv_fwd.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                       vp, i32, vp]
    lib.kda_short_conv_update.restype = i32
    lib.kda_short_conv_update.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    if path is None:
        _LIB = lib
    return lib


def _check(lib, status: int):
    if status != 0:
        raise KdaError(status, lib.kda_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _on_stream(fn):
    """Run the call with ``stream`` (when given) as torch's current stream, so that every
    buffer the binding allocates (outputs, the internal workspace) comes from the stream the
    kernels run on. torch's caching allocator ties a block to the stream current when it was
    allocated: a workspace taken from another stream and freed on return could be handed to
    that stream's next allocation while the kernels on ``stream`` still use it."""
    import functools

    @functools.wraps(fn)
    def call(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, stream=None, **kw)
        import torch
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kw)
    return call


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported input dtype {t.dtype}")


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _req(t, name, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a torch tensor on the HIP device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def check_cu_seqlens(cu_seqlens, T: int) -> None:
    """Raise ValueError unless the packed offsets are valid for T tokens: int32, one
    dimension, cu[0] = 0, nondecreasing, cu[-1] = T. Accepts a torch tensor (copied to the
    host) or anything numpy can read."""
    import numpy as np
    try:
        import torch
        if isinstance(cu_seqlens, torch.Tensor):
            if cu_seqlens.dtype != torch.int32:
                raise ValueError(f"cu_seqlens must be int32, got {cu_seqlens.dtype}")
            cu_seqlens = cu_seqlens.detach().cpu().numpy()
    except ImportError:
        pass
    cu = np.asarray(cu_seqlens)
    if cu.ndim != 1 or cu.size < 1:
        raise ValueError("cu_seqlens must be one-dimensional with N + 1 >= 1 entries")
    if cu.dtype != np.int32:
        raise ValueError(f"cu_seqlens must be int32, got {cu.dtype}")
    if cu[0] != 0:
        raise ValueError(f"cu_seqlens[0] must be 0, got {int(cu[0])}")
    d = np.diff(cu.astype(np.int64))
    if (d < 0).any():
        i = int(np.argmax(d < 0))
        raise ValueError(f"cu_seqlens must be nondecreasing: cu[{i}] = {int(cu[i])} > cu[{i + 1}] = {int(cu[i + 1])}")
    if int(cu[-1]) != T:
        raise ValueError(f"cu_seqlens[-1] must equal the token count {T}, got {int(cu[-1])}")


def _prefill_layout(q, k, v, beta, cu_seqlens):
    """(B, T, N, H, Dk, Dv) of a prefill call, after checking q, k, v, beta, cu_seqlens."""
    import torch
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _req(t, nm, q.dtype)
    _req(beta, "beta", torch.float32)
    if cu_seqlens is not None:
        _req(cu_seqlens, "cu_seqlens", torch.int32)
        if q.dim() == 4:
            if q.shape[0] != 1:
                raise ValueError("cu_seqlens requires B == 1")
        B, T = 1, q.shape[-3]
        N = cu_seqlens.numel() - 1
    else:
        if q.dim() != 4:
            raise ValueError("q must be [B, T, H, Dk] without cu_seqlens")
        B, T = q.shape[0], q.shape[1]
        N = B
    H, Dk = q.shape[-2], q.shape[-1]
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1] or beta.shape != q.shape[:-1]:
        raise ValueError("inconsistent q/k/v/beta shapes")
    if cu_seqlens is not None and CHECK_CU_SEQLENS:
        check_cu_seqlens(cu_seqlens, T)
    return B, T, N, H, Dk, Dv


def _prefill_states(q, N, H, Dk, Dv, initial_state, final_state, output_final_state):
    import torch
    if initial_state is not None:
        _req(initial_state, "initial_state", torch.float32)
        if tuple(initial_state.shape) != (N, H, Dk, Dv):
            raise ValueError(f"initial_state must be [{N}, {H}, {Dk}, {Dv}]")
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    elif final_state is not None:
        _req(final_state, "final_state", torch.float32)
        if tuple(final_state.shape) != (N, H, Dk, Dv):
            raise ValueError(f"final_state must be [{N}, {H}, {Dk}, {Dv}]")
    return final_state


def _prefill_workspace(lib, q, B, T, N, H, Dk, Dv, chunk, split, workspace):
    import torch
    if not split:
        return None, 0
    if workspace is not None:
        _req(workspace, "workspace", torch.uint8)
        return workspace, workspace.numel()
    ws = lib.kda_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, chunk, _dtype_code(q), N)
    return (torch.empty(ws, dtype=torch.uint8, device=q.device) if ws else None), ws


def _fusion(q, k, gate_x, A_log, dt_bias, normalize_qk, o_gate, o_weight, o_eps, v):
    """Check the fused-step tensors and build the C struct (the tensors stay referenced by
    the caller for the duration of the call)."""
    import torch
    _req(gate_x, "gate_x", q.dtype)
    if gate_x.shape != q.shape:
        raise ValueError("gate_x must have q's shape")
    H, Dk = q.shape[-2], q.shape[-1]
    _req(A_log, "A_log", torch.float32)
    _req(dt_bias, "dt_bias", torch.float32)
    if tuple(A_log.shape) != (H,) or tuple(dt_bias.shape) != (H, Dk):
        raise ValueError(f"A_log must be [{H}] and dt_bias [{H}, {Dk}]")
    if o_gate is not None:
        _req(o_gate, "o_gate", q.dtype)
        if o_gate.shape != v.shape:
            raise ValueError("o_gate must have v's shape")
        _req(o_weight, "o_weight", torch.float32)
        if tuple(o_weight.shape) != (v.shape[-1],):
            raise ValueError(f"o_weight must be [{v.shape[-1]}]")
    return _Fusion(gate_x.data_ptr(), A_log.data_ptr(), dt_bias.data_ptr(),
                   1 if normalize_qk else 0,
                   None if o_gate is None else o_gate.data_ptr(),
                   None if o_gate is None else o_weight.data_ptr(), float(o_eps))


def _out(o, like, dtype, name="o"):
    import torch
    if o is None:
        return torch.empty(like.shape, dtype=dtype, device=like.device)
    _req(o, name, dtype)
    if o.shape != like.shape:
        raise ValueError(f"{name} must have shape {tuple(like.shape)}")
    return o


@_on_stream
def kda_chunk_fwd(q, k, v, g, beta, *, initial_state=None, output_final_state: bool = True,
                  final_state=None, cu_seqlens=None, chunk: int = 64, scale: float = 1.0,
                  o=None, stream=None, split: bool = True, workspace=None):
    """Chunked KDA prefill (C: kda_chunk_fwd).

    q, k: [B, T, H, Dk] (or [T, H, Dk] with ``cu_seqlens``), bf16 or float32, unit L2 norm
    per token and head; v: [.., H, Dv] same dtype; g: float32 log-decay like q; beta:
    float32 [.., H]; initial_state: float32 [N, H, Dk, Dv] or None (zeros); cu_seqlens:
    int32 [N + 1] on the device (packed sequences, B = 1). ``final_state`` may be given
    (it may be ``initial_state`` itself) or is allocated when ``output_final_state``.
    ``split`` provides the optional workspace with which the library cuts long sequences
    into segments run in parallel (few chains); False computes each chain in one pass.
    ``workspace`` (a device uint8 tensor of at least ``chunk_fwd_workspace_bytes(...)``
    bytes) is used instead of allocating one per call.
    Returns (o float32 [.., H, Dv], final_state or None).
    """
    import torch
    lib = load_library()
    B, T, N, H, Dk, Dv = _prefill_layout(q, k, v, beta, cu_seqlens)
    _req(g, "g", torch.float32)
    if g.shape != q.shape:
        raise ValueError("g must have q's shape")
    final_state = _prefill_states(q, N, H, Dk, Dv, initial_state, final_state, output_final_state)
    o = _out(o, v, torch.float32)
    workspace, ws = _prefill_workspace(lib, q, B, T, N, H, Dk, Dv, chunk, split, workspace)
    st = lib.kda_chunk_fwd(B, T, H, Dk, Dv, chunk, _dtype_code(q), KDA_F32, float(scale),
                           _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                           _ptr(initial_state), _ptr(final_state), _ptr(o),
                           _ptr(cu_seqlens), N, _ptr(workspace), ws, _stream(stream))
    _check(lib, st)
    return o, final_state


@_on_stream
def kda_chunk_bwd(q, k, v, g, beta, do, *, initial_state=None, dfinal_state=None,
                  cu_seqlens=None, chunk: int = 64, scale: float = 1.0,
                  want_dinitial_state: bool = True, grads=None, workspace=None, stream=None):
    """Backward pass of ``kda_chunk_fwd`` (C: kda_chunk_bwd).

    q, k, v, g, beta, initial_state, cu_seqlens, chunk and scale are those of the forward
    call; do: float32 like v (dL/do); dfinal_state: float32 [N, H, Dk, Dv] (dL/dS_final) or
    None (zero). ``grads`` may supply the five output tensors (dq, dk, dv, dg, dbeta) and
    ``workspace`` a device uint8 tensor of at least ``chunk_bwd_workspace_bytes(...)`` bytes;
    otherwise they are allocated. Returns (dq, dk, dv, dg, dbeta, dinitial_state or None),
    all float32.
    """
    import torch
    lib = load_library()
    B, T, N, H, Dk, Dv = _prefill_layout(q, k, v, beta, cu_seqlens)
    _req(g, "g", torch.float32)
    if g.shape != q.shape:
        raise ValueError("g must have q's shape")
    _req(do, "do", torch.float32)
    if do.shape != v.shape:
        raise ValueError("do must have v's shape")
    _prefill_states(q, N, H, Dk, Dv, initial_state, None, False)
    if dfinal_state is not None:
        _req(dfinal_state, "dfinal_state", torch.float32)
        if tuple(dfinal_state.shape) != (N, H, Dk, Dv):
            raise ValueError(f"dfinal_state must be [{N}, {H}, {Dk}, {Dv}]")
    if grads is None:
        grads = (None,) * 5
    dq, dk, dv, dg, db = grads
    dq = _out(dq, q, torch.float32, "dq")
    dk = _out(dk, q, torch.float32, "dk")
    dv = _out(dv, v, torch.float32, "dv")
    dg = _out(dg, q, torch.float32, "dg")
    db = _out(db, beta, torch.float32, "dbeta")
    ds0 = (torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
           if want_dinitial_state else None)
    need = lib.kda_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, chunk, _dtype_code(q), N)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    else:
        _req(workspace, "workspace", torch.uint8)
    st = lib.kda_chunk_bwd(B, T, H, Dk, Dv, chunk, _dtype_code(q), float(scale),
                           _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                           _ptr(do), _ptr(dfinal_state), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                           _ptr(db), _ptr(ds0), _ptr(cu_seqlens), N, _ptr(workspace),
                           workspace.numel(), _stream(stream))
    _check(lib, st)
    return dq, dk, dv, dg, db, ds0


@_on_stream
def kda_chunk_bwd_noalloc(q, k, v, g, beta, do, *, grads, dinitial_state=None, initial_state=None,
                          dfinal_state=None, cu_seqlens=None, chunk: int = 64, scale: float = 1.0,
                          stream=None):
    """Backward pass with the library's fixed scratch in place of a workspace (C:
    kda_chunk_bwd_noalloc), for callers that cannot allocate: the five gradient tensors
    (dq, dk, dv, dg, dbeta) must be given in ``grads``, and ``dinitial_state`` (float32
    [N, H, Dk, Dv]) if that gradient is wanted; nothing is allocated. Arguments otherwise as
    ``kda_chunk_bwd``; returns (dq, dk, dv, dg, dbeta, dinitial_state)."""
    import torch
    lib = load_library()
    B, T, N, H, Dk, Dv = _prefill_layout(q, k, v, beta, cu_seqlens)
    _req(g, "g", torch.float32)
    if g.shape != q.shape:
        raise ValueError("g must have q's shape")
    _req(do, "do", torch.float32)
    if do.shape != v.shape:
        raise ValueError("do must have v's shape")
    _prefill_states(q, N, H, Dk, Dv, initial_state, None, False)
    if dfinal_state is not None:
        _req(dfinal_state, "dfinal_state", torch.float32)
        if tuple(dfinal_state.shape) != (N, H, Dk, Dv):
            raise ValueError(f"dfinal_state must be [{N}, {H}, {Dk}, {Dv}]")
    if dinitial_state is not None:
        _req(dinitial_state, "dinitial_state", torch.float32)
        if tuple(dinitial_state.shape) != (N, H, Dk, Dv):
            raise ValueError(f"dinitial_state must be [{N}, {H}, {Dk}, {Dv}]")
    dq, dk, dv, dg, db = grads
    for t, like, nm in ((dq, q, "dq"), (dk, q, "dk"), (dv, v, "dv"), (dg, q, "dg"), (db, beta, "dbeta")):
        _req(t, nm, torch.float32)
        if t.shape != like.shape:
            raise ValueError(f"{nm} must have shape {tuple(like.shape)}")
    st = lib.kda_chunk_bwd_noalloc(B, T, H, Dk, Dv, chunk, _dtype_code(q), float(scale),
                                   _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                   _ptr(do), _ptr(dfinal_state), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                                   _ptr(db), _ptr(dinitial_state), _ptr(cu_seqlens), N, _stream(stream))
    _check(lib, st)
    return dq, dk, dv, dg, db, dinitial_state


def kda_probe_copy(src, dst, stream=None):
    """dst = src with the library's copy probe (C: kda_probe_copy); both contiguous device
    tensors of the same byte size (a multiple of 16)."""
    lib = load_library()
    _req(src, "src")
    _req(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same byte size")
    _check(lib, lib.kda_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def kda_probe_read(src, stream=None):
    """Read all of ``src`` (a contiguous device tensor, a multiple of 16 bytes) with the
    library's read probe (C: kda_probe_read)."""
    lib = load_library()
    _req(src, "src")
    _check(lib, lib.kda_probe_read(_ptr(src), src.numel() * src.element_size(), _stream(stream)))


def kda_probe_rmw(buf, factor: float = 1.0, stream=None):
    """buf *= factor in place with the library's read-modify-write probe (C: kda_probe_rmw);
    ``buf`` is a contiguous float32 device tensor."""
    import torch
    lib = load_library()
    _req(buf, "buf", torch.float32)
    _check(lib, lib.kda_probe_rmw(_ptr(buf), buf.numel() * 4, float(factor), _stream(stream)))


def kda_probe_mfma_f16(iters: int, blocks: int, sink, shape: int = 0, stream=None) -> float:
    """Run the fp16 matrix-core probe (C: kda_probe_mfma_f16; shape 0: 16x16x32, 1: 32x32x16
    instructions) into ``sink`` (float32, at least blocks * 256 elements); returns the launch's
    dense fp16 flops."""
    import torch
    lib = load_library()
    _req(sink, "sink", torch.float32)
    if sink.numel() < blocks * 256:
        raise ValueError("sink needs blocks * 256 elements")
    _check(lib, lib.kda_probe_mfma_f16(int(shape), int(iters), int(blocks), _ptr(sink), _stream(stream)))
    return float(lib.kda_probe_mfma_f16_flops(int(iters), int(blocks)))


def kda_probe_mfma_bf16(iters: int, blocks: int, sink, shape: int = 0, stream=None) -> float:
    """The same probe with bf16 operands (C: kda_probe_mfma_bf16); returns the launch's dense
    bf16 flops."""
    import torch
    lib = load_library()
    _req(sink, "sink", torch.float32)
    if sink.numel() < blocks * 256:
        raise ValueError("sink needs blocks * 256 elements")
    _check(lib, lib.kda_probe_mfma_bf16(int(shape), int(iters), int(blocks), _ptr(sink), _stream(stream)))
    return float(lib.kda_probe_mfma_f16_flops(int(iters), int(blocks)))


def chunk_bwd_workspace_bytes(q, v, *, chunk: int = 64, num_seqs: int | None = None) -> int:
    """Bytes of workspace kda_chunk_bwd needs for q [B, T, H, Dk] (or [T, H, Dk] packed) / v
    (C: kda_chunk_bwd_workspace_bytes)."""
    lib = load_library()
    B, T, H, Dk = q.shape if q.dim() == 4 else (1, *q.shape)
    N = B if num_seqs is None else num_seqs
    return int(lib.kda_chunk_bwd_workspace_bytes(B, T, H, Dk, v.shape[-1], chunk,
                                                 _dtype_code(q), N))


def chunk_fwd_workspace_bytes(q, v, *, chunk: int = 64, num_seqs: int | None = None) -> int:
    """Bytes of optional workspace kda_chunk_fwd can use for q [B, T, H, Dk] / v (C:
    kda_chunk_fwd_workspace_bytes); 0 when no sequence split applies."""
    lib = load_library()
    B, T, H, Dk = q.shape if q.dim() == 4 else (1, *q.shape)
    N = B if num_seqs is None else num_seqs
    return int(lib.kda_chunk_fwd_workspace_bytes(B, T, H, Dk, v.shape[-1], chunk,
                                                 _dtype_code(q), N))


@_on_stream
def kda_decode_step(q, k, v, g, beta, state, *, scale: float = 1.0, o=None, stream=None):
    """One KDA decode step (C: kda_decode_step): q, k, g [N, H, Dk]; v [N, H, Dv]; beta
    [N, H]; ``state`` float32 [N, H, Dk, Dv] is updated in place. Returns o float32 [N, H, Dv]."""
    import torch
    lib = load_library()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _req(t, nm, q.dtype)
    _req(g, "g", torch.float32)
    _req(beta, "beta", torch.float32)
    _req(state, "state", torch.float32)
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or tuple(v.shape) != (N, H, Dv) or \
            tuple(beta.shape) != (N, H) or tuple(state.shape) != (N, H, Dk, Dv):
        raise ValueError("inconsistent decode shapes")
    if o is None:
        o = torch.empty((N, H, Dv), dtype=torch.float32, device=q.device)
    else:
        _req(o, "o", torch.float32)
    st = lib.kda_decode_step(N, H, Dk, Dv, _dtype_code(q), KDA_F32, float(scale),
                             _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                             _ptr(o), _stream(stream))
    _check(lib, st)
    return o


@_on_stream
def kda_chunk_fwd_fused(q, k, v, gate_x, A_log, dt_bias, beta, *, normalize_qk: bool = True,
                        o_gate=None, o_weight=None, o_eps: float = 1e-6, out_dtype=None,
                        initial_state=None, output_final_state: bool = True, final_state=None,
                        cu_seqlens=None, chunk: int = 64, scale: float = 1.0, o=None,
                        stream=None, split: bool = True, workspace=None):
    """Chunked KDA prefill with the layer's fused steps (C: kda_chunk_fwd_fused).

    As ``kda_chunk_fwd``, but the log-decay comes from the gate's pre-activation:
    gate_x (q's shape and dtype), A_log float32 [H], dt_bias float32 [H, Dk]; q and k may be
    raw (``normalize_qk``); with ``o_gate`` (v's shape and dtype), ``o_weight`` float32 [Dv]
    and ``o_eps`` the output is the gated RMSNorm of o, in ``out_dtype`` (float32 by
    default, or torch.bfloat16). Returns (o or y, final_state or None).
    """
    import torch
    lib = load_library()
    B, T, N, H, Dk, Dv = _prefill_layout(q, k, v, beta, cu_seqlens)
    fz = _fusion(q, k, gate_x, A_log, dt_bias, normalize_qk, o_gate, o_weight, o_eps, v)
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    final_state = _prefill_states(q, N, H, Dk, Dv, initial_state, final_state, output_final_state)
    o = _out(o, v, out_dtype)
    workspace, ws = _prefill_workspace(lib, q, B, T, N, H, Dk, Dv, chunk, split, workspace)
    st = lib.kda_chunk_fwd_fused(B, T, H, Dk, Dv, chunk, _dtype_code(q), _dtype_code(o),
                                 float(scale), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(fz),
                                 _ptr(beta), _ptr(initial_state), _ptr(final_state), _ptr(o),
                                 _ptr(cu_seqlens), N, _ptr(workspace), ws, _stream(stream))
    _check(lib, st)
    return o, final_state


@_on_stream
def kda_decode_step_fused(q, k, v, gate_x, A_log, dt_bias, beta, state, *,
                          normalize_qk: bool = True, o_gate=None, o_weight=None,
                          o_eps: float = 1e-6, out_dtype=None, scale: float = 1.0, o=None,
                          stream=None):
    """One KDA decode step with the layer's fused steps (C: kda_decode_step_fused): inputs as
    ``kda_decode_step`` with gate_x/A_log/dt_bias in place of g, optional raw q/k and optional
    output norm (see ``kda_chunk_fwd_fused``). ``state`` is updated in place."""
    import torch
    lib = load_library()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _req(t, nm, q.dtype)
    _req(beta, "beta", torch.float32)
    _req(state, "state", torch.float32)
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or tuple(v.shape) != (N, H, Dv) or tuple(beta.shape) != (N, H) or \
            tuple(state.shape) != (N, H, Dk, Dv):
        raise ValueError("inconsistent decode shapes")
    fz = _fusion(q, k, gate_x, A_log, dt_bias, normalize_qk, o_gate, o_weight, o_eps, v)
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    o = _out(o, v, out_dtype)
    st = lib.kda_decode_step_fused(N, H, Dk, Dv, _dtype_code(q), _dtype_code(o), float(scale),
                                   _ptr(q), _ptr(k), _ptr(v), ctypes.byref(fz), _ptr(beta),
                                   _ptr(state), _ptr(o), _stream(stream))
    _check(lib, st)
    return o


_ACT = {None: 0, "none": 0, "silu": 1}


@_on_stream
def kda_short_conv_fwd(x, weight, bias=None, *, initial_state=None, final_state=None,
                       output_final_state: bool = True, cu_seqlens=None, activation="silu",
                       y=None, stream=None):
    """The short causal convolution over a prefill batch (C: kda_short_conv_fwd).

    x: [B, T, C] (or [T, C] with ``cu_seqlens``), bf16 or float32; weight: float32 [C, W]
    (the last tap on the current token); bias: float32 [C] or None; initial_state: [N, W-1, C]
    in x's dtype or None. Returns (y like x, final_state [N, W-1, C] or None); the final state
    may be given as ``final_state`` (``initial_state`` itself for an in-place cache update).
    """
    import torch
    lib = load_library()
    _req(x, "x")
    _req(weight, "weight", torch.float32)
    if bias is not None:
        _req(bias, "bias", torch.float32)
    if cu_seqlens is not None:
        _req(cu_seqlens, "cu_seqlens", torch.int32)
        if x.dim() == 3 and x.shape[0] != 1:
            raise ValueError("cu_seqlens requires B == 1")
        B, T, N = 1, x.shape[-2], cu_seqlens.numel() - 1
        if CHECK_CU_SEQLENS:
            check_cu_seqlens(cu_seqlens, T)
    else:
        if x.dim() != 3:
            raise ValueError("x must be [B, T, C] without cu_seqlens")
        B, T, N = x.shape[0], x.shape[1], x.shape[0]
    C, W = x.shape[-1], weight.shape[-1]
    if tuple(weight.shape) != (C, W) or (bias is not None and tuple(bias.shape) != (C,)):
        raise ValueError(f"weight must be [{C}, W] and bias [{C}]")
    for t, nm in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None:
            _req(t, nm, x.dtype)
            if tuple(t.shape) != (N, W - 1, C):
                raise ValueError(f"{nm} must be [{N}, {W - 1}, {C}]")
    if final_state is None and output_final_state:
        final_state = torch.empty((N, W - 1, C), dtype=x.dtype, device=x.device)
    y = _out(y, x, x.dtype, "y")
    st = lib.kda_short_conv_fwd(B, T, C, W, _dtype_code(x), _ACT[activation], _ptr(x),
                                _ptr(weight), _ptr(bias), _ptr(initial_state), _ptr(final_state),
                                _ptr(y), _ptr(cu_seqlens), N, _stream(stream))
    _check(lib, st)
    return y, final_state


@_on_stream
def kda_short_conv_update(x, weight, bias, state, *, activation="silu", y=None, stream=None):
    """One decode token per sequence (C: kda_short_conv_update): x [N, C]; state [N, W-1, C]
    in x's dtype, shifted in place. Returns y like x."""
    import torch
    lib = load_library()
    _req(x, "x")
    _req(weight, "weight", torch.float32)
    if bias is not None:
        _req(bias, "bias", torch.float32)
    _req(state, "state", x.dtype)
    N, C = x.shape
    W = weight.shape[-1]
    if tuple(weight.shape) != (C, W) or tuple(state.shape) != (N, W - 1, C):
        raise ValueError("inconsistent short-convolution shapes")
    y = _out(y, x, x.dtype, "y")
    st = lib.kda_short_conv_update(N, C, W, _dtype_code(x), _ACT[activation], _ptr(x),
                                   _ptr(weight), _ptr(bias), _ptr(state), _ptr(y), _stream(stream))
    _check(lib, st)
    return y


@_on_stream
def kda_recurrent_fwd(q, k, v, g, beta, state, *, scale: float = 1.0, o=None, stream=None):
    """L tokens per (sequence, head) on the persistent state (C: kda_recurrent_fwd): q, k, g
    [N, L, H, Dk]; v [N, L, H, Dv]; beta [N, L, H]; ``state`` float32 [N, H, Dk, Dv] is
    updated in place. Returns o float32 [N, L, H, Dv]."""
    import torch
    lib = load_library()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _req(t, nm, q.dtype)
    _req(g, "g", torch.float32)
    _req(beta, "beta", torch.float32)
    _req(state, "state", torch.float32)
    N, L, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or tuple(v.shape) != (N, L, H, Dv) or \
            tuple(beta.shape) != (N, L, H) or tuple(state.shape) != (N, H, Dk, Dv):
        raise ValueError("inconsistent recurrent shapes")
    o = _out(o, v, torch.float32)
    st = lib.kda_recurrent_fwd(N, L, H, Dk, Dv, _dtype_code(q), KDA_F32, float(scale),
                               _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                               _ptr(o), _stream(stream))
    _check(lib, st)
    return o
