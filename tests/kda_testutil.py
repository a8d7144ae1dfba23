"""Helpers shared by the GPU parity tests: upload seeded inputs, run the oracle on the same
values, and compare with the max-error / RMS statistic."""

from __future__ import annotations

import os
import sys

import numpy as np
import pytest

import oracle
import synth

DEV = "cuda"


def torch_mod():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no HIP device visible: GPU tests need an MI355X")
    return torch


def note(msg: str):
    """Name the case on stderr before its GPU step (survives a crash of the process)."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def to_dev(arr: np.ndarray, stored: str | None = None):
    torch = torch_mod()
    a = np.ascontiguousarray(arr)
    if stored == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def f64(arr: np.ndarray, stored: str | None = None) -> np.ndarray:
    if stored in ("bf16", "f32") and arr.dtype in (np.uint16, np.float32):
        return synth.stored_to_f64(arr, stored)
    return np.asarray(arr, dtype=np.float64)


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    err = float(np.max(np.abs(got - ref)))
    return err / rms if rms > 0 else err


def assert_close(got, ref, tol: float, what: str):
    e = rel_err(got, ref)
    print(f"[parity] {what}: max|err|/RMS = {e:.3e} (tol {tol:.0e})", file=sys.stderr, flush=True)
    assert np.all(np.isfinite(np.asarray(got))), f"{what}: non-finite values"
    assert e <= tol, f"{what}: max|err|/RMS(ref) = {e:.3e} > {tol:.1e}"
    return e


def assert_close_bf16_out(got, ref, tol: float, what: str):
    """For outputs stored as bf16: every element within tol * RMS(ref) * (1 + 2^-8) plus its
    own rounding, half a bf16 ulp (at most 2^-8 |ref| relative)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    bound = tol * rms * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref)
    worst = float(np.max(err / bound)) if err.size else 0.0
    print(f"[parity] {what}: max|err|/RMS = {float(np.max(err)) / rms:.3e}, "
          f"max err/bound = {worst:.3f}", file=sys.stderr, flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert worst <= 1.0, f"{what}: error exceeds tol*RMS + 2^-8|ref| (ratio {worst:.3f})"


def oracle_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def run_oracle(x: dict, stored: str, scale: float = 1.0, initial_state=None, cu=None):
    return oracle.kda_fwd(f64(x["q"], stored), f64(x["k"], stored), f64(x["v"], stored),
                          f64(x["g"]), f64(x["beta"]), scale=scale,
                          initial_state=None if initial_state is None else f64(initial_state),
                          cu_seqlens=cu, threads=oracle_threads())


def random_inputs(seed: int, T: int, H: int, D: int, stored: str, g_const: float | None = None,
                  beta_mu: float = 0.0):
    """Seeded token-major inputs [T, H, D] from the workload generator's distributions."""
    w = synth.Workload(f"case{seed}", 1000 + seed, H=H, K=D, V=D, chunk=64, dtype=stored,
                       B=1, T=T, beta_mu=beta_mu)
    x = synth.make_inputs(w)
    if g_const is not None:
        x["g"][:] = np.float32(g_const)
    return x


def random_states(seed: int, N: int, H: int, D: int) -> np.ndarray:
    w = synth.Workload(f"state{seed}", 2000 + seed, H=H, K=D, V=D, chunk=64, dtype="f32")
    return np.stack([np.stack([synth.initial_state(w, n, h) for h in range(H)])
                     for n in range(N)])
