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


class WholeTensor:
    """The parity statistic of one returned tensor, accumulated slab by slab: max over all its
    elements of |gpu - ref| against tol * RMS(ref), the RMS also over all its elements.

    For a bf16-stored output every element may add its own rounding, half a bf16 ulp (at most
    2^-8 |ref|): each element within tol * RMS * (1 + 2^-8) + 2^-8 |ref|.

    For a row-normalised output (``pre`` = the oracle's values before the gated RMSNorm, and
    its epsilon): the core's bound on the pre-norm values, tol * RMS(pre) per element, grows
    through the normalisation of row t by 1 / sqrt(mean_t(pre^2) + eps), so a row whose RMS
    is a fraction of the tensor's gets its bound scaled by kappa_t = RMS(pre) /
    sqrt(mean_t(pre^2) + eps) where kappa_t > 1 (a well-conditioned row keeps the plain
    bound)."""

    def __init__(self, what: str, tol: float, bf16_out: bool = False):
        self.what, self.tol, self.bf16_out = what, tol, bf16_out
        self.max_err = 0.0
        self.max_excess = -np.inf  # max of |err| - 2^-8 |ref| (bf16 outputs)
        self.ss = 0.0
        self.n = 0
        self.rows = []             # (per-row max excess, per-row pre-norm RMS) of normalised outputs
        self.ss_pre = 0.0
        self.n_pre = 0

    def add(self, got, ref, pre=None, eps: float = 0.0):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        if got.shape != ref.shape:
            raise AssertionError(f"{self.what}: shape {got.shape} against {ref.shape}")
        if not np.all(np.isfinite(got)):
            raise AssertionError(f"{self.what}: non-finite values")
        if ref.size == 0:
            return
        err = np.abs(got - ref)
        self.max_err = max(self.max_err, float(err.max()))
        excess = err - 2.0 ** -8 * np.abs(ref) if self.bf16_out else err
        self.max_excess = max(self.max_excess, float(excess.max()))
        if pre is not None:
            pre = np.asarray(pre, dtype=np.float64)
            if pre.shape != ref.shape:
                raise AssertionError(f"{self.what}: pre-norm shape {pre.shape} against {ref.shape}")
            self.rows.append((excess.max(axis=-1).ravel(),
                              np.sqrt(np.mean(pre * pre, axis=-1) + eps).ravel()))
            self.ss_pre += float(np.sum(pre * pre))
            self.n_pre += pre.size
        self.ss += float(np.sum(ref * ref))
        self.n += ref.size

    def check(self, expect_n: int | None = None) -> float:
        if expect_n is not None and self.n != expect_n:
            raise AssertionError(f"{self.what}: compared {self.n} elements, expected {expect_n}")
        rms = float(np.sqrt(self.ss / self.n)) if self.n else 0.0
        e = self.max_err / rms if rms > 0 else self.max_err
        msg = f"[parity] {self.what}: max|err|/RMS = {e:.3e} over all {self.n} elements (tol {self.tol:.0e})"
        if self.bf16_out or self.rows:
            bound = self.tol * rms * ((1 + 2.0 ** -8) if self.bf16_out else 1.0)
            worst = max(self.max_excess, 0.0) / bound
            if self.rows:
                rms_pre = np.sqrt(self.ss_pre / self.n_pre)
                exc = np.concatenate([r[0] for r in self.rows])
                kappa = np.maximum(1.0, rms_pre / np.maximum(np.concatenate([r[1] for r in self.rows]), 1e-300))
                ratio = np.maximum(exc, 0.0) / kappa / bound
                i = int(np.argmax(ratio))
                worst = float(ratio[i])
                msg += (f", max err/bound = {worst:.3f} (row {i}: kappa {kappa[i]:.3g}; rows with kappa > 1: "
                        f"{int(np.sum(kappa > 1))} of {kappa.size}; unscaled max err/bound "
                        f"{max(self.max_excess, 0.0) / bound:.3f})")
            else:
                msg += f", max err/bound = {worst:.3f} (bf16 output)"
            print(msg, file=sys.stderr, flush=True)
            assert worst <= 1.0, f"{self.what}: error exceeds its bound (ratio {worst:.3f})"
        else:
            print(msg, file=sys.stderr, flush=True)
            assert e <= self.tol, f"{self.what}: max|err|/RMS(ref) = {e:.3e} > {self.tol:.1e}"
        return e
