"""kda_chunk_bwd on the GPU against the float64 oracle's backward (oracle.kda_bwd).

Every returned gradient (dq, dk, dv, dg, dbeta, dS_init) is compared separately with the
statistic of the forward tests: max |gpu - oracle| <= tol * RMS(oracle). The backward runs
in float32 throughout, so the float32-input instantiations take the float32 tolerance 1e-4.
The bf16-input instantiation sees the same bf16 values as the oracle and also computes in
float32; it is held to the float32 bound times 10 (1e-3), well inside the 2e-2 budget of the
bf16 forward: its only extra error over float32 inputs is the longer chunk (64) and larger
head dimension (128) over which rounding accumulates.
"""

import numpy as np
import pytest

import gated_delta_rule_26_amd as kda
import oracle
import synth
from kda_testutil import (assert_close, f64, note, oracle_threads, random_inputs, random_states,
                          to_dev, torch_mod)

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 1e-3
NAMES = ["dq", "dk", "dv", "dg", "dbeta", "dS_init"]


def upstream(seed, lens, H, V, K, with_state=True):
    """Seeded dL/do [T, H, V] for packed sequences of the given lengths, and dL/dS_final."""
    w = synth.Workload(f"grad{seed}", 3000 + seed, H=H, K=K, V=V, chunk=64, dtype="f32")
    do = np.zeros((int(np.sum(lens)), H, V), np.float32)
    t = 0
    for n, L in enumerate(lens):
        for h in range(H):
            do[t:t + L, h] = synth.grad_out(w, n, h, int(L))
        t += int(L)
    dsT = synth.grad_state(w, len(lens)) if with_state else None
    return do, dsT


def run_case(x, stored, lens, *, chunk, s0=None, dsT=None, do, batched=False, scale=1.0):
    torch = torch_mod()
    H = x["q"].shape[1]
    N = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    if batched:
        T = int(lens[0])
        sh = lambda a: a.reshape(N, T, *a.shape[1:])  # noqa: E731
        cu_t = None
    else:
        sh = lambda a: a  # noqa: E731
        cu_t = to_dev(cu.astype(np.int32))
    q, k, v = (to_dev(sh(x[key]), stored) for key in ("q", "k", "v"))
    g, beta = to_dev(sh(x["g"])), to_dev(sh(x["beta"]))
    init = None if s0 is None else to_dev(np.ascontiguousarray(s0, np.float32))
    dfin = None if dsT is None else to_dev(np.ascontiguousarray(dsT, np.float32))
    got = kda.kda_chunk_bwd(q, k, v, g, beta, to_dev(sh(do)), initial_state=init, dfinal_state=dfin,
                            cu_seqlens=cu_t, chunk=chunk, scale=scale)
    torch.cuda.synchronize()
    got = [t.reshape(-1, *t.shape[-2:]).cpu().numpy() if i < 4 else t.cpu().numpy()
           for i, t in enumerate(got)]
    got[4] = got[4].reshape(-1, H)
    ref = oracle.kda_bwd(f64(x["q"], stored), f64(x["k"], stored), f64(x["v"], stored), f64(x["g"]),
                         f64(x["beta"]), f64(do), scale=scale,
                         initial_state=None if s0 is None else f64(s0),
                         dfinal_state=None if dsT is None else f64(dsT), cu_seqlens=cu,
                         threads=oracle_threads())
    return got, ref


def check(got, ref, tol):
    for name, a, b in zip(NAMES, got, ref):
        assert_close(a, b, tol, name)


def test_tiny_f32_workload():
    """The fp32 workload (T=256, H=2, Dk=Dv=16, chunk 16) with dL/do only."""
    w = synth.WORKLOADS["tiny_f32"]
    x = synth.make_inputs(w)
    do, _ = upstream(1, [256], 2, 16, 16, with_state=False)
    note("bwd tiny_f32")
    got, ref = run_case(x, "f32", [256], chunk=16, do=do)
    check(got, ref, TOL_F32)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 50, 100])
def test_f32_d16_ragged_with_states(T):
    H = 3
    x = random_inputs(500 + T, T, H, 16, "f32")
    s0 = random_states(501 + T, 1, H, 16)
    do, dsT = upstream(502 + T, [T], H, 16, 16)
    note(f"bwd f32 D=16 T={T}")
    got, ref = run_case(x, "f32", [T], chunk=16, s0=s0, dsT=dsT, do=do, scale=0.5)
    check(got, ref, TOL_F32)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_f32_d128_ragged_with_states(T):
    H = 2
    x = random_inputs(520 + T, T, H, 128, "f32")
    s0 = random_states(521 + T, 1, H, 128)
    do, dsT = upstream(522 + T, [T], H, 128, 128)
    note(f"bwd f32 D=128 T={T}")
    got, ref = run_case(x, "f32", [T], chunk=64, s0=s0, dsT=dsT, do=do, scale=0.7)
    check(got, ref, TOL_F32)


@pytest.mark.parametrize("stored", ["f32", "bf16"])
def test_d128_packed_with_empty_sequences(stored):
    lens = [0, 70, 1, 128, 5, 0, 300]
    H = 2
    x = random_inputs(540, int(np.sum(lens)), H, 128, stored)
    s0 = random_states(541, len(lens), H, 128)
    do, dsT = upstream(542, lens, H, 128, 128)
    note(f"bwd packed {stored}")
    got, ref = run_case(x, stored, lens, chunk=64, s0=s0, dsT=dsT, do=do)
    check(got, ref, TOL_F32 if stored == "f32" else TOL_BF16)


@pytest.mark.parametrize("stored", ["f32", "bf16"])
def test_d128_packed_many_chunk_aligned_sequences(stored):
    """40 packed sequences, many of whole chunks and some empty, over 4 heads: the record
    slots past each sequence's last chunk are unused, and with more (slot, head) items than
    compute units the persistent prep takes several items per workgroup with unused slots
    between them."""
    lens = [64, 0, 128, 64, 1, 192, 0, 64] * 5
    H = 4
    x = random_inputs(590, int(np.sum(lens)), H, 128, stored)
    s0 = random_states(591, len(lens), H, 128)
    do, dsT = upstream(592, lens, H, 128, 128)
    note(f"bwd packed chunk-aligned {stored}")
    got, ref = run_case(x, stored, lens, chunk=64, s0=s0, dsT=dsT, do=do)
    check(got, ref, TOL_F32 if stored == "f32" else TOL_BF16)


@pytest.mark.parametrize("stored", ["f32", "bf16"])
def test_d128_batched(stored):
    B, T, H = 3, 150, 2
    x = random_inputs(560, B * T, H, 128, stored)
    do, dsT = upstream(561, [T] * B, H, 128, 128)
    note(f"bwd batched {stored}")
    got, ref = run_case(x, stored, [T] * B, chunk=64, dsT=dsT, do=do, batched=True)
    check(got, ref, TOL_F32 if stored == "f32" else TOL_BF16)


def test_bf16_strong_decay_and_degenerate_gates():
    """Decay far beyond e^-60 inside a chunk (exact pairwise factors), zero write strengths
    and zero decay on some tokens."""
    T, H = 256, 2
    x = random_inputs(580, T, H, 128, "bf16")
    x["g"][40:90] *= 40.0           # about -40 per token in places
    x["beta"][100:120] = 0.0
    x["g"][150:200] = 0.0
    do, dsT = upstream(581, [T], H, 128, 128)
    note("bwd bf16 strong decay")
    got, ref = run_case(x, "bf16", [T], chunk=64, dsT=dsT, do=do)
    check(got, ref, TOL_BF16)


def test_f32_d16_extreme_decay():
    """The fp32 16-token-chunk instantiation with decay far beyond e^-60 inside a chunk (the
    pair-by-pair paths of prep and grad2), write strengths of zero on some tokens."""
    T, H = 70, 2
    x = random_inputs(600, T, H, 16, "f32")
    x["g"][10:40] *= 60.0
    x["beta"][45:50] = 0.0
    s0 = random_states(601, 1, H, 16)
    do, dsT = upstream(602, [T], H, 16, 16)
    note("bwd f32 D=16 extreme decay")
    got, ref = run_case(x, "f32", [T], chunk=16, s0=s0, dsT=dsT, do=do, scale=0.9)
    check(got, ref, TOL_F32)


def test_empty_sequence_hands_back_the_state_gradient():
    """B = 1, T = 0: no tokens, dS_init = dL/dS_final exactly."""
    torch = torch_mod()
    H, D = 2, 128
    dsT = random_states(610, 1, H, D)
    e = torch.empty((1, 0, H, D), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((1, 0, H, D), dtype=torch.float32, device="cuda")
    b = torch.empty((1, 0, H), dtype=torch.float32, device="cuda")
    note("bwd empty batch")
    got = kda.kda_chunk_bwd(e, e, e, g, b, g, dfinal_state=to_dev(dsT))
    torch.cuda.synchronize()
    assert np.array_equal(got[5].cpu().numpy(), dsT)
    assert all(t.numel() == 0 for t in got[:5])


def test_bf16_long_sequence_with_states():
    """One 16K-token sequence (256 chunks per chain: the state passes' long recurrences),
    an initial state and a final-state gradient, two heads."""
    T, H = 16384, 2
    x = random_inputs(620, T, H, 128, "bf16")
    s0 = random_states(621, 1, H, 128)
    do, dsT = upstream(622, [T], H, 128, 128)
    note("bwd bf16 T=16384")
    got, ref = run_case(x, "bf16", [T], chunk=64, s0=s0, dsT=dsT, do=do)
    check(got, ref, TOL_BF16)
