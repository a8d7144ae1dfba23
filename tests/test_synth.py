"""The seeded input generator: reproducibility, dtype rounding and distributions."""

import math

import numpy as np
import pytest

import synth
from synth import WORKLOADS


def _bf16_neighbours(bits):
    b = bits.astype(np.int32)
    return [synth.bf16_bits_to_f64(((b + d) & 0xFFFF).astype(np.uint16)) for d in (-1, 0, 1)]


def test_bf16_rounding_is_nearest_even_from_float64():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))
    # add exact ties between two bf16 values
    base = synth.bf16_bits_to_f64(synth.f64_to_bf16_bits(x[:1000]))
    _, e = np.frexp(base)
    ties = base + np.sign(base) * np.ldexp(1.0, e - 9)  # halfway to the next bf16 away from 0
    x = np.concatenate([x, ties])
    bits = synth.f64_to_bf16_bits(x)
    lo, mid, hi = _bf16_neighbours(bits)
    err = np.abs(mid - x)
    assert np.all(err <= np.abs(lo - x))
    assert np.all(err <= np.abs(hi - x))
    tie = (err == np.abs(lo - x)) | (err == np.abs(hi - x))
    assert np.all((bits[tie] & 1) == 0)
    assert tie.sum() >= 1000


def test_slabs_are_reproducible_and_subsets_match():
    w = WORKLOADS["prefill_4k_h16"].with_(T=300)
    s1 = synth.slab(w, 0, 3)
    s2 = synth.slab(w, 0, 3)
    for key in s1:
        np.testing.assert_array_equal(s1[key], s2[key])
    full = synth.make_inputs(w)
    for key in ("q", "k", "v", "g", "beta"):
        np.testing.assert_array_equal(full[key][:, 3], s1[key])
    w4 = WORKLOADS["varlen_64seq_h16"]
    lens = synth.seq_lengths(w4)
    sub = synth.make_inputs(w4.with_(len_max=1100, len_min=64), seqs=[2, 5])
    assert sub["q"].shape[0] == sub["cu_seqlens"][-1]
    assert len(lens) == 64


def test_distributions():
    w = WORKLOADS["prefill_4k_h16"].with_(T=2048)
    s = synth.slab(w, 0, 1)
    qf = synth.stored_to_f64(s["q"], "bf16")
    kf = synth.stored_to_f64(s["k"], "bf16")
    assert np.all(np.abs(np.linalg.norm(qf, axis=1) - 1) < 4e-3)
    assert np.all(np.abs(np.linalg.norm(kf, axis=1) - 1) < 4e-3)
    assert np.all(s["g"] < 0)
    assert np.all((s["beta"] > 0) & (s["beta"] < 1))
    assert abs(float(np.mean(s["beta"])) - 0.5) < 0.03
    alpha = np.exp(s["g"].astype(np.float64))
    # retention-biased forget gate: per-token alpha mostly close to 1
    assert 0.85 < float(np.mean(alpha)) < 0.999
    a, b = synth.gate_params(w)
    assert np.all((a >= math.log(0.01)) & (a <= math.log(0.5)))
    assert abs(float(np.mean(b)) + 2.0) < 0.1


def test_long_context_gates_retain_more():
    w1 = WORKLOADS["prefill_4k_h16"].with_(T=512)
    w2 = WORKLOADS["prefill_128k_h32"].with_(T=512)
    a1 = np.exp(synth.slab(w1, 0, 0)["g"].astype(np.float64)).mean()
    a2 = np.exp(synth.slab(w2, 0, 0)["g"].astype(np.float64)).mean()
    assert a2 > a1
    assert float(synth.slab(w2, 0, 0)["beta"].mean()) > 0.55


def test_packed_lengths_and_spectral_states():
    w = WORKLOADS["varlen_64seq_h16"]
    lens = synth.seq_lengths(w)
    assert lens.min() >= 1024 and lens.max() <= 65536
    assert 0.6e6 < lens.sum() < 1.6e6
    S = synth.initial_state(w, 3, 7)
    assert S.dtype == np.float32 and S.shape == (128, 128)
    assert abs(np.linalg.norm(S.astype(np.float64), 2) - 1) < 1e-6


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_shapes(name):
    w = WORKLOADS[name]
    assert w.K in (16, 128) and w.chunk in (16, 64)
    if w.decode:
        small = synth.make_inputs(w.with_(prefill_T=70, decode_steps=3), seqs=[0, 1])
        assert small["q"].shape == (140, w.H, w.K)
        assert small["dec_q"].shape == (3, 2, w.H, w.K)
        s = synth.slab(w.with_(prefill_T=70, decode_steps=3), 1, 2)
        np.testing.assert_array_equal(small["dec_k"][:, 1, 2], s["k"][70:73])
        np.testing.assert_array_equal(small["k"][70:140, 2], s["k"][:70])
