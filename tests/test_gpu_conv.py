"""The short causal convolution on the GPU (kda_short_conv_fwd, kda_short_conv_update)
against the float64 oracle (oracle.short_conv).

Tolerance: float32 sums of 4 products and a bias, so max |gpu - oracle| <= 1e-5 * RMS(oracle)
for float32 outputs; bf16 outputs add their own rounding, half a bf16 ulp (2^-8 relative):
|gpu - oracle| <= 1e-5 * RMS * (1 + 2^-8) + 2^-8 * |oracle| per element. The conv states are
copies of inputs, so they must match bit for bit.
"""

import numpy as np
import pytest

import gated_delta_rule_26_amd as kda
import oracle
import synth
from kda_testutil import assert_close, assert_close_bf16_out, f64, note, to_dev, torch_mod

pytestmark = pytest.mark.gpu

TOL = 1e-5
ACTS = [None, "silu"]


def conv_case(seed, T, C, stored, N=1):
    w = synth.Workload(f"conv{seed}", 4000 + seed, H=1, K=C, V=C, chunk=64, dtype=stored, B=1, T=T)
    x = synth.fused_slab(w, 0, 0, T)["q"]                       # [T, C] raw values, stored dtype
    weight, bias = synth.conv_params(w, C)
    s0 = synth.conv_state(w, N, C)
    return x, weight, bias, s0


def check_out(got, ref, stored, what):
    if stored == "bf16":
        return assert_close_bf16_out(got, ref, TOL, what)
    return assert_close(got, ref, TOL, what)


def dev_out(t):
    return t.float().cpu().numpy()


def raw(t, stored):
    """Storage bits of a device tensor (bf16 as uint16), for bitwise state checks."""
    torch = torch_mod()
    a = t.cpu()
    return a.view(torch.int16).numpy().view(np.uint16) if stored == "bf16" else a.numpy()


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("stored", ["f32", "bf16"])
@pytest.mark.parametrize("T,C", [(1, 8), (3, 256), (33, 2056), (100, 4096), (300, 64)])
def test_conv_batched_matches_oracle(T, C, stored, act):
    """B = 2 sequences of T tokens (strips of 64 tokens loaded in batches of 8 rows, a
    sequence starting inside a strip and inside a batch, partial strips and channel blocks),
    initial states, final states."""
    B = 2
    x, w, b, s0 = conv_case(T * 7 + C, B * T, C, stored, N=B)
    note(f"conv batched T={T} C={C} {stored} {act}")
    y, sf = kda.kda_short_conv_fwd(to_dev(x.reshape(B, T, C), stored), to_dev(w), to_dev(b),
                                   initial_state=to_dev(s0, stored), activation=act)
    torch_mod().cuda.synchronize()
    y_ref, f_ref = oracle.short_conv(f64(x, stored), w, b, initial_state=f64(s0, stored),
                                     cu_seqlens=np.arange(B + 1) * T, activation=act)
    check_out(dev_out(y).reshape(B * T, C), y_ref, stored, "y")
    assert np.array_equal(raw(sf, stored), np.asarray(
        synth.f64_to_bf16_bits(f_ref) if stored == "bf16" else f_ref.astype(np.float32))), "final state"


@pytest.mark.parametrize("stored", ["f32", "bf16"])
def test_conv_packed_empty_short_and_aliased(stored):
    """Packed sequences including empty, 1- and 2-token ones; no initial state for one call,
    and an in-place state update (final_state = initial_state) for the other."""
    lens = [0, 1, 2, 5, 40, 0, 100, 31, 33]
    cu = np.concatenate([[0], np.cumsum(lens)])
    C = 512
    x, w, b, s0 = conv_case(90, int(cu[-1]), C, stored, N=len(lens))
    cu_t = to_dev(cu.astype(np.int32))
    note(f"conv packed {stored}")
    y, sf = kda.kda_short_conv_fwd(to_dev(x, stored), to_dev(w), to_dev(b), cu_seqlens=cu_t)
    y_ref, f_ref = oracle.short_conv(f64(x, stored), w, b, cu_seqlens=cu)
    check_out(dev_out(y), y_ref, stored, "y (zero states)")
    assert np.array_equal(f64(raw(sf, stored), stored), f_ref), "final states (zero states)"
    st = to_dev(s0, stored)
    y2, sf2 = kda.kda_short_conv_fwd(to_dev(x, stored), to_dev(w), to_dev(b), initial_state=st,
                                     final_state=st, cu_seqlens=cu_t, activation=None)
    torch_mod().cuda.synchronize()
    y2_ref, f2_ref = oracle.short_conv(f64(x, stored), w, b, initial_state=f64(s0, stored),
                                       cu_seqlens=cu, activation=None)
    check_out(dev_out(y2), y2_ref, stored, "y (initial states)")
    assert sf2.data_ptr() == st.data_ptr()
    assert np.array_equal(f64(raw(st, stored), stored), f2_ref), "final states in place"


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("stored", ["f32", "bf16"])
def test_conv_prefill_then_updates_equal_prefill(stored, act):
    """A prefill of P tokens per sequence, then decode updates, reproduce the oracle's single
    pass over the concatenated tokens (outputs, and the state bit for bit)."""
    N, P, steps, C = 3, 37, 5, 1024
    L = P + steps
    x, w, b, s0 = conv_case(91, N * L, C, stored, N=N)
    xs = x.reshape(N, L, C)
    note(f"conv prefill then updates {stored} {act}")
    y_p, st = kda.kda_short_conv_fwd(to_dev(np.ascontiguousarray(xs[:, :P]), stored), to_dev(w),
                                     to_dev(b), initial_state=to_dev(s0, stored), activation=act)
    ys = []
    for i in range(steps):
        ys.append(dev_out(kda.kda_short_conv_update(to_dev(np.ascontiguousarray(xs[:, P + i]), stored),
                                                    to_dev(w), to_dev(b), st, activation=act)))
    torch_mod().cuda.synchronize()
    y_ref, f_ref = oracle.short_conv(f64(x, stored), w, b, initial_state=f64(s0, stored),
                                     cu_seqlens=np.arange(N + 1) * L, activation=act)
    y_ref = y_ref.reshape(N, L, C)
    check_out(dev_out(y_p), y_ref[:, :P], stored, "prefill part")
    check_out(np.stack(ys, 1), y_ref[:, P:], stored, "decode part")
    assert np.array_equal(f64(raw(st, stored), stored), f_ref), "state after the updates"
