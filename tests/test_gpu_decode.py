"""kda_decode_step on the GPU against the float64 oracle (one step and chained steps)."""

import numpy as np
import pytest

import gated_delta_rule_26_amd as kda
import oracle
from kda_testutil import (assert_close, f64, note, random_inputs, random_states, to_dev,
                          torch_mod)

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4  # float32 arithmetic on exactly-represented inputs


@pytest.mark.parametrize("stored", ["f32", "bf16"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
def test_decode_steps_match_oracle(stored, D):
    torch = torch_mod()
    N, H, steps = 5, 3, 12
    x = random_inputs(30 + D, N * steps, H, D, stored)
    s0 = random_states(31 + D, N, H, D)
    # token (step s, sequence n) = row s * N + n
    rs = lambda a: a.reshape(steps, N, *a.shape[1:])  # noqa: E731
    q, k, v, g, beta = (rs(x[key]) for key in ("q", "k", "v", "g", "beta"))
    note(f"decode D={D} {stored} N={N} H={H} steps={steps}")
    state = to_dev(s0.copy())
    S_ref = f64(s0)
    for s in range(steps):
        o = kda.kda_decode_step(to_dev(q[s], stored), to_dev(k[s], stored), to_dev(v[s], stored),
                                to_dev(g[s]), to_dev(beta[s]), state, scale=0.75)
        o_ref, S_ref = oracle.kda_decode_step(f64(q[s], stored), f64(k[s], stored),
                                              f64(v[s], stored), f64(g[s]), f64(beta[s]), S_ref,
                                              scale=0.75)
        torch.cuda.synchronize()
        assert_close(o.cpu().numpy(), o_ref, TOL_F32, f"o step {s}")
    assert_close(state.cpu().numpy(), S_ref, TOL_F32, "state")


def test_decode_bitwise_deterministic():
    torch = torch_mod()
    N, H, D = 64, 4, 128
    x = random_inputs(40, N, H, D, "bf16")
    s0 = random_states(41, N, H, D)
    outs = []
    note("decode determinism")
    for _ in range(2):
        st = to_dev(s0.copy())
        o = kda.kda_decode_step(*(to_dev(x[key], "bf16") for key in ("q", "k", "v")),
                                to_dev(x["g"]), to_dev(x["beta"]), st)
        torch.cuda.synchronize()
        outs.append((o.cpu().numpy(), st.cpu().numpy()))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])
