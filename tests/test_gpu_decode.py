"""kda_decode_step and kda_recurrent_fwd on the GPU against the float64 oracle (one step,
chained steps, several tokens per call). Both compute in float32 on exactly represented
inputs, so the float32 tolerance applies to bf16 inputs too."""

import numpy as np
import pytest

import gated_delta_rule_26_amd as kda
import oracle
from kda_testutil import (assert_close, f64, note, random_inputs, random_states, run_oracle,
                          to_dev, torch_mod)

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


# ----------------------------------------------------- several tokens per call (recurrent)

@pytest.mark.parametrize("L", [1, 2, 7, 64])
@pytest.mark.parametrize("stored", ["f32", "bf16"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
def test_recurrent_tokens_match_oracle(D, stored, L):
    """kda_recurrent_fwd: N sequences of L tokens on their initial states, against the oracle
    over the same packed sequences."""
    N, H = 4, 3
    x = random_inputs(300 + D + L, N * L, H, D, stored)
    s0 = random_states(301 + D, N, H, D)
    torch = torch_mod()
    shp = lambda a: np.ascontiguousarray(a.reshape(N, L, *a.shape[1:]))  # noqa: E731
    q, k, v = (to_dev(shp(x[n]), stored) for n in ("q", "k", "v"))
    g, beta = to_dev(shp(x["g"])), to_dev(shp(x["beta"]))
    state = to_dev(s0.copy())
    note(f"recurrent D={D} {stored} L={L}")
    o = kda.kda_recurrent_fwd(q, k, v, g, beta, state, scale=0.7)
    torch.cuda.synchronize()
    o_ref, S_ref = run_oracle(x, stored, scale=0.7, initial_state=s0, cu=np.arange(N + 1) * L)
    assert_close(o.cpu().numpy().reshape(N * L, H, D), o_ref, TOL_F32, "o")
    assert_close(state.cpu().numpy(), S_ref, TOL_F32, "state")


def test_recurrent_equals_successive_decode_steps_bitwise():
    """L tokens in one call give the same bits as L decode steps (the same arithmetic per
    token, with the state kept in registers instead of HBM in between)."""
    N, L, H, D = 8, 5, 4, 128
    x = random_inputs(310, N * L, H, D, "bf16")
    s0 = random_states(311, N, H, D)
    torch = torch_mod()
    shp = lambda a: np.ascontiguousarray(a.reshape(N, L, *a.shape[1:]))  # noqa: E731
    q, k, v = (to_dev(shp(x[n]), "bf16") for n in ("q", "k", "v"))
    g, beta = to_dev(shp(x["g"])), to_dev(shp(x["beta"]))
    st1, st2 = to_dev(s0.copy()), to_dev(s0.copy())
    note("recurrent vs decode steps")
    o1 = kda.kda_recurrent_fwd(q, k, v, g, beta, st1)
    o2 = torch.stack([kda.kda_decode_step(q[:, t].contiguous(), k[:, t].contiguous(),
                                          v[:, t].contiguous(), g[:, t].contiguous(),
                                          beta[:, t].contiguous(), st2) for t in range(L)], 1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "outputs differ"
    assert torch.equal(st1, st2), "states differ"
