"""Calls on a stream other than torch's current one (``stream=``): the binding allocates its
outputs and the internal workspace on that stream, so a block freed on return cannot be handed
to another stream while the kernels still use it. Results must equal the current-stream ones
bit for bit (the kernels are deterministic), even while the current stream allocates and
overwrites memory as soon as the calls return."""

import numpy as np
import pytest

import gated_delta_rule_26_amd as kda
from kda_testutil import note, random_inputs, to_dev, torch_mod

pytestmark = pytest.mark.gpu


def test_side_stream_prefill_and_backward_bit_identical():
    torch = torch_mod()
    T, H, D = 2048, 4, 128
    x = random_inputs(71, T, H, D, "bf16")
    q, k, v = (to_dev(x[n][None], "bf16") for n in ("q", "k", "v"))
    g, beta = to_dev(x["g"][None]), to_dev(x["beta"][None])
    do = torch.from_numpy(np.random.default_rng(5).standard_normal((1, T, H, D)).astype(np.float32)).cuda()
    assert kda.chunk_fwd_workspace_bytes(q, v) > 0, "expected the split (an internal workspace)"
    note("side stream: current-stream references")
    o0, S0 = kda.kda_chunk_fwd(q, k, v, g, beta)
    gr0 = kda.kda_chunk_bwd(q, k, v, g, beta, do)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    note("side stream: the same calls on a side stream")
    o1, S1 = kda.kda_chunk_fwd(q, k, v, g, beta, stream=side)
    gr1 = kda.kda_chunk_bwd(q, k, v, g, beta, do, stream=side)
    # the current stream allocates right away and overwrites what it gets
    junk = [torch.full((1 << 26,), float("nan"), device="cuda") for _ in range(4)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(o0, o1), "o differs on the side stream"
    assert torch.equal(S0, S1), "final state differs on the side stream"
    for name, a, b in zip(["dq", "dk", "dv", "dg", "dbeta", "dS_init"], gr0, gr1):
        assert torch.equal(a, b), f"{name} differs on the side stream"


def test_side_stream_decode_bit_identical():
    torch = torch_mod()
    N, H, D = 8, 4, 128
    x = random_inputs(72, N, H, D, "bf16")
    q, k, v = (to_dev(x[n].reshape(N, H, D), "bf16") for n in ("q", "k", "v"))
    g, beta = to_dev(x["g"].reshape(N, H, D)), to_dev(x["beta"].reshape(N, H))
    s_a = torch.from_numpy(np.random.default_rng(6).standard_normal((N, H, D, D)).astype(np.float32) * 0.1).cuda()
    s_b = s_a.clone()
    o0 = kda.kda_decode_step(q, k, v, g, beta, s_a)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    note("side stream: decode step")
    o1 = kda.kda_decode_step(q, k, v, g, beta, s_b, stream=side)
    side.synchronize()
    assert torch.equal(o0, o1) and torch.equal(s_a, s_b)
