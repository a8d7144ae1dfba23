"""Malformed packed offsets on the GPU: the kernels clamp cu_seqlens to [0, T] (end >= start),
so offsets that break the precondition (cu[0] < 0, cu[N] > T, a decreasing pair) give exactly
the result of their clamped equivalent and write nothing outside the caller's arrays.

Offsets [-5, 40, 100, 300, 90] over T = 100 tokens clamp to [0, 40, 100, 100, 100]: two
sequences of 40 and 60 tokens and two empty ones; no two clamped ranges overlap, so both runs
are deterministic and compared bit for bit. Every output is a view of a NaN-filled buffer
with extra rows after it, which must stay NaN.
"""

import numpy as np
import pytest

import gated_delta_rule_26_amd as kda
from kda_testutil import note, random_inputs, random_states, to_dev, torch_mod

pytestmark = pytest.mark.gpu

T, H, D, PAD = 100, 2, 16, 16
BAD = [-5, 40, 100, 300, 90]
CLAMPED = [0, 40, 100, 100, 100]
N = len(BAD) - 1


def padded(torch, shape):
    """A NaN-filled buffer with PAD extra leading-dimension rows, and its first rows."""
    big = torch.full((shape[0] + PAD, *shape[1:]), float("nan"), dtype=torch.float32, device="cuda")
    return big, big[:shape[0]]


def cu_dev(torch, cu):
    return torch.tensor(cu, dtype=torch.int32, device="cuda")


def test_clamped_offsets_forward_and_backward():
    torch = torch_mod()
    x = random_inputs(700, T, H, D, "f32")
    q, k, v = (to_dev(x[n], "f32") for n in ("q", "k", "v"))
    g, b = to_dev(x["g"]), to_dev(x["beta"])
    s0 = to_dev(random_states(701, N, H, D))
    do = to_dev(np.random.default_rng(702).standard_normal((T, H, D)).astype(np.float32))
    dsT = to_dev(random_states(703, N, H, D))
    res = {}
    for name, cu in (("bad", BAD), ("clamped", CLAMPED)):
        note(f"offsets {name} {cu}: forward")
        obig, o = padded(torch, (T, H, D))
        fbig, fs = padded(torch, (N, H, D, D))
        kda.kda_chunk_fwd(q, k, v, g, b, initial_state=s0, final_state=fs, o=o,
                          cu_seqlens=cu_dev(torch, cu), chunk=16)
        note(f"offsets {name} {cu}: backward")
        gbig = [padded(torch, tuple(t.shape)) for t in (g, g, do, g, b)]
        got = kda.kda_chunk_bwd(q, k, v, g, b, do, initial_state=s0, dfinal_state=dsT,
                                cu_seqlens=cu_dev(torch, cu), chunk=16,
                                grads=tuple(view for _, view in gbig))
        torch.cuda.synchronize()
        res[name] = [o.clone(), fs.clone(), *(t.clone() for t in got)]
        for big, n in [(obig, T), (fbig, N)] + [(bb, bb.shape[0] - PAD) for bb, _ in gbig]:
            assert bool(torch.isnan(big[n:]).all()), f"{name}: a write past the output"
    for i, (a, c) in enumerate(zip(res["bad"], res["clamped"])):
        assert torch.equal(a, c), f"output {i} differs from the clamped offsets' result"
    # the empty sequences hand their states through
    assert torch.equal(res["bad"][1][2:], s0[2:])


def test_clamped_offsets_short_convolution():
    torch = torch_mod()
    C, W = 16, 4
    rng = np.random.default_rng(710)
    xx = to_dev(rng.standard_normal((T, C)).astype(np.float32))
    w = to_dev(rng.standard_normal((C, W)).astype(np.float32))
    bias = to_dev(rng.standard_normal(C).astype(np.float32))
    st0 = to_dev(rng.standard_normal((N, W - 1, C)).astype(np.float32))
    res = {}
    for name, cu in (("bad", BAD), ("clamped", CLAMPED)):
        note(f"offsets {name} {cu}: short convolution")
        ybig, y = padded(torch, (T, C))
        sbig, fs = padded(torch, (N, W - 1, C))
        kda.kda_short_conv_fwd(xx, w, bias, initial_state=st0, final_state=fs, y=y,
                               cu_seqlens=cu_dev(torch, cu))
        torch.cuda.synchronize()
        assert bool(torch.isnan(ybig[T:]).all()) and bool(torch.isnan(sbig[N:]).all())
        res[name] = (y.clone(), fs.clone())
    assert torch.equal(res["bad"][0], res["clamped"][0])
    assert torch.equal(res["bad"][1], res["clamped"][1])
