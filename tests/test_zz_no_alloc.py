"""kda_chunk_bwd_noalloc (the backward pass for callers that cannot allocate: its records live
in the library's fixed per-device scratch) through the C ABI, against kda_chunk_bwd (the
entry point with a caller-provided workspace) on the same inputs: two calls in a row, the
second on a smaller problem that finds the first one's records still in the scratch. The two
entry points run the same kernels, so every gradient must match bit for bit; the first call is
also held to the oracle."""

import numpy as np
import pytest

import gated_delta_rule_26_amd as kda
import synth
from kda_testutil import assert_close, f64, note, oracle_threads, random_inputs, random_states, to_dev, torch_mod

import oracle

pytestmark = pytest.mark.gpu

NAMES = ["dq", "dk", "dv", "dg", "dbeta", "dS_init"]


def _run_both(x, do, *, B=1, cu=None, s0=None, dsT=None, scale=1.0):
    torch = torch_mod()
    T = x["q"].shape[0] // B
    sh = (lambda a: a.reshape(B, T, *a.shape[1:])) if cu is None else (lambda a: a)
    q, k, v = (to_dev(sh(x[n]), "bf16") for n in ("q", "k", "v"))
    g, beta = to_dev(sh(x["g"])), to_dev(sh(x["beta"]))
    d_o = to_dev(sh(do))
    s0_t = None if s0 is None else to_dev(s0)
    dsT_t = None if dsT is None else to_dev(dsT)
    cu_t = None if cu is None else to_dev(np.asarray(cu, dtype=np.int32))
    N = B if cu is None else len(cu) - 1
    H, D = q.shape[-2], q.shape[-1]
    ref = kda.kda_chunk_bwd(q, k, v, g, beta, d_o, initial_state=s0_t, dfinal_state=dsT_t,
                            cu_seqlens=cu_t, scale=scale)
    grads = tuple(torch.full_like(t, float("nan"), dtype=torch.float32) for t in (g, g, d_o, g, beta))
    ds0 = torch.full((N, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
    got = kda.kda_chunk_bwd_noalloc(q, k, v, g, beta, d_o, grads=grads, dinitial_state=ds0,
                                    initial_state=s0_t, dfinal_state=dsT_t, cu_seqlens=cu_t, scale=scale)
    torch.cuda.synchronize()
    for name, a, b in zip(NAMES, ref, got):
        assert torch.equal(a, b), f"{name}: the allocation-free call differs from kda_chunk_bwd"
    return [t.cpu().numpy() for t in got]


def test_noalloc_backward_matches_workspace_entry_point_twice():
    # call 1: the 4K-token, 16-head training shape (494 MB of records in the 512 MiB scratch)
    w = synth.WORKLOADS["prefill_4k_h16"]
    x = synth.make_inputs(w)
    do = np.stack([synth.grad_out(w, 0, h) for h in range(w.H)], axis=1)
    dsT = synth.grad_state(w, 1)
    note("noalloc backward: 4096 x 16")
    got = _run_both(x, do, dsT=dsT)
    ref = oracle.kda_bwd(f64(x["q"], "bf16"), f64(x["k"], "bf16"), f64(x["v"], "bf16"), f64(x["g"]),
                         f64(x["beta"]), f64(do), dfinal_state=f64(dsT), threads=oracle_threads())
    for name, a, b in zip(NAMES, got, ref):
        assert_close(a.reshape(b.shape), b, 1e-3, name)

    # call 2, smaller: packed sequences with an empty one, initial states and a query scale,
    # over the first call's leftover records
    lens = [300, 0, 777, 65]
    cu = np.concatenate([[0], np.cumsum(lens)])
    H, D = 3, 128
    x = random_inputs(801, int(cu[-1]), H, D, "bf16")
    s0 = random_states(802, len(lens), H, D)
    do = np.random.default_rng(803).standard_normal((int(cu[-1]), H, D)).astype(np.float32)
    dsT = np.random.default_rng(804).standard_normal((len(lens), H, D, D)).astype(np.float32)
    note("noalloc backward: packed 4 sequences x 3 heads")
    got = _run_both(x, do, cu=cu, s0=s0, dsT=dsT, scale=D ** -0.5)
    ref = oracle.kda_bwd(f64(x["q"], "bf16"), f64(x["k"], "bf16"), f64(x["v"], "bf16"), f64(x["g"]),
                         f64(x["beta"]), f64(do), scale=D ** -0.5, initial_state=f64(s0),
                         dfinal_state=f64(dsT), cu_seqlens=cu, threads=oracle_threads())
    for name, a, b in zip(NAMES, got, ref):
        assert_close(a.reshape(b.shape), b, 1e-3, name)


def test_noalloc_backward_rejects_beyond_scratch():
    """Records beyond the fixed scratch: refused before any launch, the outputs untouched."""
    torch = torch_mod()
    # the fewest heads whose records at 4096 tokens exceed the fixed scratch (512 MiB)
    T, D = 4096, 128
    one = torch.zeros((1, T, 1, D), dtype=torch.bfloat16)
    per_head = kda.chunk_bwd_workspace_bytes(one, one)
    H = (512 << 20) // per_head + 1
    assert per_head * H > 512 << 20 >= per_head * (H - 1)
    q = torch.zeros((1, T, H, D), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((1, T, H, D), dtype=torch.float32, device="cuda")
    beta = torch.zeros((1, T, H), dtype=torch.float32, device="cuda")
    grads = tuple(torch.full_like(t, 7.0) for t in (g, g, g, g, beta))
    with pytest.raises(kda.KdaError) as e:
        kda.kda_chunk_bwd_noalloc(q, q, q, g, beta, g, grads=grads)
    assert e.value.status == 3 and "fixed scratch" in str(e.value)
    torch.cuda.synchronize()
    assert all(bool((t == 7.0).all()) for t in grads)
