"""The four bf16 workloads at their full sizes, in the launch configuration the benchmark
times, against the float64 oracle on sampled (sequence, head) chains.

Chains are independent, so the oracle recomputes a sample of them one by one from the same
seeded inputs; every other chain still runs on the GPU in the same launches. Tolerance: max
|gpu - oracle| <= 2e-2 * RMS(oracle) per returned tensor (over the sampled chains), and every
output element finite.
"""

import numpy as np
import pytest

import gated_delta_rule_26_amd as kda
import synth
from kda_testutil import (assert_close, assert_close_bf16_out, f64, note, oracle_threads,
                          to_dev, torch_mod)

import oracle

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

TOL = 2e-2


def _oracle(x, rows, cu, s0=None):
    """Oracle over token rows ``rows`` of the token-major arrays in ``x`` (all heads)."""
    return oracle.kda_fwd(f64(x["q"][rows], "bf16"), f64(x["k"][rows], "bf16"),
                          f64(x["v"][rows], "bf16"), f64(x["g"][rows]), f64(x["beta"][rows]),
                          initial_state=None if s0 is None else f64(s0), cu_seqlens=cu,
                          threads=oracle_threads())


def test_prefill_128k_h32_full_size():
    """B=1, T=131072, H=32: the split launch (transition, combine, forward) the benchmark
    times; heads 0, 13 and 31 checked over the whole sequence."""
    torch = torch_mod()
    w = synth.WORKLOADS["prefill_128k_h32"]
    x = synth.make_inputs(w)
    T, H = w.T, w.H
    q, k, v = (to_dev(x[n][None], "bf16") for n in ("q", "k", "v"))
    g, beta = to_dev(x["g"][None]), to_dev(x["beta"][None])
    assert kda.chunk_fwd_workspace_bytes(q, v) > 0, "expected the sequence split"
    note("prefill_128k_h32 full size")
    o, S = kda.kda_chunk_fwd(q, k, v, g, beta)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()), "non-finite outputs"
    heads = [0, 13, 31]
    o_s = o[0][:, heads].cpu().numpy()
    S_s = S[0, heads].cpu().numpy()
    del q, k, v, g, beta, o
    xs = {n: x[n][:, heads] for n in ("q", "k", "v", "g", "beta")}
    o_ref, S_ref = _oracle(xs, slice(None), None)
    assert_close(o_s, o_ref, TOL, "o (heads 0, 13, 31)")
    assert_close(S_s, S_ref[0], TOL, "final state (heads 0, 13, 31)")


def test_prefill_128k_h32_fused_full_size():
    """The fused layer steps at the long-context size, in the launch configuration the
    benchmark times (split; raw q/k, the gate's pre-activation, bf16 normalised output);
    heads 0 and 31 checked over the whole sequence against the oracle's composition."""
    torch = torch_mod()
    w = synth.WORKLOADS["prefill_128k_h32"]
    x = synth.make_inputs(w, fused=True)
    q, k, v, gx, z = (to_dev(x[n][None], "bf16") for n in ("q", "k", "v", "x", "z"))
    beta = to_dev(x["beta"][None])
    A, dtb, wt = to_dev(x["A_log"]), to_dev(x["dt_bias"]), to_dev(x["norm_weight"])
    assert kda.chunk_fwd_workspace_bytes(q, v) > 0, "expected the sequence split"
    note("prefill_128k_h32 fused full size")
    y, S = kda.kda_chunk_fwd_fused(q, k, v, gx, A, dtb, beta, o_gate=z, o_weight=wt,
                                   o_eps=x["norm_eps"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y.float()).all()), "non-finite outputs"
    heads = [0, 31]
    y_s = y[0][:, heads].float().cpu().numpy()
    S_s = S[0, heads].cpu().numpy()
    del q, k, v, gx, z, beta, y
    st = lambda n: f64(x[n][:, heads], "bf16")  # noqa: E731
    y_ref, S_ref = oracle.kda_fused_fwd(st("q"), st("k"), st("v"), st("x"), f64(x["A_log"][heads]),
                                        f64(x["dt_bias"][heads]), f64(x["beta"][:, heads]),
                                        o_gate=st("z"), o_weight=f64(x["norm_weight"]),
                                        o_eps=x["norm_eps"], threads=oracle_threads())
    assert_close_bf16_out(y_s, y_ref, TOL, "y (heads 0, 31)")
    assert_close(S_s, S_ref[0], TOL, "final state (heads 0, 31)")


def test_short_conv_128k_h32_full_size():
    """The short convolution (SiLU) over the long-context workload's raw q projection,
    [131072, 32 * 128] bf16, in one launch; heads 0 and 31 (channels 0-127, 3968-4095)
    checked against the oracle, the final state bit for bit."""
    torch = torch_mod()
    w = synth.WORKLOADS["prefill_128k_h32"]
    x = synth.make_inputs(w, fused=True)["q"].reshape(w.T, w.H * w.K)
    weight, bias = synth.conv_params(w, w.H * w.K)
    note("short conv 128k x 4096 full size")
    y, sf = kda.kda_short_conv_fwd(to_dev(x[None], "bf16"), to_dev(weight), to_dev(bias))
    torch.cuda.synchronize()
    chans = np.r_[0:128, 3968:4096]
    y_s = y[0][:, torch.from_numpy(chans).cuda()].float().cpu().numpy()
    f_s = sf[0][:, torch.from_numpy(chans).cuda()].float().cpu().numpy()
    y_ref, f_ref = oracle.short_conv(f64(x[:, chans], "bf16"), weight[chans], bias[chans])
    assert_close_bf16_out(y_s, y_ref, 1e-5, "y (channels of heads 0, 31)")
    assert np.array_equal(f_s, f_ref[0]), "final conv state"


def test_decode_256x32_full_size():
    """256 sequences x 32 heads: a 2048-token prefill builds the states, then 1000 decode steps
    over all of them; sequences 0, 97 and 255 (all heads) checked against the oracle over the
    concatenated 3048 tokens, and a single GPU prefill over those 3048 tokens checked too."""
    torch = torch_mod()
    w = synth.WORKLOADS["decode_256x32"]
    x = synth.make_inputs(w)
    N, P, H, K, V, steps = w.B, w.prefill_T, w.H, w.K, w.V, w.decode_steps
    dq, dk, dv = (to_dev(x[n].reshape(N, P, H, K), "bf16") for n in ("q", "k", "v"))
    dg = to_dev(x["g"].reshape(N, P, H, K))
    db = to_dev(x["beta"].reshape(N, P, H))
    note("decode_256x32: 2048-token prefill")
    _, state = kda.kda_chunk_fwd(dq, dk, dv, dg, db)
    del dq, dk, dv, dg, db
    tq, tk, tv = (to_dev(x["dec_" + n], "bf16") for n in ("q", "k", "v"))
    tg, tb = to_dev(x["dec_g"]), to_dev(x["dec_beta"])
    out = torch.empty((steps, N, H, V), dtype=torch.float32, device="cuda")
    note("decode_256x32: 1000 steps")
    for i in range(steps):
        kda.kda_decode_step(tq[i], tk[i], tv[i], tg[i], tb[i], state, o=out[i])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "non-finite decode outputs"
    seqs = [0, 97, 255]
    o_dec = out[:, seqs].cpu().numpy()          # [steps, 3, H, V]
    S_dec = state[seqs].cpu().numpy()
    del out, tq, tk, tv, tg, tb, state

    # the concatenated sequences: prefill rows of sequence n, then its decode tokens
    cat = {}
    for n_ in ("q", "k", "v", "g", "beta"):
        parts = []
        for n in seqs:
            parts.append(x[n_][n * P:(n + 1) * P])
            parts.append(x["dec_" + n_][:, n])
        cat[n_] = np.concatenate(parts)
    L = P + steps
    cu = np.arange(len(seqs) + 1) * L
    o_ref, S_ref = _oracle(cat, slice(None), cu)
    o_ref = o_ref.reshape(len(seqs), L, H, V)
    assert_close(o_dec.transpose(1, 0, 2, 3), o_ref[:, P:], TOL, "decode o (1000 steps)")
    assert_close(S_dec, S_ref, TOL, "state after 1000 steps")

    # the same 3048-token sequences through one chunked prefill on the GPU
    q, k, v = (to_dev(cat[n].reshape(len(seqs), L, H, -1), "bf16") for n in ("q", "k", "v"))
    g = to_dev(cat["g"].reshape(len(seqs), L, H, K))
    beta = to_dev(cat["beta"].reshape(len(seqs), L, H))
    note("decode_256x32: single 3048-token prefill")
    o_p, S_p = kda.kda_chunk_fwd(q, k, v, g, beta)
    torch.cuda.synchronize()
    assert_close(o_p.cpu().numpy(), o_ref, TOL, "prefill over 3048 tokens: o")
    assert_close(S_p.cpu().numpy(), S_ref, TOL, "prefill over 3048 tokens: state")


def test_varlen_64seq_h16_full_size():
    """64 packed sequences (lengths 1K-64K, about 1M tokens), H=16, spectral-norm initial
    states; the shortest, the longest, the median and the first sequence checked."""
    torch = torch_mod()
    w = synth.WORKLOADS["varlen_64seq_h16"]
    x = synth.make_inputs(w)
    cu = x["cu_seqlens"]
    lens = x["lengths"]
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    g, beta = to_dev(x["g"]), to_dev(x["beta"])
    s0 = to_dev(x["initial_state"])
    cu_t = to_dev(cu.astype(np.int32))
    note(f"varlen_64seq_h16 full size: {int(cu[-1])} tokens")
    o, S = kda.kda_chunk_fwd(q, k, v, g, beta, initial_state=s0, cu_seqlens=cu_t)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()), "non-finite outputs"
    order = np.argsort(lens, kind="stable")
    seqs = sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2]), 0})
    rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs])
    o_s = o[torch.from_numpy(rows).cuda()].cpu().numpy()
    S_s = S[seqs].cpu().numpy()
    del q, k, v, g, beta, o
    sub_cu = np.concatenate([[0], np.cumsum(lens[seqs])])
    o_ref, S_ref = _oracle(x, rows, sub_cu, s0=x["initial_state"][seqs])
    assert_close(o_s, o_ref, TOL, f"o (sequences {seqs}, lengths {lens[seqs].tolist()})")
    assert_close(S_s, S_ref, TOL, "final states (sampled sequences)")


def test_backward_4k_h16_full_size():
    """kda_chunk_bwd at the 4K-token, 16-head training shape (bf16 q/k/v, the launch the
    benchmark times), dL/do and dL/dS_final seeded; every head checked against the oracle's
    backward over the whole sequence (the bf16 backward bound of the backward tests, 1e-3)."""
    torch = torch_mod()
    w = synth.WORKLOADS["prefill_4k_h16"]
    x = synth.make_inputs(w)
    do = np.stack([synth.grad_out(w, 0, h) for h in range(w.H)], axis=1)     # [T, H, V]
    dsT = synth.grad_state(w, 1)
    q, k, v = (to_dev(x[n][None], "bf16") for n in ("q", "k", "v"))
    g, beta = to_dev(x["g"][None]), to_dev(x["beta"][None])
    note("backward 4k_h16 full size")
    got = kda.kda_chunk_bwd(q, k, v, g, beta, to_dev(do[None]), dfinal_state=to_dev(dsT))
    torch.cuda.synchronize()
    got = [t.cpu().numpy() for t in got]
    ref = oracle.kda_bwd(f64(x["q"], "bf16"), f64(x["k"], "bf16"), f64(x["v"], "bf16"),
                         f64(x["g"]), f64(x["beta"]), f64(do), dfinal_state=f64(dsT),
                         threads=oracle_threads())
    for name, a, b in zip(["dq", "dk", "dv", "dg", "dbeta", "dS_init"], got, ref):
        assert_close(a.reshape(b.shape), b, 1e-3, name)
