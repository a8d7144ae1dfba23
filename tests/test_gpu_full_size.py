"""The bf16 workloads at their full sizes, in the launch configuration the benchmark times,
against the float64 oracle over EVERY (sequence, head) chain.

Chains are independent, so the oracle runs over groups of chains (a group of heads, or a
group of sequences) one after the other on the same seeded inputs, and each group's outputs
are compared with the GPU's as they come. The statistic is that of the parity bar, per
returned tensor over all of its elements: max |gpu - oracle| <= 2e-2 * RMS(oracle), with the
RMS over the whole tensor (``WholeTensor`` accumulates both across the groups). A rounding
error that builds up over long sequences, or an addressing slip in one late chain or
segment, cannot hide in an unchecked chain.
"""

import numpy as np
import pytest

import gated_delta_rule_26_amd as kda
import synth
from kda_testutil import WholeTensor, assert_close, f64, note, oracle_threads, to_dev, torch_mod

import oracle

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]

TOL = 2e-2


def _oracle(x, cu, s0=None, threads=None):
    """Oracle over the token-major arrays in ``x`` (bf16 q, k, v; float32 g, beta)."""
    return oracle.kda_fwd(f64(x["q"], "bf16"), f64(x["k"], "bf16"), f64(x["v"], "bf16"),
                          f64(x["g"]), f64(x["beta"]),
                          initial_state=None if s0 is None else f64(s0), cu_seqlens=cu,
                          threads=threads or oracle_threads())


def _head_groups(H: int, size: int = 16):
    return [list(range(h, min(h + size, H))) for h in range(0, H, size)]


def test_prefill_128k_h32_full_size():
    """B=1, T=131072, H=32: the split launch (forward with records, segment maps, combine,
    output replay) the benchmark times; all 32 heads over the whole sequence."""
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
    o_h = o[0].cpu().numpy()
    S_h = S[0].cpu().numpy()
    del q, k, v, g, beta, o, S
    po, pS = WholeTensor("o [131072, 32, 128]", TOL), WholeTensor("final state [1, 32, 128, 128]", TOL)
    for hs in _head_groups(H):
        xs = {n: x[n][:, hs] for n in ("q", "k", "v", "g", "beta")}
        o_ref, S_ref = _oracle(xs, None)
        po.add(o_h[:, hs], o_ref)
        pS.add(S_h[hs], S_ref[0])
        note(f"prefill_128k_h32: heads {hs[0]}-{hs[-1]} compared")
    po.check(T * H * w.V)
    pS.check(H * w.K * w.V)


def test_prefill_128k_h32_fused_full_size():
    """The fused layer steps at the long-context size, in the launch configuration the
    benchmark times (split; raw q/k, the gate's pre-activation, bf16 normalised output); all
    32 heads over the whole sequence against the oracle's composition."""
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
    y_h = y[0].float().cpu().numpy()
    S_h = S[0].cpu().numpy()
    del q, k, v, gx, z, beta, y, S
    py = WholeTensor("y [131072, 32, 128] (bf16, row-normalised)", TOL, bf16_out=True)
    pS = WholeTensor("final state [1, 32, 128, 128]", TOL)
    for hs in _head_groups(w.H):
        st = lambda n: f64(x[n][:, hs], "bf16")  # noqa: E731
        # the oracle's output before its gated RMSNorm, then the norm: the pre-norm values set
        # each row's conditioning (a row of small norm amplifies the core's error on it)
        o_ref, S_ref = oracle.kda_fused_fwd(st("q"), st("k"), st("v"), st("x"), f64(x["A_log"][hs]),
                                            f64(x["dt_bias"][hs]), f64(x["beta"][:, hs]),
                                            threads=oracle_threads())
        y_ref = oracle.fused.gated_rmsnorm(o_ref, st("z"), f64(x["norm_weight"]), x["norm_eps"])
        py.add(y_h[:, hs], y_ref, pre=o_ref, eps=x["norm_eps"])
        pS.add(S_h[hs], S_ref[0])
        note(f"prefill_128k_h32 fused: heads {hs[0]}-{hs[-1]} compared")
    py.check(w.T * w.H * w.V)
    pS.check(w.H * w.K * w.V)


def test_short_conv_128k_h32_full_size():
    """The short convolution (SiLU) over the long-context workload's raw q projection,
    [131072, 32 * 128] bf16, in one launch; every channel checked against the oracle, the
    final state bit for bit."""
    torch = torch_mod()
    w = synth.WORKLOADS["prefill_128k_h32"]
    x = synth.make_inputs(w, fused=True)["q"].reshape(w.T, w.H * w.K)
    C = w.H * w.K
    weight, bias = synth.conv_params(w, C)
    note("short conv 128k x 4096 full size")
    y, sf = kda.kda_short_conv_fwd(to_dev(x[None], "bf16"), to_dev(weight), to_dev(bias))
    torch.cuda.synchronize()
    y_h = y[0].float().cpu().numpy()
    f_h = sf[0].float().cpu().numpy()
    del y, sf
    py = WholeTensor("y [131072, 4096] (bf16)", 1e-5, bf16_out=True)
    for c0 in range(0, C, 1024):
        ch = slice(c0, c0 + 1024)
        y_ref, f_ref = oracle.short_conv(f64(x[:, ch], "bf16"), weight[ch], bias[ch])
        py.add(y_h[:, ch], y_ref)
        assert np.array_equal(f_h[:, ch], f_ref[0]), f"final conv state, channels {c0}.."
    py.check(w.T * C)


def test_decode_256x32_full_size():
    """256 sequences x 32 heads: a 2048-token prefill builds the states, then 1000 decode
    steps over all of them. Every chain is checked against the oracle over its concatenated
    3048 tokens: the decode outputs of all 1000 steps ([1000, 256, 32, 128]) and the states
    after the last step. One GPU chunked prefill over the same 3048-token sequences is checked
    against the same oracle run."""
    torch = torch_mod()
    w = synth.WORKLOADS["decode_256x32"]
    x = synth.make_inputs(w)
    N, P, H, K, V, steps = w.B, w.prefill_T, w.H, w.K, w.V, w.decode_steps
    L = P + steps
    dq, dk, dv = (to_dev(x[n].reshape(N, P, H, -1), "bf16") for n in ("q", "k", "v"))
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
    del tq, tk, tv, tg, tb

    def concat(seqs):
        """The concatenated sequences: prefill rows of sequence n, then its decode tokens."""
        cat = {}
        for name in ("q", "k", "v", "g", "beta"):
            cat[name] = np.concatenate([np.concatenate([x[name][n * P:(n + 1) * P], x["dec_" + name][:, n]])
                                        for n in seqs])
        return cat

    # the same 3048-token sequences through one chunked prefill over the whole batch
    groups = [list(range(n, n + 16)) for n in range(0, N, 16)]
    q = torch.empty((N, L, H, K), dtype=torch.bfloat16, device="cuda")
    k, v = torch.empty_like(q), torch.empty_like(q)
    g = torch.empty((N, L, H, K), dtype=torch.float32, device="cuda")
    beta = torch.empty((N, L, H), dtype=torch.float32, device="cuda")
    for grp in groups:
        cat = concat(grp)
        sl = slice(grp[0], grp[-1] + 1)
        for t, name in ((q, "q"), (k, "k"), (v, "v")):
            t[sl] = to_dev(cat[name].reshape(len(grp), L, H, -1), "bf16")
        g[sl] = to_dev(cat["g"].reshape(len(grp), L, H, K))
        beta[sl] = to_dev(cat["beta"].reshape(len(grp), L, H))
    note("decode_256x32: single 3048-token prefill of all 256 sequences")
    o_p, S_p = kda.kda_chunk_fwd(q, k, v, g, beta)
    torch.cuda.synchronize()
    del q, k, v, g, beta

    pd = WholeTensor("decode o, 1000 steps [1000, 256, 32, 128]", TOL)
    ps = WholeTensor("state after 1000 steps [256, 32, 128, 128]", TOL)
    pp = WholeTensor("prefill over 3048 tokens: o [256, 3048, 32, 128]", TOL)
    pps = WholeTensor("prefill over 3048 tokens: final state", TOL)
    for grp in groups:
        cat = concat(grp)
        cu = np.arange(len(grp) + 1) * L
        o_ref, S_ref = _oracle(cat, cu)
        o_ref = o_ref.reshape(len(grp), L, H, V)
        sl = slice(grp[0], grp[-1] + 1)
        pd.add(out[:, sl].cpu().numpy().transpose(1, 0, 2, 3), o_ref[:, P:])
        ps.add(state[sl].cpu().numpy(), S_ref)
        pp.add(o_p[sl].cpu().numpy(), o_ref)
        pps.add(S_p[sl].cpu().numpy(), S_ref)
        note(f"decode_256x32: sequences {grp[0]}-{grp[-1]} compared")
    pd.check(steps * N * H * V)
    ps.check(N * H * K * V)
    pp.check(N * L * H * V)
    pps.check(N * H * K * V)


def test_varlen_64seq_h16_full_size():
    """64 packed sequences (lengths 1K-64K, about 1M tokens), H=16, spectral-norm initial
    states, longest first; every sequence and head checked: the packed o and all 64 final
    states."""
    torch = torch_mod()
    w = synth.WORKLOADS["varlen_64seq_h16"]
    x = synth.make_inputs(w)
    cu = x["cu_seqlens"]
    N = len(x["lengths"])
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    g, beta = to_dev(x["g"]), to_dev(x["beta"])
    s0 = to_dev(x["initial_state"])
    cu_t = to_dev(cu.astype(np.int32))
    assert kda.chunk_fwd_workspace_bytes(q, v, num_seqs=N) > 0, "expected the longest-first order"
    note(f"varlen_64seq_h16 full size: {int(cu[-1])} tokens")
    o, S = kda.kda_chunk_fwd(q, k, v, g, beta, initial_state=s0, cu_seqlens=cu_t)
    torch.cuda.synchronize()
    del q, k, v, g, beta, s0
    S_h = S.cpu().numpy()
    po = WholeTensor(f"o [{int(cu[-1])}, 16, 128]", TOL)
    pS = WholeTensor("final states [64, 16, 128, 128]", TOL)
    for n in range(N):
        rows = slice(int(cu[n]), int(cu[n + 1]))
        xs = {name: x[name][rows] for name in ("q", "k", "v", "g", "beta")}
        o_ref, S_ref = _oracle(xs, None, s0=x["initial_state"][n:n + 1])
        po.add(o[rows].cpu().numpy(), o_ref)
        pS.add(S_h[n:n + 1], S_ref)
        if n % 8 == 7:
            note(f"varlen_64seq_h16: sequences 0-{n} compared")
    po.check(int(cu[-1]) * w.H * w.V)
    pS.check(N * w.H * w.K * w.V)


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
