"""Benchmark of the KDA core on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  1. kda_chunk_fwd on the long-context prefill workload (B=1, T=131072, H=32,
     Dk=Dv=128, chunk 64, bf16 q/k/v, float32 gates, zero initial state, float32 o and
     final state), and
  2. one kda_decode_step on the decode workload (256 sequences x 32 heads of float32
     128x128 states, built by a 2048-token prefill of the same-style inputs; one bf16 token
     per sequence and head per step).

Inputs are generated on the host (seeded, synth/) and are resident in HBM before the timed
region, as is the prefill's optional split workspace. The headline value is prefill tokens/s
(H=32, d=128); the decode step's state bandwidth is reported next to it. Times come from HIP
events recorded on the stream the kernels run on (one kda_chunk_fwd call = the transition,
combine and chunked-forward kernels). The roofline fraction uses algorithmic bytes per call.

Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
  python bench.py --counter-pass [--steps K]
      only the prefill calls (then two backward calls at the 4K-token, 16-head shape), then a
      plain copy-like kernel (out = -x over COPY_BYTES) as the HBM-counter calibration; run it
      under rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE (and MfmaUtil MfmaFlopsF16 MfmaFlopsF32
      for the matrix-core counters)
  python bench.py --traffic-from FETCH_CSV WRITE_CSV
      turn the two counter_collection.csv files of those runs into the per-call HBM traffic
      (profiles/kda_chunk_fwd_prefill_128k_h32_traffic.json), tagged with the kernel source hash
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s (H=32,d=128) + decode state-update HBM GB/s, 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak, published
MFMA_F32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix peak, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kda_chunk_fwd_prefill_128k_h32_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "gated_delta_rule_26_amd", "csrc", "kda_chunk.hip")
PREFILL_KERNELS = ("chunk_fwd_kernel", "replay_kernel", "split_combine_kernel")  # one call
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kda_decode_step_decode_256x32_traffic.json")
DECODE_SRC = os.path.join(ROOT, "gated_delta_rule_26_amd", "csrc", "kda_decode.hip")
DECODE_KERNELS = ("decode_kernel",)
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kda_chunk_bwd_backward_4k_h16_traffic.json")
BWD_SRC = os.path.join(ROOT, "gated_delta_rule_26_amd", "csrc", "kda_chunk_bwd.hip")
BWD_KERNELS = ("bwd_prep_kernel", "bwd_state_kernel", "bwd_grad_kernel")
DECODE_STEPS = 1000   # the decode workload: 1000 consecutive steps per timed block
COPY_BYTES = 1 << 30  # calibration: read 1 GiB, write 1 GiB


def prefill_bytes_per_token_head(K: int, V: int) -> int:
    """Algorithmic HBM bytes per (token, head): bf16 q and k, bf16 v, float32 g, float32
    beta, float32 o."""
    return 2 * K * 2 + V * 2 + K * 4 + 4 + V * 4


def prefill_flops_per_token_head(K: int, V: int, C: int) -> float:
    """Algorithmic flops per (token, head) of the chunkwise form: per chunk 3C^2K + 2C^2V +
    6CKV + C^3/3 (A, M and W; U~ and M U; W S, (q e^G) S and the state update; the
    triangular inverse)."""
    return (3 * C * C * K + 2 * C * C * V + 6 * C * K * V + C ** 3 / 3) / C


def bwd_bytes_per_token_head(K: int, V: int) -> int:
    """Algorithmic HBM bytes of the backward pass per (token, head): q, k, v bf16, g, beta
    and dL/do float32 read once; dq, dk, dg, dv, dbeta float32 written once."""
    return (2 * K * 2 + V * 2 + K * 4 + 4 + V * 4) + (3 * K * 4 + V * 4 + 4)


def bwd_flops_per_token_head(K: int, V: int, C: int) -> float:
    """Algorithmic flops per (token, head) of the chunked backward pass, per chunk (triangular
    products counted at half, as in the forward): recomputing A~, M, W (3 C^2 K), U~ (C^2 V),
    T (C^3/3), U = U~ - W S and the state update (4 CKV); the reverse state pass M^T dO (C^2 V),
    Kd dS', Qg^T dO, W^T dU (6 CKV); the gradient products dO S^T, U dS'^T, dU S^T (6 CKV),
    dM = dO U^T (C^2 V), dT = dU (beta v)^T + dW (beta K e^G)^T (C^2 V + C^2 K), T^T dU (C^2 V),
    T^T dW (C^2 K), T^T dT and its product with T^T (2 C^3/3), and the pair terms of A~ and M
    (4 C^2 K). Total 9 C^2 K + 5 C^2 V + 16 C K V + C^3 per chunk."""
    return (9 * C * C * K + 5 * C * C * V + 16 * C * K * V + C ** 3) / C


def fused_prefill_bytes_per_token_head(K: int, V: int) -> int:
    """Algorithmic HBM bytes per (token, head) of the fused prefill: bf16 raw q and k, bf16 v,
    the gate's bf16 pre-activation, float32 beta, the output gate's bf16 pre-activation and
    the bf16 normalised output."""
    return 2 * K * 2 + V * 2 + K * 2 + 4 + V * 2 + V * 2


def fused_decode_bytes_per_step(N: int, H: int, K: int, V: int) -> int:
    """State read + write (float32) plus bf16 q, k, v, gate and output-gate pre-activations,
    float32 beta and the bf16 output per (sequence, head)."""
    return 2 * N * H * K * V * 4 + N * H * (2 * K * 2 + V * 2 + K * 2 + 4 + V * 2) + N * H * V * 2


def decode_bytes_per_step(N: int, H: int, K: int, V: int) -> int:
    """State read + write (float32) plus one bf16 q, k, v, float32 g, beta and float32 o per
    (sequence, head)."""
    return 2 * N * H * K * V * 4 + N * H * (2 * K * 2 + V * 2 + K * 4 + 4) + N * H * V * 4


def kernel_sha(src: str | None = None) -> str:
    with open(src or KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(launch_bytes: float, path: str | None = None, src: str | None = None):
    """HBM traffic per launch from a committed rocprofv3 counter summary (the prefill's by
    default), or None when it is missing or was taken on a different version of the kernel
    source."""
    try:
        with open(path or TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_sha(src):
        return None
    return t.get("hbm_bytes_per_launch")


def _counter_rows(path: str):
    import csv
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            yield row["Kernel_Name"], int(row["Dispatch_Id"]), row["Counter_Name"], float(row["Counter_Value"])


def kernel_label(name: str) -> str:
    """Readable label of a prefill kernel from its (possibly mangled) name: the split flag and
    the fused steps come from the template arguments (chunk_fwd_kernel<..., STORE, FUSE>,
    replay_kernel<..., XMODE, FOUT>)."""
    import re
    m = re.search(r"chunk_fwd_kernel<[^>]*?(true|false), (\d+)>", name) or \
        re.search(r"chunk_fwd_kernel\w*?ELb(\d)ELi(\d)EEEv", name)
    if m:
        store = m.group(1) in ("true", "1")
        fuse = int(m.group(2))
        tag = "split forward, records" if store else "forward"
        if fuse & 1:
            tag += ", fused gate and q/k norm"
        if fuse & 2:
            tag += ", fused output norm"
        return f"chunk_fwd_kernel ({tag})"
    m = re.search(r"replay_kernel<[^>]*?(true|false), (true|false)>", name) or \
        re.search(r"replay_kernel\w*?ELb(\d)ELb(\d)EEEv", name)
    if m:
        if m.group(1) in ("true", "1"):
            return "replay_kernel (segment maps X)"
        return "replay_kernel (outputs" + (", fused output norm)" if m.group(2) in ("true", "1") else ")")
    if "replay_kernel" in name or "chunk_fwd_kernel" in name:
        return name
    return "split_combine_kernel"


def traffic_from(fetch_csv: str, write_csv: str, kernels=PREFILL_KERNELS,
                 call_kernel: str = "chunk_fwd_kernel") -> dict:
    """Per-call HBM bytes of one entry point (the prefill's kernels by default; one dispatch of
    ``call_kernel`` per call) from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each
    scaled by known bytes / counted bytes of the copy-like calibration kernel (it reads and
    writes COPY_BYTES)."""
    out = {}
    for key, path in (("fetch", fetch_csv), ("write", write_csv)):
        per_kernel, copy, calls = {}, [], set()
        for name, disp, cname, val in _counter_rows(path):
            if cname not in ("FETCH_SIZE", "WRITE_SIZE"):
                continue
            if any(k in name for k in kernels):
                short = kernel_label(name) if kernels == PREFILL_KERNELS else next(k for k in kernels if k in name)
                kib, n = per_kernel.get(short, (0.0, 0))
                per_kernel[short] = (kib + val, n + 1)
                if call_kernel in name:
                    calls.add(disp)
            elif "neg_kernel" in name:
                copy.append(val)
        if not copy or not calls:
            raise SystemExit(f"{path}: no {call_kernel} or calibration dispatches found")
        copy_kib = sum(copy) / len(copy)
        scale = (COPY_BYTES / 1024.0) / copy_kib
        total_kib = sum(kib for kib, _ in per_kernel.values())
        out[key] = {
            "calls": len(calls),
            "copy_counter_kib": copy_kib,
            "scale": scale,
            "bytes_per_call": total_kib / len(calls) * 1024.0 * scale,
            "per_kernel_kib_per_dispatch": {k: kib / n for k, (kib, n) in per_kernel.items()},
        }
    return out


def write_traffic(fetch_csv: str, write_csv: str) -> None:
    """The prefill call's, the decode step's and the backward call's traffic files from the
    counter pass."""
    for path, src, workload, kernels, call in (
            (TRAFFIC_FILE, KERNEL_SRC, "prefill_128k_h32 (one kda_chunk_fwd call)", PREFILL_KERNELS,
             "chunk_fwd_kernel"),
            (DECODE_TRAFFIC_FILE, DECODE_SRC, "decode_256x32 (one kda_decode_step call)", DECODE_KERNELS,
             "decode_kernel"),
            (BWD_TRAFFIC_FILE, BWD_SRC, "backward_4k_h16 (one kda_chunk_bwd call)", BWD_KERNELS,
             "bwd_grad_kernel")):
        t = traffic_from(fetch_csv, write_csv, kernels, call)
        res = {
            "kernel_source_sha": kernel_sha(src),
            "workload": workload,
            "hbm_bytes_per_launch": round(t["fetch"]["bytes_per_call"] + t["write"]["bytes_per_call"]),
            "fetch_bytes_per_launch": round(t["fetch"]["bytes_per_call"]),
            "write_bytes_per_launch": round(t["write"]["bytes_per_call"]),
            "calibration": {"kernel": "torch.neg over 1 GiB float32 (reads 1 GiB, writes 1 GiB)",
                            "fetch_scale": t["fetch"]["scale"], "write_scale": t["write"]["scale"]},
            "counters": t,
        }
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "w") as f:
            json.dump(res, f, indent=1)
        print(json.dumps(res, indent=1))


def other_workloads(kda, synth, to_dev, torch, np, log, state) -> dict:
    """Prefill tokens/s on the 4K-token and the packed variable-length workloads, the fused
    layer steps on the long-context prefill and on the decode step (``state``: the decode
    workload's states), and the device's copy bandwidth as a practical HBM reference (events
    on the current stream)."""
    out = {}

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # The 4K-token workloads' working sets (about 0.1 GB) fit in the 256 MB Infinity Cache, so
    # back-to-back calls find their inputs cached. Each is also timed cold: before every call a
    # reduction reads a 512 MiB buffer, which evicts the cache without leaving dirty lines to
    # be written back during the call, and events bracket the call alone.
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")

    def timed_cold(fn, reps):
        fn()
        evs = []
        for _ in range(reps):
            flush.max()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / reps

    w = synth.WORKLOADS["prefill_4k_h16"]
    x = synth.make_inputs(w)
    q, k, v = (to_dev(x[n][None], True) for n in ("q", "k", "v"))
    g, b = to_dev(x["g"][None]), to_dev(x["beta"][None])
    ws = torch.empty(max(kda.chunk_fwd_workspace_bytes(q, v), 1), dtype=torch.uint8, device="cuda")
    fwd = lambda: kda.kda_chunk_fwd(q, k, v, g, b, workspace=ws)  # noqa: E731
    ms, ms_cold = timed(fwd, 20), timed_cold(fwd, 20)
    pb = w.T * w.H * prefill_bytes_per_token_head(w.K, w.V) + w.H * w.K * w.V * 4
    out["prefill_4k_h16"] = {"ms": round(ms, 4), "tokens_per_s": round(w.T / (ms * 1e-3), 1),
                             "cache": "resident (back to back)",
                             "algorithmic_gbs": round(pb / (ms * 1e-3) / 1e9, 1),
                             "frac_hbm": round(pb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             "ms_cold": round(ms_cold, 4),
                             "tokens_per_s_cold": round(w.T / (ms_cold * 1e-3), 1),
                             "algorithmic_gbs_cold": round(pb / (ms_cold * 1e-3) / 1e9, 1),
                             "frac_hbm_cold": round(pb / (ms_cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             "algorithmic_bytes": pb,
                             "B": 1, "T": w.T, "H": w.H, "dk": w.K, "dv": w.V, "chunk": w.chunk}
    del q, k, v, g, b, ws, x
    log("timed prefill_4k_h16")

    # backward pass at the same shape (the training side): dL/do seeded, dL/dS_final zero
    x = synth.make_inputs(w)
    q, k, v = (to_dev(x[n][None], True) for n in ("q", "k", "v"))
    g, b = to_dev(x["g"][None]), to_dev(x["beta"][None])
    do = torch.from_numpy(np.stack([synth.grad_out(w, 0, h) for h in range(w.H)], axis=1)[None]).cuda()
    wsb = torch.empty(kda.chunk_bwd_workspace_bytes(q, v), dtype=torch.uint8, device="cuda")
    grads = tuple(torch.empty_like(t, dtype=torch.float32) for t in (g, g, do, g, b))
    bwd = lambda: kda.kda_chunk_bwd(q, k, v, g, b, do, grads=grads, workspace=wsb,  # noqa: E731
                                    want_dinitial_state=False)
    ms, ms_cold = timed(bwd, 20), timed_cold(bwd, 20)
    bb = w.T * w.H * bwd_bytes_per_token_head(w.K, w.V)
    bf = w.T * w.H * bwd_flops_per_token_head(w.K, w.V, w.chunk)
    out["backward_4k_h16"] = {
        "ms": round(ms, 4), "tokens_per_s": round(w.T / (ms * 1e-3), 1),
        "cache": "resident (back to back)",
        "ms_cold": round(ms_cold, 4), "tokens_per_s_cold": round(w.T / (ms_cold * 1e-3), 1),
        # float32-accurate throughout (products in float32 or as three bf16 products of split
        # factors): the matrix cores bind (about 99 flop per algorithmic byte against a ridge
        # of about 20), priced at the fp32 matrix peak
        "roofline": {"bound": "mfma_f32", "achieved": round(bf / (ms * 1e-3) / 1e12, 2),
                     "peak": MFMA_F32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(bf / (ms * 1e-3) / 1e12 / MFMA_F32_PEAK_TFLOPS, 4),
                     "algorithmic_flops": round(bf)},
        "algorithmic_gbs": round(bb / (ms * 1e-3) / 1e9, 1),
        "frac_hbm": round(bb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "bytes_per_token_head": bwd_bytes_per_token_head(w.K, w.V),
        "workspace_bytes": wsb.numel(),
        "traffic": load_traffic(bb, BWD_TRAFFIC_FILE, BWD_SRC),
        "what": "kda_chunk_bwd: dq, dk, dv, dg, dbeta from dL/do (float32 accuracy)"}
    del q, k, v, g, b, do, wsb, grads, x, flush
    log("timed backward_4k_h16")

    w = synth.WORKLOADS["varlen_64seq_h16"]
    x = synth.make_inputs(w)
    cu = torch.from_numpy(x["cu_seqlens"].astype(np.int32)).cuda()
    q, k, v = (to_dev(x[n], True) for n in ("q", "k", "v"))
    g, b = to_dev(x["g"]), to_dev(x["beta"])
    s0 = to_dev(x["initial_state"])
    n_tok = int(x["cu_seqlens"][-1])
    ws = torch.empty(max(kda.chunk_fwd_workspace_bytes(q, v, num_seqs=len(x["lengths"])), 1),
                     dtype=torch.uint8, device="cuda")
    ms = timed(lambda: kda.kda_chunk_fwd(q, k, v, g, b, initial_state=s0, cu_seqlens=cu,
                                         workspace=ws), 3)
    vb = n_tok * w.H * prefill_bytes_per_token_head(w.K, w.V) + 2 * len(x["lengths"]) * w.H * w.K * w.V * 4
    out["varlen_64seq_h16"] = {"ms": round(ms, 4), "tokens_per_s": round(n_tok / (ms * 1e-3), 1),
                               "algorithmic_gbs": round(vb / (ms * 1e-3) / 1e9, 1),
                               "frac_hbm": round(vb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                               "algorithmic_bytes": vb,
                               "sequences": len(x["lengths"]), "tokens": n_tok,
                               "longest": int(max(x["lengths"])), "H": w.H, "dk": w.K,
                               "order": "longest first"}
    del q, k, v, g, b, s0, cu, ws, x
    log("timed varlen_64seq_h16")

    # fused layer steps, long-context prefill shape: raw q/k normalised in-kernel, the gate
    # from its bf16 pre-activation, the gated RMSNorm of the output written as bf16
    w = synth.WORKLOADS["prefill_128k_h32"]
    x = synth.make_inputs(w, fused=True)
    q, k, v, gx, z = (to_dev(x[n][None], True) for n in ("q", "k", "v", "x", "z"))
    b = to_dev(x["beta"][None])
    A, dtb, wt = to_dev(x["A_log"]), to_dev(x["dt_bias"]), to_dev(x["norm_weight"])
    y = torch.empty((1, w.T, w.H, w.V), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((1, w.H, w.K, w.V), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(kda.chunk_fwd_workspace_bytes(q, v), 1), dtype=torch.uint8, device="cuda")
    ms = timed(lambda: kda.kda_chunk_fwd_fused(q, k, v, gx, A, dtb, b, o_gate=z, o_weight=wt,
                                               o_eps=x["norm_eps"], out_dtype=torch.bfloat16,
                                               final_state=S, o=y, workspace=ws), 10)
    fb = w.T * w.H * fused_prefill_bytes_per_token_head(w.K, w.V) + w.H * w.K * w.V * 4
    out["prefill_128k_h32_fused"] = {
        "ms": round(ms, 4), "tokens_per_s": round(w.T / (ms * 1e-3), 1),
        "algorithmic_gbs": round(fb / (ms * 1e-3) / 1e9, 1),
        "frac_hbm": round(fb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "bytes_per_token_head": fused_prefill_bytes_per_token_head(w.K, w.V),
        "steps": "gate from bf16 pre-activation, q/k L2 norm, gated RMSNorm, bf16 output"}
    del q, k, v, gx, z, b, y, S, ws, x
    log("timed prefill_128k_h32_fused")

    # 8 tokens per sequence and head in one call (the recurrent mode for short queries) on the
    # decode workload's states: the state is read and written once for the 8
    N, H = state.shape[0], state.shape[1]
    wd = synth.WORKLOADS["decode_256x32"].with_(prefill_T=0, decode_steps=8)
    x = synth.make_inputs(wd, seqs=range(N))
    dq, dk, dv = (to_dev(x["dec_" + n], True) for n in ("q", "k", "v"))
    dg, db = to_dev(x["dec_g"]), to_dev(x["dec_beta"])
    L8 = wd.decode_steps
    rq, rk, rv = (t.transpose(0, 1).contiguous() for t in (dq, dk, dv))    # [N, 8, H, D]
    rg, rb = dg.transpose(0, 1).contiguous(), db.transpose(0, 1).contiguous()
    ro = torch.empty((N, L8, H, wd.V), dtype=torch.float32, device="cuda")
    us = timed(lambda: kda.kda_recurrent_fwd(rq, rk, rv, rg, rb, state, o=ro), 20) * 1e3
    rbytes = 2 * N * H * wd.K * wd.V * 4 + N * L8 * H * (2 * wd.K * 2 + wd.V * 2 + wd.K * 4 + 4 + wd.V * 4)
    out["decode_256x32_8_tokens_per_call"] = {
        "avg_launch_us": round(us, 2), "tokens_per_s": round(N * L8 * 1e6 / us, 1),
        "us_per_token_step": round(us / L8, 2), "achieved_gbs": round(rbytes / (us * 1e-6) / 1e9, 1),
        "frac_hbm": round(rbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes": rbytes,
        "what": "kda_recurrent_fwd: 256 sequences x 32 heads x 8 tokens, state read and written once"}
    del dq, dk, dv, dg, db, x, rq, rk, rv, rg, rb, ro
    log("timed decode_256x32 with 8 tokens per call")

    x = synth.make_inputs(wd, seqs=range(N), fused=True)
    dq, dk, dv, dgx, dz = (to_dev(x["dec_" + n], True) for n in ("q", "k", "v", "x", "z"))
    db = to_dev(x["dec_beta"])
    A, dtb, wt = to_dev(x["A_log"]), to_dev(x["dt_bias"]), to_dev(x["norm_weight"])
    yd = torch.empty((N, H, wd.V), dtype=torch.bfloat16, device="cuda")
    it = iter(range(1 << 30))

    def dstep():
        i = next(it) % wd.decode_steps
        kda.kda_decode_step_fused(dq[i], dk[i], dv[i], dgx[i], A, dtb, db[i], state, o_gate=dz[i],
                                  o_weight=wt, o_eps=x["norm_eps"], out_dtype=torch.bfloat16,
                                  o=yd)
    us = timed(dstep, 50) * 1e3
    db_ = fused_decode_bytes_per_step(N, H, wd.K, wd.V)
    out["decode_256x32_fused"] = {
        "avg_launch_us": round(us, 2), "steps_per_s": round(1e6 / us, 1),
        "achieved_gbs": round(db_ / (us * 1e-6) / 1e9, 1),
        "frac_hbm": round(db_ / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": db_,
        "steps": "gate from bf16 pre-activation, q/k L2 norm, gated RMSNorm, bf16 output"}
    del dq, dk, dv, dgx, dz, db, yd, x
    log("timed decode_256x32_fused")

    # the layer's short convolutions (SiLU) on the long-context shape: raw q, k and v
    # projections, [131072, 32 * 128] bf16 each, one launch per tensor; and one decode update
    # of the decode workload's 256 sequences over all three (12288 channels)
    w = synth.WORKLOADS["prefill_128k_h32"]
    x = synth.make_inputs(w, fused=True)
    C = w.H * w.K
    xs = [to_dev(x[n].reshape(1, w.T, C), True) for n in ("q", "k", "v")]
    prm = [synth.conv_params(w, C, i) for i in range(3)]
    ws_ = [(to_dev(a), to_dev(b)) for a, b in prm]
    ys = [torch.empty_like(t) for t in xs]
    fs = [torch.empty((1, 3, C), dtype=torch.bfloat16, device="cuda") for _ in xs]

    def conv3():
        for i in range(3):
            kda.kda_short_conv_fwd(xs[i], ws_[i][0], ws_[i][1], final_state=fs[i], y=ys[i])
    ms = timed(conv3, 10)
    cb = 3 * w.T * C * (2 + 2)
    out["short_conv_128k_h32"] = {
        "ms": round(ms, 4), "tokens_per_s": round(w.T / (ms * 1e-3), 1),
        "algorithmic_gbs": round(cb / (ms * 1e-3) / 1e9, 1),
        "frac_hbm": round(cb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "bytes": cb, "what": "q, k, v: 3 x [131072, 4096] bf16, width-4 depthwise causal conv + SiLU"}
    del xs, ys, fs, ws_, x
    log("timed short_conv_128k_h32")
    N3 = 256
    wd = synth.WORKLOADS["decode_256x32"]
    C3 = 3 * wd.H * wd.K
    xt = to_dev(synth.fused_slab(wd.with_(K=C3), 0, 0, N3)["q"], True)      # [256, 12288]
    st = to_dev(synth.conv_state(wd, N3, C3), True)
    cw, cbias = (to_dev(a) for a in synth.conv_params(wd, C3))
    yt = torch.empty_like(xt)
    us = timed(lambda: kda.kda_short_conv_update(xt, cw, cbias, st, y=yt), 50) * 1e3
    ub = N3 * C3 * (2 + 2 + 2 * 3 * 2)
    out["short_conv_update_256"] = {
        "avg_launch_us": round(us, 2), "achieved_gbs": round(ub / (us * 1e-6) / 1e9, 1),
        "frac_hbm": round(ub / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "bytes": ub, "what": "256 sequences x 12288 channels (q, k, v), state [3, C] bf16 in place"}
    log("timed short_conv_update_256")

    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
    dst = torch.empty_like(src)
    ms = timed(lambda: dst.copy_(src), 10)
    out["copy_reference"] = {"bytes": 2 << 30, "gbs": round((2 << 30) / (ms * 1e-3) / 1e9, 1),
                             "what": "device-to-device copy of 1 GiB (read + write)"}
    # the device's practical peaks, from the library's probes: a copy with 16-byte
    # non-temporal loads; a read-only stream (the bound of the read-mostly prefill); an
    # in-place read-modify-write stream (the decode step's state pattern); and a loop of
    # independent fp16 / bf16 matrix-core products on every CU
    ms = timed(lambda: kda.kda_probe_copy(src, dst), 10)
    copy_gbs = (2 << 30) / (ms * 1e-3) / 1e9
    ms = timed(lambda: kda.kda_probe_read(src), 10)
    read_gbs = (1 << 30) / (ms * 1e-3) / 1e9
    ms = timed(lambda: kda.kda_probe_rmw(src, 1.0), 10)
    rmw_gbs = (2 << 30) / (ms * 1e-3) / 1e9
    blocks, iters = 2048, 2000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    tf, tb = {}, {}
    for probe, rates in ((kda.kda_probe_mfma_f16, tf), (kda.kda_probe_mfma_bf16, tb)):
        for shape, name in ((0, "16x16x32"), (1, "32x32x16")):
            flops = probe(iters, blocks, sink, shape=shape)
            ms = timed(lambda: probe(iters, blocks, sink, shape=shape), 5)
            rates[name] = flops / (ms * 1e-3) / 1e12
    best = max(tf.values())
    best_copy = max(copy_gbs, out["copy_reference"]["gbs"])
    out["measured_peaks"] = {
        "hbm_read_gbs": round(read_gbs, 1), "hbm_read_frac_of_published": round(read_gbs / HBM_PEAK_GBS, 4),
        "hbm_rmw_gbs": round(rmw_gbs, 1), "hbm_rmw_frac_of_published": round(rmw_gbs / HBM_PEAK_GBS, 4),
        "hbm_copy_gbs": round(best_copy, 1),
        "hbm_gbs_by_copy": {"kda_probe_copy": round(copy_gbs, 1), "torch copy_": out["copy_reference"]["gbs"]},
        "mfma_f16_tflops": round(best, 1),
        "mfma_f16_tflops_by_instruction": {k: round(v, 1) for k, v in tf.items()},
        "mfma_bf16_tflops_by_instruction": {k: round(v, 1) for k, v in tb.items()},
        "mfma_frac_of_published": round(best / MFMA_F16_PEAK_TFLOPS, 4),
        "what": ("1 GiB: kda_probe_read (non-temporal loads, 64 KB per workgroup), kda_probe_rmw (in place, "
                 "non-temporal loads and stores, 16 KB per workgroup), the better of two copies; "
                 "kda_probe_mfma_f16 / _bf16, 2048 x 256 threads")}
    del src, dst, sink
    log("measured the read, read-modify-write, copy and matrix-core peaks")
    return out


def cpu_baseline(x: dict, sample_tokens: int) -> dict:
    """The float64 oracle (unchanged) on the first ``sample_tokens`` tokens of the prefill
    workload, all heads, on the host's cores."""
    import numpy as np

    import oracle
    import synth
    threads = min(os.cpu_count() or 1, x["q"].shape[1], 16)
    sl = slice(0, sample_tokens)
    args = (synth.stored_to_f64(x["q"][sl], "bf16"), synth.stored_to_f64(x["k"][sl], "bf16"),
            synth.stored_to_f64(x["v"][sl], "bf16"), x["g"][sl].astype(np.float64),
            x["beta"][sl].astype(np.float64))
    t0 = time.perf_counter()
    oracle.kda_fwd(*args, threads=threads)
    dt = time.perf_counter() - t0
    # one thread on a shorter prefix (the rate per token is the same: every token costs the
    # same recurrence step)
    t1 = min(sample_tokens, 4096)
    s1 = slice(0, t1)
    t0 = time.perf_counter()
    oracle.kda_fwd(*(a[s1] for a in args), threads=1)
    dt1 = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": sample_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"prefill_128k_h32, " +
                       ("all" if sample_tokens == x["q"].shape[0] else "first") +
                       f" {sample_tokens} tokens x {x['q'].shape[1]} heads "
                       f"(float64 recurrence, {dt:.1f} s wall)"),
            "single_thread": {"value": t1 / dt1, "unit": "tokens/s",
                              "sample": f"first {t1} tokens x {x['q'].shape[1]} heads ({dt1:.1f} s wall)"},
            "host": {"nproc": os.cpu_count(), "cpu": model}}



def cpu_baseline_decode(tok: dict, N: int, H: int, K: int, V: int) -> dict:
    """The float64 oracle's decode step (unchanged) over consecutive tokens of the decode
    workload, all N x H states, on the host's cores. The states start at zero: a step costs
    the same whatever their values, and starting from the 2048-token prefill would add its
    own minutes of oracle time to the baseline."""
    import numpy as np

    import oracle
    import synth
    steps = tok["q"].shape[0]
    threads = min(os.cpu_count() or 1, 16)
    st = lambda a: synth.stored_to_f64(a, "bf16")  # noqa: E731
    args = [(st(tok["q"][j]), st(tok["k"][j]), st(tok["v"][j]), tok["g"][j].astype(np.float64),
             tok["beta"][j].astype(np.float64)) for j in range(steps)]
    state = np.zeros((N, H, K, V))
    t0 = time.perf_counter()
    for a in args:
        _, state = oracle.kda_decode_step(*a, state, threads=threads)
    dt = time.perf_counter() - t0
    return {"value": steps / dt, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"decode_256x32: {steps} consecutive steps over all {N} x {H} states "
                      f"(float64 recurrence, {dt:.1f} s wall)"}

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=131072)
    ap.add_argument("--cpu-decode-steps", type=int, default=8,
                    help="consecutive oracle decode steps timed for the CPU baseline")
    ap.add_argument("--decode-seqs", type=int, default=256)
    ap.add_argument("--decode-steps", type=int, default=DECODE_STEPS,
                    help="consecutive decode steps in each step's timed block (the workload's 1000)")
    ap.add_argument("--counter-pass", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads (4K prefill, packed varlen) and the copy reference")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic(*args.traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported "
              "(the KDA core needs no collectives: (sequence, head) chains are independent)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_delta_rule_26_amd as kda
    import synth

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    dev = "cuda"
    to_dev = lambda a, bf=False: (torch.from_numpy(np.ascontiguousarray(a).view(np.int16))  # noqa: E731
                                  .view(torch.bfloat16) if bf else torch.from_numpy(a)).to(dev)

    # ---------------------------------------------------------------- prefill workload
    wp = synth.WORKLOADS["prefill_128k_h32"]
    t0 = time.perf_counter()
    xp = synth.make_inputs(wp)
    log(f"generated prefill inputs in {time.perf_counter() - t0:.1f}s")
    T, H, K, V, C = wp.T, wp.H, wp.K, wp.V, wp.chunk
    pq, pk, pv = (to_dev(xp[n][None], True) for n in ("q", "k", "v"))
    pg, pb = to_dev(xp["g"][None]), to_dev(xp["beta"][None])
    po = torch.empty((1, T, H, V), dtype=torch.float32, device=dev)
    pS = torch.empty((1, H, K, V), dtype=torch.float32, device=dev)
    ws_bytes = kda.chunk_fwd_workspace_bytes(pq, pv, chunk=C)
    pws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    if args.counter_pass:
        # prefill calls only, then decode steps, then the copy-like calibration kernel
        for _ in range(args.warmup + args.steps):
            kda.kda_chunk_fwd(pq, pk, pv, pg, pb, final_state=pS, o=po, workspace=pws)
        torch.cuda.synchronize()
        # decode steps on 256 x 32 states (the traffic does not depend on the values)
        wd = synth.WORKLOADS["decode_256x32"].with_(prefill_T=0, decode_steps=8)
        xd = synth.make_inputs(wd, seqs=range(args.decode_seqs))
        tq, tk, tv = (to_dev(xd["dec_" + n], True) for n in ("q", "k", "v"))
        tg, tb = to_dev(xd["dec_g"]), to_dev(xd["dec_beta"])
        state = torch.zeros((args.decode_seqs, H, K, V), dtype=torch.float32, device=dev)
        to = torch.empty((args.decode_seqs, H, V), dtype=torch.float32, device=dev)
        for i in range(args.steps):
            j = i % wd.decode_steps
            kda.kda_decode_step(tq[j], tk[j], tv[j], tg[j], tb[j], state, o=to)
        torch.cuda.synchronize()
        del tq, tk, tv, tg, tb, state, to, xd
        # two backward calls at the 4K-token, 16-head training shape (matrix-core counters)
        wb = synth.WORKLOADS["prefill_4k_h16"]
        xb = synth.make_inputs(wb)
        bq, bk, bv = (to_dev(xb[n][None], True) for n in ("q", "k", "v"))
        bg, bb = to_dev(xb["g"][None]), to_dev(xb["beta"][None])
        bdo = torch.from_numpy(np.stack([synth.grad_out(wb, 0, h) for h in range(wb.H)], axis=1)[None]).to(dev)
        for _ in range(2):
            kda.kda_chunk_bwd(bq, bk, bv, bg, bb, bdo, want_dinitial_state=False)
        torch.cuda.synchronize()
        del bq, bk, bv, bg, bb, bdo, xb
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"counter pass: {args.warmup + args.steps} prefill calls (workspace {ws_bytes} B), "
            f"{args.steps} decode steps, 3 calibration copies of {COPY_BYTES} B")
        return

    # ----------------------------------------------------------------- decode workload
    # 256 sequences x 32 heads; the states come from a 2048-token prefill, then each step of
    # the benchmark runs the workload's consecutive decode steps (one token per sequence and
    # head per step, the state updated in place and read back by the next step)
    nd = args.decode_steps
    wd = synth.WORKLOADS["decode_256x32"].with_(decode_steps=nd)
    t0 = time.perf_counter()
    xd = synth.make_inputs(wd, seqs=range(args.decode_seqs))
    log(f"generated decode inputs in {time.perf_counter() - t0:.1f}s")
    N = args.decode_seqs
    dq, dk, dv = (to_dev(xd[n].reshape(N, wd.prefill_T, H, K), True) for n in ("q", "k", "v"))
    dg = to_dev(xd["g"].reshape(N, wd.prefill_T, H, K))
    db = to_dev(xd["beta"].reshape(N, wd.prefill_T, H))
    state = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    kda.kda_chunk_fwd(dq, dk, dv, dg, db, final_state=state)  # the 2048-token prefill
    del dq, dk, dv, dg, db
    tq, tk, tv = (to_dev(xd["dec_" + n], True) for n in ("q", "k", "v"))
    tg, tb = to_dev(xd["dec_g"]), to_dev(xd["dec_beta"])
    dec_tok = {n: xd["dec_" + n][:args.cpu_decode_steps] for n in ("q", "k", "v", "g", "beta")}
    del xd
    tokens = [(tq[j], tk[j], tv[j], tg[j], tb[j]) for j in range(nd)]
    to = torch.empty((N, H, V), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log("inputs resident in HBM")

    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        kda.kda_chunk_fwd(pq, pk, pv, pg, pb, final_state=pS, o=po, workspace=pws)
        if ev:
            ev[1].record(stream)
        for t in tokens:
            kda.kda_decode_step(*t, state, o=to)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    pre_ms = [e[0].elapsed_time(e[1]) for e in evs]
    blk_ms = [e[1].elapsed_time(e[2]) for e in evs]
    pre_avg = sum(pre_ms) / len(pre_ms)
    dec_avg = sum(blk_ms) / len(blk_ms) / nd   # ms per decode step, over blocks of nd steps

    tok_s = T / (pre_avg * 1e-3)
    p_bytes = T * H * prefill_bytes_per_token_head(K, V) + H * K * V * 4  # + final state
    p_flops = T * H * prefill_flops_per_token_head(K, V, C)
    achieved_gbs = p_bytes / (pre_avg * 1e-3) / 1e9
    d_bytes = decode_bytes_per_step(N, H, K, V)
    d_gbs = d_bytes / (dec_avg * 1e-3) / 1e9

    traffic = load_traffic(p_bytes)
    d_traffic = load_traffic(d_bytes, DECODE_TRAFFIC_FILE, DECODE_SRC) if N == 256 else None
    res = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"prefill_128k_h32 + decode_256x32 ({nd} consecutive steps)",
            "prefill": {"B": 1, "T": T, "H": H, "dk": K, "dv": V, "chunk": C,
                        "inputs": "bf16 q/k/v, f32 g/beta", "outputs": "f32 o and final state"},
            "decode": {"N": N, "H": H, "dk": K, "dv": V, "state": "f32, updated in place",
                       "state_init": "2048-token prefill", "steps_per_step": nd},
            "compute": "fp16 matrix-core operands, f32 accumulation and state",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "kda_chunk_fwd (prefill_128k_h32)",
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": p_bytes,
            "avg_launch_ms": round(pre_avg, 4),
            "mfma_frac_algorithmic": round(p_flops / (pre_avg * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
        },
        "decode": {
            "kernel": "kda_decode_step (decode_256x32)",
            "protocol": f"{nd} consecutive steps between one pair of events (each step reads the "
                        "state the previous one wrote)",
            "avg_launch_us": round(dec_avg * 1e3, 2),
            "steps_per_s": round(1e3 / dec_avg, 1),
            "tokens_per_s": round(N * 1e3 / dec_avg, 1),
            "achieved_gbs": round(d_gbs, 1),
            "peak_gbs": HBM_PEAK_GBS,
            "frac": round(d_gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_step": d_bytes,
            "traffic": d_traffic,
        },
        "cpu_baseline": None,
        "other_workloads": None,
    }
    if not args.no_extra:
        del pq, pk, pv, pg, pb, po, pws, tq, tk, tv, tg, tb, tokens
        res["other_workloads"] = other_workloads(kda, synth, to_dev, torch, np, log, state)
        mp = res["other_workloads"]["measured_peaks"]
        res["roofline"]["frac_of_measured_peak"] = round(res["roofline"]["achieved"] / mp["hbm_read_gbs"], 4)
        res["decode"]["frac_of_measured_peak"] = round(res["decode"]["achieved_gbs"] / mp["hbm_rmw_gbs"], 4)
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(xp, min(args.cpu_sample_tokens, T))
        res["cpu_baseline"]["decode"] = cpu_baseline_decode(dec_tok, N, H, K, V)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
