"""kda_chunk_fwd on the GPU against the float64 oracle.

Tolerances (max |gpu - oracle| <= tol * RMS(oracle), per returned tensor):
  float32 instantiations: 1e-4;  bf16-input / float32-accumulate instantiation: 2e-2."""

import numpy as np
import pytest

import gated_delta_rule_26_amd as kda
import synth
from kda_testutil import (assert_close, f64, note, random_inputs, random_states, run_oracle,
                          to_dev, torch_mod)

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def gpu_chunk(x, stored, *, B=1, chunk, s0=None, cu=None, scale=1.0, alias=False, split=True):
    torch = torch_mod()
    T = x["q"].shape[0] // B
    sh = lambda a: a.reshape(B, T, *a.shape[1:]) if cu is None else a  # noqa: E731
    q, k, v = (to_dev(sh(x[key]), stored) for key in ("q", "k", "v"))
    g, beta = to_dev(sh(x["g"])), to_dev(sh(x["beta"]))
    init = None if s0 is None else to_dev(np.ascontiguousarray(s0, dtype=np.float32))
    cu_t = None if cu is None else to_dev(np.asarray(cu, dtype=np.int32))
    o, S = kda.kda_chunk_fwd(q, k, v, g, beta, initial_state=init, cu_seqlens=cu_t, chunk=chunk,
                             scale=scale, final_state=init if alias else None, split=split)
    torch.cuda.synchronize()
    return o.reshape(x["v"].shape).cpu().numpy(), S.cpu().numpy()


# ------------------------------------------------------------------- float32 instantiations

def test_tiny_f32_workload():
    """fp32 everywhere, B=1, T=256, H=2, Dk=Dv=16, chunk 16, zero initial state."""
    w = synth.WORKLOADS["tiny_f32"]
    x = synth.make_inputs(w)
    note("tiny_f32 full")
    o, S = gpu_chunk(x, "f32", chunk=16)
    o_ref, S_ref = run_oracle(x, "f32")
    assert_close(o, o_ref, TOL_F32, "o")
    assert_close(S, S_ref, TOL_F32, "final state")


@pytest.mark.parametrize("D,C", [(16, 16), (32, 16), (32, 64), (64, 64), (128, 32)])
@pytest.mark.parametrize("T", [1, 15, 50, 64, 65, 200, 333])
def test_f32_ragged_lengths_with_state(D, C, T):
    H = 3
    x = random_inputs(100 + T, T, H, D, "f32")
    s0 = random_states(101 + T, 1, H, D)
    note(f"f32 D={D} C={C} T={T}")
    o, S = gpu_chunk(x, "f32", chunk=C, s0=s0, scale=0.5)
    o_ref, S_ref = run_oracle(x, "f32", scale=0.5, initial_state=s0)
    assert_close(o, o_ref, TOL_F32, "o")
    assert_close(S, S_ref, TOL_F32, "final state")


@pytest.mark.parametrize("D,C", [(16, 16), (32, 16), (32, 64), (128, 32)])
def test_f32_batched_sequences(D, C):
    B, T, H = 3, 150, 2
    x = random_inputs(110 + D, B * T, H, D, "f32")
    s0 = random_states(111, B, H, D)
    note(f"f32 batched B={B} D={D}")
    o, S = gpu_chunk(x, "f32", B=B, chunk=C, s0=s0)
    o_ref, S_ref = run_oracle(x, "f32", initial_state=s0, cu=np.arange(B + 1) * T)
    assert_close(o, o_ref, TOL_F32, "o")
    assert_close(S, S_ref, TOL_F32, "final state")


@pytest.mark.parametrize("D,C", [(16, 16), (32, 16), (32, 64), (64, 64), (128, 32)])
def test_f32_packed_with_empty_sequences(D, C):
    lens = [0, 70, 1, 128, 5, 0, 300]
    cu = np.concatenate([[0], np.cumsum(lens)])
    H = 2
    x = random_inputs(120 + D, int(cu[-1]), H, D, "f32")
    s0 = random_states(121, len(lens), H, D)
    note(f"f32 packed D={D}")
    o, S = gpu_chunk(x, "f32", chunk=C, s0=s0, cu=cu)
    o_ref, S_ref = run_oracle(x, "f32", initial_state=s0, cu=cu)
    assert_close(o, o_ref, TOL_F32, "o")
    assert_close(S, S_ref, TOL_F32, "final states")
    np.testing.assert_array_equal(S[0], s0[0])   # empty sequences keep their state
    np.testing.assert_array_equal(S[5], s0[5])


@pytest.mark.parametrize("D,C", [(16, 16), (32, 64), (128, 32)])
def test_f32_strong_decay(D, C):
    """g = -3 per token: the decay over a 64-token chunk is e^-192, far below float32's range;
    the per-16-token factorisation keeps every operand finite."""
    T, H = 200, 2
    x = random_inputs(130, T, H, D, "f32", g_const=-3.0)
    s0 = random_states(131, 1, H, D)
    note(f"f32 strong decay D={D}")
    o, S = gpu_chunk(x, "f32", chunk=C, s0=s0)
    o_ref, S_ref = run_oracle(x, "f32", initial_state=s0)
    assert_close(o, o_ref, TOL_F32, "o")
    assert_close(S, S_ref, TOL_F32, "final state")


def extreme_gates(x, seed: int, g_min: float):
    """Overwrite a seeded half of the channels of every head with per-token log-decays drawn
    uniformly from [g_min, 0.8 g_min] on a random third of the tokens: the mix of decays that
    no single reference per 16-token block can represent (a factor e^{16 |g|} overflows
    float32 for |g| > 5.5) next to ordinary channels."""
    rng = np.random.default_rng(seed)
    T, H, K = x["g"].shape
    tok = rng.random(T) < 1 / 3
    ch = rng.random((H, K)) < 0.5
    sel = tok[:, None, None] & ch[None]
    vals = rng.uniform(g_min, 0.8 * g_min, size=x["g"].shape).astype(np.float32)
    x["g"][sel] = vals[sel]
    return x


@pytest.mark.parametrize("D,C", [(16, 16), (32, 64), (64, 64), (128, 32)])
@pytest.mark.parametrize("g_min", [-8.0, -40.0, -400.0])
def test_f32_extreme_decay(D, C, g_min):
    """Per-token decays down to e^-400 (block decays far below e^-60): the diagonal blocks are
    summed pair by pair from the cumulative log-decay."""
    T, H = 333, 2
    x = extreme_gates(random_inputs(135, T, H, D, "f32"), 136, g_min)
    s0 = random_states(137, 1, H, D)
    note(f"f32 extreme decay D={D} g_min={g_min}")
    o, S = gpu_chunk(x, "f32", chunk=C, s0=s0, scale=D ** -0.5)
    o_ref, S_ref = run_oracle(x, "f32", scale=D ** -0.5, initial_state=s0)
    assert_close(o, o_ref, TOL_F32, "o")
    assert_close(S, S_ref, TOL_F32, "final state")


def test_f32_prefill_4k_h16_inputs_at_head_size_128():
    """The 4K-token, 16-head workload's bf16 inputs upcast exactly to float32, through the
    float32 instantiation at the real head size (Dk = Dv = 128, 32-token chunks): the 1e-4
    float32 bound at D = 128 separates the algorithm's own error from the bf16 path's fp16
    operand rounding."""
    w = synth.WORKLOADS["prefill_4k_h16"]
    x = synth.make_inputs(w)
    for key in ("q", "k", "v"):
        x[key] = synth.bf16_bits_to_f32(x[key])
    note("prefill_4k_h16 inputs, float32 instantiation (C=32, D=128)")
    o, S = gpu_chunk(x, "f32", chunk=32)
    o_ref, S_ref = run_oracle(x, "f32")
    assert_close(o, o_ref, TOL_F32, "o")
    assert_close(S, S_ref, TOL_F32, "final state")
    o1, S1 = gpu_chunk(x, "f32", chunk=32, split=False)
    assert_close(o1, o_ref, TOL_F32, "o (one pass)")
    assert_close(S1, S_ref, TOL_F32, "final state (one pass)")


# ----------------------------------------------------------------------- bf16 instantiation

def test_bf16_prefill_4k_h16_workload():
    """bf16 q/k/v, fp32 gates and state: B=1, T=4096, H=16, Dk=Dv=128, chunk 64, zero state."""
    w = synth.WORKLOADS["prefill_4k_h16"]
    x = synth.make_inputs(w)
    note("prefill_4k_h16 full")
    o, S = gpu_chunk(x, "bf16", chunk=64)
    o_ref, S_ref = run_oracle(x, "bf16")
    assert_close(o, o_ref, TOL_BF16, "o")
    assert_close(S, S_ref, TOL_BF16, "final state")


@pytest.mark.parametrize("T", [1, 17, 63, 64, 65, 130, 1000])
def test_bf16_ragged_batched_with_state(T):
    B, H, D = 2, 2, 128
    x = random_inputs(140 + T, B * T, H, D, "bf16")
    s0 = random_states(141, B, H, D)
    note(f"bf16 T={T}")
    o, S = gpu_chunk(x, "bf16", B=B, chunk=64, s0=s0, scale=0.9)
    o_ref, S_ref = run_oracle(x, "bf16", scale=0.9, initial_state=s0, cu=np.arange(B + 1) * T)
    assert_close(o, o_ref, TOL_BF16, "o")
    assert_close(S, S_ref, TOL_BF16, "final state")


def test_bf16_packed_aliasing_and_empty():
    lens = [300, 0, 64, 1, 777, 0, 129]
    cu = np.concatenate([[0], np.cumsum(lens)])
    H, D = 3, 128
    x = random_inputs(150, int(cu[-1]), H, D, "bf16")
    s0 = random_states(151, len(lens), H, D)
    note("bf16 packed aliasing")
    o, S = gpu_chunk(x, "bf16", chunk=64, s0=s0, cu=cu, alias=True)
    o_ref, S_ref = run_oracle(x, "bf16", initial_state=s0, cu=cu)
    assert_close(o, o_ref, TOL_BF16, "o")
    assert_close(S, S_ref, TOL_BF16, "final states")
    np.testing.assert_array_equal(S[1], s0[1])


def test_bf16_strong_decay():
    T, H, D = 300, 2, 128
    x = random_inputs(160, T, H, D, "bf16", g_const=-3.0)
    note("bf16 strong decay")
    o, S = gpu_chunk(x, "bf16", chunk=64)
    o_ref, S_ref = run_oracle(x, "bf16")
    assert_close(o, o_ref, TOL_BF16, "o")
    assert_close(S, S_ref, TOL_BF16, "final state")


@pytest.mark.parametrize("split", [False, True])
def test_bf16_large_values_within_fp16_range(split):
    """Values and states 512 times larger than the workloads' (v ~ N(0, 512^2), initial
    states of spectral norm 512): the fp16 matrix-core operands (S, U~, U, v) stay below fp16's
    largest value 65504, the range precondition of the bf16 instantiation, and the result
    holds the bf16 bound. (The scale is a power of two: the bf16 values are exact.)"""
    T, H, D = 2500, 2, 128
    x = random_inputs(185, T, H, D, "bf16")
    x["v"] = synth.f64_to_bf16_bits(512.0 * synth.bf16_bits_to_f64(x["v"]))
    s0 = 512.0 * random_states(186, 1, H, D)
    note(f"bf16 large values split={split}")
    o, S = gpu_chunk(x, "bf16", chunk=64, s0=s0, split=split)
    o_ref, S_ref = run_oracle(x, "bf16", initial_state=s0)
    assert float(np.max(np.abs(S_ref))) < 65504 and float(np.max(np.abs(o_ref))) < 65504
    assert_close(o, o_ref, TOL_BF16, "o")
    assert_close(S, S_ref, TOL_BF16, "final state")


def test_f32_large_values_have_no_range_limit():
    """The float32 instantiations carry no fp16 operands: values 10^6 times the workloads'."""
    T, H, D = 700, 2, 64
    x = random_inputs(187, T, H, D, "f32")
    x["v"] = (x["v"].astype(np.float64) * 1e6).astype(np.float32)
    s0 = (1e6 * random_states(188, 1, H, D)).astype(np.float32)
    note("f32 large values")
    o, S = gpu_chunk(x, "f32", chunk=64, s0=s0)
    o_ref, S_ref = run_oracle(x, "f32", initial_state=s0)
    assert float(np.max(np.abs(S_ref))) > 1e6
    assert_close(o, o_ref, TOL_F32, "o")
    assert_close(S, S_ref, TOL_F32, "final state")


@pytest.mark.parametrize("g_min", [-2.0, -8.0, -40.0, -400.0])
def test_bf16_extreme_decay(g_min):
    """Chunks whose blocks decay below e^-20 in some channels: bf16 off-diagonal operands and
    float32 pair-by-pair diagonal blocks, for decays up to e^-400 per token."""
    T, H, D = 1000, 2, 128
    x = extreme_gates(random_inputs(165, T, H, D, "bf16"), 166, g_min)
    s0 = random_states(167, 1, H, D)
    note(f"bf16 extreme decay g_min={g_min}")
    o, S = gpu_chunk(x, "bf16", chunk=64, s0=s0, scale=D ** -0.5)
    o_ref, S_ref = run_oracle(x, "bf16", scale=D ** -0.5, initial_state=s0)
    assert_close(o, o_ref, TOL_BF16, "o")
    assert_close(S, S_ref, TOL_BF16, "final state")


@pytest.mark.parametrize("g_c", [-0.6, -0.74, -1.2, -3.0])
def test_bf16_constant_channel_decay(g_c):
    """Half the channels decay by e^{g_c} on every token (16-token block decay e^{16 g_c}):
    around e^-12 the balanced fp16 factors meet the pair-by-pair diagonal path."""
    T, H, D = 640, 2, 128
    x = random_inputs(175, T, H, D, "bf16")
    ch = np.random.default_rng(176).random((H, D)) < 0.5
    x["g"][:, ch] = np.float32(g_c)
    s0 = random_states(177, 1, H, D)
    note(f"bf16 constant channel decay g={g_c}")
    o, S = gpu_chunk(x, "bf16", chunk=64, s0=s0, scale=D ** -0.5)
    o_ref, S_ref = run_oracle(x, "bf16", scale=D ** -0.5, initial_state=s0)
    assert_close(o, o_ref, TOL_BF16, "o")
    assert_close(S, S_ref, TOL_BF16, "final state")


@pytest.mark.parametrize("where", ["block0", "block2"])
def test_bf16_single_channel_extreme(where):
    """One channel alone (77, odd, owned by neither the first lane nor the first wave) decays
    by e^-5 per token for 16 tokens inside one chunk: a single thread's vote must switch the
    whole chunk to the pair-by-pair diagonal path."""
    T, H, D = 256, 2, 128
    x = random_inputs(178, T, H, D, "bf16")
    t0 = 64 + (0 if where == "block0" else 32)
    x["g"][t0:t0 + 16, :, 77] = np.float32(-5.0)
    s0 = random_states(179, 1, H, D)
    note(f"bf16 single channel extreme {where}")
    o, S = gpu_chunk(x, "bf16", chunk=64, s0=s0, scale=D ** -0.5)
    o_ref, S_ref = run_oracle(x, "bf16", scale=D ** -0.5, initial_state=s0)
    assert_close(o, o_ref, TOL_BF16, "o")
    assert_close(S, S_ref, TOL_BF16, "final state")


def test_bf16_prefill_then_decode_equals_prefill():
    torch = torch_mod()
    P, steps, H, D = 200, 24, 2, 128
    x = random_inputs(170, P + steps, H, D, "bf16")
    note("bf16 prefill then decode")
    o_all, S_all = gpu_chunk(x, "bf16", chunk=64)
    head = {key: val[:P] for key, val in x.items() if key in ("q", "k", "v", "g", "beta")}
    _, S = gpu_chunk(head, "bf16", chunk=64)
    state = to_dev(S)
    outs = []
    for t in range(P, P + steps):
        o = kda.kda_decode_step(*(to_dev(x[key][t:t + 1], "bf16") for key in ("q", "k", "v")),
                                to_dev(x["g"][t:t + 1]), to_dev(x["beta"][t:t + 1]), state)
        outs.append(o.cpu().numpy()[0])
    torch.cuda.synchronize()
    o_ref, S_ref = run_oracle(x, "bf16")
    assert_close(np.stack(outs), o_ref[P:], TOL_BF16, "decode o vs oracle")
    assert_close(state.cpu().numpy(), S_ref, TOL_BF16, "state vs oracle")
    assert_close(np.stack(outs), o_all[P:], TOL_BF16, "decode o vs one prefill")


def test_bf16_bitwise_deterministic():
    x = random_inputs(180, 1000, 4, 128, "bf16")
    note("bf16 determinism")
    o1, S1 = gpu_chunk(x, "bf16", chunk=64)
    o2, S2 = gpu_chunk(x, "bf16", chunk=64)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def test_zero_length_batch_keeps_state():
    torch = torch_mod()
    H, D = 2, 128
    s0 = random_states(190, 3, H, D)
    note("zero-length batch")
    e = torch.empty((3, 0, H, D), dtype=torch.bfloat16, device="cuda")
    ef = torch.empty((3, 0, H, D), dtype=torch.float32, device="cuda")
    eb = torch.empty((3, 0, H), dtype=torch.float32, device="cuda")
    o, S = kda.kda_chunk_fwd(e, e, e, ef, eb, initial_state=to_dev(s0))
    torch.cuda.synchronize()
    assert o.shape == (3, 0, H, D)
    np.testing.assert_array_equal(S.cpu().numpy(), s0)


# --------------------------------------------------------------- sequence split (few chains)

def split_bytes(B, T, H, D, C, stored):
    lib = kda.load_library()
    return lib.kda_chunk_fwd_workspace_bytes(B, T, H, D, D, C, 1 if stored == "bf16" else 0, B)


SPLIT_CASES = [
    # (stored, D, C, B, T, H): each gives few chains and enough chunks for several segments
    ("bf16", 128, 64, 1, 5000, 2),
    ("bf16", 128, 64, 2, 8192 + 37, 3),
    ("bf16", 128, 64, 1, 2048, 1),
    ("f32", 16, 16, 1, 700, 1),
    ("f32", 32, 64, 1, 3000, 2),
    ("f32", 64, 64, 2, 4100, 2),
    ("f32", 128, 32, 1, 3000, 2),
    ("f32", 128, 32, 2, 1500 + 17, 1),
]


@pytest.mark.parametrize("stored,D,C,B,T,H", SPLIT_CASES)
def test_split_matches_oracle_and_unsplit(stored, D, C, B, T, H):
    """Long sequences on few chains run as parallel segments chained through their state
    maps; outputs and final states match the oracle and the one-pass computation."""
    assert split_bytes(B, T, H, D, C, stored) > 0, "case does not exercise the split"
    x = random_inputs(300 + T + D, B * T, H, D, stored)
    s0 = random_states(301 + T, B, H, D)
    tol = TOL_BF16 if stored == "bf16" else TOL_F32
    note(f"split {stored} D={D} C={C} B={B} T={T} H={H}")
    o, S = gpu_chunk(x, stored, B=B, chunk=C, s0=s0, scale=D ** -0.5)
    cu = np.arange(B + 1) * T
    o_ref, S_ref = run_oracle(x, stored, scale=D ** -0.5, initial_state=s0, cu=cu)
    assert_close(o, o_ref, tol, "o (split)")
    assert_close(S, S_ref, tol, "final state (split)")
    o1, S1 = gpu_chunk(x, stored, B=B, chunk=C, s0=s0, scale=D ** -0.5, split=False)
    assert_close(o, o1, tol, "o split vs one pass")
    assert_close(S, S1, tol, "state split vs one pass")


# Few segments: the combine's first steps and its three-step register rotation end at every
# position (no segment map at all with two segments, one with three, two with four).
FEW_SEGMENT_CASES = [
    # (stored, D, C, T, H, segments, chunks per segment) on a 256-compute-unit device
    ("bf16", 128, 64, 768, 1, 3, 4),
    ("bf16", 128, 64, 837, 1, 4, 4),
    ("bf16", 128, 64, 1100, 100, 2, 9),
    ("f32", 128, 32, 384, 1, 3, 4),
    ("f32", 128, 32, 448, 1, 4, 4),
    ("f32", 128, 32, 560, 100, 2, 9),
]


def split_plan_bytes(T, H, D, C, stored, nseg, per):
    """Workspace bytes of a split into nseg segments of per chunks: maps R and X, start
    states, and per-chunk records (2 C Dk + Dk C + C Dv operands, the part of M that M U
    reads, and Dk decays). M U runs in steps of ks reduction indices (32 with fp16 operands,
    16 with float32, two or one 16-column tiles per step); 16-row band i reads its first
    ks * (i // tiles + 1) columns."""
    sz = 2 if stored == "bf16" else 4
    ks, tiles = (32, 2) if stored == "bf16" else (16, 1)
    m_elems = sum(16 * ks * (i // tiles + 1) for i in range(C // 16))
    rec = (2 * C * D + D * C + C * D + m_elems) * sz + D * 4
    rec = (rec + 255) // 256 * 256
    return (nseg - 1) * H * (D * D + D * D) * 4 + nseg * H * D * D * 4 + nseg * H * per * rec


@pytest.mark.parametrize("stored,D,C,T,H,nseg,per", FEW_SEGMENT_CASES)
def test_split_few_segments(stored, D, C, T, H, nseg, per):
    torch = torch_mod()
    got = split_bytes(1, T, H, D, C, stored)
    assert got > 0, "case does not exercise the split"
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert got == split_plan_bytes(T, H, D, C, stored, nseg, per), "not the intended plan"
    x = random_inputs(700 + T + H, T, H, D, stored)
    s0 = random_states(701 + T, 1, H, D)
    tol = TOL_BF16 if stored == "bf16" else TOL_F32
    note(f"split {stored} D={D} C={C} T={T} H={H} into {nseg} segments")
    o, S = gpu_chunk(x, stored, chunk=C, s0=s0, scale=D ** -0.5)
    o_ref, S_ref = run_oracle(x, stored, scale=D ** -0.5, initial_state=s0)
    assert_close(o, o_ref, tol, "o (split)")
    assert_close(S, S_ref, tol, "final state (split)")


def test_split_bf16_strong_decay_and_aliasing():
    """Split with near-total forgetting (tiny state maps) and final_state == initial_state."""
    B, T, H, D = 1, 4096 + 100, 2, 128
    x = random_inputs(320, T, H, D, "bf16")
    x["g"][: T // 3] = np.float32(-6.0)
    s0 = random_states(321, B, H, D)
    note("split bf16 strong decay + aliasing")
    o, S = gpu_chunk(x, "bf16", chunk=64, s0=s0, alias=True)
    o_ref, S_ref = run_oracle(x, "bf16", initial_state=s0)
    assert_close(o, o_ref, TOL_BF16, "o (split, strong decay)")
    assert_close(S, S_ref, TOL_BF16, "final state (split, strong decay, aliased)")


def test_split_without_initial_state():
    B, T, H, D = 1, 3 * 1024 + 64 * 16, 2, 128
    x = random_inputs(330, T, H, D, "bf16")
    note("split bf16 zero initial state")
    o, S = gpu_chunk(x, "bf16", chunk=64)
    o_ref, S_ref = run_oracle(x, "bf16")
    assert_close(o, o_ref, TOL_BF16, "o (split, no s0)")
    assert_close(S, S_ref, TOL_BF16, "final state (split, no s0)")


# --------------------------------------------------------------- the method's degenerate cases

DEGEN = [("bf16", 128, 64), ("f32", 32, 64), ("f32", 16, 16), ("f32", 128, 32)]


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("stored,D,C", DEGEN)
def test_no_decay_is_deltanet(stored, D, C, split):
    """g = 0 (alpha = 1): the plain delta rule, with an initial state; unsplit and split."""
    T, H = 2100, 2
    x = random_inputs(400 + D, T, H, D, stored, g_const=0.0)
    s0 = random_states(401, 1, H, D)
    note(f"no decay {stored} D={D} split={split}")
    o, S = gpu_chunk(x, stored, chunk=C, s0=s0, split=split)
    o_ref, S_ref = run_oracle(x, stored, initial_state=s0)
    tol = TOL_F32 if stored == "f32" else TOL_BF16
    assert_close(o, o_ref, tol, "o")
    assert_close(S, S_ref, tol, "final state")


@pytest.mark.parametrize("stored,D,C", DEGEN)
def test_zero_write_strength_is_pure_decay(stored, D, C):
    """beta = 0: nothing is written; the state only decays, row by row (key channels), and
    o_t reads the decayed initial state."""
    T, H = 500, 2
    x = random_inputs(410 + D, T, H, D, stored)
    x["beta"][:] = 0.0
    s0 = random_states(411, 1, H, D)
    note(f"pure decay {stored} D={D}")
    o, S = gpu_chunk(x, stored, chunk=C, s0=s0)
    o_ref, S_ref = run_oracle(x, stored, initial_state=s0)
    tol = TOL_F32 if stored == "f32" else TOL_BF16
    assert_close(o, o_ref, tol, "o")
    assert_close(S, S_ref, tol, "final state")
    decay = np.exp(np.sum(f64(x["g"]), axis=0))               # [H, D]: per key channel
    np.testing.assert_allclose(S_ref[0], s0[0] * decay[:, :, None], rtol=1e-10, atol=1e-300)


@pytest.mark.parametrize("stored,D,C", DEGEN)
def test_full_write_with_query_on_key_overwrites(stored, D, C):
    """beta = 1 and q = k: each token overwrites the state along its key, so o_t is v_t
    scaled by ||k_t||^2 plus what the decayed state held off that direction, which is
    exactly 0 for a unit key (the rounded keys are off unit norm by ~3e-3 in bf16)."""
    T, H = 300, 2
    x = random_inputs(420 + D, T, H, D, stored)
    x["beta"][:] = 1.0
    x["q"] = x["k"].copy()
    s0 = random_states(421, 1, H, D)
    note(f"overwrite {stored} D={D}")
    o, S = gpu_chunk(x, stored, chunk=C, s0=s0)
    o_ref, S_ref = run_oracle(x, stored, initial_state=s0)
    tol = TOL_F32 if stored == "f32" else TOL_BF16
    assert_close(o, o_ref, tol, "o")
    assert_close(S, S_ref, tol, "final state")
    if stored == "f32":  # unit keys to float32 rounding: o_t = v_t
        np.testing.assert_allclose(o_ref, f64(x["v"]), rtol=0, atol=1e-5 * np.sqrt(np.mean(o_ref ** 2)))


@pytest.mark.parametrize("split", [False, True])
def test_chunk_size_invariance(split):
    """The chunk size changes only the rounding: chunks of 16 and of 64 tokens on the same
    inputs (float32, D = 32, a ragged 333-token sequence with an initial state) each match
    the oracle within the float32 bound, and each other within twice it."""
    T, H, D = 333, 2, 32
    x = random_inputs(700, T, H, D, "f32")
    s0 = random_states(701, 1, H, D)
    note(f"chunk-size invariance split={split}")
    o16, S16 = gpu_chunk(x, "f32", chunk=16, s0=s0, split=split)
    o64, S64 = gpu_chunk(x, "f32", chunk=64, s0=s0, split=split)
    o_ref, S_ref = run_oracle(x, "f32", initial_state=s0)
    assert_close(o16, o_ref, TOL_F32, "o, chunk 16")
    assert_close(o64, o_ref, TOL_F32, "o, chunk 64")
    assert_close(S16, S_ref, TOL_F32, "final state, chunk 16")
    assert_close(S64, S_ref, TOL_F32, "final state, chunk 64")
    assert_close(o16, o64, 2 * TOL_F32, "o, chunk 16 against chunk 64")
    assert_close(S16, S64, 2 * TOL_F32, "final state, chunk 16 against chunk 64")
