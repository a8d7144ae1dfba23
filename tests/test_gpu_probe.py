"""The measurement probes on the GPU: the copy reproduces its input bit for bit, the in-place
read-modify-write scales exactly its buffer and nothing past it; the fp16
matrix-core loop gives the sums its fixed operands imply (every product of every iteration
was done)."""

import numpy as np
import pytest

import gated_delta_rule_26_amd as kda
from kda_testutil import note, torch_mod

pytestmark = pytest.mark.gpu


def test_probe_copy_is_exact():
    torch = torch_mod()
    src = torch.randn(1 << 22, device="cuda")
    dst = torch.zeros_like(src)
    note("probe copy 16 MiB")
    kda.kda_probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("n", [1 << 22, (1 << 22) + 12])
def test_probe_rmw_is_exact_and_bounded(n):
    """buf *= 2 in place, a power of two (exact); a ragged tail past the last full 16 KB slab
    is scaled too, and nothing past the buffer's end is touched."""
    torch = torch_mod()
    big = torch.randn(n + 1024, device="cuda")
    ref = big.clone()
    note(f"probe rmw {n} floats")
    kda.kda_probe_rmw(big[:n], 2.0)
    kda.kda_probe_read(big[:n])
    torch.cuda.synchronize()
    assert torch.equal(big[:n], 2 * ref[:n])
    assert torch.equal(big[n:], ref[n:])


def probe_expected(shape, iters, blocks, bf16=False):
    """What every thread of the probe writes: the sum of its accumulator elements after
    `iters` products. Each lane's A fragment holds 8 fp16 values 1e-3 * (thread + e) and its
    B fragment 1e-3 * (block + e), e = 0..7, so B does not depend on the column and every
    column of D = A B is the same vector d[row] = sum over the k slices of A[row, k] b[k].
    16x16x32: lane 16 s + i holds row i, k = 8 s + e of A; the lane's 4 accumulator elements
    are rows 4 s .. 4 s + 3; 8 accumulators. 32x32x16: lane 32 s + i holds row i, k = 8 s + e;
    its 16 elements are rows 8 u + 4 s + r (u, r = 0..3); 4 accumulators."""
    if bf16:  # round to nearest even to 8 significant bits
        def f16(x):
            u = (np.float32(1e-3) * np.asarray(x, np.float32)).view(np.uint32).astype(np.uint64)
            u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
            return u.astype(np.uint32).view(np.float32).astype(np.float64)
    else:
        f16 = lambda x: (np.float32(1e-3) * np.asarray(x, np.float32)).astype(np.float16).astype(np.float64)  # noqa: E731
    e = np.arange(8)
    out = np.zeros((blocks, 256))
    rows, nk, nacc = (16, 4, 8) if shape == 0 else (32, 2, 4)
    for blk in range(blocks):
        bb = f16(blk + e)
        for w in range(4):
            d = np.zeros(rows)
            for i in range(rows):
                d[i] = sum(float(f16(64 * w + rows * s + i + e) @ bb) for s in range(nk))
            for lane in range(64):
                s_ = lane // rows
                own = ([4 * s_ + r for r in range(4)] if shape == 0 else
                       [8 * u + 4 * s_ + r for u in range(4) for r in range(4)])
                out[blk, 64 * w + lane] = nacc * iters * d[own].sum()
    return out.reshape(-1)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("shape", [0, 1])
def test_probe_mfma_result(shape, bf16):
    torch = torch_mod()
    iters, blocks = 10, 4
    sink = torch.full((blocks * 256,), float("nan"), device="cuda")
    note(f"probe mfma shape {shape} {'bf16' if bf16 else 'fp16'}, {blocks} blocks")
    probe = kda.kda_probe_mfma_bf16 if bf16 else kda.kda_probe_mfma_f16
    flops = probe(iters, blocks, sink, shape=shape)
    torch.cuda.synchronize()
    assert flops == iters * blocks * 4 * 8 * 2 * 16 * 16 * 32
    got = sink.cpu().numpy().astype(np.float64)
    ref = probe_expected(shape, iters, blocks, bf16)
    np.testing.assert_allclose(got, ref, rtol=1e-4)
