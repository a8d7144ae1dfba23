"""The measurement probes on the GPU: the copy reproduces its input bit for bit; the fp16
matrix-core loop runs and leaves finite accumulators."""

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


@pytest.mark.parametrize("shape", [0, 1])
def test_probe_mfma_runs(shape):
    torch = torch_mod()
    sink = torch.full((4 * 256,), float("nan"), device="cuda")
    note(f"probe mfma shape {shape}, 4 blocks")
    flops = kda.kda_probe_mfma_f16(10, 4, sink, shape=shape)
    torch.cuda.synchronize()
    assert flops == 10 * 4 * 4 * 8 * 2 * 16 * 16 * 32
    assert bool(torch.isfinite(sink).all())
