"""The whole-tensor parity statistic of the GPU tests (kda_testutil.WholeTensor), on the CPU:
accumulating over slabs gives the statistic of the whole tensor, the bf16 allowance is half an
ulp per element, and a row-normalised output widens the bound only on rows whose pre-norm RMS
is below the tensor's, by exactly that ratio."""

import numpy as np
import pytest

from kda_testutil import WholeTensor


def test_slabs_give_the_whole_tensor_statistic():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((40, 8))
    got = ref + 1e-3 * rng.standard_normal(ref.shape)
    a, b = WholeTensor("a", 1.0), WholeTensor("b", 1.0)
    a.add(got, ref)
    for i in range(0, 40, 7):
        b.add(got[i:i + 7], ref[i:i + 7])
    assert a.check(320) == pytest.approx(b.check(320), rel=1e-12)
    e = np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2))
    assert a.check() == pytest.approx(e, rel=1e-12)


def test_tolerance_and_nonfinite():
    ref = np.ones((4, 4))
    t = WholeTensor("t", 1e-2)
    t.add(ref + 0.02, ref)
    with pytest.raises(AssertionError):
        t.check()
    t = WholeTensor("t", 1e-2)
    with pytest.raises(AssertionError):
        t.add(np.full((4, 4), np.nan), ref)


def test_row_conditioning_scales_only_small_rows():
    # row 0 has pre-norm RMS 1e-3 of the others: its bound is 1000x wider, the others unchanged
    V = 16
    pre = np.ones((4, V))
    pre[0] *= 1e-3
    ref = np.ones((4, V))                    # normalised rows
    rms_pre = np.sqrt(np.mean(pre ** 2))
    kappa0 = rms_pre / 1e-3
    tol = 2e-2
    ok = WholeTensor("ok", tol, bf16_out=True)
    got = ref.copy()
    got[0] += 0.9 * tol * kappa0 * (1 + 2.0 ** -8)        # within the widened bound
    got[1] += 0.9 * tol * (1 + 2.0 ** -8) + 2.0 ** -8      # within the plain bound
    ok.add(got, ref, pre=pre)
    ok.check()
    bad = WholeTensor("bad", tol, bf16_out=True)
    got = ref.copy()
    got[1] += 1.1 * tol * (1 + 2.0 ** -8) + 2.0 ** -8      # a well-conditioned row over its bound
    bad.add(got, ref, pre=pre)
    with pytest.raises(AssertionError):
        bad.check()
    bad = WholeTensor("bad", tol, bf16_out=True)
    got = ref.copy()
    got[0] += 1.1 * tol * kappa0 * (1 + 2.0 ** -8) + 2.0 ** -8
    bad.add(got, ref, pre=pre)
    with pytest.raises(AssertionError):
        bad.check()
