"""The binding's host-side check of packed offsets (check_cu_seqlens), on the CPU."""

import numpy as np
import pytest
import torch

import gated_delta_rule_26_amd as kda


@pytest.mark.parametrize("cu, T", [([0], 0), ([0, 0], 0), ([0, 5], 5), ([0, 0, 3, 3, 10], 10)])
def test_valid_offsets_pass(cu, T):
    kda.check_cu_seqlens(np.array(cu, np.int32), T)
    kda.check_cu_seqlens(torch.tensor(cu, dtype=torch.int32), T)


@pytest.mark.parametrize("cu, T, what", [
    ([1, 5], 5, r"cu_seqlens\[0\] must be 0"),
    ([-5, 5], 5, r"cu_seqlens\[0\] must be 0"),
    ([0, 6, 4, 10], 10, r"nondecreasing: cu\[1\] = 6 > cu\[2\] = 4"),
    ([0, 4, 12], 10, r"must equal the token count 10"),
    ([0, 4, 8], 10, r"must equal the token count 10"),
])
def test_invalid_offsets_are_named(cu, T, what):
    with pytest.raises(ValueError, match=what):
        kda.check_cu_seqlens(np.array(cu, np.int32), T)
    with pytest.raises(ValueError, match=what):
        kda.check_cu_seqlens(torch.tensor(cu, dtype=torch.int32), T)


def test_wrong_dtype_and_rank():
    with pytest.raises(ValueError, match="int32"):
        kda.check_cu_seqlens(torch.tensor([0, 3], dtype=torch.int64), 3)
    with pytest.raises(ValueError, match="int32"):
        kda.check_cu_seqlens(np.array([0, 3], np.int64), 3)
    with pytest.raises(ValueError, match="one-dimensional"):
        kda.check_cu_seqlens(np.zeros((2, 2), np.int32), 0)
    with pytest.raises(ValueError, match="one-dimensional"):
        kda.check_cu_seqlens(np.zeros(0, np.int32), 0)
