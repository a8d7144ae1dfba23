"""The oracle reproduces its frozen small-case outputs (tests/golden/oracle_small.json)."""

import json
import os
import sys

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))


def test_oracle_matches_frozen_fixture():
    import make_golden

    with open(os.path.join(HERE, "golden", "oracle_small.json")) as f:
        doc = json.load(f)
    x, cu, s0 = make_golden.case_inputs()
    assert cu.tolist() == doc["cu_seqlens"]
    o, S = oracle.kda_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], initial_state=s0,
                          cu_seqlens=cu)
    np.testing.assert_allclose(o, np.array(doc["o"]), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(S, np.array(doc["final_state"]), rtol=1e-13, atol=1e-15)
