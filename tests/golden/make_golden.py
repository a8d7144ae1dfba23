"""Writes tests/golden/oracle_small.json: the float64 oracle's outputs on one small seeded
case (two packed sequences, one of them with a ragged tail, with initial states).

It calls only the oracle and the seeded input generator. The fixture freezes the oracle:
a later change to the oracle's arithmetic shows up as a mismatch and must be justified,
then the fixture regenerated with this script.
"""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402

CASE = dict(H=2, K=4, V=3, lengths=[5, 3])


def case_inputs():
    w = synth.Workload("golden_small", 900, H=CASE["H"], K=CASE["K"], V=CASE["V"], chunk=16,
                       dtype="f32", n_seqs=2, len_min=1, len_max=10)
    lens = CASE["lengths"]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    arrs = {key: [] for key in ("q", "k", "v", "g", "beta")}
    for n, L in enumerate(lens):
        # one slab per (sequence, head); stack heads on axis 1
        per_h = [synth.slab(w, n, h, L) for h in range(w.H)]
        for key in arrs:
            arrs[key].append(np.stack([s[key] for s in per_h], axis=1))
    out = {key: np.concatenate(v).astype(np.float64) for key, v in arrs.items()}
    s0 = np.stack([np.stack([synth.initial_state(w, n, h)
                             for h in range(w.H)]) for n in range(len(lens))])
    return out, cu, s0.astype(np.float64)


def main():
    x, cu, s0 = case_inputs()
    o, S = oracle.kda_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], scale=1.0,
                          initial_state=s0, cu_seqlens=cu)
    doc = {
        "what": "float64 oracle outputs on a small seeded packed case (written by make_golden.py)",
        "case": CASE,
        "cu_seqlens": cu.tolist(),
        "o": o.tolist(),
        "final_state": S.tolist(),
    }
    with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
