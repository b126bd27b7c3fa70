"""Writes readme_example.json: the packed layout of the rnnt-loss-ascend README
usage example (section "Usage": two samples, T = [4, 6], target lengths
[2, 1], V = 8, blank = -1, i.e. 24 packed rows), with seeded logits and the
loss and gradient the oracle and the brute-force enumerator give for it.

Calls only ``oracle/``.  The README prints shapes only (its logits are
unseeded), so the values here are the oracle's, cross-checked against brute
force before they are written.
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle  # noqa: E402
from oracle import bruteforce  # noqa: E402


def main():
    rng = np.random.default_rng(2024)
    V = 8
    T = [4, 6]
    U = [2, 1]
    targets = [[2, 3], [1, 0]]          # the README's targets; padding 0 is never read
    N = sum(t * (u + 1) for t, u in zip(T, U))
    logits = np.round(rng.normal(0.0, 1.0, size=(N, V)), 6)   # 6 decimals: exact in the JSON text
    out = {"source": "rnnt-loss-ascend README, section 'Usage' (shape-level example)",
           "V": V, "logit_lengths": T, "target_lengths": U, "targets": targets, "blank": -1,
           "logits": logits.tolist(), "cases": []}
    for reduction in ("none", "mean", "sum"):
        loss, red, g, gr = oracle.batch(logits, np.array(targets, np.int32), T, U, blank=-1,
                                        reduction=reduction)
        off = 0
        for i in range(2):
            rows = T[i] * (U[i] + 1)
            bl, bg = bruteforce.sample(logits[off:off + rows], T[i], U[i], targets[i], V - 1, True)
            assert abs(bl - loss[i]) < 1e-12 and np.abs(bg - g[off:off + rows]).max() < 1e-12
            off += rows
        out["cases"].append({"reduction": reduction, "loss": np.atleast_1d(red).tolist(),
                             "loss_per_sample": loss.tolist(), "grad": gr.tolist()})
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "readme_example.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
