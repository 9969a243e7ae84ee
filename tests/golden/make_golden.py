"""Write tests/golden/e4_trajectory_64.json from the oracle alone.

Three packed-E4 steps on 64 parameters drawn with the single-tensor workload's
generators (workloads.host_params(1, limit=64), host_grads(1, t, limit=64)),
hyperparameters lr 1e-3, betas (0.9, 0.999), eps 1e-8, weight decay 0.01.
The file freezes the oracle's output so that a later change to its
arithmetic shows up as a diff that has to be justified.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "e4_trajectory_64.json")


def main():
    h = workloads.HYPER
    p = workloads.host_params(1, limit=64)[0]
    w = np.zeros(64, np.uint32)
    steps = []
    for t in range(1, 4):
        g = workloads.host_grads(1, t, limit=64)[0]
        s = oracle.scalars(h["lr"], h["beta1"], h["beta2"], h["eps"], h["weight_decay"], t)
        oracle.step_packed(oracle.PACKED_E4, p, g, w, s)
        steps.append({"step": t,
                      "params_hex": [f"{x:08x}" for x in p.view(np.uint32)],
                      "words_hex": [f"{x:08x}" for x in w]})
    with open(OUT, "w") as f:
        json.dump({"recipe": __doc__.strip().splitlines()[2:6], "hyper": h, "steps": steps}, f, indent=1)
    print(OUT)


if __name__ == "__main__":
    main()
