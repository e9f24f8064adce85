"""Writes llama7b_up_search_losses.json: the exact search losses of the full
Llama-7B-shaped MLP up-projection workload (K = 4096 -> N = 11008, fp16,
65536 calibration tokens, 20 candidate exponents alpha_i = i / 19), computed by
the CPU oracle alone in float64 from the seeded inputs.

"AWQ Math", section "Searching the scale -- no backprop required": the loss of
a candidate is the mean squared error between W x and
Q(W diag(s)) diag(s)^-1 x over the calibration tokens, s_j = (s_X,j)^alpha.

Run from the repository root:  python tests/golden/make_llama7b_up_search_losses.py
(about 1.2e14 floating-point operations: several minutes on 8 cores).
"""
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle as O  # noqa: E402
import workloads as WL  # noqa: E402


def main():
    w = WL.workload(2)
    W = WL.weight(w).float().numpy()
    X = WL.calibration(w).float().numpy()
    alphas = WL.alpha_grid(20)
    t0 = time.time()
    m = O.act_mean_abs(X)
    S = O.candidate_scales(m, alphas)
    L = O.search_losses(W, X, S)
    best = O.choose_candidate(L)
    order = np.argsort(L)
    gap = float((L[order[1]] - L[order[0]]) / L[order[0]])
    out = {
        "workload": w.name,
        "N": w.N, "K": w.K, "T": w.T, "group": 128, "bits": 4,
        "source": "oracle.search_losses (float64) on workloads.weight / workloads.calibration of "
                  "the Llama-7B MLP up-projection; \"AWQ Math\", Searching the scale",
        "alphas": [float(a) for a in alphas],
        "losses": [float(v) for v in L],
        "argmin": best,
        "relative_gap_best_to_runner_up": gap,
        "mean_abs_sha": __import__("hashlib").sha256(m.tobytes()).hexdigest(),
    }
    path = os.path.join(ROOT, "tests", "golden", "llama7b_up_search_losses.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {path}: argmin {best}, gap {gap:.3e}, {time.time() - t0:.0f} s")


if __name__ == "__main__":
    main()
