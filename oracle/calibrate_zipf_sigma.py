"""Calibrate the draft-noise sigma of the Zipf workload (test infrastructure only).

The workload asks for a draft whose mean acceptance rate alpha is about 0.7,
where alpha at one position is sum_x min(p(x), q(x)) (the probability that a
token drawn from q passes the accept test of Step 3 in the Speculative Sampling
explainer).  This script bisects sigma on a calibration draw of the workload's
own generator (8 sequences x 4 positions at V = 128256, bf16) using the
oracle's softmax, and prints the sigma that the generator then uses as
ZIPF_DRAFT_SIGMA.

    python -m oracle.calibrate_zipf_sigma
"""

import numpy as np

from oracle.chain import softmax_fp64, widen
from rejection_sampling_verify_chain_amd import inputs


def mean_alpha(sigma, seed=12345, B=8):
    b = inputs.chain_zipf(seed, B, 4, 128256, "bf16", sigma)
    vals = []
    for s in range(B):
        T = float(b.temperature[s])
        for i in range(b.gamma):
            p = softmax_fp64(widen(b.target[s, i], "bf16"), T)
            q = softmax_fp64(widen(b.draft[s, i], "bf16"), T)
            vals.append(np.minimum(p, q).sum())
    return float(np.mean(vals))


def main(target=0.7):
    lo, hi = 0.3, 1.5
    for _ in range(12):
        mid = 0.5 * (lo + hi)
        a = mean_alpha(mid)
        print(f"sigma={mid:.4f} alpha={a:.4f}")
        if a > target:
            lo = mid
        else:
            hi = mid
    print(f"calibrated sigma ~ {0.5 * (lo + hi):.3f}")


if __name__ == "__main__":
    main()
