"""Set the cumulative-mass threshold tau_p of the 480p pooled workload.

Bisection on the oracle's pooled mask (seed 1002 inputs) for ~85% tile
sparsity, the sparsity named for that workload. Writes pooled_tau.json next
to this file. Calls only the oracle and the input generator.

    python tests/golden/tune_pooled_threshold.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth   # noqa: E402

TARGET_SPARSITY = 0.85


def main():
    w = synth.workload("wan13b_480p")
    x = synth.make_qkv(w, want=("q", "k"))
    lo, hi = 0.0, 1.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        m, _, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, 1, mid)
        sp = 1.0 - m.mean()
        if sp > TARGET_SPARSITY:
            lo = mid
        else:
            hi = mid
    tau = round(hi, 6)
    m, _, margin = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, 1, tau)
    out = {"tau_p": tau, "tile_sparsity": float(1.0 - m.mean()), "seed": w.seed,
           "min_margin": float(margin.min()), "target_sparsity": TARGET_SPARSITY}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "pooled_tau.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(out)


if __name__ == "__main__":
    main()
