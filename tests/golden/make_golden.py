"""Write the stored expected values of the tiny fp32 prefill case.

Calls only the oracle and the seeded input generator.  The pages print no
worked example, so these values are the oracle's own, kept as a regression
pin: a change to the oracle's arithmetic that moves them must be justified
by a reading of the pages.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import sparse_attention as sa  # noqa: E402
from synth import workloads as W  # noqa: E402


def c1_values():
    cfg = W.C1
    q, k, v, _ = W.prefill_inputs_host(cfg)
    r = sa.prefill_pipeline(q, k, v, theta=cfg.theta, block=cfg.block,
                            split_pair=cfg.band_split_pair, calibrate=True,
                            sm_scale=cfg.d ** -0.5, causal=True,
                            budget=sa.keep_budget(cfg.N, keep_const=cfg.keep_const),
                            n_sink=cfg.n_sink, n_local=cfg.n_local)
    sc = r["scores"][0, 0]
    return {
        "case": cfg.name,
        "block_scores_lower": [[float(sc[i, j]) for j in range(i + 1)] for i in range(cfg.N)],
        "selected_blocks": [s.tolist() for s in r["sel"][0][0]],
        "out_rows": {str(t): [float(x) for x in r["out"][0, 0, t]] for t in (0, 63, 64, 300, 511)},
        "lse_rows": {str(t): float(r["lse"][0, 0, t]) for t in (0, 63, 64, 300, 511)},
    }


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c1_oracle.json")
    with open(path, "w") as f:
        json.dump(c1_values(), f, indent=1)
    print("wrote", path)
