"""Write the oracle's results on the 512-token fp32 workload to tiny_f32_512.json.

Calls only the fp64 oracle (and the seeded input generator, which holds no method
arithmetic). The fixture is a regression record for the oracle: a later change to
its arithmetic shows up as a diff here, and the commit that regenerates it must name
the passage or reading that justifies the change.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from long_context_approximate_amd.inputs import CONFIGS, make_inputs  # noqa: E402

ROWS = [0, 1, 31, 32, 100, 255, 256, 257, 300, 511]


def main():
    cfg = CONFIGS["tiny_f32_512"]
    sh = oracle.shape_of(cfg)
    x = make_inputs(cfg)
    res = oracle.run(sh, x["q"], x["k"], x["v"])
    rec = {
        "workload": cfg.name,
        "source": "oracle/spava_oracle.py via tests/golden/make_golden.py",
        "idx": res["idx"].tolist(),
        "min_margin": float(np.nanmin(res["margins"])),
        "score_sums": res["scores"].sum(axis=2).tolist(),
        "rows": ROWS,
        "lse": [[repr(float(res["lse"][h, i])) for i in ROWS] for h in range(cfg.num_q_heads)],
        "o_row_sums": [[repr(float(res["o"][i, h].sum())) for i in ROWS]
                       for h in range(cfg.num_q_heads)],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_f32_512.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
