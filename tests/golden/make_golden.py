"""Write tests/golden/oracle_small.json: float64 oracle results on small seeded
cases, used as a regression fixture for the oracle (a later change to the
oracle's arithmetic must reproduce these or justify the change).

Calls only the oracle and the seeded input generator.  Run from the repository
root:  python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import WORKLOADS, generate, reduced  # noqa: E402

SAMPLE_ROWS = [0, 1, 17, 100, 255]


def summarize(o):
    o = np.asarray(o, dtype=np.float64)
    return {
        "shape": list(o.shape),
        "sum": float(o.sum()),
        "sum_abs": float(np.abs(o).sum()),
        "sum_sq": float((o * o).sum()),
    }


def main():
    cases = {}
    # the fp32 parity workload at full size (1 head, 256 tokens)
    w = WORKLOADS["noncausal_f32_b1h1n256"]
    x = generate(w).f64
    o = oracle.linattn(x["q"], x["k"], x["v"], w.eps)
    cases[w.name] = dict(summarize(o), rows={str(r): o[0, 0, r].tolist() for r in SAMPLE_ROWS})
    # small bf16 RoPE case on a 2x3x5 grid
    wr = reduced(WORKLOADS["video720p_rope3d"], H=2, N=30, grid=(2, 3, 5))
    x = generate(wr).f64
    ang = oracle.rope3d_angles(*wr.grid)
    o = oracle.linattn(x["q"], x["k"], x["v"], wr.eps, angles=ang)
    cases["rope3d_2x3x5_h2"] = dict(summarize(o), rows={str(r): o[0, 1, r].tolist() for r in (0, 7, 29)})
    # small bf16 block-causal case: 3 chunks of 20 tokens
    wb = reduced(WORKLOADS["video480p_blockcausal"], H=2, N=60, chunk=20)
    x = generate(wb).f64
    o, S, z = oracle.block_causal(x["q"], x["k"], x["v"], wb.chunk, wb.eps)
    cases["blockcausal_3x20_h2"] = dict(summarize(o), S=summarize(S), z=z[0, 0].tolist(),
                                        rows={str(r): o[0, 0, r].tolist() for r in (0, 19, 20, 59)})
    out = {
        "_about": "float64 oracle outputs on small seeded inputs (numpy PCG64 seed 0, draws Q, K, V). "
                  "Written by tests/golden/make_golden.py, which calls only the oracle and the input generator.",
        "numpy_version": np.__version__,
        "cases": cases,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
