"""Write the decimal brute-force fixture used by the oracle pin tests.

Calls only the oracle package (its 40-digit brute force) on a seeded input
from tests/workloads.py.  Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path[:0] = [ROOT, os.path.join(ROOT, "tests")]

import workloads  # noqa: E402
from oracle.brute import brute_fwd  # noqa: E402

SPEC = dict(name="golden_k128_T5", seed=21, B=1, T=5, H=2, K=128, V=128, head=1)


def main():
    s = SPEC
    x = workloads.random_inputs(s["name"], s["seed"], s["B"], s["T"], s["H"], s["K"], s["V"],
                                init_std=None)
    out, fin = brute_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias,
                         x.lower_bound, None, head=s["head"])
    rows = [0, 1, 63, 127]
    doc = {
        "what": "KDA forward, 40-digit decimal brute force of the unrolled product form "
                "(oracle/brute.py); zero initial state; inputs from tests/workloads.py "
                "random_inputs with the spec below",
        "spec": s,
        "out": [[str(v) for v in row] for row in out],
        "final_rows": rows,
        "final": [[str(v) for v in fin[r]] for r in rows],
    }
    with open(os.path.join(HERE, "brute_k128_T5.json"), "w") as f:
        json.dump(doc, f, indent=0)


if __name__ == "__main__":
    main()
