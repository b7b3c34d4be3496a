"""Write tests/golden/tiny_greedy.json from the CPU oracle alone.

Run from the repository root: ``python tests/golden/make_golden.py``.  The file
records the oracle's 4-step greedy decode of the tiny MoE workload (2 layers,
d=256, 8 experts top-2, 64-token pre-filled cache, seed 0): the fed tokens,
the routed expert ids per layer, and a few logits per step.  The test that
reads it checks that the oracle still reproduces its own seeded decode.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import decode as O  # noqa: E402
from persistent_moe_amd import workloads as W  # noqa: E402


def main():
    wl = W.WORKLOADS["tiny"]
    fed, res = O.greedy_decode(wl, 4)
    out = {
        "workload": wl.name,
        "steps": [
            {
                "fed_token": f[0],
                "argmax": r[0].token,
                "experts": [t.route.ids.tolist() for t in r[0].layers],
                "logits_head": [float(v) for v in r[0].logits[:8]],
                "logits_std": float(r[0].logits.std()),
            }
            for f, r in zip(fed, res)
        ],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_greedy.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
