"""Writes ring_schedules.txt: for each workload and computed rank, the ring step
order and block classes.  Calls only oracle/ (ring order from the glossary page
"sequence parallelism transformers", section "Ring Attention", item "Ring
Communication"; classes from the causal visibility rule).

Run from the repository root:  python tests/golden/make_ring_schedules.py
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from sequence_transformer_attention_amd import workloads  # noqa: E402

NAMES = {0: "SKIP", 1: "FULL", 2: "PARTIAL"}


def lines():
    out = ["# workload rank step block kv_off class   (q_off = rank * N/P, block length N/P)"]
    for w in workloads.ALL:
        nb = w.N // w.P
        ranks = sorted(set(w.ranks) | {0, w.P - 1, w.P // 2})
        for r in ranks:
            for s in range(w.P):
                j = oracle.ring_block(w.P, r, s)
                c = oracle.classify(r * nb, nb, j * nb, nb, w.causal)
                out.append(f"{w.name} {r} {s} {j} {j * nb} {NAMES[c]}")
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "ring_schedules.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines()) + "\n")
    print(path)
