"""Write tests/golden/tagged_gather.txt from the CPU oracle (oracle/ only).

Inputs are the peer-tagged payloads (byte i of payload r is (r*131 + i*7 + 1)
mod 251); each line holds "W<w>_S<s>" and the hex of the gathered output.
Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import oracle  # noqa: E402
from deterministic_collective_movement_amd.workloads import tagged_payload  # noqa: E402

CASES = [(1, 1), (2, 1), (2, 7), (3, 5), (3, 16), (4, 17), (8, 3), (5, 33)]

HEADER = """# Rank-ordered gather of peer-tagged payloads, written by make_golden.py from the
# CPU oracle (oracle/rog_oracle.c).  Definition: RL-Align/RL-Kernel PR #491,
# "perf(cuda): vectorize the deterministic all-gather copy and right-size its
# single-block path", section "What" (copy_rank_ordered places the bytes as the
# all-gather does): output = payload 0 | payload 1 | ...
# Input byte i of payload r is (r*131 + i*7 + 1) mod 251.
"""


def main():
    lines = [HEADER]
    for W, S in CASES:
        payloads = [tagged_payload(r, S) for r in range(W)]
        out = np.empty(W * S, np.uint8)
        oracle.gather_c(payloads, out)
        lines.append("W%d_S%d %s\n" % (W, S, out.tobytes().hex()))
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tagged_gather.txt"), "w") as f:
        f.writelines(lines)


if __name__ == "__main__":
    main()
