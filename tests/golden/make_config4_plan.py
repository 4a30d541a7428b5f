"""Writes config4_perturbation.txt: which key of each chosen (head, chunk) pair
the 131072-token workload scales by 8 so that its score leaves the safe band.

The (head, chunk) pairs -- 1% of the 32 x 128 pairs -- come from the seeded
generator; inside each pair the key with the largest float64 score is chosen,
scores taken from the oracle.  Scaling that key by 8 (exact in bf16) multiplies
its score by 8, pushing it far above phi + b (FlashDecoding++ theory page,
section 3: a score past the unified-max criterion sends its block to the
online-softmax recompute).

Run from the repository root:  python tests/golden/make_config4_plan.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synthetic  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "config4_perturbation.txt")


def plan():
    c = synthetic.CONFIGS[4]
    prob = synthetic.make_config(4, perturb=False)
    C = c["chunk_size"]
    nch = c["max_seq_len"] // C
    pairs = synthetic.perturbation_pairs(c["num_q_heads"], nch, c["perturb_fraction"],
                                         synthetic.SEED_BASE + 4)
    rows = []
    cache = {}
    for h, ch in pairs:
        if h not in cache:
            cache[h] = oracle.scores(**prob.args(), batch_index=0, head=int(h))
        s = cache[h][ch * C:(ch + 1) * C]
        rows.append((int(h), int(ch), int(ch * C + np.argmax(s))))
    return rows


if __name__ == "__main__":
    rows = plan()
    with open(OUT, "w") as f:
        f.write("# 131072-token MHA workload (batch 1, 32 heads, chunk 1024, seed 0x5EED0004):\n")
        f.write("# keys scaled by 8 -- one per listed (head, chunk) pair, the key with the\n")
        f.write("# largest float64 oracle score in that chunk.  Written by make_config4_plan.py.\n")
        f.write("# head chunk token\n")
        for r in rows:
            f.write("%d %d %d\n" % r)
    print("wrote", OUT, len(rows), "rows")
