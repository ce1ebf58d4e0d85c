"""Writes ce_b8_v1000_f32.txt: the oracle's results on the [8, 1000] fp32 workload.

Calls only ``oracle/`` and the seeded generator ``workloads``; the stored
values are regression pins of the oracle itself (the pages print no worked
numeric example of cross-entropy). Run from the repository root:

    python tests/golden/make_golden.py
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    w = workloads.CE_B8_V1000_F32
    logits, target = workloads.ce_inputs(w)
    lines = ["# oracle cross-entropy of the seeded [8, 1000] fp32 workload (rows 3 and 6 ignored)",
             "# columns: z_loss_multiplier reduction n_valid loss(float.hex)"]
    for z in w.z_loss:
        for red in w.reductions:
            out = oracle.cross_entropy(logits, target, -100, red, z)
            lines.append(f"{z!r} {red} {out['n_valid']} {float(out['loss']).hex()}")
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "ce_b8_v1000_f32.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(open(path).read())


if __name__ == "__main__":
    main()
