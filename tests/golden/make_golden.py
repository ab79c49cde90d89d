"""Writes tests/golden/tiny_fp32_oracle.txt from the fp64 oracle alone.

The pages print no worked example, so this fixture is not a page value: it is the oracle's
own output on the tiny fp32 workload (1 request, H=8, P=64, T=4 chain, seed 0), kept as a
regression anchor. Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_fp32_oracle.txt")


def main():
    w = workloads.tiny(0)
    out, lse, am = oracle.run_workload(w)
    with open(OUT, "w") as f:
        f.write("# tiny fp32 workload, seed 0: 1 request, H=8, P=64, T=4 chain, scale 1/sqrt(192)\n")
        f.write("# written by tests/golden/make_golden.py from the fp64 oracle (regression anchor)\n")
        f.write("# row token head argmax lse out_sum out[0] out[1] out[511]\n")
        for n in range(out.shape[0]):
            f.write(f"{n} {n // 8} {n % 8} {am[n]} {lse[n]:.17g} {out[n].sum():.17g} "
                    f"{out[n, 0]:.17g} {out[n, 1]:.17g} {out[n, 511]:.17g}\n")


if __name__ == "__main__":
    main()
