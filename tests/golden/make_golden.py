"""Writes the stored expected values under tests/golden/ from the oracle only.

Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle.planner import plan_rand_attn  # noqa: E402


def main():
    ra = plan_rand_attn(3, 16, 3, 1)
    with open(os.path.join(HERE, "plan_H3_nb16_r3_seed1.txt"), "w") as f:
        f.write("# rand_attn [H=3][nb-2=14][r=3], SplitMix64 seed 1, written by make_golden.py\n")
        for h in range(3):
            for row in ra[h]:
                f.write(" ".join(str(int(x)) for x in row) + "\n")


if __name__ == "__main__":
    main()
