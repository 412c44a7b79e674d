"""Writes input_sha256.txt: the SHA-256 of every seeded input array of every
workload (dtype, shape and bytes; workloads), so a change
in the input generator shows up as a failing CPU test.  Uses only the input
generator, no part of the method.

    python tests/golden/make_input_sha256.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workloads as W  # noqa: E402


def main():
    lines = ["# workload input dtype shape sha256 (workloads.sha256_hex)"]
    for name in W.WORKLOADS:
        for inp, a in W.input_arrays(name):
            lines.append(f"{name} {inp} {a.dtype.str} {'x'.join(map(str, a.shape))} {W.sha256_hex(a)}")
    with open(os.path.join(HERE, "input_sha256.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
