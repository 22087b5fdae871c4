"""Writes the oracle's frozen known-answer vectors (calls only `oracle`).

Run from the repository root:  python tests/golden/make_golden.py
The files guard the oracle's counter-based r16 and stochastic rounding against
accidental change; the published SplitMix64 sequence pins the generator itself.
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import rounding  # noqa: E402


def main():
    cases = [(0, 1, 0), (0, 1, 1), (0x5EED0001, 1, 12345), (0x5EED0001, 10, 16777215),
             (0xFFFFFFFFFFFFFFFF, 3, 4294967295), (42, 20, 58720255), (7, 1 << 20, 89128959)]
    lines = ["# seed step idx r16   (r16 = top 16 bits of SplitMix64 output number (step<<32|idx)+1)"]
    for seed, step, idx in cases:
        r = int(rounding.rand16(seed, step, np.array([idx], dtype=np.uint64))[0])
        lines.append(f"{seed} {step} {idx} {r}")
    with open(os.path.join(HERE, "rand16_kat.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    xs = np.array([1.0, 1.00390625, 1.0039062, -3.14159, 0.0, -0.0, 6.5e-39, 3.3895314e38, -1e-20],
                  dtype=np.float32)
    rs = [0, 1, 0x7FFF, 0x8000, 0xFFFF]
    lines = ["# x32_bits r16 bf16_bits   (stochastic rounding: (bits(x)+r16)>>16)"]
    for x in xs:
        for r in rs:
            b = int(rounding.sr_bf16(np.array([x]), np.array([r]))[0])
            lines.append(f"{int(np.array([x]).view(np.uint32)[0]):#010x} {r:#06x} {b:#06x}")
    with open(os.path.join(HERE, "sr_bf16_kat.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
