#!/usr/bin/env python3
"""Writes input_sha256.txt: the SHA-256 of the fp16 bytes of Q, K and V of
every workload, as the seeded generator produces them.  Calls only the input
generator (no attention arithmetic); run from the repository root."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from scaled_dot_product_attn_amd import inputs  # noqa: E402


def main():
    lines = ["# SHA-256 of the fp16 input tensors (little-endian bytes, C order) of each",
             "# workload: name tensor shape sha256.  Written by make_input_sha256.py."]
    for table in (inputs.WORKLOADS, inputs.DECODE_WORKLOADS):
        for c, w in sorted(table.items()):
            for name, x in zip("QKV", w.qkv()):
                lines.append(f"{w.name} {name} {'x'.join(map(str, x.shape))} {inputs.sha256(x)}")
    with open(os.path.join(HERE, "input_sha256.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
