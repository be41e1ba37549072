"""Write tests/golden/tiny_128_int4.txt from the oracle (and nothing else).

Run:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from workloads import WORKLOADS, generate  # noqa: E402


def main():
    w = WORKLOADS["tiny_128_int4"]
    x, s = generate(w, "cpu")
    out = O.forward(x.numpy().astype(np.float64), s, "int4", 0, "f32")
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_128_int4.txt")
    with open(path, "w") as f:
        f.write("# oracle output for workload tiny_128_int4 (64 x 128 fp32, seed 1, signs seed 0)\n")
        f.write("# written by tests/golden/make_golden.py; one line per row:\n")
        f.write("# <fp32 scale as hex bits> <64 packed bytes as hex>\n")
        for t in range(w.tokens):
            sb = np.float32(out["scales"][t, 0]).view(np.uint32)
            f.write(f"{int(sb):08x} {out['packed'][t].tobytes().hex()}\n")


if __name__ == "__main__":
    main()
