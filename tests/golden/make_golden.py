"""Writes tests/golden/tiny_probe_row.txt from the CPU oracle alone.

The file pins the oracle's output for the probe row of the tiny fp32
workload (X[M,256], W[32,256], b[32], all N(0,1)/16, seed 0), so that a later
change to the oracle's arithmetic shows up as a diff of this file.
Run:  python tests/golden/make_golden.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads as wl  # noqa: E402


def main():
    w = wl.tiny_weights(0)
    y = oracle.linear_f32(w.probes, w.w, w.b)[0]
    lines = ["# oracle.linear_f32 of the tiny workload's probe row (seed 0): index, fp32 bits, value",
             f"# input sha: probe={hash_arr(w.probes)} w={hash_arr(w.w)} b={hash_arr(w.b)}"]
    for n, v in enumerate(y):
        lines.append(f"{n} 0x{np.float32(v).view(np.uint32):08x} {float(v)!r}")
    with open(os.path.join(HERE, "tiny_probe_row.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


def hash_arr(a):
    import hashlib
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


if __name__ == "__main__":
    main()
