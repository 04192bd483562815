"""Regenerate nf4_ties.txt: scan fp32 values within 8192 ulps of each midpoint
between consecutive NF4 levels (the oracle's table) and list the exact ties of
the fp32 distance rule.  Calls only oracle/ and numpy."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "..", ".."))
import oracle  # noqa: E402


def ties():
    L = oracle.nf4_levels()
    out = []
    offs = np.arange(-8192, 8193, dtype=np.int64)
    for j in range(15):
        mid = np.float32((np.float64(L[j]) + np.float64(L[j + 1])) / 2)
        base = np.int64(mid.view(np.int32))
        ints = base + offs if mid >= 0 else base - offs
        v = ints.astype(np.int32).view(np.float32)
        for x in v[np.abs(v - L[j]) == np.abs(v - L[j + 1])]:
            out.append((j, int(np.float32(x).view(np.uint32)), float(x)))
    return out


if __name__ == "__main__":
    for j, h, x in ties():
        print(f"{j} {h:08x} {np.float32(x)}")
