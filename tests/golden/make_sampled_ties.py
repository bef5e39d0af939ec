"""Writes sampled_ties.json: decoding steps at which two chosen vocabulary ids
of position (0, 0) draw the same Gumbel noise, so that equal logits there give
exactly equal sampling scores (a planted tie: the lower id must win).

The noise of id v is u = ((w >> 9) + 0.5) 2^-23 from word v % 4 of the
Philox4x32-10 block (v // 4, l, b, step) (oracle/philox.py), so two ids tie when
their words agree in the top 23 bits.  The search runs over the step counter
with the oracle's own generator; nothing here reads a GPU result.

    python tests/golden/make_sampled_ties.py
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "..", ".."))
from oracle.philox import philox4x32_10  # noqa: E402

SEED = 0x5EED_0001_0002

# (dtype, elements the rows start past a 16-byte boundary, V, [(v1, v2), ...]):
# bf16 rows 3 elements in have a 5-element head [0, 5), 16-byte spans from 5,
# and a 3-element tail [4093, 4096); f32 rows 1 element in have a 3-element
# head, spans from 3 and a 1-element tail [4095, 4096).
CASES = [
    ("bf16", 3, 4096, [(2, 2000), (102, 105), (3000, 4094), (1, 4095), (4093, 4095), (0, 4),
                       (60, 1500)]),
    ("f32", 1, 4096, [(2, 2000), (103, 105), (3000, 4095), (1, 4095), (0, 2), (60, 1500)]),
]


def word(step, v):
    """Word v % 4 of block (v // 4, l=0, b=0, step) for an array of steps."""
    key = (SEED & 0xFFFFFFFF, SEED >> 32)
    w = philox4x32_10((np.uint64(v // 4), 0, 0, step), key)
    return w[v % 4]


def find_step(v1, v2, chunk=1 << 22):
    for start in range(0, 1 << 32, chunk):
        steps = np.arange(start, start + chunk, dtype=np.uint64)
        hit = np.flatnonzero((word(steps, v1) >> np.uint64(9)) == (word(steps, v2) >> np.uint64(9)))
        if hit.size:
            return int(steps[hit[0]])
    raise RuntimeError("no tie found")


def main():
    out = {"seed": SEED, "cases": []}
    for dtype, off, V, pairs in CASES:
        for v1, v2 in pairs:
            s = find_step(v1, v2)
            out["cases"].append({"dtype": dtype, "off": off, "V": V, "v1": v1, "v2": v2,
                                 "step": s})
            print(dtype, v1, v2, s, flush=True)
    path = os.path.join(os.path.dirname(__file__), "sampled_ties.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
