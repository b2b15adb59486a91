"""Writes search_full_4096.json: the oracle's MSE-searched per-tensor scale
of the fp32 4096 x 4096 N(0,1) workload tensor (seed 1) at block 16, for
abs-max, 4-over-6 and brute force (32 exhaustive searches of the tensor:
about half an hour).  Calls only oracle/ and the seeded input generator;
the search over the full tensor takes the oracle minutes, too long to redo
inside a GPU test.  Run: python tests/golden/make_search_golden.py"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from microscaling_fp4_block_fp4q_amd import synth as S  # noqa: E402
from oracle import oracle as O  # noqa: E402


def main():
    x = S.config2()["normal"]
    out = {"what": "oracle search_global_scale on synth.config2()['normal'] (fp32 4096x4096 N(0,1), seed 1), "
                   "E4M3 block 16; g as fp32 bits, j = argmin candidate, totals = fp64 tree sums",
           "cases": {}}
    for name, st in (("absmax", O.ABSMAX), ("4-over-6", O.FOUR_OVER_SIX), ("brute-force", O.BRUTE_FORCE)):
        g, totals = O.global_scale_search(x, block=16, strategy=st)
        out["cases"][name] = {"g_bits": int(np.float32(g).view(np.uint32)), "g": float(g),
                              "j": int(np.argmin(totals)), "totals": [float(t) for t in totals]}
        print(name, g, int(np.argmin(totals)), flush=True)
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "search_full_4096.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
