"""Write tests/golden/inputs_sha256.json from the input generator and oracle/ only.

Usage: python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from ring_context_parallelism_amd.inputs import WORKLOADS, workload_qkv, sha256_of, to_numpy_f64  # noqa: E402

SMALL = ["causal_s256_cp2_zigzag_h2_d64_fp32", "causal_s8192_cp4_zigzag_h32_d128_bf16"]


def main():
    out = {"inputs": {}, "oracle": {}}
    for name in SMALL:
        w = WORKLOADS[name]
        q, k, v = workload_qkv(w)
        out["inputs"][name] = sha256_of(q, k, v)
    w = WORKLOADS[SMALL[0]]
    q, k, v = (to_numpy_f64(t) for t in workload_qkv(w))
    o, lse = oracle.attention(q, k, v, causal=True)
    out["oracle"][SMALL[0]] = {
        "sum_O": float(o.sum()),
        "sum_abs_O": float(np.abs(o).sum()),
        "sum_LSE": float(lse.sum()),
        "O_row255_h1_d0_3": [float(x) for x in o[255, 1, :4]],
        "LSE_h0_rows_0_1_128_255": [float(lse[0, i]) for i in (0, 1, 128, 255)],
    }
    with open(os.path.join(HERE, "inputs_sha256.json"), "w") as f:
        json.dump(out, f, indent=2)
        f.write("\n")


if __name__ == "__main__":
    main()
