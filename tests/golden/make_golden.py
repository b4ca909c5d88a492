"""Writes the oracle regression fixture next to this script.

It calls only ``oracle`` (and the seeded ``workloads`` generator), so every stored
value comes from the CPU oracle.  The MoBA pages print no worked numeric example, so
there is no fixture of the pages' own numbers; this file only guards the oracle
against unintended change.  Run from the repository root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from workloads import small_workload, make_inputs, bf16_to_f64  # noqa: E402

CASES = [
    dict(name="small_gqa_ragged", batch=1, hq=2, hkv=1, head_dim=8, seqlen=44, block=8,
         topk=3, recipe="offset", seed=21),
    dict(name="small_b2", batch=2, hq=2, hkv=2, head_dim=4, seqlen=24, block=4,
         topk=2, recipe="iid", seed=22),
]


def main():
    out = []
    for c in CASES:
        w = small_workload(c["name"], c["batch"], c["hq"], c["hkv"], c["head_dim"],
                           c["seqlen"], c["block"], c["topk"], c["recipe"], c["seed"])
        inp = make_inputs(w)
        Q, K, V = (bf16_to_f64(inp[x]) for x in "qkv")
        o, lse, idx, _ = oracle.moba_forward(Q, K, V, w.block, w.topk, w.sm_scale)
        out.append(dict(case=c, scale=w.sm_scale, idx=idx.tolist(),
                        out=[float.hex(float(x)) for x in o.ravel()],
                        lse=[float.hex(float(x)) for x in lse.ravel()]))
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(out, f, indent=0)


if __name__ == "__main__":
    main()
