"""Write tests/golden/oracle_tiny.json: digests of the oracle's outputs on the
seeded tiny workload (T=16, H=512, I=256, E=8, top-2, clamp 7) in W4A16 and A4
mode.  Calls only the oracle and the seeded input generator; rerun it (and say
which passage or reading justifies the change) whenever the oracle's arithmetic
changes on purpose."""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from mxfp4_block_scaled_router_amd import workloads  # noqa: E402


def digest(a):
    return hashlib.sha256(a.tobytes()).hexdigest()


def run():
    wl = workloads.WORKLOADS["tiny"]
    inp = workloads.make_inputs(wl)
    rec = {"workload": "tiny", "seed": wl.seed}
    for a4 in (False, True):
        r = oracle.moe_forward(inp["x"], inp["logits"], inp["w13"], inp["w13s"], inp["w2"],
                               inp["w2s"], top_k=wl.top_k, clamp_limit=wl.clamp_limit, a4=a4)
        tag = "a4" if a4 else "w4a16"
        rec[tag] = {
            "inputs": {k: digest(v) for k, v in sorted(inp.items())},
            "ids": digest(r.ids), "w": digest(r.w), "sorted": digest(r.sorted),
            "inv": digest(r.inv), "counts": r.counts.tolist(), "act": digest(r.act),
            "out32": digest(r.out32), "out": digest(r.out),
            "out32_first8": [float(v) for v in r.out32[0, :8]],
        }
        if a4:
            rec[tag].update(xq=digest(r.xq), xs=digest(r.xs), actq=digest(r.actq),
                            acts=digest(r.acts))
    return rec


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json")
    with open(out, "w") as f:
        json.dump(run(), f, indent=1, sort_keys=True)
    print("wrote", out)
