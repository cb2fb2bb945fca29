"""Writes the golden fixtures in this folder.  Calls only the oracle and the
seeded input generator; run from the repository root:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def plan_tiny_decode():
    b = workloads.tiny_decode_f32()
    params = dict(num_qo_heads=8, num_kv_heads=2, tile_q=16, tile_kv=16, num_workers=8, split_factor=2,
                  min_chunk=32, max_chunk=0, item_overhead=0, max_items_per_worker=16, max_slots=64,
                  max_merge=64, causal=True, window=0, sink=0)
    plan = oracle.plan_ref(b.qo_len, b.kv_len, oracle.PlanParams(**params))
    return {
        "what": "plan of the tiny fp32 paged GQA decode (kv 17/64/130/255, 8 q / 2 kv heads) on 8 workers; "
                "C = 2*(17+64+130+255) = 932, L_c = roundup(ceil(932*17/(16*16)), 16) = roundup(62, 16) = 64 "
                "(decode tiles: an even share plus a sixteenth), so request 2 splits "
                "into [0,64) [64,128) [128,130) and request 3 into four 64-token chunks",
        "source": "plan defined in oracle/plan.py (the pages give no algorithm; FlashInfer paper summary, "
                  "research methodology 3: dynamic load-balanced scheduling)",
        "params": params,
        "qo_len": [int(x) for x in b.qo_len],
        "kv_len": [int(x) for x in b.kv_len],
        "chunk": int(plan["chunk"]),
        "items": plan["items"].tolist(),
        "worker_items": plan["worker_items"],
        "merge": plan["merge"][:, :6].tolist(),  # the two prefix fields are zero without a shared prefix
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "plan_tiny_decode.json"), "w") as f:
        json.dump(plan_tiny_decode(), f, indent=1)
    print("wrote plan_tiny_decode.json")
