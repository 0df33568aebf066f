"""Writes search_llama2_7b_block.json: the oracle's scale search (the C++ oracle,
oracle/awq_oracle.cpp) on the seven linears of a Llama-2-7B-shaped block with 65,536
seeded calibration rows per input.

Calls only the seeded generator (gen) and the oracle.  Run from the repository root:
    python tests/golden/make_search_llama2_7b_block.py
The GPU test test_search_llama2_7b_block_full regenerates the same inputs and
compares the device's alpha index, losses and packed output with this file.
"""
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from gen import activations_fp16, normal_fp16, seed_for  # noqa: E402
from gen.workloads import layer_inputs_7b_block  # noqa: E402

M = 65536
INPUT_K = {"attn_in": 4096, "o_in": 4096, "mlp_in": 4096, "down_in": 11008}
LAYER_KN = {"q_proj": (4096, 4096), "k_proj": (4096, 4096), "v_proj": (4096, 4096), "o_proj": (4096, 4096),
            "gate_proj": (4096, 11008), "up_proj": (4096, 11008), "down_proj": (11008, 4096)}


def calib_input(name):
    i = list(INPUT_K).index(name)
    return activations_fp16(M, INPUT_K[name], seed=seed_for(5, 10 + i), lognormal=True)


def layer_weight(li, K, N):
    return normal_fp16((N, K), 0.02, seed=seed_for(5, 100 + li))


def main():
    alphas = oracle.alpha_grid(20)
    out = {"_about": "oracle.search (C++ oracle) on the 7B-block search workload (65,536 calibration rows, "
                      "lognormal channel profile, 1% outliers x20, 20 alphas, group 128); written by "
                      "make_search_llama2_7b_block.py",
           "calib_rows": M, "alphas": [float(a) for a in alphas], "layers": {}}
    cache = {}
    for li, (lname, src) in enumerate(layer_inputs_7b_block()):
        K, N = LAYER_KN[lname]
        if src not in cache:
            cache.clear()
            cache[src] = calib_input(src)
        X = cache[src]
        W = layer_weight(li, K, N)
        t0 = time.time()
        r = oracle.search(W, X, alphas=alphas)
        dt = time.time() - t0
        out["layers"][lname] = {"K": K, "N": N, "alpha_index": int(r["alpha_index"]),
                                "losses": [float(v) for v in r["losses"]], "oracle_seconds": round(dt, 1),
                                "oracle_threads": os.cpu_count()}
        print(f"{lname}: alpha*={alphas[r['alpha_index']]:.2f} L*/L0={r['losses'][r['alpha_index']] / r['losses'][0]:.4f} "
              f"({dt:.0f} s)", flush=True)
    path = os.path.join(ROOT, "tests", "golden", "search_llama2_7b_block.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
