"""Writes tests/golden/oracle_small.json: the oracle's outputs on one small
seeded case (a regression fixture for the oracle; every value comes from the
oracle package alone).  Run: python tests/golden/make_oracle_golden.py"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synthetic_inputs as si  # noqa: E402


def compute():
    wl = si.make("tiny", N=300, H=1, seed=4242)
    q, k, v = (si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))
    res = {"workload": "tiny recipe, B=1 H=1 N=300 d=128, seed 4242", "rows": [0, 129, 299]}
    for pv in ("fp8", "fp16"):
        out, z, vq, vs = oracle.attention(q, k, v, False, wl.sm_scale, pv, rows=res["rows"])
        res[pv] = {
            "q8_sha256": hashlib.sha256(z["q8"].tobytes()).hexdigest(),
            "k8_sha256": hashlib.sha256(z["k8"].tobytes()).hexdigest(),
            "vq_sha256": hashlib.sha256(vq.tobytes()).hexdigest(),
            "q_scale": z["q_scale"].ravel().tolist(),
            "k_scale": z["k_scale"].ravel().tolist(),
            "k_mean_head": z["k_mean"].ravel()[:8].tolist(),
            "v_scale_head": vs.ravel()[:8].tolist(),
            "out": out[0, 0].tolist(),
        }
    return res


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")
    with open(path, "w") as f:
        json.dump(compute(), f, indent=0)
    print("wrote", path)
