"""The oracle still reproduces its stored outputs on one small seeded case
(tests/golden/oracle_small.json, written by tests/golden/make_oracle_golden.py
from the oracle alone).  A change here means the oracle's arithmetic changed."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))


def test_oracle_matches_stored_golden():
    import make_oracle_golden as g

    with open(os.path.join(HERE, "golden", "oracle_small.json")) as f:
        stored = json.load(f)
    now = g.compute()
    for pv in ("fp8", "fp16"):
        for key in ("q8_sha256", "k8_sha256", "vq_sha256"):
            assert now[pv][key] == stored[pv][key], (pv, key)
        for key in ("q_scale", "k_scale", "k_mean_head", "v_scale_head"):
            assert np.array_equal(np.float32(now[pv][key]), np.float32(stored[pv][key])), (pv, key)
        assert np.allclose(np.float32(now[pv]["out"]), np.float32(stored[pv]["out"]), rtol=0, atol=1e-6)
