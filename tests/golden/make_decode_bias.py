"""Writes decode_router_bias.json: the threshold-router biases of the 360M-shape MoR-4 decode
workload, calibrated by the CPU oracle (oracle.calibrate_threshold_bias) on the seed-4
calibration batch (4 sequences x 128 tokens of N(0, 1) hidden states) with the seed-0 weights.

The biases stand in for a trained router: with them, the static sigmoid > 0.5 test keeps about
3/4, 2/3 and 1/2 of the tokens that reach recursions 2, 3 and 4 (capacities 4/4, 3/4, 2/4, 1/4).

    python tests/golden/make_decode_bias.py
"""
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workload  # noqa: E402

CONFIG, CAL_B, CAL_T = "smol360m_mor4_decode", 4, 128


def main():
    cfg = workload.get_config(CONFIG)
    W = workload.make_weights(cfg)
    H = workload.make_calibration_inputs(cfg, CAL_B, CAL_T)
    t0 = time.time()
    b = oracle.calibrate_threshold_bias(cfg, W, H)
    rec = {"config": CONFIG, "calibration": f"seed {workload.SEED_CALIB}, {CAL_B} x {CAL_T} tokens",
           "router_b": [float(x) for x in b], "seconds": round(time.time() - t0, 1)}
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "decode_router_bias.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
