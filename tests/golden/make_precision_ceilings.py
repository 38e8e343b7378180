"""Writes tests/golden/precision_ceilings.json: the rounding model's predicted error
ratios (oracle/rounding.py: the oracle's formulas with bf16 rounding at the bf16 path's
storage points) for the full-size parity cases, whose model evaluation takes minutes of
CPU time. Small cases are predicted inside the tests themselves.

    python tests/golden/make_precision_ceilings.py [key ...]

Each entry maps a tensor to [max|err| / RMS, RMS(err) / RMS] of the model against the
unrounded oracle. Calls only oracle/ and the seeded input generators.
"""
from __future__ import annotations

import fcntl
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import seeded_inputs as si  # noqa: E402
from oracle import rounding  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "precision_ceilings.json")

LAYERS = ["gpt_h1024", "gpt175b_tp8", "gpt1t_tp8"]
STAGES = ["gpt_h8192_stage_mb1", "gpt_h8192_stage_mb2", "gpt_h8192_stage_mb4"]
KEYS = [f"{w}:{m}" for w in LAYERS + STAGES for m in ("bf16", "bf16qk")]


def predict(key: str):
    name, mode = key.split(":")
    w = si.WORKLOADS[name]
    case = si.workload_case(name)
    sh = w.shape
    args = (case.x, case.dout)
    if w.layers == 1:
        ref = rounding.layer(*args, case.layers, sh.micro_batch, sh.seq, sh.head_dim, ())
        mod = rounding.layer(*args, case.layers, sh.micro_batch, sh.seq, sh.head_dim, rounding.MODES[mode])
        pairs = [("out", mod[0], ref[0]), ("dx", mod[1], ref[1])]
        pairs += [(k, mod[2][0][k], ref[2][0][k]) for k in sorted(ref[2][0])]
    else:
        ref = rounding.stage(*args, case.layers, sh.micro_batch, sh.seq, sh.head_dim, ())
        mod = rounding.stage(*args, case.layers, sh.micro_batch, sh.seq, sh.head_dim, rounding.MODES[mode])
        pairs = [("out", mod[0], ref[0]), ("dx", mod[1], ref[1])]
        pairs += [(f"l{l}.{k}", mod[2][l][k], ref[2][l][k]) for l in range(w.layers) for k in sorted(ref[2][l])]
    return {k: [round(v, 6) for v in rounding.ratios(a, b)[:2]] for k, a, b in pairs}


def main(keys):
    for key in keys:
        t0 = time.time()
        pred = predict(key)
        # read-modify-write under a lock, so that runs over disjoint keys can go in parallel
        with open(OUT + ".lock", "w") as lk:
            fcntl.flock(lk, fcntl.LOCK_EX)
            data = {}
            if os.path.exists(OUT):
                with open(OUT) as f:
                    data = json.load(f)
            data[key] = pred
            with open(OUT, "w") as f:
                json.dump(data, f, indent=1, sort_keys=True)
        print(f"{key}: {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or KEYS)
