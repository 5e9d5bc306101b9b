"""Write tests/golden/fp8_noise_floor.json: for each workload, how far two
evaluations of the oracle that differ only in the dot products' accumulation
(float64 rounded once vs fp32 sums) land apart on the layer output y --
relative L2 and max|dy| / RMS(y).  Calls oracle/ only.

    python tests/golden/make_noise_floor.py
"""
import json
import sys
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parents[2]
sys.path.insert(0, str(ROOT))

from oracle import moe  # noqa: E402
from workloads import make_workload  # noqa: E402

NAMES = ["prefill_fp8_small", "decode_fp8_small", "toy_bf16_fp8w", "skewed_bf16_small",
         "manyrow_fp8_small", "prefill_fp8"]


def floor(name):
    wl = make_workload(name)
    ew = moe.ExpertWeights(wl.cfg, wl.w, cache=False)
    y64 = moe.moe_layer(wl, ew=ew)["y"].astype(np.float64)
    y32 = moe.moe_layer(wl, ew=ew, acc="f32")["y"].astype(np.float64)
    d = y32 - y64
    return {"rel_l2": float(np.linalg.norm(d) / np.linalg.norm(y64)),
            "maxabs_over_rms": float(np.max(np.abs(d)) / np.sqrt(np.mean(y64 ** 2)))}


if __name__ == "__main__":
    out = {"source": "the oracle itself (oracle/moe.py moe_layer, acc='f64' vs acc='f32'); "
                     "written by tests/golden/make_noise_floor.py",
           "floors": {n: floor(n) for n in NAMES}}
    (Path(__file__).parent / "fp8_noise_floor.json").write_text(json.dumps(out, indent=1) + "\n")
    print(json.dumps(out, indent=1))
