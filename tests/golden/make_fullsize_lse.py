"""Writes the fp64 oracle's per-token log-sum-exp, target logit and mean loss
for the three large seeded workloads, so that the full-size GPU parity test
can compare every token without spending minutes of host time per run.

Calls only the oracle (``oracle.forward``, ``oracle.target_logits``) on the
seeded inputs of ``workloads`` (seed 0); nothing here comes from the HIP
path. Output, per workload NAME:
  tests/golden/fullsize_NAME_lse.npy   float64 [N]  oracle lse_i
  tests/golden/fullsize_NAME_tgt.npy   float64 [N]  H_i . W_{y_i} (NaN where
                                                    the label is ignored)
  tests/golden/fullsize_oracle.json    input fingerprint, n_valid, loss

    python tests/golden/make_fullsize_lse.py [NAME ...]

About 18 minutes of fp64 BLAS on 8 cores for all three.
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads as WL  # noqa: E402

NAMES = [w.name for w in WL.WORKLOADS[2:]]
INDEX = os.path.join(HERE, "fullsize_oracle.json")


def main(names):
    index = {}
    if os.path.exists(INDEX):
        with open(INDEX) as f:
            index = json.load(f)
    for name in names:
        w = WL.BY_NAME[name]
        t0 = time.perf_counter()
        inp = WL.make_inputs(w, 0)
        fp = WL.fingerprint(inp)
        H, W = inp.H_f64(), inp.W_f64()
        loss, lse = oracle.forward(H, W, inp.labels)
        tgt = oracle.target_logits(H, W, inp.labels)
        tgt[inp.labels == WL.IGNORE_INDEX] = np.nan
        del H, W
        np.save(os.path.join(HERE, f"fullsize_{name}_lse.npy"), lse)
        np.save(os.path.join(HERE, f"fullsize_{name}_tgt.npy"), tgt)
        index[name] = {
            "fingerprint": fp,
            "seed": 0,
            "N": w.N, "d": w.d, "V": w.V,
            "n_valid": int((inp.labels != WL.IGNORE_INDEX).sum()),
            "loss": float(loss),
            "lse": f"fullsize_{name}_lse.npy",
            "tgt": f"fullsize_{name}_tgt.npy",
            "written_by": "tests/golden/make_fullsize_lse.py (oracle.forward,"
                          " oracle.target_logits; fp64)",
        }
        with open(INDEX, "w") as f:
            json.dump(index, f, indent=1, sort_keys=True)
        print(f"{name}: loss {loss:.9f} in {time.perf_counter() - t0:.0f} s",
              flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or NAMES)
