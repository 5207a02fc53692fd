"""Writes the CPU oracle's per-row results for a full-size workload.

Runs only `oracle/` on the seeded inputs of `workloads/`; the stored values
let the full-size GPU test compare sampled rows of dW, which need every row's
log-sum-exp. Usage: python tests/golden/make_fullsize_oracle.py gptoss20b_32k
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads as wl  # noqa: E402


def main(name):
    w = wl.get_config(name)
    x = wl.generate(w)
    t0 = time.time()
    out = oracle.forward(x["H"], x["W"], x["ids"], x["logits"], w.T, block=512)
    path = os.path.join(HERE, f"oracle_{name}_rows.npz")
    np.savez_compressed(path, row_lse=out["row_lse"], row_kl=out["row_kl"],
                        loss=np.array(out["loss"]), seed=np.array(wl.seed_for(w)))
    print(f"{name}: loss {out['loss']:.12f} in {time.time() - t0:.0f} s -> {path}")


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "gptoss20b_32k")
