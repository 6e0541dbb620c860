"""How often the step's two nonlinear branches act on each workload.

TEST INFRASTRUCTURE ONLY (like the rest of this package).  The step of the
page "TV solver: the FGP step on the GPU" (section "What one step does") has
two nonlinear parts: the clip z = max(b - lambda L(r), 0) and the projection
p' = q / max(1, |q|).  A parity test only exercises them if the inputs drive
them, so this reports, after each workload's outer x inner steps of the fp32
oracle:

  clipped    the fraction of voxels where the read-out z is 0 (the clip acts);
  projected  the fraction of voxels where |p| is within 1e-6 of 1, i.e. the
             last step projected there (|q| > 1 gives |p'| = 1 up to
             rounding; |q| <= 1 leaves p' = q, inside the ball).

    python -m oracle.branches 0 1 2 [3] [4]
"""
import json
import sys
import time

import numpy as np

import oracle
import phantoms


def fractions(idx):
    w = phantoms.workload(idx)
    b, p0, r0 = phantoms.make_inputs(idx)
    t = time.perf_counter()
    p, _ = oracle.run(b, p0, r0, w["lam"], w["n_outer"], w["n_inner"])
    z = oracle.primal(b, p, w["lam"])
    norm2 = (p.astype(np.float64) ** 2).sum(axis=0)
    return {"workload": phantoms.BASE_NAMES[idx], "steps": w["n_outer"] * w["n_inner"],
            "clipped": round(float(np.mean(z == 0.0)), 4),
            "projected": round(float(np.mean(norm2 > (1.0 - 1e-6) ** 2)), 4),
            "seconds": round(time.perf_counter() - t, 1), "threads": oracle.get_threads()}


def main(argv):
    for a in argv or ["0", "1", "2"]:
        print(json.dumps(fractions(int(a))), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
