"""Distance of the fp32 oracle from the fp64 oracle after a full solve.

TEST INFRASTRUCTURE ONLY (like the rest of this package).  The fp32 oracle is
the parity reference of the GPU kernels, which match it bit for bit; the fp64
run of the same iteration (the same steps of the page "TV solver: the FGP
step on the GPU", section "What one step does", in double precision) is the
accuracy reference.  This prints, per workload, the largest absolute
difference between the two on p, r and the read-out z after the workload's
outer x inner steps, as context for the 1e-5 parity gate: it is not a gate.

    python -m oracle.accuracy 0 1 2 [3]
"""
import json
import sys
import time

import numpy as np

import oracle
import phantoms


def distance(idx):
    w = phantoms.workload(idx)
    b, p0, r0 = phantoms.make_inputs(idx)
    t = time.perf_counter()
    p32, r32 = oracle.run(b, p0, r0, w["lam"], w["n_outer"], w["n_inner"])
    z32 = oracle.primal(b, p32, w["lam"])
    b64 = b.astype(np.float64)
    p64, r64 = oracle.run(b64, p0, r0, w["lam"], w["n_outer"], w["n_inner"], dtype=np.float64)
    z64 = oracle.primal(b64, p64, w["lam"])

    def d(x, y):
        return float(np.max(np.abs(x.astype(np.float64) - y)))

    return {"workload": phantoms.BASE_NAMES[idx], "steps": w["n_outer"] * w["n_inner"],
            "lambda": w["lam"], "max_abs_p": d(p32, p64), "max_abs_r": d(r32, r64),
            "max_abs_z": d(z32, z64), "max_abs_z64": float(np.max(np.abs(z64))),
            "seconds": round(time.perf_counter() - t, 1), "threads": oracle.get_threads()}


def main(argv):
    for a in argv or ["0", "1", "2"]:
        print(json.dumps(distance(int(a))), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
