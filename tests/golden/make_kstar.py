"""Writes kstar.json: the Newton budget K*(T) -- the smallest iteration count whose iterate agrees
with the sequential unroll to tau = 1e-4 (max abs over every element and state component) -- for
the diagonal GRU and LSTM, zero and warm first iterates, on a grid of sequence lengths.  With it, the
residual history R_0 .. R_7 of 8 Newton iterations on the same inputs and, from it, the iteration count
of tolerance mode (the first k with R_k < tol, plus one) at tol = 1e-4, 1e-5 and 1e-6.

The protocol is the one the pararnn-torch README describes: K*(T) and the warm start in section
"Method", the long-context campaign (iterates within 1e-4 of the unroll, one batch row) in section "Benchmarks".  Inputs are the seeded synthetic ones of the benchmark workloads (GRU: bf16 gate
inputs, LSTM: fp32), B = 1, D = 1024.  Everything is computed by the fp64 CPU oracle: the iterates
by Newton with sequential linear solves, the reference by the sequential unroll.

    python tests/golden/make_kstar.py     # several minutes on 8 cores
"""
import json
import os
import sys
import time

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle  # noqa: E402
from nonlinear_rnn_solve_amd import synth  # noqa: E402

TAU = 1e-4
T_GRID = [1024, 4096, 16384, 65536, 131072]
CELLS = [("gru", "bf16"), ("lstm", "f32")]
B, D, K_MAX = 1, 1024, 8
STOP_TOLS = (1e-4, 1e-5, 1e-6)


def main():
    out = {"tau": TAU, "B": B, "D": D, "t_grid": T_GRID, "seed_rule": "3000 + T // 1024 (+ 500 for lstm)",
           "stop_tols": list(STOP_TOLS), "entries": []}
    for cell, dtype in CELLS:
        for T in T_GRID:
            seed = 3000 + T // 1024 + (500 if cell == "lstm" else 0)
            inp = synth.make_inputs(cell, B, T, D, dtype=dtype, seed=seed)
            prob = oracle.Problem(cell, inp.pre, inp.w, inp.bias, dtype=oracle.BF16 if dtype == "bf16" else oracle.F32)
            U = oracle.unroll(prob)
            for warm in (False, True):
                t0 = time.time()
                errs = []
                for K in range(1, K_MAX + 1):
                    H = oracle.newton(prob, K, warm=warm)[0]
                    errs.append(float(np.max(np.abs(H - U))))
                    if errs[-1] <= TAU:
                        break
                kstar = len(errs) if errs[-1] <= TAU else None
                _, res, _, _, _ = oracle.newton(prob, K_MAX, warm=warm)
                stops = {}
                for tol in STOP_TOLS:
                    below = [k for k, r in enumerate(res) if r < tol]
                    stops["%g" % tol] = below[0] + 1 if below else None
                out["entries"].append({"cell": cell, "dtype": dtype, "init": "warm" if warm else "zero", "T": T,
                                       "seed": seed, "kstar": kstar, "max_err_by_k": errs,
                                       "residuals": [float(r) for r in res], "stop_iters": stops})
                print(cell, T, "warm" if warm else "zero", "K* =", kstar, ["%.2e" % e for e in errs], "stops", stops,
                      "%.0fs" % (time.time() - t0), flush=True)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "kstar.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
