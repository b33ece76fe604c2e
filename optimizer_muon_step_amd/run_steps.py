"""Run a fixed number of Muon steps on named workloads, for a profiler.

    python -m optimizer_muon_step_amd.run_steps c1:10:50 c2:10:50

Each argument is WORKLOAD:WARM:STEPS.  A workload gets seeded inputs from
workloads.py, WARM untimed steps, a device synchronisation, then STEPS
steps enqueued back to back on one stream and a synchronisation; one line
per workload reports the wall time of those STEPS.  The workloads run in
the order given, so a kernel trace of the run holds, for each of them,
WARM + STEPS consecutive steps (momentum ... apply)."""
from __future__ import annotations

import os
import sys
import time

if __package__ in (None, ""):  # run as a file: make the package importable
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))


def main(argv: list[str]) -> int:
    import torch

    import optimizer_muon_step_amd as mu
    from optimizer_muon_step_amd import workloads as wl

    if not torch.cuda.is_available():
        raise SystemExit("run_steps needs a GPU")
    mu._lib.load()
    lr, beta, ns_steps, coeffs = 0.02, 0.95, 5, (3.4445, -4.7750, 2.0315)
    for arg in argv:
        name, warm, steps = arg.split(":")
        warm, steps = int(warm), int(steps)
        specs = wl.config_specs(name)
        W = [torch.from_numpy(wl.make_params(name, i, s)).cuda() for i, s in enumerate(specs)]
        G = [torch.from_numpy(wl.make_grad(name, i, s, 1)).cuda() for i, s in enumerate(specs)]
        M = [torch.zeros((s.rows, s.cols), device="cuda") for s in specs]
        torch.cuda.synchronize()
        for _ in range(warm):
            mu.muon_step(W, G, M, lr, beta, ns_steps, coeffs)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            mu.muon_step(W, G, M, lr, beta, ns_steps, coeffs)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        print(f"{name}: {len(specs)} matrices, {warm} warm + {steps} steps, "
              f"{1e3 * dt / steps:.4f} ms per step (wall), {steps / dt:.1f} steps/s", flush=True)
        del W, G, M
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
