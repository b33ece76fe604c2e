"""Explore the slope-at-zero versus closeness-to-1 trade-off of Newton-Schulz
coefficient schedules (host-side design aid; nothing here runs on the GPU).

The "new optimizer" thread (tweet 6/8) picks the quintic's coefficients to
maximise the slope at zero, accepting that the iteration no longer converges
exactly, and notes a trade-off space there.  In exact arithmetic each
iteration X <- a X + (b A + c A^2) X maps every singular value s of the
normalised input through p(s) = a s + b s^3 + c s^5, so a schedule of K
triples maps s through the composition P = p_K o ... o p_1.  Two numbers
summarise a schedule:

  slope0   P'(0) = a_1 a_2 ... a_K: how much the smallest singular values
           are amplified (bigger is better for ill-conditioned updates)
  band     [min P, max P] over s in [s_min, 1]: how far the orthogonalised
           update's singular values spread around 1 (narrower is closer to
           an exact orthogonalisation)

Run `python -m optimizer_muon_step_amd.coeff_tradeoff` for a table of the
default triple, the textbook convergent quintic and a few schedules.
"""
from __future__ import annotations

import numpy as np

DEFAULT_TRIPLE = (3.4445, -4.7750, 2.0315)
TEXTBOOK_TRIPLE = (15 / 8, -10 / 8, 3 / 8)  # p(1) = 1, p'(1) = 0: converges to the polar factor


def as_schedule(coeffs, ns_steps):
    arr = np.asarray(coeffs, np.float64)
    if arr.shape == (3,):
        return [tuple(arr)] * ns_steps
    if arr.shape == (ns_steps, 3):
        return [tuple(r) for r in arr]
    raise ValueError(f"expected one triple or {ns_steps} triples")


def compose(schedule, s):
    """P(s) for an array of singular values s (fp64)."""
    s = np.asarray(s, np.float64)
    for a, b, c in schedule:
        s2 = s * s
        s = s * (a + s2 * (b + c * s2))
    return s


def profile(schedule, s_min=1e-3, points=20001):
    """slope0, band over [s_min, 1] (log-spaced grid plus the end points) and
    the grid point where P is largest."""
    grid = np.unique(np.concatenate([np.geomspace(s_min, 1.0, points), [s_min, 1.0]]))
    P = compose(schedule, grid)
    slope0 = float(np.prod([a for a, _, _ in schedule]))
    return {"slope0": slope0, "band": (float(P.min()), float(P.max())), "argmax": float(grid[np.argmax(P)]),
            "P(1)": float(compose(schedule, [1.0])[0])}


def main():
    cases = {
        "default x5": as_schedule(DEFAULT_TRIPLE, 5),
        "textbook x5": as_schedule(TEXTBOOK_TRIPLE, 5),
        "default x3 + textbook x2": [DEFAULT_TRIPLE] * 3 + [TEXTBOOK_TRIPLE] * 2,
        "default x4 + textbook x1": [DEFAULT_TRIPLE] * 4 + [TEXTBOOK_TRIPLE],
        "default x6": as_schedule(DEFAULT_TRIPLE, 6),
    }
    print(f"{'schedule':28s} {'slope0':>10s} {'band over [1e-3, 1]':>22s} {'P(1)':>8s}")
    for name, sch in cases.items():
        r = profile(sch)
        lo, hi = r["band"]
        print(f"{name:28s} {r['slope0']:10.1f} [{lo:8.4f}, {hi:8.4f}]   {r['P(1)']:8.4f}")


if __name__ == "__main__":
    main()
