"""Calibrate γ of the 8K needle prefill workload with the oracle's routing.

TEST INFRASTRUCTURE: calls only the oracle and the seeded input generator.
Deterministic bisection on log γ over [1, 1024]: the oracle's group routing is
evaluated on every 16th query row and γ is moved until the group sparsity
(fraction of visible chunks with zero group weight) is 0.75 +- 0.01.

Usage:  python oracle/calibrate_gamma.py        (prints the frozen γ)
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from oracle import dash_oracle as O  # noqa: E402
from long_context_amd import inputs  # noqa: E402


def sparsity_at(w, kbar, gamma, rows):
    rt = O.route(w.Q[:, :, rows], rows[None, :], kbar, w.B, w.alpha, gamma, w.sigma,
                 True, w.n)
    return O.group_sparsity(rt)


def calibrate(target=0.75, tol=0.01, seed=0):
    w = inputs.prefill_8k_gqa8_needles(seed=seed, gamma=1.0)
    kbar = O.stage0_summaries(w.K, w.qbar, w.B)
    rows = np.arange(0, w.n, 16)
    lo, hi = math.log(1.0), math.log(1024.0)
    g = math.exp(0.5 * (lo + hi))
    for _ in range(60):
        g = math.exp(0.5 * (lo + hi))
        s = sparsity_at(w, kbar, g, rows)
        if abs(s - target) <= tol:
            return g, s
        if s < target:
            lo = math.log(g)
        else:
            hi = math.log(g)
    return g, sparsity_at(w, kbar, g, rows)


if __name__ == "__main__":
    gamma, s = calibrate()
    print(f"gamma={gamma!r} sparsity={s:.4f}")
