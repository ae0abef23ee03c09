"""Calibrate γ of synthetic workloads with the oracle's routing.

TEST INFRASTRUCTURE: calls only the oracle and the seeded input generators.
Deterministic bisection on log γ: the oracle's group routing is evaluated on
sampled query rows and γ is moved until the group sparsity (fraction of visible
chunks with zero group weight) reaches the target.

Usage:
  python oracle/calibrate_gamma.py                 the 8K needle prefill (target 0.75 +- 0.01)
  python oracle/calibrate_gamma.py --efficiency    the efficiency replicas (prefill 16K and
                                                   96K, decode 96K x 24) at group sparsity
                                                   0.75 / 0.875 / 0.9375 (+- 0.005)
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


def bisect(sp_fn, target, tol, lo=1.0, hi=4096.0, steps=60):
    lo, hi = math.log(lo), math.log(hi)
    g = math.exp(0.5 * (lo + hi))
    s = None
    for _ in range(steps):
        g = math.exp(0.5 * (lo + hi))
        s = sp_fn(g)
        if abs(s - target) <= tol:
            break
        if s < target:
            lo = math.log(g)
        else:
            hi = math.log(g)
    return g, s


def calibrate_efficiency(tol=0.005):
    out = {}
    for n, step in ((16 * 1024, 64), (96 * 1024, 256)):
        w = inputs.efficiency_prefill(n, gamma=1.0)
        kbar = O.stage0_summaries(w.K, w.qbar, w.B)
        rows = np.arange(w.B, w.n, step)
        for t in inputs.EFFICIENCY_SPARSITY:
            g, s = bisect(lambda gm: sparsity_at(w, kbar, gm, rows), t, tol)
            print(f"prefill_{n // 1024}k target {t}: gamma={g!r} sparsity={s:.4f}", flush=True)
            if abs(s - t) <= 2 * tol:
                out[(f"prefill_{n // 1024}k", t)] = g
            else:
                print(f"  target {t} not reachable at {n // 1024}K, left out", flush=True)
        del w, kbar
    w = inputs.efficiency_decode(gamma=1.0)
    kbar = O.stage0_summaries(w.K, w.qbar, w.B)
    pos = (w.seq_len - 1)[:, None]

    def dec_sparsity(gm):
        rt = O.route(w.Q, pos, kbar, w.B, w.alpha, gm, w.sigma, True, w.n)
        return O.group_sparsity(rt)

    for t in inputs.EFFICIENCY_SPARSITY:
        g, s = bisect(dec_sparsity, t, tol)
        if abs(s - t) <= 2 * tol:
            out[(f"decode_{w.n // 1024}k_b{w.b}", t)] = g
        print(f"decode_{w.n // 1024}k_b{w.b} target {t}: gamma={g!r} sparsity={s:.4f}", flush=True)
    return out


if __name__ == "__main__":
    if "--efficiency" in sys.argv:
        print("GAMMA_EFFICIENCY =", calibrate_efficiency())
    else:
        gamma, s = calibrate()
        print(f"gamma={gamma!r} sparsity={s:.4f}")
