"""Seeded synthetic workloads for the DashAttention forward pass.

This module only draws data: shapes, seeds, value distributions and the planted
structure (needle chunks, key clusters, flat/sharp decode queries). It holds none
of the method's arithmetic (no summaries, scores, entmax, bias or attention), so
both the CPU oracle and the HIP path can consume exactly the same inputs.

Conventions
-----------
* Layout is BHSD: Q is [b, h_q, n_q, d]; K and V are [b, h_kv, n_kv, d].
* One ``numpy.random.default_rng(seed)`` per workload. Tensors are drawn in a
  fixed order: Q, K, V, q̄, then planted structure, then per-head scalings.
* Values are drawn in float32; for bf16 workloads they are then rounded to the
  nearest bfloat16 (ties to even) and kept as float32 arrays holding
  bf16-exact values, so converting them to bfloat16 on the device is exact.
* q̄ (the learned per-KV-head summary query) is drawn N(0, 0.1^2) in float32.

Workload names follow what they are (mode, context, shape):
``prefill_1k_fp32``, ``prefill_8k_gqa8_needles``, ``decode_32k_b16``,
``prefill_32k_clusters`` and ``decode_128k_b4``.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

# γ of the 8K needle prefill workload: the value at which the oracle's group
# routing (on every 16th query row) leaves 75% +- 1% of the visible chunks with
# zero weight. Written by oracle/calibrate_gamma.py; the CPU test suite
# re-checks the sparsity it produces.
GAMMA_PREFILL_8K = 5.3586700962132126


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns a float32 array whose values are exactly representable in bf16.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    mode: str               # "prefill" or "decode"
    dtype: str              # "f32" or "bf16": the stored dtype of Q, K, V
    b: int
    h_q: int
    h_kv: int
    d: int
    n: int                  # prefill: sequence length; decode: KV length L (incl. the new token)
    B: int                  # chunk size
    alphas: Tuple[float, ...]
    gamma: float
    sigma: float
    causal: bool
    Q: np.ndarray           # prefill [b,h_q,n,d]; decode [b,h_q,1,d]
    K: np.ndarray           # [b,h_kv,n,d]
    V: np.ndarray           # [b,h_kv,n,d]
    qbar: np.ndarray        # [h_kv,d] float32
    seq_len: Optional[np.ndarray] = None   # decode: [b] int32 KV length incl. the new token
    notes: str = ""

    @property
    def alpha(self) -> float:
        return self.alphas[0]

    @property
    def g(self) -> int:
        return self.h_q // self.h_kv

    @property
    def num_chunks(self) -> int:
        return self.n // self.B


def _unit(v: np.ndarray) -> np.ndarray:
    return v / np.linalg.norm(v, axis=-1, keepdims=True)


def _orth_unit(rng: np.random.Generator, u: np.ndarray, count: int) -> np.ndarray:
    """`count` random unit vectors orthogonal to the unit vector u (float64)."""
    e = rng.standard_normal((count, u.shape[-1]))
    e -= (e @ u)[:, None] * u[None, :]
    return _unit(e)


def _plant_direction(rng: np.random.Generator, rows: np.ndarray, u: np.ndarray,
                     cos: float = 0.8) -> np.ndarray:
    """Rotate each row to cosine `cos` with u, keeping its norm: |r|(cos u + sin e)."""
    norms = np.linalg.norm(rows.astype(np.float64), axis=-1, keepdims=True)
    e = _orth_unit(rng, u, rows.shape[0])
    sin = np.sqrt(1.0 - cos * cos)
    return (norms * (cos * u[None, :] + sin * e)).astype(np.float32)


def _draw_qkv(rng, b, h_q, h_kv, n_q, n_kv, d):
    Q = rng.standard_normal((b, h_q, n_q, d), dtype=np.float32)
    K = rng.standard_normal((b, h_kv, n_kv, d), dtype=np.float32)
    V = rng.standard_normal((b, h_kv, n_kv, d), dtype=np.float32)
    qbar = (0.1 * rng.standard_normal((h_kv, d))).astype(np.float32)
    return Q, K, V, qbar


def _finish(w: Workload) -> Workload:
    if w.dtype == "bf16":
        w.Q = round_bf16(w.Q)
        w.K = round_bf16(w.K)
        w.V = round_bf16(w.V)
    return w


def make_prefill(b=1, h_q=1, h_kv=1, d=64, n=1024, B=64, alphas=(1.5,), gamma=1.0,
                 sigma=1.0, causal=True, dtype="f32", seed=0, name="prefill_custom",
                 qbar_scale=0.1) -> Workload:
    """Plain N(0,1) Q, K, V prefill workload of the given shape."""
    rng = np.random.default_rng(seed)
    Q, K, V, qbar = _draw_qkv(rng, b, h_q, h_kv, n, n, d)
    if qbar_scale != 0.1:
        qbar = (qbar * np.float32(qbar_scale / 0.1)).astype(np.float32)
    return _finish(Workload(name, "prefill", dtype, b, h_q, h_kv, d, n, B, tuple(alphas),
                            float(gamma), float(sigma), bool(causal), Q, K, V, qbar))


def upstream_grad(shape, seed=0, dtype="f32") -> np.ndarray:
    """N(0,1) upstream gradient dO of a given shape (rounded to bf16 for dtype bf16)."""
    g = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    return round_bf16(g) if dtype == "bf16" else g


def make_decode(b=2, h_q=4, h_kv=2, d=64, L=1024, B=64, alphas=(1.5,), gamma=1.0,
                sigma=1.0, dtype="bf16", seed=0, name="decode_custom",
                seq_len=None) -> Workload:
    """Plain N(0,1) decode workload: one new query per sequence, KV length L."""
    rng = np.random.default_rng(seed)
    Q, K, V, qbar = _draw_qkv(rng, b, h_q, h_kv, 1, L, d)
    sl = np.full((b,), L, np.int32) if seq_len is None else np.asarray(seq_len, np.int32)
    return _finish(Workload(name, "decode", dtype, b, h_q, h_kv, d, L, B, tuple(alphas),
                            float(gamma), float(sigma), True, Q, K, V, qbar, sl))


# --------------------------------------------------------------------------------------
# The five reference workloads.
# --------------------------------------------------------------------------------------

def prefill_1k_fp32(seed=0, gamma=1.0) -> Workload:
    """Causal prefill, fp32, b=1, 1 query / 1 KV head, n=1024, d=64, B=64, α=1.5, γ=1."""
    return make_prefill(1, 1, 1, 64, 1024, 64, (1.5,), gamma, 1.0, True, "f32", seed,
                        name="prefill_1k_fp32")


def prefill_8k_gqa8_needles(seed=0, gamma=None) -> Workload:
    """Causal prefill, bf16, b=1, 16 query / 2 KV heads, d=128, n=8192, B=64, α=1.5.

    Eight needle chunks per KV head at distinct chunk positions in [1, T_c-2]: every
    key of a needle chunk is rotated to cosine 0.8 with a needle direction u_m
    (norm kept), and 64 query rows after the chunk have every head of the group
    set to |q| u_m. γ is the calibrated value that gives ~75% group sparsity.
    """
    b, h_q, h_kv, d, n, B = 1, 16, 2, 128, 8192, 64
    g = h_q // h_kv
    T = n // B
    rng = np.random.default_rng(seed)
    Q, K, V, qbar = _draw_qkv(rng, b, h_q, h_kv, n, n, d)
    for r in range(h_kv):
        chunks = rng.choice(np.arange(1, T - 1), size=8, replace=False)
        taken = np.zeros(n, bool)
        for c in chunks:
            u = _unit(rng.standard_normal(d))
            sl = slice(c * B, (c + 1) * B)
            K[0, r, sl] = _plant_direction(rng, K[0, r, sl], u)
            eligible = np.nonzero(~taken[(c + 1) * B:])[0] + (c + 1) * B
            rows = rng.choice(eligible, size=min(64, eligible.size), replace=False)
            taken[rows] = True
            for hh in range(r * g, (r + 1) * g):
                qn = np.linalg.norm(Q[0, hh, rows].astype(np.float64), axis=-1, keepdims=True)
                Q[0, hh, rows] = (qn * u[None, :]).astype(np.float32)
    gam = GAMMA_PREFILL_8K if gamma is None else float(gamma)
    return _finish(Workload("prefill_8k_gqa8_needles", "prefill", "bf16", b, h_q, h_kv, d, n, B,
                            (1.5,), gam, 1.0, True, Q, K, V, qbar,
                            notes="8 needle chunks per KV head, 64 aligned query rows each"))


def decode_32k_b16(seed=0) -> Workload:
    """Decode, bf16, b=16, 32 query / 2 KV heads, d=128, L=32768, B=64, α=1.5, γ=1.

    Each (b, h) query is scaled by s ~ LogNormal(0, 0.5) so that per-head support
    sizes range from sharp to flat.
    """
    b, h_q, h_kv, d, L, B = 16, 32, 2, 128, 32768, 64
    rng = np.random.default_rng(seed)
    Q, K, V, qbar = _draw_qkv(rng, b, h_q, h_kv, 1, L, d)
    s = rng.lognormal(0.0, 0.5, size=(b, h_q)).astype(np.float32)
    Q *= s[:, :, None, None]
    return _finish(Workload("decode_32k_b16", "decode", "bf16", b, h_q, h_kv, d, L, B, (1.5,),
                            1.0, 1.0, True, Q, K, V, qbar, np.full((b,), L, np.int32),
                            notes="per-head query scale ~ LogNormal(0, 0.5)"))


def prefill_32k_clusters(seed=0, alphas=(1.25, 1.5, 2.0)) -> Workload:
    """Causal prefill, bf16, b=1, 32 query / 2 KV heads, d=128, n=32768, B=64, γ=1.

    32 clusters per KV head, each of 4 adjacent chunks starting at a multiple of 4;
    every key in a cluster is rotated to cosine 0.8 with the cluster's direction.
    """
    b, h_q, h_kv, d, n, B = 1, 32, 2, 128, 32768, 64
    T = n // B
    rng = np.random.default_rng(seed)
    Q, K, V, qbar = _draw_qkv(rng, b, h_q, h_kv, n, n, d)
    for r in range(h_kv):
        starts = 4 * rng.choice(np.arange(T // 4), size=32, replace=False)
        for c0 in starts:
            u = _unit(rng.standard_normal(d))
            sl = slice(c0 * B, (c0 + 4) * B)
            K[0, r, sl] = _plant_direction(rng, K[0, r, sl], u)
    return _finish(Workload("prefill_32k_clusters", "prefill", "bf16", b, h_q, h_kv, d, n, B,
                            tuple(alphas), 1.0, 1.0, True, Q, K, V, qbar,
                            notes="32 clusters x 4 adjacent chunks per KV head, cosine 0.8"))


def decode_128k_b4(seed=0) -> Workload:
    """Decode, bf16, b=4, 32 query / 2 KV heads, d=128, L=131072, B=128, α=1.5, γ=1.

    Per (b, r) group: 8 needle chunks at uniform-random visible positions with keys
    at cosine 0.8 to a unit direction u_{b,r}. Four of the eight groups are flat
    (every head's query has norm 0.2), four sharp (norm 4); each head's query is
    norm * unit(0.8 u_{b,r} + 0.6 e_h) with e_h a random unit vector orthogonal to u.
    """
    b, h_q, h_kv, d, L, B = 4, 32, 2, 128, 131072, 128
    g = h_q // h_kv
    vis = (L - 1) // B
    rng = np.random.default_rng(seed)
    Q, K, V, qbar = _draw_qkv(rng, b, h_q, h_kv, 1, L, d)
    sharp = rng.permutation(np.array([0] * 4 + [1] * 4)).reshape(b, h_kv)
    for bi in range(b):
        for r in range(h_kv):
            u = _unit(rng.standard_normal(d))
            for c in rng.choice(np.arange(vis), size=8, replace=False):
                sl = slice(c * B, (c + 1) * B)
                K[bi, r, sl] = _plant_direction(rng, K[bi, r, sl], u)
            norm = 4.0 if sharp[bi, r] else 0.2
            e = _orth_unit(rng, u, g)
            q = norm * _unit(0.8 * u[None, :] + 0.6 * e)
            Q[bi, r * g:(r + 1) * g, 0] = q.astype(np.float32)
    w = Workload("decode_128k_b4", "decode", "bf16", b, h_q, h_kv, d, L, B, (1.5,), 1.0, 1.0,
                 True, Q, K, V, qbar, np.full((b,), L, np.int32),
                 notes="4 flat (|q|=0.2) and 4 sharp (|q|=4) groups, 8 needles per group")
    w.sharp = sharp
    return _finish(w)


# --------------------------------------------------------------------------------------
# Replicas of the pages' efficiency operating points (paper review section 五,
# efficiency table): causal prefill of 16K and 96K tokens at batch 1 and decode at 96K
# with batch 24, chunk size 64, group sparsity 75 / 87.5 / 93.75 % reached through γ.
# Plain N(0,1) inputs (the pages measure trained-model activations, which are not
# available); the γ values are frozen from the oracle's routing by
# oracle/calibrate_gamma.py (`--efficiency`).
# --------------------------------------------------------------------------------------

EFFICIENCY_SPARSITY = (0.75, 0.875, 0.9375)
# γ per (workload, target group sparsity), bisected by the float64 oracle on sampled
# rows (prefill: every 64th row at 16K, every 256th at 96K; decode: all 24 queries).
# 93.75% is out of reach at 16K on these inputs: with only up to 256 visible chunks,
# the union over 16 query heads of near-argmax weights still leaves about 11% of the
# chunks routed (0.889 at γ = 4096).
GAMMA_EFFICIENCY = {
    ("prefill_16k", 0.75): 34.52, ("prefill_16k", 0.875): 304.4,
    ("prefill_96k", 0.75): 8.819, ("prefill_96k", 0.875): 16.35, ("prefill_96k", 0.9375): 29.34,
    ("decode_96k_b24", 0.75): 6.583, ("decode_96k_b24", 0.875): 11.07, ("decode_96k_b24", 0.9375): 19.87,
}


def efficiency_prefill(n, sparsity=None, seed=0, gamma=None) -> Workload:
    """Causal prefill, bf16, b=1, 32 query / 2 KV heads, d=128, B=64, α=1.5, N(0,1)."""
    rng = np.random.default_rng(seed)
    b, h_q, h_kv, d, B = 1, 32, 2, 128, 64
    Q, K, V, qbar = _draw_qkv(rng, b, h_q, h_kv, n, n, d)
    key = (f"prefill_{n // 1024}k", sparsity)
    gam = float(gamma) if gamma is not None else GAMMA_EFFICIENCY.get(key, 1.0)
    return _finish(Workload(f"efficiency_prefill_{n // 1024}k", "prefill", "bf16", b, h_q, h_kv, d, n, B,
                            (1.5,), gam, 1.0, True, Q, K, V, qbar,
                            notes=f"target group sparsity {sparsity}"))


def efficiency_decode(sparsity=None, seed=0, gamma=None, b=24, L=96 * 1024) -> Workload:
    """Decode, bf16, b=24, 32 query / 2 KV heads, d=128, L=96K, B=64, α=1.5, N(0,1)."""
    rng = np.random.default_rng(seed)
    h_q, h_kv, d, B = 32, 2, 128, 64
    Q, K, V, qbar = _draw_qkv(rng, b, h_q, h_kv, 1, L, d)
    key = (f"decode_{L // 1024}k_b{b}", sparsity)
    gam = float(gamma) if gamma is not None else GAMMA_EFFICIENCY.get(key, 1.0)
    sl = np.full((b,), L, np.int32)
    return _finish(Workload(f"efficiency_decode_{L // 1024}k_b{b}", "decode", "bf16", b, h_q, h_kv, d, L, B,
                            (1.5,), gam, 1.0, True, Q, K, V, qbar, sl,
                            notes=f"target group sparsity {sparsity}"))


WORKLOADS = {
    "prefill_1k_fp32": prefill_1k_fp32,
    "prefill_8k_gqa8_needles": prefill_8k_gqa8_needles,
    "decode_32k_b16": decode_32k_b16,
    "prefill_32k_clusters": prefill_32k_clusters,
    "decode_128k_b4": decode_128k_b4,
}


def make(name: str, seed: int = 0, **kw) -> Workload:
    return WORKLOADS[name](seed=seed, **kw)
