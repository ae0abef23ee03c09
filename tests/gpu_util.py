"""Helpers of the GPU parity tests: run the HIP path through the C ABI and compare
with the oracle under the stated tolerances.

Tolerances (the method's own readings):
  * chunk summaries k̄: max |Δ| <= 1e-4;
  * group routing weights w: max |Δ| <= 1e-3 on every row;
  * routed chunk lists: identical on every row that is not exempt; a (b, r, row) is
    exempt when some head of its group has a visible chunk whose thresholded score
    x = (α-1)γz̄ lies within 1e-6 of that head's τ (oracle, float64);
  * exempt rows are at most MAX_EXEMPT_FRAC of the checked rows plus MAX_EXEMPT_ABS
    (so a broken margin cannot silently exempt everything);
  * the routed bias d = (ln w - μ)/σ of Proposition 4.1, element by element on every
    listed chunk of a non-exempt row, within the per-entry bound of bias_tolerance;
  * outputs of non-exempt rows: fp32 inputs max |ΔO| <= 1e-4; bf16 inputs
    max_d |ΔO| / rms_d(O_oracle) <= 2e-2 per (head, row).
"""
from __future__ import annotations

import numpy as np
import torch

from long_context_amd import dash
from oracle import dash_oracle as O

MARGIN = 1e-6
TOL_KBAR = 1e-4
TOL_W = 1e-3
TOPK_MARGIN = 1e-5
TOL_F32 = 1e-4
TOL_BF16_ROW = 2e-2
# A row is exempt when some head has a visible chunk within 1e-6 of τ. Over a window
# of width 2e-6 the thresholded scores of the <= 16 x 1023 (head, chunk) values of a
# row are sparse enough that a few percent of rows at most are exempt; a margin that
# broke would exempt most rows.
MAX_EXEMPT_FRAC = 0.03
MAX_EXEMPT_ABS = 2
U32 = 2.0 ** -24                       # unit roundoff of fp32
# The bias bound is checked to stay informative: its median over the listed entries
# must be small enough that an error of μ of 1e-2 (shifting every d of a row) fails.
BIAS_MEDIAN_MAX = 5e-3


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def gpu_prefill(w, alpha=None, gamma=None, sigma=None, causal=None, with_w=True, out_dtype=torch.float32,
                top_k=0):
    alpha = w.alpha if alpha is None else alpha
    gamma = w.gamma if gamma is None else gamma
    sigma = w.sigma if sigma is None else sigma
    causal = w.causal if causal is None else causal
    Q, K, V = to_dev(w.Q, w.dtype), to_dev(w.K, w.dtype), to_dev(w.V, w.dtype)
    qbar = torch.from_numpy(w.qbar).cuda()
    b, h_q, n, d = w.Q.shape
    T = n // w.B
    kbar = dash.alloc_kbar(b, w.h_kv, T, d)
    dash.dash_summarize(K, qbar, kbar, w.B)
    idx, bias, cnt, wo = dash.alloc_route(b, w.h_kv, n, T, with_w=with_w)
    if with_w:
        wo.zero_()
    dash.dash_route(Q, kbar, w.B, alpha, gamma, sigma, causal, idx, bias, cnt, wo, top_k=top_k)
    Oo = torch.empty((b, h_q, n, d), dtype=out_dtype, device="cuda")
    dash.dash_attend_prefill(Q, K, V, idx, bias, cnt, Oo, w.B, causal)
    torch.cuda.synchronize()
    return dict(kbar=kbar, idx=idx, bias=bias, cnt=cnt, w=wo, O=Oo, T=T)


def oracle_prefill_rows(w, rows, kbar_or=None, alpha=None, gamma=None, sigma=None, causal=None, top_k=0):
    alpha = w.alpha if alpha is None else alpha
    gamma = w.gamma if gamma is None else gamma
    sigma = w.sigma if sigma is None else sigma
    causal = w.causal if causal is None else causal
    kb = O.stage0_summaries(w.K, w.qbar, w.B) if kbar_or is None else kbar_or
    rows = np.asarray(rows)
    b = w.Q.shape[0]
    pos = np.broadcast_to(rows, (b, rows.size))
    rt = O.route(w.Q[:, :, rows], pos, kb, w.B, alpha, gamma, sigma, causal, w.n, top_k=top_k,
                 keep_heads=True)
    rt["tol_bias"] = bias_tolerance(w.Q[:, :, rows], kb, rt, alpha, gamma, sigma)
    out = O.attend(w.Q[:, :, rows], pos, w.K, w.V, rt, w.B, causal, w.n)
    return kb, rt, out


def bias_tolerance(Qr, kbar, rt, alpha, gamma, sigma):
    """Per-entry bound on |d_gpu - d_oracle| for the routed bias (Proposition 4.1,
    d_c = (ln w_c - μ)/σ), derived from the fp32 arithmetic of the router. Needs the
    oracle's per-head scores x and thresholds τ (route(..., keep_heads=True)).

    * Scores. y_c = (α-1)γ(z̄_c - max z̄) (α = 1: γ(z̄_c - max z̄)) is formed from fp32
      dot products of d terms. Their rounding error behaves like a random walk of at
      most d steps, bounded here by 8u·A with A = scale·Σ_k |q_k k̄_ck| (over 5
      standard deviations of it for d <= 128), so with the shift and the scaling
      |δy| <= ε = 16u·max A + 4u·max|y| per (head, row).
    * Threshold. τ is a weighted mean of the y it balances (∂τ/∂y_c >= 0, summing to
      1), plus the rounding of the fp32 Newton sums of at most 1023 terms: |δτ| <= ε +
      32u. Hence |δt| <= e = 2ε + 32u for t = y - τ.
    * Weights. ln w_c = ln Σ_h t_hc^p - ln g with p = 1/(α-1), so
      |δ ln w_c| <= p Σ_h t_hc^(p-1) e_h / Σ_h t_hc^p + η (softmax routing: max_h 2ε_h + η);
      η = 2^-20 (1 + p max|log2 t|) covers the power (exp2/log2 for non-integer p),
      the head sum and the fp32 log.
    * Bias. δd_c σ = δ ln w_c - mean_S δ ln w + the rounding of μ (a mean of |S|
      fp32 logs: 64u max|ln w|) and of the subtraction (2^-20 (1 + |ln w_c|)).
    Rows whose chunks sit close to the threshold (small t) get a large bound: the bias
    itself is ill-conditioned there (∂ ln w/∂t = p/t). Returns [b, h_kv, R, T]
    (zero off the support; 1e-30 everywhere when σ = inf, where d = 0 exactly)."""
    w = rt["w"]
    b, hkv, R, T = w.shape
    if np.isinf(sigma) or T == 0:
        return np.full(w.shape, 1e-30)
    Qr = np.asarray(Qr, np.float64)
    hq, d = Qr.shape[1], Qr.shape[-1]
    g = hq // hkv
    kb = np.asarray(kbar, np.float64)[:, :, :T]
    valid = np.arange(T)[None, None, :] < np.asarray(rt["vis"])[:, :, None]      # [b, R, T]
    validh = np.broadcast_to(valid[:, None], (b, hq, R, T))
    soft = alpha == 1.0
    scale = gamma * (1.0 if soft else alpha - 1.0) / np.sqrt(d)
    A = np.empty((b, hq, R, T))
    for bi in range(b):
        for h in range(hq):
            A[bi, h] = scale * (np.abs(Qr[bi, h]) @ np.abs(kb[bi, h // g]).T)
    x = rt["x"]
    xmax = np.where(validh, x, -np.inf).max(-1, keepdims=True)
    xmax = np.where(np.isfinite(xmax), xmax, 0.0)
    eps = (16 * U32 * np.where(validh, A, 0.0).max(-1)
           + 4 * U32 * np.where(validh, np.abs(x - xmax), 0.0).max(-1))              # [b, hq, R]
    if soft:
        dl = np.repeat((2 * eps).reshape(b, hkv, g, R).max(2)[..., None], T, -1) + 2.0 ** -20
    else:
        p = 1.0 / (alpha - 1.0)
        e = 2 * eps + 32 * U32
        t = np.where(validh, x - rt["tau"][..., None], 0.0)
        tp = np.where(t > 0, t, 0.0)
        with np.errstate(divide="ignore", invalid="ignore"):
            num = np.where(tp > 0, p * tp ** (p - 1.0), 0.0) * e[..., None]
            lt = np.where(tp > 0, np.abs(np.log2(np.where(tp > 0, tp, 1.0))), 0.0)
        num = num.reshape(b, hkv, g, R, T).sum(2)
        den = (tp ** p).reshape(b, hkv, g, R, T).sum(2)
        eta = 2.0 ** -20 * (1.0 + p * lt.reshape(b, hkv, g, R, T).max(2))
        with np.errstate(divide="ignore", invalid="ignore"):
            dl = np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0) + eta
    sup = rt["support"]
    cnt = np.maximum(sup.sum(-1, keepdims=True), 1)
    lnw = np.where(sup, rt["bias"] * sigma + rt["mu"][..., None], 0.0)
    mean_dl = np.where(sup, dl, 0.0).sum(-1, keepdims=True) / cnt
    mu_err = 64 * U32 * np.abs(lnw).max(-1, keepdims=True)
    tol = (dl + mean_dl + mu_err + 2.0 ** -20 * (1.0 + np.abs(lnw))) / sigma
    return np.where(sup, tol, 0.0)


def exempt_rows(rt):
    """Rows whose support the float64 oracle decides within rounding distance: a chunk
    with |x - τ| <= MARGIN, or (top-k budget) a log-weight gap <= TOPK_MARGIN at the cut."""
    return (rt["margin"] <= MARGIN) | (rt["margin_topk"] <= TOPK_MARGIN)


def check_exempt_count(n_exempt, n_rows):
    lim = MAX_EXEMPT_FRAC * n_rows + MAX_EXEMPT_ABS
    assert n_exempt <= lim, f"{n_exempt} of {n_rows} rows exempt (limit {lim:.1f})"


def compare_bias(bias_g, ref_idx, rt_bias, tol, where):
    """bias_g: the GPU's bias entries of one row's list; ref_idx its chunks (equal to
    the oracle's support); returns the largest |Δd| / tolerance."""
    diff = np.abs(bias_g.astype(np.float64) - rt_bias[ref_idx])
    lim = tol[ref_idx]
    bad = diff > lim
    assert not bad.any(), (f"{where}: bias differs by {diff[bad].max():.3e} at chunk "
                           f"{ref_idx[bad][0]} (bound {lim[bad][0]:.3e})")
    return float((diff / np.maximum(lim, 1e-30)).max()) if diff.size else 0.0


def compare_route(g, rt, rows, T):
    """Returns (n_exempt, n_rows) after asserting lists, biases, weights and the
    exempt count; logs the bias check's worst error-to-bound ratio and the median
    bound (the bound must stay informative: median <= BIAS_MEDIAN_MAX)."""
    cnt = g["cnt"][:, :, rows].cpu().numpy()
    idx = g["idx"][:, :, rows].cpu().numpy()
    exempt = exempt_rows(rt)                             # [b, h_kv, R]
    check_exempt_count(int(exempt.sum()), exempt.size)
    tolb = rt.get("tol_bias") if g.get("bias") is not None else None
    bia = g["bias"][:, :, rows].cpu().numpy() if tolb is not None else None
    if g.get("w") is not None and T > 0:
        wg = g["w"][:, :, rows, :T].cpu().numpy()
        dw = np.abs(wg - rt["w"]).max()
        assert dw <= TOL_W, f"routing weights differ by {dw}"
    b, hkv, R = cnt.shape
    worst, tols = 0.0, []
    for bi in range(b):
        for r in range(hkv):
            for k in range(R):
                if exempt[bi, r, k]:
                    continue
                ref = np.nonzero(rt["support"][bi, r, k])[0]
                c = cnt[bi, r, k]
                where = f"(b={bi}, r={r}, row={rows[k]})"
                assert c == ref.size, f"{where}: cnt {c} != {ref.size}"
                assert np.array_equal(idx[bi, r, k, :c], ref), f"{where}: lists differ"
                if tolb is not None:
                    worst = max(worst, compare_bias(bia[bi, r, k, :c], ref, rt["bias"][bi, r, k],
                                                    tolb[bi, r, k], where))
                    tols.append(tolb[bi, r, k][ref])
    if tolb is not None and tols and np.concatenate(tols).size:
        med = float(np.median(np.concatenate(tols)))
        print(f"  bias: worst |Δd|/bound {worst:.3e}, median bound {med:.2e}", flush=True)
        assert med <= BIAS_MEDIAN_MAX, f"bias bound uninformative (median {med:.2e})"
    return int(exempt.sum()), exempt.size


def compare_out(Og, Oref, exempt, g_per_kv, dtype):
    """Og, Oref [b, h_q, R, d]; exempt [b, h_kv, R]."""
    ex = np.repeat(exempt, g_per_kv, axis=1)             # per query head
    keep = ~ex
    diff = np.abs(Og - Oref)
    if dtype == "f32":
        err = diff.max(-1)[keep].max() if keep.any() else 0.0
        assert err <= TOL_F32, f"fp32 output error {err}"
        return err
    rms = np.sqrt((Oref ** 2).mean(-1))
    rel = diff.max(-1) / np.maximum(rms, 1e-30)
    err = rel[keep].max() if keep.any() else 0.0
    assert err <= TOL_BF16_ROW, f"bf16 per-row relative output error {err}"
    return err
