"""Helpers of the GPU parity tests: run the HIP path through the C ABI and compare
with the oracle under the stated tolerances.

Tolerances (the method's own readings):
  * chunk summaries k̄: max |Δ| <= 1e-4;
  * group routing weights w: max |Δ| <= 1e-3 on every row;
  * routed chunk lists: identical on every row that is not exempt; a (b, r, row) is
    exempt when some head of its group has a visible chunk whose thresholded score
    x = (α-1)γz̄ lies within 1e-6 of that head's τ (oracle, float64);
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
    rt = O.route(w.Q[:, :, rows], pos, kb, w.B, alpha, gamma, sigma, causal, w.n, top_k=top_k)
    out = O.attend(w.Q[:, :, rows], pos, w.K, w.V, rt, w.B, causal, w.n)
    return kb, rt, out


def exempt_rows(rt):
    """Rows whose support the float64 oracle decides within rounding distance: a chunk
    with |x - τ| <= MARGIN, or (top-k budget) a log-weight gap <= TOPK_MARGIN at the cut."""
    return (rt["margin"] <= MARGIN) | (rt["margin_topk"] <= TOPK_MARGIN)


def compare_route(g, rt, rows, T):
    """Returns (n_exempt, n_rows) after asserting lists and weights."""
    cnt = g["cnt"][:, :, rows].cpu().numpy()
    idx = g["idx"][:, :, rows].cpu().numpy()
    exempt = exempt_rows(rt)                             # [b, h_kv, R]
    if g.get("w") is not None and T > 0:
        wg = g["w"][:, :, rows, :T].cpu().numpy()
        dw = np.abs(wg - rt["w"]).max()
        assert dw <= TOL_W, f"routing weights differ by {dw}"
    b, hkv, R = cnt.shape
    for bi in range(b):
        for r in range(hkv):
            for k in range(R):
                if exempt[bi, r, k]:
                    continue
                ref = np.nonzero(rt["support"][bi, r, k])[0]
                c = cnt[bi, r, k]
                assert c == ref.size, f"(b={bi}, r={r}, row={rows[k]}): cnt {c} != {ref.size}"
                assert np.array_equal(idx[bi, r, k, :c], ref), f"(b={bi}, r={r}, row={rows[k]}): lists differ"
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
