"""Plain float64 CPU oracle of the DashAttention forward pass.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP implementation.

Every function follows the equations of the xllm-io paper review of
"DashAttention: Differentiable and Adaptive Sparse Hierarchical Attention"
(section 三, technical architecture), written out directly in float64:

* background: SDPA (Z = QK^T/sqrt(d), P = pi(Z+M), O = PV) and the α-entmax
  transform [(α-1)s - τ]_+^{1/(α-1)} with τ the unique normaliser;
* Stage 0, Eq. 4: chunk summary by local SDPA under the learned query q̄;
* Stage 1, Eq. 6: chunk logits, γ-scaled α-entmax per query head, GQA average
  and support union within each KV group;
* Stage 2, Eq. 9 with the σ-tempered prior of Eq. 11 and the mass split of
  Eq. 12, and the equivalent additive-bias form of Proposition 4.1.

Readings taken where the page leaves a step open (each is listed in the design
notes of this repository):
* a causal query at position p routes to chunks c < floor(p/B); its diagonal
  branch D is its own chunk up to and including p (no summary exists for it);
  non-causal queries route to every complete chunk and D is the trailing
  partial chunk;
* Stage 2 uses the group weights w (unhatted in Eq. 9-12), not per-head ŵ;
* only complete chunks (T_c = floor(n/B)) get a summary;
* decode is the prefill computation for the single query at position L-1.

Parity status: pinned by tests/test_oracle.py (entmax against its variational
definition, brute-force KKT supports, sparsemax/softmax limits; Stage 0 mean
pooling and B=1; the Eq. 9 form against the Prop. 4.1 form; σ=inf against a
library masked SDPA; full support against library causal SDPA). The backward
functions (attend_backward, route_backward, summary_backward: gradients with the
support held fixed) are pinned by central finite differences of the forward
oracle, chained through all three stages, and by torch autograd of masked SDPA.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _f64(x):
    return np.asarray(x, dtype=F64)


# ----------------------------------------------------------------------------------
# α-entmax (background formula of section 三)
# ----------------------------------------------------------------------------------

def entmax_tau_bisect(x, valid=None, alpha=1.5, iters=200):
    """τ with sum_c [x_c - τ]_+^{1/(α-1)} = 1, by bisection, for every row of x.

    x is the thresholded argument (α-1)·s, shape [..., T]; `valid` masks the
    entries that take part (default: all). The root lies in
    [max x - 1, max x - |V|^{-(α-1)}]: at the left end the top term alone is 1,
    at the right end every term is at most 1/|V|.
    Rows with no valid entry get τ = nan.
    """
    x = _f64(x)
    if valid is None:
        valid = np.ones(x.shape, bool)
    if x.shape[-1] == 0:
        return np.full(x.shape[:-1], np.nan)
    p = 1.0 / (alpha - 1.0)
    cnt = valid.sum(-1)
    xm = np.where(valid, x, -np.inf)
    mx = np.where(cnt > 0, xm.max(-1), 0.0)
    y = xm - mx[..., None]                       # shift: entmax is shift-invariant
    lo = np.full(mx.shape, -1.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        hi = -np.power(np.maximum(cnt, 1).astype(F64), -(alpha - 1.0))
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        f = np.sum(np.power(np.clip(y - mid[..., None], 0.0, None), p), axis=-1)
        big = f >= 1.0
        lo = np.where(big, mid, lo)
        hi = np.where(big, hi, mid)
        if np.all(hi - lo <= 1e-16):
            break
    tau = 0.5 * (lo + hi) + mx
    return np.where(cnt > 0, tau, np.nan)


def entmax_tau_sorted(x, valid=None, alpha=1.5):
    """Exact τ for α = 2 (sparsemax) and α = 1.5, by sorting, for every row of x.

    With the values sorted in decreasing order, the support is a prefix of size k*.
    α = 2: τ_k = (sum_{j<=k} x_(j) - 1)/k and k* is the largest k with x_(k) > τ_k.
    α = 1.5: on a prefix of size k, sum_j (x_(j) - τ)^2 = 1 gives
    τ_k = M_k - sqrt((1 - SS_k)/k), with M_k the prefix mean and SS_k the prefix sum
    of squared deviations; k* is the largest k with SS_k <= 1 and x_(k) > τ_k.
    """
    if alpha not in (1.5, 2.0):
        raise ValueError("exact sorted threshold exists here only for alpha in {1.5, 2}")
    x = _f64(x)
    if valid is None:
        valid = np.ones(x.shape, bool)
    if x.shape[-1] == 0:
        return np.full(x.shape[:-1], np.nan)
    cnt = valid.sum(-1)
    xm = np.where(valid, x, -np.inf)
    mx = np.where(cnt > 0, xm.max(-1), 0.0)
    y = xm - mx[..., None]
    ys = -np.sort(-y, axis=-1)                   # decreasing; invalid (-inf) last
    T = ys.shape[-1]
    k = np.arange(1, T + 1, dtype=F64)
    inrange = k <= cnt[..., None]
    ysafe = np.where(inrange, ys, 0.0)
    c1 = np.cumsum(ysafe, -1)
    if alpha == 2.0:
        tau_k = (c1 - 1.0) / k
        ok = inrange & (ysafe > tau_k)
    else:
        mean = c1 / k
        c2 = np.cumsum(ysafe * ysafe, -1)
        ss = np.maximum(c2 - k * mean * mean, 0.0)
        delta = (1.0 - ss) / k
        tau_k = mean - np.sqrt(np.maximum(delta, 0.0))
        ok = inrange & (delta >= 0.0) & (ysafe > tau_k)
    kstar = np.where(ok, np.arange(T), -1).max(-1)          # index of the last valid k
    tau = np.take_along_axis(tau_k, np.maximum(kstar, 0)[..., None], -1)[..., 0]
    return np.where(cnt > 0, tau + mx, np.nan)


def entmax_tau(x, valid=None, alpha=1.5):
    """The oracle's τ: exact sorted form for α in {1.5, 2}, bisection otherwise."""
    if alpha in (1.5, 2.0):
        return entmax_tau_sorted(x, valid, alpha)
    return entmax_tau_bisect(x, valid, alpha)


def entmax(s, alpha=1.5, valid=None):
    """α-entmax(s) = [(α-1)s - τ]_+^{1/(α-1)} over the last axis; α = 1 is softmax.

    Returns (p, tau, x) with x = (α-1)s; invalid entries get p = 0.
    """
    s = _f64(s)
    if valid is None:
        valid = np.ones(s.shape, bool)
    if alpha == 1.0:
        z = np.where(valid, s, -np.inf)
        m = z.max(-1, keepdims=True) if z.shape[-1] else np.zeros(z.shape[:-1] + (1,))
        z = z - np.where(np.isfinite(m), m, 0.0)
        e = np.where(valid, np.exp(z), 0.0)
        tot = e.sum(-1, keepdims=True)
        return np.where(tot > 0, e / np.where(tot > 0, tot, 1.0), 0.0), None, s
    x = (alpha - 1.0) * s
    tau = entmax_tau(x, valid, alpha)
    t = np.clip(x - tau[..., None], 0.0, None)
    p = np.where(valid, np.power(t, 1.0 / (alpha - 1.0)), 0.0)
    return p, tau, x


# ----------------------------------------------------------------------------------
# Stage 0 (Eq. 4)
# ----------------------------------------------------------------------------------

def stage0_summaries(K, qbar, B):
    """k̄_c^(r) = sum_{t in C_c} softmax_t(<q̄^(r), k_t^(r)>/sqrt(d)) k_t^(r).

    K [b, h_kv, n, d], q̄ [h_kv, d] -> k̄ [b, h_kv, floor(n/B), d]; keys are also the
    values of this local attention. A trailing partial chunk gets no summary.
    """
    K = _f64(K)
    qbar = _f64(qbar)
    b, hkv, n, d = K.shape
    T = n // B
    out = np.empty((b, hkv, T, d))
    for bi in range(b):
        for r in range(hkv):
            Kc = K[bi, r, :T * B].reshape(T, B, d)
            s = (Kc @ qbar[r]) / np.sqrt(d)                  # [T, B]
            s = s - s.max(-1, keepdims=True)
            a = np.exp(s)
            a = a / a.sum(-1, keepdims=True)
            out[bi, r] = np.einsum("tj,tjd->td", a, Kc)
    return out


# ----------------------------------------------------------------------------------
# Stage 1 (Eq. 6, GQA average and union) and the Prop. 4.1 bias
# ----------------------------------------------------------------------------------

def visible_chunks(pos, B, T, causal):
    """Number of routable chunks for a query at position `pos` (chunks 0..count-1)."""
    pos = np.asarray(pos)
    if causal:
        return np.minimum(pos // B, T)
    return np.full(pos.shape, T)


def route(Qr, pos, kbar, B, alpha, gamma, sigma, causal, n_kv, keep_heads=False,
          row_block=256, top_k=0):
    """Stage 1 routing for query rows Qr [b, h_q, R, d] at token positions pos [b, R].

    For every query head h (KV group r = floor(h/g)) and row i:
      z̄_c = <q_i, k̄_c>/sqrt(d) over visible chunks, ŵ = α-entmax(γ z̄)
      (α = 1: ŵ = softmax(γ z̄), the α -> 1 limit, and every visible chunk is in
      the support; log w is then formed in log space);
    then per KV group: w = mean over the group's heads of ŵ, support S = {c: w_c > 0}
    (the union of the head supports), μ = mean_{c in S} log w_c and the
    Prop. 4.1 bias d_c = (log w_c - μ)/σ on S (σ = inf gives d = 0).

    Returns a dict of float64/bool arrays:
      w [b,h_kv,R,T], support [b,h_kv,R,T], bias [b,h_kv,R,T] (0 off support),
      mu [b,h_kv,R], vis [b,R], tau [b,h_q,R], margin [b,h_kv,R]
      (min over the group's heads and visible chunks of |x - τ|, x = (α-1)γz̄),
      margin_topk [b,h_kv,R] (top_k > 0: log-weight gap between the last kept and the
      first dropped chunk, inf where nothing is dropped),
      and when keep_heads: what [b,h_q,R,T], x [b,h_q,R,T].
    top_k > 0 keeps only the top_k largest group weights of each row's support (a
    fixed routing budget for ablations; equal weights go to the lower chunk id), and
    μ and d are taken over the kept chunks.
    """
    Qr = _f64(Qr)
    kbar = _f64(kbar)
    b, hq, R, d = Qr.shape
    hkv = kbar.shape[1]
    g = hq // hkv
    T = n_kv // B
    kb = kbar[:, :, :T]
    vis = visible_chunks(np.broadcast_to(np.asarray(pos), (b, R)), B, T, causal)
    w = np.zeros((b, hkv, R, T))
    tau = np.full((b, hq, R), np.nan)
    margin = np.full((b, hkv, R), np.inf)
    if keep_heads:
        what_all = np.zeros((b, hq, R, T))
        x_all = np.zeros((b, hq, R, T))
    valid_full = np.arange(T)[None, None, :] < vis[:, :, None]          # [b, R, T]
    logw_soft = np.zeros((b, hkv, R, T))
    for r0 in range(0, R, row_block):
        r1 = min(R, r0 + row_block)
        for bi in range(b):
            valid = valid_full[bi, r0:r1]                                 # [rows, T]
            for r in range(hkv):
                acc = np.zeros((r1 - r0, T))
                lacc = np.full((r1 - r0, T), -np.inf)     # α = 1: log Σ_h ŵ_h
                for h in range(r * g, (r + 1) * g):
                    z = (Qr[bi, h, r0:r1] @ kb[bi, r].T) / np.sqrt(d)      # [rows, T]
                    p, t, x = entmax(gamma * z, alpha, valid)
                    acc += p
                    if alpha == 1.0:
                        # softmax routing has no threshold and no support boundary
                        # (every visible chunk is routed): keep log ŵ for a stable log w
                        zz = np.where(valid, gamma * z, -np.inf)
                        m = np.max(zz, -1, keepdims=True) if T else np.zeros((r1 - r0, 1))
                        m = np.where(np.isfinite(m), m, 0.0)
                        tot = np.exp(zz - m).sum(-1, keepdims=True)
                        lse = np.log(np.where(tot > 0, tot, 1.0))
                        lp = np.where(valid, zz - m - lse, -np.inf)
                        lacc = np.logaddexp(lacc, lp)
                    else:
                        tau[bi, h, r0:r1] = t
                        with np.errstate(invalid="ignore"):
                            gap = np.where(valid, np.abs(x - t[:, None]), np.inf)
                        if T > 0:
                            margin[bi, r, r0:r1] = np.minimum(margin[bi, r, r0:r1], gap.min(-1))
                    if keep_heads:
                        what_all[bi, h, r0:r1] = p
                        x_all[bi, h, r0:r1] = np.where(valid, x, 0.0)
                w[bi, r, r0:r1] = acc / g
                if alpha == 1.0:
                    logw_soft[bi, r, r0:r1] = np.where(valid, lacc - np.log(g), 0.0)
    if alpha == 1.0:
        support = np.broadcast_to(valid_full[:, None], w.shape).copy()
        logw = np.where(support, logw_soft, 0.0)
    else:
        support = w > 0.0
        with np.errstate(divide="ignore"):
            logw = np.where(support, np.log(np.where(support, w, 1.0)), 0.0)
    margin_topk = np.full(w.shape[:-1], np.inf)
    if top_k > 0:
        # fixed budget: the top_k largest weights of each row's support, equal weights
        # to the lower chunk id; margin_topk is the log-weight gap at the cut
        for ix in np.ndindex(*w.shape[:-1]):
            cs = np.nonzero(support[ix])[0]
            if cs.size <= top_k:
                continue
            order = sorted(cs.tolist(), key=lambda c: (-logw[ix][c], c))
            keep = np.zeros(w.shape[-1], bool)
            keep[order[:top_k]] = True
            margin_topk[ix] = logw[ix][order[top_k - 1]] - logw[ix][order[top_k]]
            support[ix] = keep
            logw[ix] = np.where(keep, logw[ix], 0.0)
    cnt = support.sum(-1)
    mu = np.where(cnt > 0, logw.sum(-1) / np.maximum(cnt, 1), 0.0)
    if np.isinf(sigma):
        bias = np.zeros_like(w)
    else:
        bias = np.where(support, (logw - mu[..., None]) / sigma, 0.0)
    out = dict(w=w, support=support, bias=bias, mu=mu, vis=vis, tau=tau, margin=margin,
               cnt=cnt, margin_topk=margin_topk)
    if keep_heads:
        out["what"] = what_all
        out["x"] = x_all
    return out


def route_mask(support, words):
    """Bitpacked block mask of a routing (paper review section 三, GPU kernel table:
    M_i in {0,1}^{T_c}, 32 chunks per 32-bit word): bit c % 32 of word c // 32 is
    set iff chunk c is in the support. support [..., T] bool -> [..., words] uint32."""
    support = np.asarray(support, bool)
    T = support.shape[-1]
    out = np.zeros(support.shape[:-1] + (words,), np.uint32)
    for c in range(T):
        out[..., c // 32] |= support[..., c].astype(np.uint32) << np.uint32(c % 32)
    return out


def diagonal_range(pos, B, T, n_kv, causal):
    """Token range [lo, hi) of the diagonal branch D for a query at `pos`."""
    if causal:
        return (pos // B) * B, pos + 1
    return T * B, n_kv


# ----------------------------------------------------------------------------------
# Stage 2: Prop. 4.1 form (the form the kernels compute) and the Eq. 9 form
# ----------------------------------------------------------------------------------

def attend(Qr, pos, K, V, rt, B, causal, n_kv, row_block=64):
    """o_i = sum_{j in R_i ∪ D_i} softmax_j(z_ij + d_ij) v_j  (Prop. 4.1).

    z_ij = <q_i, k_j>/sqrt(d); d_ij = bias of chunk c(j) on routed tokens R_i
    (tokens of the chunks in the group support S_i), 0 on the diagonal branch D_i,
    and every other token is masked. Computed as a dense masked product over
    blocks of rows. Returns O [b, h_q, R, d] float64.
    """
    Qr = _f64(Qr)
    K = _f64(K)
    V = _f64(V)
    b, hq, R, d = Qr.shape
    hkv = K.shape[1]
    g = hq // hkv
    T = n_kv // B
    pos = np.broadcast_to(np.asarray(pos), (b, R))
    O = np.zeros((b, hq, R, d))
    for bi in range(b):
        for r0 in range(0, R, row_block):
            r1 = min(R, r0 + row_block)
            p = pos[bi, r0:r1]
            jmax = n_kv if not causal else int(p.max()) + 1
            tok = np.arange(jmax)
            chunk_of = tok // B
            for r in range(hkv):
                # additive bias per (row, token): routed chunks get d, D gets 0, rest -inf
                L = np.full((r1 - r0, jmax), -np.inf)
                full = chunk_of < T
                sup = rt["support"][bi, r, r0:r1][:, chunk_of[full]]
                bia = rt["bias"][bi, r, r0:r1][:, chunk_of[full]]
                L[:, full] = np.where(sup, bia, -np.inf)
                for k, pk in enumerate(p):
                    lo, hi = diagonal_range(int(pk), B, T, n_kv, causal)
                    L[k, lo:min(hi, jmax)] = 0.0
                for h in range(r * g, (r + 1) * g):
                    Z = (Qr[bi, h, r0:r1] @ K[bi, r, :jmax].T) / np.sqrt(d) + L
                    Z = Z - Z.max(-1, keepdims=True)
                    P = np.exp(Z)
                    P = P / P.sum(-1, keepdims=True)
                    O[bi, h, r0:r1] = P @ V[bi, r, :jmax]
    return O


def attend_backward(Qr, pos, K, V, rt, B, causal, n_kv, dO, row_block=64):
    """Gradients of Stage 2 (Prop. 4.1 form, the support and the bias held fixed) for
    an upstream gradient dO [b, h_q, R, d] of o_i (paper review section 三: Stage 2 is
    an ordinary softmax attention with an additive per-chunk bias, so its backward is
    the softmax-attention backward with that bias):
      P = softmax(Z), Z = QK^T/sqrt(d) + L;  dV = P^T dO;  dP = dO V^T;
      dZ = P ∘ (dP - rowsum(dP ∘ P));  dQ = dZ K/sqrt(d);  dK = dZ^T Q/sqrt(d);
      d(bias)_{i,c} = sum over the group's heads and the tokens j of chunk c of dZ_ij.
    Returns dQ [b,h_q,R,d], dK, dV [b,h_kv,n_kv,d], dbias [b,h_kv,R,T] (0 off the
    support) and lse [b,h_q,R] = log sum_j exp(Z_ij), all float64.
    """
    Qr = _f64(Qr)
    K = _f64(K)
    V = _f64(V)
    dO = _f64(dO)
    b, hq, R, d = Qr.shape
    hkv = K.shape[1]
    g = hq // hkv
    T = n_kv // B
    pos = np.broadcast_to(np.asarray(pos), (b, R))
    dQ = np.zeros((b, hq, R, d))
    dK = np.zeros((b, hkv, n_kv, d))
    dV = np.zeros((b, hkv, n_kv, d))
    dbias = np.zeros((b, hkv, R, T))
    lse = np.zeros((b, hq, R))
    sc = 1.0 / np.sqrt(d)
    for bi in range(b):
        for r0 in range(0, R, row_block):
            r1 = min(R, r0 + row_block)
            p = pos[bi, r0:r1]
            jmax = n_kv if not causal else int(p.max()) + 1
            tok = np.arange(jmax)
            chunk_of = tok // B
            for r in range(hkv):
                L = np.full((r1 - r0, jmax), -np.inf)
                full = chunk_of < T
                sup = rt["support"][bi, r, r0:r1][:, chunk_of[full]]
                bia = rt["bias"][bi, r, r0:r1][:, chunk_of[full]]
                L[:, full] = np.where(sup, bia, -np.inf)
                routed = np.zeros((r1 - r0, jmax), bool)
                routed[:, full] = sup
                for k, pk in enumerate(p):
                    lo, hi = diagonal_range(int(pk), B, T, n_kv, causal)
                    L[k, lo:min(hi, jmax)] = 0.0
                    routed[k, lo:min(hi, jmax)] = False
                for h in range(r * g, (r + 1) * g):
                    Z = (Qr[bi, h, r0:r1] @ K[bi, r, :jmax].T) * sc + L
                    m = Z.max(-1, keepdims=True)
                    E = np.exp(Z - m)
                    ssum = E.sum(-1, keepdims=True)
                    P = E / ssum
                    lse[bi, h, r0:r1] = (m + np.log(ssum))[:, 0]
                    g_o = dO[bi, h, r0:r1]
                    dV[bi, r, :jmax] += P.T @ g_o
                    dP = g_o @ V[bi, r, :jmax].T
                    dZ = P * (dP - (dP * P).sum(-1, keepdims=True))
                    dQ[bi, h, r0:r1] = (dZ @ K[bi, r, :jmax]) * sc
                    dK[bi, r, :jmax] += (dZ.T @ Qr[bi, h, r0:r1]) * sc
                    dzr = np.where(routed, dZ, 0.0)
                    for c in range(T):
                        dbias[bi, r, r0:r1, c] += dzr[:, c * B:(c + 1) * B].sum(-1) if c * B < jmax else 0.0
    dbias = np.where(rt["support"], dbias, 0.0)
    return dict(dQ=dQ, dK=dK, dV=dV, dbias=dbias, lse=lse)


def route_backward(Qr, pos, kbar, B, alpha, gamma, sigma, causal, n_kv, dbias):
    """Gradients of Stage 1 for an upstream gradient dbias [b, h_kv, R, T] of the
    Prop. 4.1 bias (paper review section 三: Eq. 6 routing, the GQA average and the
    bias of Prop. 4.1), the support S held fixed (it changes only on a set of
    measure zero):
      d_c = (log w_c - μ)/σ, μ = mean over S of log w
          -> g_c = ∂L/∂log w_c = (dbias_c - mean over S of dbias)/σ on S;
      w = (1/g) Σ_h ŵ_h                    -> ∂L/∂ŵ_h = g_c / (g w_c) on S;
      ŵ_h = α-entmax(x_h), x_h = γ z_h, whose Jacobian is diag(s) - s sᵀ/Σ s with
          s = ŵ_h^(2-α) on the head's support (α = 1, softmax: s = ŵ_h)
          -> ∂L/∂x_h = s (∂L/∂ŵ_h - Σ s ∂L/∂ŵ_h / Σ s);
      z_h = q_h k̄ᵀ/sqrt(d)                 -> dq_h = γ ∂L/∂x_h k̄/sqrt(d),
                                              dk̄ = Σ_h γ (∂L/∂x_h)ᵀ q_h/sqrt(d).
    Returns dQ [b, h_q, R, d] and dkbar [b, h_kv, T, d] (float64). A fixed top-k
    budget is not covered: its kept set drops chunks the entmax normalisation still
    couples, so the lists alone do not carry the gradient.
    """
    Qr = _f64(Qr)
    kbar = _f64(kbar)
    b, hq, R, d = Qr.shape
    hkv = kbar.shape[1]
    g = hq // hkv
    T = n_kv // B
    kb = kbar[:, :, :T]
    rt = route(Qr, pos, kbar, B, alpha, gamma, sigma, causal, n_kv, keep_heads=True)
    S = rt["support"]
    dQ = np.zeros_like(Qr)
    dkb = np.zeros((b, hkv, T, d))
    if np.isinf(sigma) or T == 0:
        return dict(dQ=dQ, dkbar=dkb)
    db = np.where(S, _f64(dbias)[..., :T], 0.0)
    cnt = S.sum(-1, keepdims=True)
    mean = db.sum(-1, keepdims=True) / np.maximum(cnt, 1)
    glogw = np.where(S, (db - mean) / sigma, 0.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        dw = np.where(S, glogw / np.where(S, rt["w"], 1.0), 0.0)       # ∂L/∂w
    sq = np.sqrt(d)
    for h in range(hq):
        r = h // g
        what = rt["what"][:, h]                                          # [b, R, T]
        dwhat = dw[:, r] / g
        if alpha == 1.0:
            s_ = what
        else:
            with np.errstate(invalid="ignore"):
                s_ = np.where(what > 0, np.power(np.where(what > 0, what, 1.0), 2.0 - alpha), 0.0)
        ssum = s_.sum(-1, keepdims=True)
        dx = s_ * (dwhat - (s_ * dwhat).sum(-1, keepdims=True) / np.where(ssum > 0, ssum, 1.0))
        dz = gamma * dx / sq
        for bi in range(b):
            dQ[bi, h] = dz[bi] @ kb[bi, r]
            dkb[bi, r] += dz[bi].T @ Qr[bi, h]
    return dict(dQ=dQ, dkbar=dkb)


def summary_backward(K, qbar, B, dkbar):
    """Gradients of Stage 0 (Eq. 4: k̄_c = Σ_j π_j k_j, π = softmax_j(<q̄, k_j>/sqrt(d))
    over the B tokens of chunk c) for dkbar [b, h_kv, T, d]:
      ∂L/∂π_j = <dk̄_c, k_j>, ∂L/∂a_j = π_j (<dk̄_c, k_j> - <dk̄_c, k̄_c>),
      dk_j = π_j dk̄_c + ∂L/∂a_j q̄/sqrt(d),  dq̄ = Σ_{c, j} ∂L/∂a_j k_j/sqrt(d)
    (summed over the batch as well). Tokens past the last complete chunk get zero.
    Returns dK [b, h_kv, n, d] and dqbar [h_kv, d] (float64).
    """
    K = _f64(K)
    qbar = _f64(qbar)
    b, hkv, n, d = K.shape
    T = n // B
    dkb = _f64(dkbar)[:, :, :T]
    dK = np.zeros_like(K)
    dq = np.zeros((hkv, d))
    sq = np.sqrt(d)
    for bi in range(b):
        for r in range(hkv):
            for c in range(T):
                Kc = K[bi, r, c * B:(c + 1) * B]
                a = Kc @ qbar[r] / sq
                pi = np.exp(a - a.max())
                pi /= pi.sum()
                kbc = pi @ Kc
                dp = Kc @ dkb[bi, r, c]
                da = pi * (dp - dkb[bi, r, c] @ kbc)
                dK[bi, r, c * B:(c + 1) * B] = pi[:, None] * dkb[bi, r, c][None, :] + da[:, None] * qbar[r][None, :] / sq
                dq[r] += da @ Kc / sq
    return dict(dK=dK, dqbar=dq)


def attend_eq9(Qr, pos, K, V, rt, B, sigma, causal, n_kv):
    """Stage 2 through the prior of Eq. 9 with Eq. 11 and Eq. 12, row by row.

    g_ij = λ_i w'_ij on routed tokens R_i and (1-λ_i)/|D_i| on D_i, with the
    σ-tempered prior w'_ij = (1/B) w_{c(j)}^{1/σ} / sum_c w_c^{1/σ} and
    λ_i = sigmoid(KL(u_R || w'_R) + log(|R_i|/|D_i|)); then
    p_ij = g_ij exp(z_ij) / sum_t g_it exp(z_it) and o_i = sum_j p_ij v_j.
    Used to pin the bias form; slow, meant for a handful of rows.
    """
    Qr = _f64(Qr)
    K = _f64(K)
    V = _f64(V)
    b, hq, R, d = Qr.shape
    hkv = K.shape[1]
    g = hq // hkv
    T = n_kv // B
    pos = np.broadcast_to(np.asarray(pos), (b, R))
    O = np.zeros((b, hq, R, d))
    for bi in range(b):
        for i in range(R):
            pk = int(pos[bi, i])
            lo, hi = diagonal_range(pk, B, T, n_kv, causal)
            D = np.arange(lo, hi)
            for r in range(hkv):
                w = rt["w"][bi, r, i]
                S = np.nonzero(rt["support"][bi, r, i])[0]
                Rtok = (S[:, None] * B + np.arange(B)[None, :]).reshape(-1)
                if S.size:
                    if np.isinf(sigma):
                        wt = np.where(w > 0, 1.0, 0.0)
                    else:
                        wt = np.where(w > 0, np.power(np.where(w > 0, w, 1.0), 1.0 / sigma), 0.0)
                    wprime = (1.0 / B) * wt[Rtok // B] / wt.sum()
                    kl = -np.log(Rtok.size) - np.mean(np.log(wprime))
                    if D.size:
                        lam = 1.0 / (1.0 + np.exp(-(kl + np.log(Rtok.size / D.size))))
                    else:
                        lam = 1.0
                else:
                    wprime = np.zeros(0)
                    lam = 0.0
                toks = np.concatenate([Rtok, D])
                prior = np.concatenate([lam * wprime,
                                        np.full(D.size, (1.0 - lam) / max(D.size, 1))])
                for h in range(r * g, (r + 1) * g):
                    z = (K[bi, r, toks] @ Qr[bi, h, i]) / np.sqrt(d)
                    z = z - z.max()
                    e = prior * np.exp(z)
                    O[bi, h, i] = (e / e.sum()) @ V[bi, r, toks]
    return O


# ----------------------------------------------------------------------------------
# Whole forward passes
# ----------------------------------------------------------------------------------

def prefill(Q, K, V, qbar, B, alpha, gamma, sigma, causal=True, rows=None, keep_heads=False):
    """Stages 0-2 for a prefill of n tokens (query row i sits at position i).

    `rows` selects the query rows to evaluate (default: all). Returns a dict with
    kbar, the route dict and O [b, h_q, len(rows), d].
    """
    Q = _f64(Q)
    b, hq, n, d = Q.shape
    rows = np.arange(n) if rows is None else np.asarray(rows)
    kbar = stage0_summaries(K, qbar, B)
    Qr = Q[:, :, rows]
    pos = np.broadcast_to(rows, (b, rows.size))
    rt = route(Qr, pos, kbar, B, alpha, gamma, sigma, causal, n, keep_heads=keep_heads)
    O = attend(Qr, pos, K, V, rt, B, causal, n)
    return dict(kbar=kbar, route=rt, O=O, rows=rows)


def decode(Q, K, V, kbar, seq_len, B, alpha, gamma, sigma, keep_heads=False, top_k=0):
    """One decode step: the query Q[b, h_q, 0] sits at position seq_len[b]-1 and sees
    KV tokens [0, seq_len[b]). Routing uses the cached summaries kbar (top_k > 0: the
    fixed routing budget of route()). Returns dict(route=..., O [b, h_q, 1, d]).
    """
    Q = _f64(Q)
    b = Q.shape[0]
    seq_len = np.asarray(seq_len)
    outs, rts = [], []
    for bi in range(b):
        L = int(seq_len[bi])
        pos = np.array([[L - 1]])
        rt = route(Q[bi:bi + 1], pos, kbar[bi:bi + 1, :, :L // B], B, alpha, gamma, sigma,
                   True, L, keep_heads=keep_heads, top_k=top_k)
        O = attend(Q[bi:bi + 1], pos, K[bi:bi + 1, :, :L], V[bi:bi + 1, :, :L], rt, B, True, L)
        outs.append(O)
        rts.append(rt)
    return dict(O=np.concatenate(outs, 0), routes=rts)


def group_sparsity(rt):
    """1 - sum|S| / sum|V| over (b, r, row) with at least one visible chunk."""
    vis = rt["vis"]                                        # [b, R]
    hkv = rt["w"].shape[1]
    visr = np.broadcast_to(vis[:, None, :], (vis.shape[0], hkv, vis.shape[1]))
    m = visr >= 1
    return 1.0 - rt["cnt"][m].sum() / visr[m].sum()
