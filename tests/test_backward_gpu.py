"""GPU parity of the Stage-2 backward (dash_attend_prefill_lse and
dash_attend_prefill_backward through the C ABI) against the oracle's attend_backward.

The routed lists come from the oracle's routing of the same inputs, so the check
isolates Stage 2: the GPU runs its forward (for O and lse) and its backward on those
lists, the oracle differentiates the same fixed-support attention in float64.

Tolerances (bf16 Q, K, V are exact; u = 2^-8 is the unit roundoff of bf16):
  * lse: max |Δ| <= 4e-3 (the forward's denominator sums bf16-rounded P);
  * dQ, dK, dV and the routed entries of dbias, each as a whole: relative L2 error
    ||Δ|| / ||ref|| <= u (independent rounding errors add in quadrature; observed
    near 0.5u);
  * every element within its first-order rounding bound (stage2_bounds): the MFMA
    operands P and dZ are rounded to bf16 (relative error <= u each, 2u allowed for
    a rounding before and after the product with P), P also carries the forward's
    lse error, dO its bf16 rounding when it comes in fp32, and Δ = <o, do> the
    rounding of O (the forward sums bf16-rounded P; O's own bf16 rounding when O is
    bf16). With E_ij the resulting bound on the error of dZ_ij,
      |ΔdQ_i| <= Σ_j E_ij |k_j| / sqrt(d),  |ΔdK_j| <= Σ_i E_ij |q_i| / sqrt(d),
      |ΔdV_j| <= Σ_i P_ij |do_i| (2u + δlse_i),  |Δdbias_ic| <= Σ_{j in c} E_ij,
    plus 2^-16 of the sum of the magnitudes of the terms for the fp32 accumulation;
  * list entries at or past cnt are exactly zero.
"""
import numpy as np
import pytest
import torch

from long_context_amd import inputs

pytestmark = pytest.mark.gpu

TOL_LSE = 4e-3
TOL_L2 = 2.0 ** -8
UB = 2.0 ** -8                 # unit roundoff of bf16
ACC = 2.0 ** -16               # fp32 accumulation of up to ~10^5 terms (random walk, wide margin)


@pytest.fixture(autouse=True)
def _need_gpu(gpu_lib):
    yield


def _log(msg):
    print(msg, flush=True)


def _gu():
    from tests import gpu_util
    return gpu_util


def lists_from_support(support, bias_dense, cap):
    b, hkv, n, T = support.shape
    idx = np.zeros((b, hkv, n, cap), np.int32)
    bias = np.zeros((b, hkv, n, cap), np.float32)
    cnt = np.zeros((b, hkv, n), np.int32)
    for bi in range(b):
        for r in range(hkv):
            for i in range(n):
                c = np.nonzero(support[bi, r, i])[0]
                idx[bi, r, i, :c.size] = c
                bias[bi, r, i, :c.size] = bias_dense[bi, r, i, c]
                cnt[bi, r, i] = c.size
    return idx, bias, cnt


def run_backward(w, causal, gamma, odt, seed=7, alpha=1.5, sigma=1.0):
    from long_context_amd import dash
    from oracle import dash_oracle as O
    b, hq, n, d = w.Q.shape
    hkv, B = w.h_kv, w.B
    T = n // B
    cap = max(T, 1)
    pos = np.broadcast_to(np.arange(n), (b, n))
    kb = O.stage0_summaries(w.K, w.qbar, B)
    rt = O.route(w.Q, pos, kb, B, alpha, gamma, sigma, causal, n)
    bias32 = rt["bias"].astype(np.float32)
    idx, bias, cnt = lists_from_support(rt["support"], bias32, cap)
    rt = dict(rt, bias=bias32.astype(np.float64))
    dO = inputs.upstream_grad((b, hq, n, d), seed=seed, dtype=odt)
    tdt = torch.bfloat16 if odt == "bf16" else torch.float32
    dev = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)
    Qd, Kd, Vd = (dev(x, torch.bfloat16) for x in (w.Q, w.K, w.V))
    ti, tb, tc = dev(idx, torch.int32), dev(bias, torch.float32), dev(cnt, torch.int32)
    Og = torch.empty((b, hq, n, d), dtype=tdt, device="cuda")
    lse = torch.full((b, hq, n), float("nan"), device="cuda")
    dash.dash_attend_prefill_lse(Qd, Kd, Vd, ti, tb, tc, Og, lse, B, causal)
    dQ = torch.full((b, hq, n, d), float("nan"), device="cuda")
    dK = torch.full((b, hkv, n, d), float("nan"), device="cuda")
    dV = torch.full((b, hkv, n, d), float("nan"), device="cuda")
    db = torch.full((b, hkv, n, cap), float("nan"), device="cuda")
    dash.dash_attend_prefill_backward(Qd, Kd, Vd, ti, tb, tc, Og, dev(dO, tdt), lse, dQ, dK, dV, db, B, causal)
    torch.cuda.synchronize()
    ref = O.attend_backward(w.Q, pos, w.K, w.V, rt, B, causal, n, dO.astype(np.float64))
    got = dict(lse=lse.cpu().numpy(), dQ=dQ.cpu().numpy(), dK=dK.cpu().numpy(), dV=dV.cpu().numpy(),
               dbias=db.cpu().numpy())
    bnd = stage2_bounds(w.Q, pos, w.K, w.V, rt, B, causal, n, dO, np.abs(got["lse"] - ref["lse"]),
                        o_bf16=odt == "bf16", do_f32=odt == "f32")
    return got, ref, idx, cnt, bnd


def stage2_bounds(Qr, pos, K, V, rt, B, causal, n_kv, dO, dlse, o_bf16, do_f32):
    """First-order bounds on the GPU's rounding errors of dQ, dK, dV, dbias (see the
    module docstring), from the float64 P and dZ of the same fixed-support attention.
    dlse [b, h_q, R] is the GPU's measured lse error. Returns dict of arrays shaped
    like the oracle's gradients."""
    from oracle import dash_oracle as O
    Qr = np.asarray(Qr, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    dO = np.asarray(dO, np.float64)
    b, hq, R, d = Qr.shape
    hkv = K.shape[1]
    g = hq // hkv
    T = n_kv // B
    sc = 1.0 / np.sqrt(d)
    pos = np.broadcast_to(np.asarray(pos), (b, R))
    out = dict(dQ=np.zeros((b, hq, R, d)), dK=np.zeros((b, hkv, n_kv, d)), dV=np.zeros((b, hkv, n_kv, d)),
               dbias=np.zeros((b, hkv, R, T)))
    for bi in range(b):
        for r0 in range(0, R, 64):
            r1 = min(R, r0 + 64)
            p = pos[bi, r0:r1]
            jmax = n_kv if not causal else int(p.max()) + 1
            chunk_of = np.arange(jmax) // B
            full = chunk_of < T
            for r in range(hkv):
                L = np.full((r1 - r0, jmax), -np.inf)
                L[:, full] = np.where(rt["support"][bi, r, r0:r1][:, chunk_of[full]],
                                      rt["bias"][bi, r, r0:r1][:, chunk_of[full]], -np.inf)
                routed = np.zeros((r1 - r0, jmax), bool)
                routed[:, full] = rt["support"][bi, r, r0:r1][:, chunk_of[full]]
                for k, pk in enumerate(p):
                    lo, hi = O.diagonal_range(int(pk), B, T, n_kv, causal)
                    L[k, lo:min(hi, jmax)] = 0.0
                    routed[k, lo:min(hi, jmax)] = False
                Kb, Vb = K[bi, r, :jmax], V[bi, r, :jmax]
                aK, aV = np.abs(Kb), np.abs(Vb)
                for h in range(r * g, (r + 1) * g):
                    q = Qr[bi, h, r0:r1]
                    Z = q @ Kb.T * sc + L
                    P = np.exp(Z - Z.max(-1, keepdims=True))
                    P /= P.sum(-1, keepdims=True)
                    do = dO[bi, h, r0:r1]
                    o = P @ Vb
                    dP = do @ Vb.T
                    dZ = P * (dP - (do * o).sum(-1, keepdims=True))
                    dl = dlse[bi, h, r0:r1][:, None]
                    # error of Δ = <o, do>: the forward's rounded P (and O's own rounding)
                    dDel = UB * (np.abs(do) * (P @ aV)).sum(-1, keepdims=True)
                    if o_bf16:
                        dDel += UB * (np.abs(o) * np.abs(do)).sum(-1, keepdims=True)
                    E = (2 * UB + dl) * np.abs(dZ) + P * dDel
                    if do_f32:                      # dO rounded to bf16 before dP
                        E += P * UB * (np.abs(do) @ aV.T)
                    aq = np.abs(q)
                    out["dQ"][bi, h, r0:r1] = sc * (E @ aK + ACC * (np.abs(dZ) @ aK))
                    out["dK"][bi, r, :jmax] += sc * (E.T @ aq + ACC * (np.abs(dZ).T @ aq))
                    dv_u = 2 * UB + (UB if do_f32 else 0.0)
                    out["dV"][bi, r, :jmax] += (P * (dv_u + dl)).T @ np.abs(do) + ACC * (P.T @ np.abs(do))
                    Er = np.where(routed, E + ACC * np.abs(dZ), 0.0)
                    for c in range(min(T, (jmax + B - 1) // B)):
                        out["dbias"][bi, r, r0:r1, c] += Er[:, c * B:(c + 1) * B].sum(-1)
    return out


def check_grads(got, ref, idx, cnt, bnd, tag=""):
    dl = np.abs(got["lse"] - ref["lse"]).max()
    ratio, l2 = {}, {}
    for name in ("dQ", "dK", "dV"):
        g, r, bd = got[name], ref[name], bnd[name]
        assert np.isfinite(g).all(), f"{name}: non-finite values"
        e = np.abs(g - r)
        ratio[name] = (e / np.maximum(bd, 1e-30)).max()
        if ratio[name] > 1:
            _log(f"{name}: worst element at {np.unravel_index((e / np.maximum(bd, 1e-30)).argmax(), e.shape)}")
        l2[name] = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    # dbias: the oracle's dense [.., T] gradient and bound gathered at the list positions
    e = np.arange(idx.shape[-1])
    live = e[None, None, None, :] < cnt[..., None]
    if ref["dbias"].shape[-1]:
        li = np.where(live, idx, 0).astype(np.int64)
        rd = np.take_along_axis(ref["dbias"], li, axis=-1)
        bd = np.take_along_axis(bnd["dbias"], li, axis=-1)
    else:
        rd = bd = np.zeros(idx.shape)
    rd = np.where(live, rd, 0.0)
    gd = got["dbias"]
    assert np.all(gd[~live] == 0.0), "dbias past cnt must be zero"
    if live.any():
        ratio["dbias"] = (np.abs(gd - rd)[live] / np.maximum(bd[live], 1e-30)).max()
        l2["dbias"] = np.linalg.norm((gd - rd)[live]) / max(np.linalg.norm(rd[live]), 1e-30)
    _log(f"{tag} lse={dl:.2e} " + " ".join(f"{k}: err/bound {ratio[k]:.2e} l2 {l2[k]:.2e}" for k in ratio))
    assert dl <= TOL_LSE, f"lse differs by {dl}"
    for name in ratio:
        assert ratio[name] <= 1.0, f"{name}: an element exceeds its rounding bound ({ratio[name]:.2f}x)"
        assert l2[name] <= TOL_L2, f"{name}: relative L2 error {l2[name]}"


BWD = [
    # b, h_q, h_kv, d, n, B, causal, gamma, O/dO dtype
    (1, 16, 2, 128, 300, 64, True, 6.0, "f32"),      # GQA 8, ragged tail
    (2, 32, 2, 64, 520, 64, False, 6.0, "f32"),      # GQA 16, d 64, non-causal tail
    (1, 16, 2, 128, 400, 128, True, 4.0, "bf16"),    # B 128: two token tiles per chunk
    (1, 32, 2, 128, 1100, 64, False, 8.0, "f32"),    # tail seen by every row: three segments
    (1, 16, 2, 128, 2048, 64, True, 3.0, "f32"),     # many chunks, dense early routing
    (1, 4, 4, 64, 300, 64, True, 6.0, "f32"),        # g = 1 (one head per list)
    (2, 8, 2, 128, 333, 64, True, 5.0, "bf16"),      # g = 4
    (1, 16, 2, 128, 300, 32, True, 6.0, "f32"),      # B 32: 32-token dQ tiles, half-used dK/dV tiles
    (2, 8, 2, 64, 250, 32, False, 5.0, "bf16"),      # B 32, d 64, non-causal tail of 26 tokens
    (1, 2, 2, 64, 200, 32, True, 4.0, "f32"),        # B 32, g = 1 (query tiles of 32 rows)
    (1, 32, 2, 128, 260, 32, True, 6.0, "bf16"),     # B 32, GQA 16 (query tiles of 8 rows)
]


@pytest.mark.parametrize("case", BWD, ids=[f"g{c[1] // c[2]}-d{c[3]}-n{c[4]}-B{c[5]}-c{int(c[6])}-{c[8]}" for c in BWD])
def test_backward_matches_oracle(case):
    b, hq, hkv, d, n, B, causal, gamma, odt = case
    _log(f"backward case {case}")
    w = inputs.make_prefill(b=b, h_q=hq, h_kv=hkv, d=d, n=n, B=B, dtype="bf16", gamma=gamma, seed=3)
    got, ref, idx, cnt, bnd = run_backward(w, causal, gamma, odt)
    check_grads(got, ref, idx, cnt, bnd, tag=str(case))


def test_backward_short_sequence_no_full_chunk():
    """n < B: no routed chunk at all, only the diagonal (causal) branch."""
    w = inputs.make_prefill(b=1, h_q=8, h_kv=1, d=64, n=50, B=64, dtype="bf16", seed=4)
    got, ref, idx, cnt, bnd = run_backward(w, True, 1.0, "f32")
    check_grads(got, ref, idx, cnt, bnd, tag="n50")


def test_backward_32k_clusters_full_size():
    """The 32K GQA-16 clustered workload at full size (α = 1.5, the benchmark's
    launch). Rows of the last two chunks and a sample of other rows take the oracle's
    routed lists (the rest keep the GPU router's); the oracle then fixes lse, dQ and
    dbias of those rows, and dK, dV of the last two chunks' tokens exactly (only rows
    in those chunks can see them). Over the whole tensors, sum_j dV_j equals the sum
    of dO over the group's rows and heads, since every row's P sums to one."""
    from long_context_amd import dash
    from oracle import dash_oracle as O
    w = inputs.prefill_32k_clusters(alphas=(1.5,))
    b, hq, n, d = w.Q.shape
    hkv, B, g = w.h_kv, w.B, hq // w.h_kv
    T = n // B
    rng = np.random.default_rng(21)
    rows = np.unique(np.concatenate([rng.choice(n - 2 * B, size=24, replace=False), np.arange(n - 2 * B, n),
                                     [0, 1, B, 2 * B - 1, n // 2]]))
    _log(f"32k backward: {rows.size} oracle rows")
    dev = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)
    Qd, Kd, Vd = (dev(x, torch.bfloat16) for x in (w.Q, w.K, w.V))
    kbar = dash.alloc_kbar(b, hkv, T, d)
    dash.dash_summarize(Kd, torch.from_numpy(w.qbar).cuda(), kbar, B)
    idx, bias, cnt, _ = dash.alloc_route(b, hkv, n, T, with_w=False)
    dash.dash_route(Qd, kbar, B, 1.5, w.gamma, w.sigma, True, idx, bias, cnt)
    pos = np.broadcast_to(rows, (b, rows.size))
    kb = O.stage0_summaries(w.K, w.qbar, B)
    rt = O.route(w.Q[:, :, rows], pos, kb, B, 1.5, w.gamma, w.sigma, True, n)
    bias32 = rt["bias"].astype(np.float32)
    li, lb, lc = lists_from_support(rt["support"], bias32, T)
    ri = torch.from_numpy(rows).cuda()
    idx[:, :, ri] = dev(li, torch.int32)
    bias[:, :, ri] = dev(lb, torch.float32)
    cnt[:, :, ri] = dev(lc, torch.int32)
    rt = dict(rt, bias=bias32.astype(np.float64))
    dO = inputs.upstream_grad((b, hq, n, d), seed=22, dtype="bf16")
    dOd = dev(dO, torch.bfloat16)
    # fp32 O: Δ = <o_i, do_i> then carries no bf16 rounding of O, which would add up
    # to 2^-9 sum_d |o_d do_d| to Δ and dominate rows whose gradient cancels (row 1)
    Og = torch.empty((b, hq, n, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((b, hq, n), device="cuda")
    dash.dash_attend_prefill_lse(Qd, Kd, Vd, idx, bias, cnt, Og, lse, B, True)
    dQ = torch.empty((b, hq, n, d), device="cuda")
    dK = torch.empty((b, hkv, n, d), device="cuda")
    dV = torch.empty((b, hkv, n, d), device="cuda")
    db = torch.empty((b, hkv, n, T), device="cuda")
    dash.dash_attend_prefill_backward(Qd, Kd, Vd, idx, bias, cnt, Og, dOd.float(), lse, dQ, dK, dV, db, B, True)
    torch.cuda.synchronize()
    # Σ_j dV_j = Σ_{h in group, i} dO_{h,i}; each row's P sums to one within its rounding
    sv = dV.double().sum(2)
    so = dOd.double().reshape(b, hkv, g, n, d).sum((2, 3))
    bound = 2.0 ** -8 * dOd.double().abs().reshape(b, hkv, g, n, d).sum((2, 3))
    assert torch.all((sv - so).abs() <= bound), float(((sv - so).abs() / bound).max())
    ref = O.attend_backward(w.Q[:, :, rows], pos, w.K, w.V, rt, B, True, n, dO[:, :, rows].astype(np.float64))
    tail = slice(n - 2 * B, n)
    got = dict(lse=lse[:, :, ri].cpu().numpy(), dQ=dQ[:, :, ri].cpu().numpy(),
               dK=dK[:, :, tail].cpu().numpy(), dV=dV[:, :, tail].cpu().numpy(), dbias=db[:, :, ri].cpu().numpy())
    dlse = np.abs(got["lse"] - ref["lse"])
    bnd = stage2_bounds(w.Q[:, :, rows], pos, w.K, w.V, rt, B, True, n, dO[:, :, rows], dlse,
                        o_bf16=False, do_f32=False)
    ref = dict(ref, dK=ref["dK"][:, :, tail], dV=ref["dV"][:, :, tail])
    bnd = dict(bnd, dK=bnd["dK"][:, :, tail], dV=bnd["dV"][:, :, tail])
    check_grads(got, ref, li, lc, bnd, tag="32k")


# ------------------------------------------------------------------------------------
# Stage 1 and Stage 0 backward, and the whole chain
# ------------------------------------------------------------------------------------
# fp32 arithmetic on exact inputs: relative L2 <= 1e-4 and per row
# max |Δ| <= 1e-3 (rms of the row + rms of the tensor) (fp32 sums of ~10^2 terms sit
# near 1e-6 relative; the threshold ŵ = t^(1/(α-1)) amplifies the error of a small t,
# but only on weights near zero).
TOL_F32_L2 = 1e-4
TOL_F32_ROW = 1e-3


def _rel(g, r, tol_l2, tol_row, name):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    assert np.isfinite(g).all(), f"{name}: non-finite"
    l2 = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    rms_all = np.sqrt((r ** 2).mean())
    rms_row = np.sqrt((r ** 2).mean(-1))
    row = (np.abs(g - r).max(-1) / (rms_all + rms_row + 1e-30)).max()
    _log(f"  {name}: l2 {l2:.2e} row {row:.2e}")
    assert l2 <= tol_l2, f"{name}: relative L2 error {l2}"
    assert row <= tol_row, f"{name}: per-row error {row}"


@pytest.mark.parametrize("dtype,d,B,n", [("f32", 64, 16, 200), ("bf16", 128, 64, 520), ("bf16", 64, 32, 96)])
def test_summary_backward_matches_oracle(dtype, d, B, n):
    from long_context_amd import dash
    from oracle import dash_oracle as O
    w = inputs.make_prefill(b=2, h_q=2, h_kv=2, d=d, n=n, B=B, dtype=dtype, seed=8)
    T = n // B
    dkb = inputs.upstream_grad((2, 2, T + 2, d), seed=9)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    K = torch.from_numpy(w.K).to("cuda", tdt)
    dK = torch.zeros((2, 2, n, d), device="cuda")
    dq = torch.zeros((2, d), device="cuda")
    dash.dash_summarize_backward(K, torch.from_numpy(w.qbar).cuda(), torch.from_numpy(dkb).cuda(), B, dK, dq)
    torch.cuda.synchronize()
    ref = O.summary_backward(w.K, w.qbar, B, dkb[:, :, :T])
    _log(f"summary backward {dtype} d={d} B={B} n={n}")
    _rel(dK.cpu().numpy(), ref["dK"], TOL_F32_L2, TOL_F32_ROW, "dK")
    _rel(dq.cpu().numpy(), ref["dqbar"], TOL_F32_L2, TOL_F32_ROW, "dqbar")
    assert np.all(dK[:, :, T * B:].cpu().numpy() == 0)      # the partial chunk has no summary


ROUTE_BWD = [
    # dtype, b, h_q, h_kv, d, n, B, alpha, gamma, sigma, causal, seed
    ("f32", 1, 1, 1, 64, 512, 32, 1.5, 6.0, 1.0, True, 10),
    ("bf16", 2, 16, 2, 128, 600, 64, 1.5, 8.0, 1.0, True, 10),       # GQA 8
    ("bf16", 1, 32, 2, 128, 384, 64, 2.0, 4.0, 0.5, True, 11),       # GQA 16, sparsemax
    ("bf16", 1, 8, 2, 64, 400, 32, 1.0, 2.0, 1.0, True, 10),         # softmax routing
    ("f32", 1, 8, 2, 64, 448, 32, 1.25, 6.0, 2.0, False, 10),        # non-causal
    ("bf16", 1, 16, 2, 128, 5200, 16, 1.5, 6.0, 1.0, True, 10),      # 325 chunks: dk̄ in two column slices
    ("f32", 1, 2, 1, 64, 9728, 16, 1.5, 4.0, 1.0, True, 10),         # 608 chunks, d 64: two slices
]

# The routing gradient is ill-conditioned near the edge of a head's support: with
# t = x - τ > 0 the weight is ŵ = t^(1/(α-1)) and ∂ log ŵ/∂x = 1/((α-1) t), so a row
# whose routed chunks sit just above the threshold turns the fp32 rounding of x and τ
# into a large relative error of its gradient. A row's conditioning is measured as
# PERTURB_FACTOR times the largest change of its float64 gradient under three random
# relative perturbations of k̄ by 2^-23 (one fp32 unit), relative to the row's rms
# plus the tensor's; the kernel's x comes from fp32 dot products of at most 128 terms
# and its τ from an fp32 threshold search, together well under 2^6 such units. Each
# row (and each tensor's L2 norm) is held to its conditioning clipped to
# [TOL_COND_MIN, TOL_COND_MAX]: well-conditioned rows, most of them, to 1e-3 relative.
# Rows whose conditioning exceeds TOL_COND_MAX are exempt, as rows within the
# forward's margin are: they take a zero upstream gradient on both sides (so they
# add nothing to dk̄), and their count is bounded by MAX_ILL_FRAC of the rows plus 2
# (the share grows with the number of chunks a row sees near its threshold: about 6%
# of the rows at 325 chunks, 3% at 608 with one head per group, 16% of a 22-row
# sample at 1300 chunks).
PERTURB_FACTOR = 64.0
TOL_COND_MIN = 1e-3
TOL_COND_MAX = 1e-2
MAX_ILL_FRAC = 0.20


def _spread(fn, kb, reps=3):
    ref = fn(kb)
    rng = np.random.default_rng(1234)
    out = {k: (np.zeros(v.shape[:-1]), 0.0) for k, v in ref.items()}
    for _ in range(reps):
        pr = fn(kb * (1.0 + 2.0 ** -23 * rng.standard_normal(kb.shape)))
        for k, v in ref.items():
            row, l2 = out[k]
            out[k] = (np.maximum(row, np.abs(pr[k] - v).max(-1)), max(l2, np.linalg.norm(pr[k] - v)))
    return ref, out


def ill_conditioned_rows(fn, kb, g):
    """[b, h_kv, R] rows of the routing backward whose dQ conditioning (see above)
    exceeds TOL_COND_MAX (fn: dbias-fixed oracle routing backward as a function of k̄)."""
    ref, sp = _spread(fn, kb)
    r = ref["dQ"]
    rms_all = np.sqrt((r ** 2).mean())
    rms_row = np.sqrt((r ** 2).mean(-1))
    bad = PERTURB_FACTOR * sp["dQ"][0] > TOL_COND_MAX * (rms_row + rms_all)    # [b, h_q, R]
    b, hq, R = bad.shape
    return bad.reshape(b, hq // g, g, R).any(2)


def _check_tiered(g, r, spread, name):
    """Every row within its conditioning clipped to [TOL_COND_MIN, TOL_COND_MAX] of
    (rms of the row + rms of the tensor), the tensor's L2 within its own clipped
    conditioning; logs the share of rows held to TOL_COND_MIN."""
    g = np.asarray(g, np.float64)
    assert np.isfinite(g).all(), f"{name}: non-finite"
    row_sp, l2_sp = spread
    rms_all = np.sqrt((r ** 2).mean())
    scale = np.sqrt((r ** 2).mean(-1)) + rms_all + 1e-300
    tol = np.clip(PERTURB_FACTOR * row_sp / scale, TOL_COND_MIN, TOL_COND_MAX)
    err = np.abs(g - r).max(-1) / scale
    nr = max(np.linalg.norm(r), 1e-300)
    l2 = np.linalg.norm(g - r) / nr
    l2_tol = float(np.clip(PERTURB_FACTOR * l2_sp / nr, TOL_COND_MIN, TOL_COND_MAX))
    k = np.unravel_index(np.argmax(err / tol), err.shape)
    _log(f"  {name}: worst row {k} err {err[k]:.2e} bound {tol[k]:.2e}; rows at the 1e-3 bound "
         f"{(tol <= TOL_COND_MIN).mean():.3f}; l2 {l2:.2e} bound {l2_tol:.2e}")
    assert err[k] <= tol[k], f"{name}: row {k} error {err[k]:.3e} above {tol[k]:.3e}"
    assert l2 <= l2_tol, f"{name}: relative L2 error {l2:.3e} above {l2_tol:.3e}"


def check_tau(stats, Qr, kb, rt, alpha, gamma, rows_ok):
    """The router's threshold (dash_route_stats, in the shifted domain y = x - max x)
    against the oracle's τ on the rows checked: |Δτ| <= ε + 32u with ε the score
    error bound of the forward's bias check (the threshold is a weighted mean of the
    scores it balances, plus the rounding of the fp32 Newton sums)."""
    from tests.gpu_util import U32
    x, tau = rt["x"], rt["tau"]                                   # [b, h_q, R, T], [b, h_q, R]
    b, hq, R, T = x.shape
    valid = np.arange(T)[None, None, :] < np.asarray(rt["vis"])[:, :, None]
    validh = np.broadcast_to(valid[:, None], x.shape)
    xmax = np.where(validh, x, -np.inf).max(-1)
    ok = np.isfinite(xmax) & np.repeat(rows_ok, hq // rt["w"].shape[1], axis=1)
    if alpha == 1.0 or not ok.any():
        return
    hkv = kb.shape[1]
    g = hq // hkv
    scale = gamma * (alpha - 1.0) / np.sqrt(Qr.shape[-1])
    A = np.stack([scale * (np.abs(Qr[:, h]) @ np.abs(kb[:, h // g, :T]).transpose(0, 2, 1)) for h in range(hq)], 1)
    eps = 16 * U32 * np.where(validh, A, 0).max(-1) + 4 * U32 * np.where(validh, np.abs(x - xmax[..., None]), 0).max(-1)
    err = np.abs(stats[..., 1] - (tau - xmax))
    ratio = (err / (eps + 32 * U32))[ok]
    _log(f"  tau: worst |Δτ|/bound {ratio.max():.2e} over {ok.sum()} (head, row) pairs")
    assert ratio.max() <= 1.0, f"router threshold off by {ratio.max():.2f}x its bound"


@pytest.mark.parametrize("case", ROUTE_BWD, ids=[f"{c[0]}-g{c[2] // c[3]}-a{c[7]}-c{int(c[10])}" for c in ROUTE_BWD])
def test_route_backward_matches_oracle(case):
    """Stage-1 backward through the C ABI against the oracle: the GPU's own routing
    (lists and statistics of dash_route_stats), one dense upstream gradient of the
    bias read at the routed entries. Rows within the exemption margin get a zero
    upstream gradient on both sides (their lists may differ, and dk̄ sums over all
    rows), so their routing gradient is exactly zero; every other row's list must
    match the oracle's."""
    from long_context_amd import dash
    from oracle import dash_oracle as O
    G = _gu()
    dtype, b, hq, hkv, d, n, B, alpha, gamma, sigma, causal, seed = case
    _log(f"route backward case {case}")
    w = inputs.make_prefill(b=b, h_q=hq, h_kv=hkv, d=d, n=n, B=B, dtype=dtype, seed=seed)
    T = n // B
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Q = torch.from_numpy(w.Q).to("cuda", tdt)
    K = torch.from_numpy(w.K).to("cuda", tdt)
    kbar = dash.alloc_kbar(b, hkv, T, d)
    dash.dash_summarize(K, torch.from_numpy(w.qbar).cuda(), kbar, B)
    idx, bias, cnt, _ = dash.alloc_route(b, hkv, n, T)
    stats = torch.empty((b, hq, n, 2), device="cuda")
    dash.dash_route_stats(Q, kbar, B, alpha, gamma, sigma, causal, idx, bias, cnt, stats)
    torch.cuda.synchronize()
    pos = np.broadcast_to(np.arange(n), (b, n))
    kb_or = O.stage0_summaries(w.K, w.qbar, B)
    rt = O.route(w.Q, pos, kb_or, B, alpha, gamma, sigma, causal, n, keep_heads=True)
    ex = G.exempt_rows(rt)                                     # [b, h_kv, n]
    up = inputs.upstream_grad((b, hkv, n, T), seed=12)
    db0 = np.where(rt["support"] & ~ex[..., None], up, 0.0)
    fn = lambda dbias: (lambda kb: O.route_backward(w.Q, pos, kb, B, alpha, gamma, sigma, causal, n, dbias))
    ill = ill_conditioned_rows(fn(db0), kb_or, hq // hkv) & ~ex
    _log(f"  exempt rows: {int(ex.sum())}, ill-conditioned rows: {int(ill.sum())} of {ex.size}")
    assert ill.sum() <= MAX_ILL_FRAC * ex.size + 2, "too many ill-conditioned rows"
    drop = ex | ill
    dense = np.where(drop[..., None], 0.0, up).astype(np.float32)
    ii = idx.cpu().numpy().astype(np.int64)
    cc = cnt.cpu().numpy()
    live = np.arange(ii.shape[-1])[None, None, None, :] < cc[..., None]
    dlist = np.where(live, np.take_along_axis(dense, np.where(live, ii, 0), -1), 0.0).astype(np.float32)
    dQ = torch.zeros((b, hq, n, d), device="cuda")
    dkb = torch.zeros((b, hkv, T, d), device="cuda")
    dash.dash_route_backward(Q, kbar, idx, cnt, torch.from_numpy(dlist).cuda(), stats, B, alpha, gamma, sigma,
                             dQ, dkb)
    torch.cuda.synchronize()
    nex, _ = G.compare_route(dict(idx=idx, cnt=cnt), rt, np.arange(n), T)
    check_tau(stats.cpu().numpy(), w.Q.astype(np.float64), kb_or, rt, alpha, gamma, ~ex)
    db = np.where(rt["support"], dense, 0.0)
    ref, spread = _spread(fn(db), kb_or)
    gq = dQ.cpu().numpy()
    exq = np.repeat(drop, hq // hkv, axis=1)                   # per query head
    assert np.all(gq[exq] == 0.0), "rows with a zero upstream gradient must get none"
    _check_tiered(gq, ref["dQ"], spread["dQ"], "dQ (routing)")
    _check_tiered(dkb.cpu().numpy(), ref["dkbar"], spread["dkbar"], "dkbar")


# In the chain, Stage 1 takes the Stage-2 dbias with its bf16-level error, and the
# routing Jacobian scales a chunk's gradient by 1/w (w its group weight), so a chunk
# routed with a tiny weight magnifies that error. The chain tolerance per element is
# the sum of: the Stage-2 rounding bound (stage2_bounds), CHAIN_FACTOR times the
# largest change of the oracle's Stage-1 and Stage-0 gradients when its dbias takes
# three random errors of the size of the Stage-2 dbias bound (the propagated part;
# the L2 bound of each tensor is likewise u plus CHAIN_FACTOR times that spread),
# and TOL_COND_MIN of the Stage-1/Stage-0 part's row rms plus its tensor rms (their
# own fp32 arithmetic on well-conditioned rows, held to TOL_COND_MIN in the standalone
# tests; the chain's case has no row within the exemption margin).
CHAIN_FACTOR = 4.0


@pytest.mark.parametrize("causal,alpha", [(True, 1.5), (False, 2.0)])
def test_full_backward_chain_matches_oracle(causal, alpha):
    """The whole backward through the C ABI (Stage 2, then Stage 1 adding to dQ and
    dk̄, then Stage 0 adding to dK and dq̄) after the GPU forward, against the oracle's
    chained backward on the same inputs."""
    from long_context_amd import dash
    from oracle import dash_oracle as O
    G = _gu()
    b, hq, hkv, d, n, B, gamma, sigma = 1, 16, 2, 128, 384, 64, 4.0, 1.0
    w = inputs.make_prefill(b=b, h_q=hq, h_kv=hkv, d=d, n=n, B=B, dtype="bf16", seed=14)
    T = n // B
    dev = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)
    Q, K, V = (dev(x, torch.bfloat16) for x in (w.Q, w.K, w.V))
    qbar = dev(w.qbar, torch.float32)
    kbar = dash.alloc_kbar(b, hkv, T, d)
    dash.dash_summarize(K, qbar, kbar, B)
    idx, bias, cnt, _ = dash.alloc_route(b, hkv, n, T)
    stats = torch.empty((b, hq, n, 2), device="cuda")
    dash.dash_route_stats(Q, kbar, B, alpha, gamma, sigma, causal, idx, bias, cnt, stats)
    Og = torch.empty((b, hq, n, d), device="cuda")
    lse = torch.empty((b, hq, n), device="cuda")
    dash.dash_attend_prefill_lse(Q, K, V, idx, bias, cnt, Og, lse, B, causal)
    dO = inputs.upstream_grad((b, hq, n, d), seed=15, dtype="bf16")
    dQ = torch.empty((b, hq, n, d), device="cuda")
    dK = torch.empty((b, hkv, n, d), device="cuda")
    dV = torch.empty((b, hkv, n, d), device="cuda")
    db = torch.empty(idx.shape, device="cuda")
    dash.dash_attend_prefill_backward(Q, K, V, idx, bias, cnt, Og, dev(dO, torch.float32), lse, dQ, dK, dV, db,
                                      B, causal)
    dkb = torch.zeros((b, hkv, T, d), device="cuda")
    dash.dash_route_backward(Q, kbar, idx, cnt, db, stats, B, alpha, gamma, sigma, dQ, dkb)
    dqb = torch.zeros((hkv, d), device="cuda")
    dash.dash_summarize_backward(K, qbar, dkb, B, dK, dqb)
    torch.cuda.synchronize()
    pos = np.broadcast_to(np.arange(n), (b, n))
    kb_or = O.stage0_summaries(w.K, w.qbar, B)
    rt = O.route(w.Q, pos, kb_or, B, alpha, gamma, sigma, causal, n)
    assert not G.exempt_rows(rt).any(), "a row sits within the exemption margin: choose another seed"
    G.compare_route(dict(idx=idx, cnt=cnt), rt, np.arange(n), T)
    rt = dict(rt, bias=rt["bias"].astype(np.float32).astype(np.float64))
    g2 = O.attend_backward(w.Q, pos, w.K, w.V, rt, B, causal, n, dO.astype(np.float64))
    up = lambda dbias: O.route_backward(w.Q, pos, kb_or, B, alpha, gamma, sigma, causal, n, dbias)
    g1 = up(g2["dbias"])
    g0 = O.summary_backward(w.K, w.qbar, B, g1["dkbar"])
    ref = dict(dQ=g2["dQ"] + g1["dQ"], dK=g2["dK"] + g0["dK"], dV=g2["dV"], dqbar=g0["dqbar"])
    part1 = dict(dQ=g1["dQ"], dK=g0["dK"], dV=np.zeros_like(g2["dV"]), dqbar=g0["dqbar"])
    dlse = np.abs(lse.cpu().numpy() - g2["lse"])
    b2 = stage2_bounds(w.Q, pos, w.K, w.V, rt, B, causal, n, dO, dlse, o_bf16=False, do_f32=False)
    bnd2 = dict(dQ=b2["dQ"], dK=b2["dK"], dV=b2["dV"], dqbar=np.zeros_like(g0["dqbar"]))
    # the Stage-2 dbias error carried through Stages 1 and 0 (oracle only)
    S = rt["support"]
    rng = np.random.default_rng(99)
    spread = {k: np.zeros(v.shape) for k, v in ref.items()}
    for _ in range(3):
        err = b2["dbias"] * rng.standard_normal(S.shape)
        p1 = up(np.where(S, g2["dbias"] + err, 0.0))
        p0 = O.summary_backward(w.K, w.qbar, B, p1["dkbar"])
        for k, v in (("dQ", p1["dQ"] - g1["dQ"]), ("dK", p0["dK"] - g0["dK"]), ("dqbar", p0["dqbar"] - g0["dqbar"])):
            spread[k] = np.maximum(spread[k], np.abs(v))
    _log(f"full chain causal={causal} alpha={alpha}")
    got = dict(dQ=dQ.cpu().numpy(), dK=dK.cpu().numpy(), dV=dV.cpu().numpy(), dqbar=dqb.cpu().numpy())
    for name in ("dQ", "dK", "dV", "dqbar"):
        g, r, sp = got[name].astype(np.float64), ref[name], spread[name]
        assert np.isfinite(g).all(), f"{name}: non-finite"
        p1r = part1[name]
        f32 = TOL_COND_MIN * (np.sqrt((p1r ** 2).mean(-1, keepdims=True)) + np.sqrt((p1r ** 2).mean()))
        tol = bnd2[name] + CHAIN_FACTOR * sp + f32
        e = np.abs(g - r)
        k = np.unravel_index(np.argmax(e / tol), e.shape)
        nr = np.linalg.norm(r)
        l2 = np.linalg.norm(g - r) / nr
        l2_tol = TOL_L2 + CHAIN_FACTOR * np.linalg.norm(sp) / nr
        _log(f"  {name}: worst element {k} err/bound {e[k] / tol[k]:.2e}; l2 {l2:.2e} bound {l2_tol:.2e}")
        assert np.all(e <= tol), f"{name}: element {k} error {e[k]} above {tol[k]}"
        assert l2 <= l2_tol, f"{name}: relative L2 error {l2}"


def _route_backward_sampled(w, alpha, rows, seed):
    """Stages 1 and 0 backward through the C ABI with the upstream dbias nonzero only on
    the given rows (their oracle-routed entries, where the oracle's list matches the
    GPU router's). Both gradients are linear in dbias: the oracle then fixes dQ of
    those rows, every other row's routing gradient is exactly zero, and dk̄ is the sum
    over the given rows alone. Stage 0 takes the oracle's dk̄ on both sides and is
    checked on the whole of dK and dq̄."""
    from long_context_amd import dash
    from oracle import dash_oracle as O
    G = _gu()
    b, hq, n, d = w.Q.shape
    hkv, B = w.h_kv, w.B
    T = n // B
    dev = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    Qd, Kd = dev(w.Q, tdt), dev(w.K, tdt)
    qbar = torch.from_numpy(w.qbar).cuda()
    kbar = dash.alloc_kbar(b, hkv, T, d)
    dash.dash_summarize(Kd, qbar, kbar, B)
    idx, bias, cnt, _ = dash.alloc_route(b, hkv, n, T)
    stats = torch.empty((b, hq, n, 2), device="cuda")
    dash.dash_route_stats(Qd, kbar, B, alpha, w.gamma, w.sigma, w.causal, idx, bias, cnt, stats)
    torch.cuda.synchronize()
    pos = np.broadcast_to(rows, (b, rows.size))
    kb = O.stage0_summaries(w.K, w.qbar, B)
    rt = O.route(w.Q[:, :, rows], pos, kb, B, alpha, w.gamma, w.sigma, w.causal, n, keep_heads=True)
    nex, _ = G.compare_route(dict(idx=idx, cnt=cnt), rt, rows, T)
    ex = G.exempt_rows(rt)                                     # [b, h_kv, R]
    up = inputs.upstream_grad((b, hkv, rows.size, T), seed=seed)
    fn = lambda dbias: (lambda k: O.route_backward(w.Q[:, :, rows], pos, k, B, alpha, w.gamma, w.sigma, w.causal,
                                                   n, dbias))
    ill = ill_conditioned_rows(fn(np.where(rt["support"] & ~ex[..., None], up, 0.0)), kb, hq // hkv) & ~ex
    _log(f"  exempt rows: {nex}, ill-conditioned rows: {int(ill.sum())} of {ex.size}")
    assert ill.sum() <= MAX_ILL_FRAC * ex.size + 2, "too many ill-conditioned rows"
    keep = ~(ex | ill)
    dense = np.where(rt["support"] & keep[..., None], up, 0.0)  # oracle layout, sampled rows
    # the same values at the GPU's list positions of the sampled rows, zero elsewhere
    ri = torch.from_numpy(rows).cuda()
    ii = idx[:, :, ri].cpu().numpy().astype(np.int64)
    cc = cnt[:, :, ri].cpu().numpy()
    live = np.arange(ii.shape[-1])[None, None, None, :] < cc[..., None]
    dl = np.where(live, np.take_along_axis(dense, np.where(live, ii, 0), -1), 0.0).astype(np.float32)
    dlist = torch.zeros(idx.shape, device="cuda")
    dlist[:, :, ri] = dev(dl, torch.float32)
    dQ = torch.zeros((b, hq, n, d), device="cuda")
    dkb = torch.zeros((b, hkv, T, d), device="cuda")
    dash.dash_route_backward(Qd, kbar, idx, cnt, dlist, stats, B, alpha, w.gamma, w.sigma, dQ, dkb)
    torch.cuda.synchronize()
    check_tau(stats[:, :, ri].cpu().numpy(), w.Q[:, :, rows].astype(np.float64), kb, rt, alpha, w.gamma, ~ex)
    gq = dQ.cpu().numpy()
    others = np.ones(n, bool)
    others[rows] = False
    assert np.all(gq[:, :, others] == 0.0), "rows with a zero upstream gradient must get none"
    ref, spread = _spread(fn(dense), kb)
    _check_tiered(gq[:, :, rows], ref["dQ"], spread["dQ"], "dQ (routing, sampled rows)")
    _check_tiered(dkb.cpu().numpy(), ref["dkbar"], spread["dkbar"], "dkbar")
    dK = torch.zeros((b, hkv, n, d), device="cuda")
    dq = torch.zeros((hkv, d), device="cuda")
    dash.dash_summarize_backward(Kd, qbar, dev(ref["dkbar"], torch.float32), B, dK, dq)
    torch.cuda.synchronize()
    r0 = O.summary_backward(w.K, w.qbar, B, ref["dkbar"])
    _rel(dK.cpu().numpy(), r0["dK"], TOL_F32_L2, TOL_F32_ROW, "dK (summaries)")
    _rel(dq.cpu().numpy(), r0["dqbar"], TOL_F32_L2, TOL_F32_ROW, "dqbar")


@pytest.mark.parametrize("alpha", [1.5, 1.25])
def test_route_and_summary_backward_32k_full_size(alpha):
    """Stages 1 and 0 backward on the 32K GQA-16 clustered workload at full size, in
    the benchmark's launch (512 chunks: dk̄ in two 64-column slices), with the upstream
    gradient on 28 sampled rows."""
    w = inputs.prefill_32k_clusters(alphas=(alpha,))
    n, B = w.n, w.B
    rng = np.random.default_rng(31)
    rows = np.unique(np.concatenate([rng.choice(n, size=24, replace=False), [B, 2 * B - 1, n // 2, n - 1]]))
    _log(f"32k routing backward alpha={alpha}: {rows.size} rows")
    _route_backward_sampled(w, alpha, rows, seed=32)


def test_route_backward_1300_chunks_sampled():
    """1300 chunks at d = 128 (B = 16, GQA 8): the dk̄ accumulator no longer fits 32
    columns per workgroup and runs in eight 16-column slices; the router splits each
    row over four wavefronts. Upstream gradient on sampled rows."""
    w = inputs.make_prefill(b=1, h_q=16, h_kv=2, d=128, n=1300 * 16, B=16, dtype="bf16", seed=41, gamma=6.0)
    rng = np.random.default_rng(42)
    rows = np.unique(np.concatenate([rng.choice(w.n, size=20, replace=False), [16, w.n - 1]]))
    _log(f"1300-chunk routing backward: {rows.size} rows")
    _route_backward_sampled(w, 1.5, rows, seed=43)
