"""Pins of the CPU oracle against what the DashAttention pages and mathematics fix.

None of these re-types an oracle formula: each checks the oracle against an
independent definition (variational form of entmax, brute-force KKT search,
library SDPA, a second formulation of Stage 2) or a closed-form special case.
Citations name the xllm-io paper review, section 三 (technical architecture).
"""
import itertools

import numpy as np
import pytest
import scipy.optimize
import scipy.special
import torch

from oracle import dash_oracle as O
from long_context_amd import inputs


# ----------------------------------------------------------------------------------
# α-entmax (background formula, section 三): outputs on the simplex, unique τ,
# α -> 1 softmax, α = 2 sparsemax, sparsity grows with α.
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("alpha", [1.1, 1.25, 1.5, 2.0, 3.0])
def test_entmax_on_simplex(alpha):
    rng = np.random.default_rng(0)
    s = rng.standard_normal((400, 33)) * 3
    valid = np.arange(33)[None] < rng.integers(1, 34, size=(400, 1))
    p, tau, x = O.entmax(s, alpha, valid)
    assert np.all(p >= 0)
    assert np.all(p[~valid] == 0)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_entmax_shift_invariance(alpha):
    rng = np.random.default_rng(1)
    s = rng.standard_normal((50, 20))
    p1, _, _ = O.entmax(s, alpha)
    p2, _, _ = O.entmax(s + 7.25, alpha)
    np.testing.assert_allclose(p1, p2, atol=1e-12)


def _tsallis_objective(p, s, alpha):
    # maximise p.s + H_alpha(p) with Tsallis entropy H = sum(p - p^alpha)/(alpha(alpha-1))
    p = np.clip(p, 0, None)
    return -(p @ s + np.sum(p - p ** alpha) / (alpha * (alpha - 1)))


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 3.0])
def test_entmax_matches_variational_definition(alpha):
    """α-entmax is the maximiser of p.s + Tsallis entropy over the simplex; its
    closed form [(α-1)s - τ]_+^{1/(α-1)} must agree with a generic optimiser."""
    rng = np.random.default_rng(2)
    for _ in range(6):
        T = int(rng.integers(2, 7))
        s = rng.standard_normal(T) * 1.5
        res = scipy.optimize.minimize(
            _tsallis_objective, np.full(T, 1.0 / T), args=(s, alpha), method="SLSQP",
            bounds=[(0, 1)] * T, constraints=[{"type": "eq", "fun": lambda p: p.sum() - 1}],
            options={"ftol": 1e-15, "maxiter": 500})
        p, _, _ = O.entmax(s[None], alpha)
        np.testing.assert_allclose(p[0], res.x, atol=2e-5)


def test_sparsemax_is_simplex_projection():
    """α = 2 is sparsemax: the Euclidean projection of s onto the simplex."""
    rng = np.random.default_rng(3)
    for _ in range(10):
        T = int(rng.integers(2, 9))
        s = rng.standard_normal(T)
        res = scipy.optimize.minimize(
            lambda p: 0.5 * np.sum((p - s) ** 2), np.full(T, 1.0 / T), method="SLSQP",
            bounds=[(0, None)] * T, constraints=[{"type": "eq", "fun": lambda p: p.sum() - 1}],
            options={"ftol": 1e-15, "maxiter": 500})
        p, _, _ = O.entmax(s[None], 2.0)
        np.testing.assert_allclose(p[0], res.x, atol=1e-6)


def test_entmax_alpha_to_one_is_softmax():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((20, 15))
    p1, _, _ = O.entmax(s, 1.0)
    np.testing.assert_allclose(p1, scipy.special.softmax(s, axis=-1), atol=1e-14)
    p, _, _ = O.entmax(s, 1.0 + 1e-4)
    assert np.abs(p - scipy.special.softmax(s, axis=-1)).max() < 2e-4


def _brute_force_tau(x, alpha):
    """Enumerate every support S, solve sum_S (x-τ)^p = 1 on it, keep the KKT-valid ones."""
    p = 1.0 / (alpha - 1.0)
    T = x.size
    found = []
    for k in range(1, T + 1):
        for S in itertools.combinations(range(T), k):
            xs = x[list(S)]
            lo, hi = xs.min() - 2.0, xs.min()
            for _ in range(200):           # on S the sum is decreasing in τ < min(xs)
                mid = 0.5 * (lo + hi)
                if np.sum((xs - mid) ** p) >= 1:
                    lo = mid
                else:
                    hi = mid
            tau = 0.5 * (lo + hi)
            off = np.setdiff1d(np.arange(T), S)
            solved = abs(np.sum((xs - tau) ** p) - 1.0) < 1e-9
            if solved and np.all(xs > tau) and np.all(x[off] <= tau):
                found.append((S, tau))
    return found


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_entmax_brute_force_support(alpha):
    """Exactly one support satisfies the KKT conditions (τ is unique) and it is the
    oracle's."""
    rng = np.random.default_rng(5)
    for _ in range(8):
        T = int(rng.integers(1, 9))
        s = rng.standard_normal(T) * 2
        x = (alpha - 1) * s
        found = _brute_force_tau(x, alpha)
        assert len(found) == 1
        S, tau = found[0]
        p, t, _ = O.entmax(s[None], alpha)
        assert set(np.nonzero(p[0] > 0)[0]) == set(S)
        assert abs(t[0] - tau) < 1e-12


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_sorted_threshold_matches_bisection(alpha):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2000, 64))
    valid = np.arange(64)[None] < rng.integers(1, 65, size=(2000, 1))
    a = O.entmax_tau_sorted(x, valid, alpha)
    b = O.entmax_tau_bisect(x, valid, alpha)
    assert np.abs(a - b).max() < 1e-13


def test_entmax_gamma_limits():
    rng = np.random.default_rng(7)
    s = rng.standard_normal((10, 12))
    p, _, _ = O.entmax(1e-9 * s, 1.5)
    np.testing.assert_allclose(p, 1.0 / 12, atol=1e-6)
    p, _, _ = O.entmax(1e4 * s, 1.5)
    np.testing.assert_array_equal(p, np.eye(12)[s.argmax(-1)])


def test_sparsity_grows_with_alpha():
    rng = np.random.default_rng(8)
    s = rng.standard_normal((500, 64)) * 2
    nnz = [np.count_nonzero(O.entmax(s, a)[0]) for a in (1.25, 1.5, 2.0, 3.0)]
    assert nnz[0] >= nnz[1] >= nnz[2] >= nnz[3]
    assert nnz[0] > nnz[3]


# ----------------------------------------------------------------------------------
# Stage 0 (Eq. 4): local SDPA under q̄ with keys as values.
# ----------------------------------------------------------------------------------

def test_stage0_is_local_sdpa():
    rng = np.random.default_rng(9)
    K = rng.standard_normal((2, 3, 100, 16))
    qbar = rng.standard_normal((3, 16))
    B = 8
    kb = O.stage0_summaries(K, qbar, B)
    assert kb.shape == (2, 3, 12, 16)          # trailing partial chunk has no summary
    Kt = torch.from_numpy(K[:, :, :96].reshape(2, 3, 12, 8, 16))
    q = torch.from_numpy(qbar)[None, :, None, None, :].expand(2, 3, 12, 1, 16)
    ref = torch.nn.functional.scaled_dot_product_attention(q, Kt, Kt)[..., 0, :]
    np.testing.assert_allclose(kb, ref.numpy(), atol=1e-13)


def test_stage0_zero_query_is_mean_pooling():
    rng = np.random.default_rng(10)
    K = rng.standard_normal((1, 2, 64, 8))
    kb = O.stage0_summaries(K, np.zeros((2, 8)), 16)
    np.testing.assert_allclose(kb, K.reshape(1, 2, 4, 16, 8).mean(3), atol=1e-14)


def test_stage0_chunk_of_one_is_the_key():
    rng = np.random.default_rng(11)
    K = rng.standard_normal((1, 1, 10, 4))
    kb = O.stage0_summaries(K, rng.standard_normal((1, 4)), 1)
    np.testing.assert_allclose(kb, K, atol=1e-15)


def test_stage0_permutation_invariant_within_chunk():
    rng = np.random.default_rng(12)
    K = rng.standard_normal((1, 1, 32, 8))
    qbar = rng.standard_normal((1, 8))
    perm = np.concatenate([rng.permutation(16), 16 + rng.permutation(16)])
    np.testing.assert_allclose(O.stage0_summaries(K, qbar, 16),
                               O.stage0_summaries(K[:, :, perm], qbar, 16), atol=1e-14)


# ----------------------------------------------------------------------------------
# Stage 1: GQA average and union (Eq. 6 and the GQA paragraph).
# ----------------------------------------------------------------------------------

def _small(seed=0, **kw):
    args = dict(b=2, h_q=4, h_kv=2, d=16, n=160, B=16, alphas=(1.5,), gamma=2.0,
                sigma=1.0, causal=True, dtype="f32", seed=seed)
    args.update(kw)
    return inputs.make_prefill(**args)


def test_group_weights_simplex_and_union():
    w = _small()
    kb = O.stage0_summaries(w.K, w.qbar, w.B)
    rows = np.arange(w.n)
    rt = O.route(w.Q, rows[None], kb, w.B, 1.5, 3.0, 1.0, True, w.n, keep_heads=True)
    has = rt["vis"][:, None, :] >= 1
    sums = rt["w"].sum(-1)
    np.testing.assert_allclose(sums[np.broadcast_to(has, sums.shape)], 1.0, atol=1e-12)
    heads_sup = (rt["what"] > 0).reshape(2, 2, 2, w.n, -1).any(2)
    np.testing.assert_array_equal(heads_sup, rt["support"])


def test_group_of_one_head_is_the_head():
    w = _small(h_q=2, h_kv=2)
    kb = O.stage0_summaries(w.K, w.qbar, w.B)
    rows = np.arange(w.n)
    rt = O.route(w.Q, rows[None], kb, w.B, 1.5, 3.0, 1.0, True, w.n, keep_heads=True)
    np.testing.assert_allclose(rt["w"], rt["what"], atol=0)


def test_query_head_to_kv_group_map():
    """r = floor(h/g): with identical heads inside each group, the group weight equals
    the single-head entmax of that group's query against that group's summaries."""
    w = _small(h_q=6, h_kv=2)
    Q = w.Q.copy()
    Q[:, 1:3] = Q[:, 0:1]
    Q[:, 4:6] = Q[:, 3:4]
    kb = O.stage0_summaries(w.K, w.qbar, w.B)
    rows = np.arange(w.n)
    rt = O.route(Q, rows[None], kb, w.B, 1.5, 3.0, 1.0, True, w.n)
    for r in range(2):
        single = O.route(Q[:, 3 * r:3 * r + 1], rows[None], kb[:, r:r + 1], w.B, 1.5, 3.0, 1.0,
                         True, w.n)
        np.testing.assert_allclose(rt["w"][:, r], single["w"][:, 0], atol=1e-14)


def test_single_visible_chunk_has_unit_weight_and_zero_bias():
    w = _small()
    kb = O.stage0_summaries(w.K, w.qbar, w.B)
    rows = np.arange(w.B, 2 * w.B)                       # exactly one visible chunk
    rt = O.route(w.Q[:, :, rows], rows[None], kb, w.B, 1.5, 3.0, 1.0, True, w.n)
    np.testing.assert_allclose(rt["w"][..., 0], 1.0, atol=1e-15)
    np.testing.assert_array_equal(rt["cnt"], 1)
    np.testing.assert_allclose(rt["bias"], 0.0, atol=1e-15)


# ----------------------------------------------------------------------------------
# Stage 2: Eq. 9 / 11 / 12 versus Proposition 4.1, and library SDPA special cases.
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("sigma", [1.0, 0.5, 3.0, np.inf])
@pytest.mark.parametrize("causal,n", [(True, 160), (False, 160), (False, 168)])
def test_bias_form_equals_prior_form(sigma, causal, n):
    """Prop. 4.1: the additive bias d = (log w - μ)/σ on R and 0 on D reproduces the
    prior-induced softmax of Eq. 9 built from Eq. 11 and Eq. 12."""
    w = _small(n=n, causal=causal, sigma=sigma)
    kb = O.stage0_summaries(w.K, w.qbar, w.B)
    rows = np.array([0, 5, 16, 17, 40, 63, 64, 100, n - 1])
    rt = O.route(w.Q[:, :, rows], rows[None], kb, w.B, 1.5, 3.0, sigma, causal, n)
    a = O.attend(w.Q[:, :, rows], rows[None], w.K, w.V, rt, w.B, causal, n)
    b = O.attend_eq9(w.Q[:, :, rows], rows[None], w.K, w.V, rt, w.B, sigma, causal, n)
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_uniform_router_gives_zero_bias_and_size_split():
    """Identical summaries make the router uniform: d = 0 and λ = |R|/(|R|+|D|)."""
    w = _small()
    kb = np.broadcast_to(O.stage0_summaries(w.K, w.qbar, w.B)[:, :, :1], (2, 2, 10, 16)).copy()
    rows = np.arange(w.n)
    rt = O.route(w.Q, rows[None], kb, w.B, 1.5, 3.0, 1.0, True, w.n)
    np.testing.assert_allclose(rt["bias"], 0.0, atol=1e-12)
    vis = rt["vis"][0]
    assert np.all(rt["cnt"][0, 0] == vis)


def _sdpa(q, k, v, mask):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(mask)).numpy()


def test_sigma_inf_is_masked_softmax():
    """σ = inf: the prior is uniform on the support, so Stage 2 is plain SDPA with the
    boolean mask of R ∪ D (checked against the library routine)."""
    w = _small(sigma=np.inf)
    kb = O.stage0_summaries(w.K, w.qbar, w.B)
    rows = np.arange(w.n)
    rt = O.route(w.Q, rows[None], kb, w.B, 2.0, 6.0, np.inf, True, w.n)
    Oa = O.attend(w.Q, rows[None], w.K, w.V, rt, w.B, True, w.n)
    T = w.n // w.B
    tok = np.arange(w.n)
    for bi in range(2):
        for r in range(2):
            mask = np.zeros((w.n, w.n), bool)
            sup = rt["support"][bi, r]                        # [rows, T]
            mask[:, :T * w.B] = sup[:, tok[:T * w.B] // w.B]
            own = (rows[:, None] // w.B == tok[None] // w.B) & (tok[None] <= rows[:, None])
            mask |= own
            for h in range(2 * r, 2 * r + 2):
                ref = _sdpa(np.asarray(w.Q[bi, h], np.float64), np.asarray(w.K[bi, r], np.float64),
                            np.asarray(w.V[bi, r], np.float64), mask)
                np.testing.assert_allclose(Oa[bi, h], ref, atol=1e-12)


def test_full_support_is_dense_causal_attention():
    """γ -> 0 routes every visible chunk with equal weight; with σ = inf Stage 2 is
    dense causal SDPA."""
    w = _small(sigma=np.inf)
    res = O.prefill(w.Q, w.K, w.V, w.qbar, w.B, 1.5, 1e-9, np.inf, True)
    assert O.group_sparsity(res["route"]) == 0.0
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.asarray(w.Q, np.float64)),
        torch.from_numpy(np.asarray(np.repeat(w.K, 2, axis=1), np.float64)),
        torch.from_numpy(np.asarray(np.repeat(w.V, 2, axis=1), np.float64)), is_causal=True)
    np.testing.assert_allclose(res["O"], ref.numpy(), atol=1e-12)


def test_no_visible_chunk_is_causal_softmax_over_own_chunk():
    w = _small()
    res = O.prefill(w.Q, w.K, w.V, w.qbar, w.B, 1.5, 3.0, 1.0, True, rows=np.arange(w.B))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.asarray(w.Q[:, :, :w.B], np.float64)),
        torch.from_numpy(np.asarray(np.repeat(w.K[:, :, :w.B], 2, axis=1), np.float64)),
        torch.from_numpy(np.asarray(np.repeat(w.V[:, :, :w.B], 2, axis=1), np.float64)),
        is_causal=True)
    np.testing.assert_allclose(res["O"], ref.numpy(), atol=1e-13)


@pytest.mark.parametrize("L", [160, 161, 175, 176])
def test_decode_equals_last_prefill_row(L):
    w = _small(n=L)
    kb = O.stage0_summaries(w.K, w.qbar, w.B)
    pre = O.prefill(w.Q, w.K, w.V, w.qbar, w.B, 1.5, 3.0, 1.0, True, rows=np.array([L - 1]))
    dec = O.decode(w.Q[:, :, L - 1:L], w.K, w.V, kb, np.full(2, L), w.B, 1.5, 3.0, 1.0)
    np.testing.assert_allclose(dec["O"], pre["O"], atol=1e-14)


def test_group_sparsity_monotone_in_alpha_on_clusters():
    """Aggregate sparsity grows with α on a small clustered workload."""
    rng = np.random.default_rng(13)
    w = _small(n=512, B=16, h_q=8, h_kv=2, d=32)
    K = w.K.copy()
    for r in range(2):
        for c0 in (4, 12, 20):
            u = rng.standard_normal(32)
            u /= np.linalg.norm(u)
            K[:, r, c0 * 16:(c0 + 4) * 16] = 0.8 * np.linalg.norm(
                K[:, r, c0 * 16:(c0 + 4) * 16], axis=-1, keepdims=True) * u + \
                0.6 * K[:, r, c0 * 16:(c0 + 4) * 16] / np.sqrt(32)
    kb = O.stage0_summaries(K, w.qbar, 16)
    rows = np.arange(0, 512, 3)
    sp = [O.group_sparsity(O.route(w.Q[:, :, rows], rows[None], kb, 16, a, 1.0, 1.0, True, 512))
          for a in (1.25, 1.5, 2.0)]
    assert sp[0] <= sp[1] <= sp[2]
    assert sp[2] > sp[0]


def test_sequence_shorter_than_a_chunk_routes_nothing():
    """n < B: no complete chunk, so no row routes anywhere and Stage 2 is causal
    softmax over the row's own (partial) chunk."""
    w = _small(n=12)
    res = O.prefill(w.Q, w.K, w.V, w.qbar, w.B, 1.5, 3.0, 1.0, True)
    assert res["kbar"].shape[2] == 0 and res["route"]["cnt"].sum() == 0
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.asarray(w.Q, np.float64)),
        torch.from_numpy(np.asarray(np.repeat(w.K, 2, axis=1), np.float64)),
        torch.from_numpy(np.asarray(np.repeat(w.V, 2, axis=1), np.float64)), is_causal=True)
    np.testing.assert_allclose(res["O"], ref.numpy(), atol=1e-13)


def test_softmax_routing_is_the_entmax_limit():
    """α = 1 routes with softmax, the α -> 1 limit of entmax (paper review section 三,
    α-entmax background): its group weights, supports and biases approach those of
    α-entmax routing as α -> 1, every visible chunk is routed, and each row's group
    weights sum to one."""
    w = _small()
    kb = O.stage0_summaries(w.K, w.qbar, w.B)
    rows = np.arange(w.n)
    soft = O.route(w.Q, rows[None], kb, w.B, 1.0, 3.0, 1.0, True, w.n)
    near = O.route(w.Q, rows[None], kb, w.B, 1.0 + 1e-5, 3.0, 1.0, True, w.n)
    np.testing.assert_allclose(soft["w"], near["w"], atol=1e-5)
    assert np.array_equal(soft["cnt"][0, 0], soft["vis"][0])
    assert np.array_equal(soft["support"], near["support"])
    np.testing.assert_allclose(soft["bias"], near["bias"], atol=1e-3)
    has = soft["vis"][0] > 0
    np.testing.assert_allclose(soft["w"].sum(-1)[..., has], 1.0, atol=1e-12)
    assert np.isinf(soft["margin"]).all()             # no support boundary to exempt


def test_softmax_routing_log_weights_stay_finite():
    """Softmax routing with a huge γ: the group log-weights (and so the biases) stay
    finite although the smallest weights underflow in floating point."""
    w = _small()
    kb = O.stage0_summaries(w.K, w.qbar, w.B)
    rows = np.arange(w.n)
    rt = O.route(w.Q, rows[None], kb, w.B, 1.0, 5000.0, 1.0, True, w.n)
    sup = rt["support"]
    assert np.isfinite(rt["bias"][sup]).all()
    assert (rt["w"][sup] == 0.0).any()


def test_topk_keeps_the_heaviest_subset():
    """A fixed budget keeps, per row, the k-subset of the support with the largest
    total group weight (brute force over all k-subsets on a small case), μ is the
    mean log-weight of the kept chunks (so the kept biases average to zero), and a
    budget at least the support size changes nothing."""
    w = _small()
    kb = O.stage0_summaries(w.K, w.qbar, w.B)
    rows = np.arange(w.B, w.n, 7)
    full = O.route(w.Q[:, :, rows], rows[None], kb, w.B, 1.5, 1.0, 1.0, True, w.n)
    k = 3
    rt = O.route(w.Q[:, :, rows], rows[None], kb, w.B, 1.5, 1.0, 1.0, True, w.n, top_k=k)
    checked = 0
    for ix in np.ndindex(*full["cnt"].shape):
        cs = np.nonzero(full["support"][ix])[0]
        kept = np.nonzero(rt["support"][ix])[0]
        assert kept.size == min(k, cs.size)
        if cs.size > k:
            best = max(itertools.combinations(cs.tolist(), k), key=lambda sub: sum(full["w"][ix][list(sub)]))
            assert set(kept.tolist()) == set(best)
            checked += 1
        np.testing.assert_allclose(rt["bias"][ix][kept].mean() if kept.size else 0.0, 0.0, atol=1e-12)
    assert checked > 0
    big = O.route(w.Q[:, :, rows], rows[None], kb, w.B, 1.5, 1.0, 1.0, True, w.n, top_k=10_000)
    assert np.array_equal(big["support"], full["support"])
    np.testing.assert_allclose(big["bias"], full["bias"], atol=0)


def test_topk_with_softmax_routing_is_a_fixed_budget():
    """α = 1 routes every visible chunk, so a budget k routes exactly min(k, visible)."""
    w = _small()
    kb = O.stage0_summaries(w.K, w.qbar, w.B)
    rows = np.arange(w.n)
    rt = O.route(w.Q, rows[None], kb, w.B, 1.0, 3.0, 1.0, True, w.n, top_k=4)
    assert np.array_equal(rt["cnt"][0, 0], np.minimum(4, rt["vis"][0]))


def _one_hot_route(xs, alpha, gamma=1.0, top_k=0):
    """Route one non-causal row whose per-head thresholded scores are exactly `xs`
    [heads, T]: summaries k̄_c = sqrt(T) e_c make z̄_c = q_c, so q = x / ((α-1)γ)
    (α = 1: x / γ)."""
    heads, T = xs.shape
    scale = gamma * (alpha - 1.0 if alpha != 1.0 else 1.0)
    Q = (xs / scale)[None, :, None, :]                   # [1, heads, 1, d = T]
    kb = (np.sqrt(T) * np.eye(T))[None, None]            # [1, 1, T, T]
    return O.route(Q, np.array([[T]]), kb, 1, alpha, gamma, 1.0, False, T, keep_heads=True, top_k=top_k)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_margin_is_the_distance_to_the_brute_force_threshold(alpha):
    """The exemption margin of a row is min over its group's heads and visible chunks
    of |x - τ| (the distance of a score to the unique KKT threshold): compared with τ
    from the brute-force support enumeration, on random tiny rows."""
    rng = np.random.default_rng(31)
    for _ in range(6):
        T = int(rng.integers(2, 8))
        xs = rng.standard_normal((2, T)) * (alpha - 1.0) * 2.0
        rt = _one_hot_route(xs, alpha)
        ref = np.inf
        for h in range(2):
            found = _brute_force_tau(xs[h], alpha)
            assert len(found) == 1
            ref = min(ref, np.abs(xs[h] - found[0][1]).min())
        assert abs(rt["margin"][0, 0, 0] - ref) < 1e-12


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_margin_separates_planted_near_threshold_scores(alpha):
    """A chunk planted 5e-7 below a head's τ (outside the support, so τ is unchanged)
    makes the row exempt (margin <= 1e-6); planted 2e-6 below, it does not. The other
    head is uniform, so its scores sit far from its own threshold."""
    base = np.array([1.0, 0.6, 0.1, -0.3]) * (alpha - 1.0) * 2.0
    (S, tau), = _brute_force_tau(base, alpha)
    for gap, exempt in ((5e-7, True), (2e-6, False)):
        xs = np.stack([np.append(base, tau - gap), np.zeros(5)])
        (S2, tau2), = _brute_force_tau(xs[0], alpha)
        assert set(S2) == set(S) and abs(tau2 - tau) < 1e-12
        rt = _one_hot_route(xs, alpha)
        assert abs(rt["margin"][0, 0, 0] - gap) < 1e-10
        assert bool(rt["margin"][0, 0, 0] <= 1e-6) == exempt


def test_topk_margin_is_the_log_weight_gap_at_the_cut():
    """With softmax routing (α = 1) log w_c - log w_c' = γ (z̄_c - z̄_c') for one head,
    so the fixed-budget margin is the logit gap between the last kept and the first
    dropped chunk: planted gaps of 5e-6 (exempt, <= 1e-5) and 2e-5 (not exempt)."""
    for gap, exempt in ((5e-6, True), (2e-5, False)):
        xs = np.array([[2.0, 1.5, 1.0, 1.0 - gap, 0.0]])
        rt = _one_hot_route(xs, 1.0, gamma=1.0, top_k=3)
        assert np.array_equal(np.nonzero(rt["support"][0, 0, 0])[0], [0, 1, 2])
        assert abs(rt["margin_topk"][0, 0, 0] - gap) < 1e-12
        assert bool(rt["margin_topk"][0, 0, 0] <= 1e-5) == exempt
    rt = _one_hot_route(np.array([[2.0, 1.0]]), 1.0, top_k=3)   # nothing dropped
    assert rt["margin_topk"][0, 0, 0] == np.inf


def test_route_mask_matches_little_endian_bit_packing():
    """The oracle's bitpacked mask equals numpy's little-endian bit packing read as
    32-bit little-endian words, and unpacks back to the support."""
    rng = np.random.default_rng(4)
    sup = rng.random((2, 3, 5, 70)) < 0.3
    words = 3
    m = O.route_mask(sup, words)
    padded = np.zeros(sup.shape[:-1] + (words * 32,), bool)
    padded[..., :70] = sup
    ref = np.packbits(padded, axis=-1, bitorder="little").view("<u4")
    assert np.array_equal(m, ref)
    back = np.unpackbits(m.view(np.uint8), axis=-1, bitorder="little")[..., :70].astype(bool)
    assert np.array_equal(back, sup)


def _stage2_setup(n=160, B=16, seed=5, sigma=1.0):
    w = _small(n=n)
    kb = O.stage0_summaries(w.K, w.qbar, B)
    rows = np.arange(n)
    rt = O.route(w.Q, rows[None], kb, B, 1.5, 3.0, sigma, True, n)
    rng = np.random.default_rng(seed)
    dO = rng.standard_normal(w.Q.shape)
    return w, rows, rt, dO


def test_stage2_backward_matches_finite_differences():
    """Stage-2 gradients of <dO, O> against central differences of the forward
    oracle in random directions, for Q, K, V and the per-chunk bias."""
    w, rows, rt, dO = _stage2_setup()
    n, B = w.n, 16
    Q, K, V = (np.asarray(x, np.float64) for x in (w.Q, w.K, w.V))
    gr = O.attend_backward(Q, rows[None], K, V, rt, B, True, n, dO)
    rng = np.random.default_rng(8)
    eps = 1e-6

    def loss(Qx, Kx, Vx, rtx):
        return float((dO * O.attend(Qx, rows[None], Kx, Vx, rtx, B, True, n)).sum())

    for name, x in (("Q", Q), ("K", K), ("V", V)):
        u = rng.standard_normal(x.shape)
        args = dict(Q=Q, K=K, V=V)
        plus = dict(args); plus[name] = x + eps * u
        minus = dict(args); minus[name] = x - eps * u
        fd = (loss(plus["Q"], plus["K"], plus["V"], rt) - loss(minus["Q"], minus["K"], minus["V"], rt)) / (2 * eps)
        an = float((gr["d" + name] * u).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    u = np.where(rt["support"], rng.standard_normal(rt["bias"].shape), 0.0)
    rp = dict(rt); rp["bias"] = rt["bias"] + eps * u
    rm = dict(rt); rm["bias"] = rt["bias"] - eps * u
    fd = (loss(Q, K, V, rp) - loss(Q, K, V, rm)) / (2 * eps)
    an = float((gr["dbias"] * u).sum())
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), ("bias", fd, an)


def test_stage2_backward_sigma_inf_is_masked_sdpa_autograd():
    """σ = inf (bias 0): the Stage-2 gradients are those of masked softmax attention,
    here from torch autograd of scaled_dot_product_attention with the same mask; and
    the log-sum-exp equals scipy's."""
    w, rows, rt, dO = _stage2_setup(sigma=np.inf)
    n, B, g = w.n, 16, 2
    Q, K, V = (np.asarray(x, np.float64) for x in (w.Q, w.K, w.V))
    gr = O.attend_backward(Q, rows[None], K, V, rt, B, True, n, dO)
    nb = Q.shape[0]
    mask = np.zeros((nb, 2, n, n), bool)
    for bi in range(nb):
        for r in range(2):
            for i in range(n):
                for c in np.nonzero(rt["support"][bi, r, i])[0]:
                    mask[bi, r, i, c * B:(c + 1) * B] = True
                mask[bi, r, i, (i // B) * B:i + 1] = True
    mask = np.repeat(mask, g, axis=1)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (Q, np.repeat(K, g, 1), np.repeat(V, g, 1)))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask))
    (out * torch.from_numpy(dO)).sum().backward()
    np.testing.assert_allclose(gr["dQ"], tq.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(gr["dK"], tk.grad.numpy().reshape(nb, 2, g, n, -1).sum(2), atol=1e-10)
    np.testing.assert_allclose(gr["dV"], tv.grad.numpy().reshape(nb, 2, g, n, -1).sum(2), atol=1e-10)
    d = Q.shape[-1]
    Z = np.einsum("bhid,bhjd->bhij", Q, np.repeat(K, g, 1)) / np.sqrt(d)
    Z = np.where(mask, Z, -np.inf)
    np.testing.assert_allclose(gr["lse"], scipy.special.logsumexp(Z, axis=-1), atol=1e-12)


def _chain(Q, K, V, qbar, dO, B, alpha, gamma, sigma, causal):
    """<dO, O> of the whole forward pass (Stage 0 summaries, Stage 1 routing, Stage 2)."""
    n = Q.shape[2]
    rows = np.arange(n)
    kb = O.stage0_summaries(K, qbar, B)
    rt = O.route(Q, rows[None], kb, B, alpha, gamma, sigma, causal, n)
    out = O.attend(Q, rows[None], K, V, rt, B, causal, n)
    return float((dO * out).sum()), kb, rt


@pytest.mark.parametrize("alpha,causal,sigma", [(1.5, True, 1.0), (2.0, True, 0.5), (1.0, True, 1.0),
                                                (1.25, False, 2.0)])
def test_backward_chain_matches_finite_differences(alpha, causal, sigma):
    """The whole backward chain (Stage 2, the bias -> group weights -> per-head entmax
    Jacobian -> logits, and Stage 0) against central differences of the forward
    oracle in random directions of Q, K, V and q̄; the support must not move under
    the perturbation (it is held fixed by construction)."""
    w = _small(n=96, seed=3)
    B, gamma = 16, 2.0
    Q, K, V, qbar = (np.asarray(x, np.float64) for x in (w.Q, w.K, w.V, w.qbar))
    rng = np.random.default_rng(11)
    dO = rng.standard_normal(Q.shape)
    n = Q.shape[2]
    rows = np.arange(n)
    loss, kb, rt = _chain(Q, K, V, qbar, dO, B, alpha, gamma, sigma, causal)
    g2 = O.attend_backward(Q, rows[None], K, V, rt, B, causal, n, dO)
    g1 = O.route_backward(Q, rows[None], kb, B, alpha, gamma, sigma, causal, n, g2["dbias"])
    g0 = O.summary_backward(K, qbar, B, g1["dkbar"])
    grads = dict(Q=g2["dQ"] + g1["dQ"], K=g2["dK"] + g0["dK"], V=g2["dV"], qbar=g0["dqbar"])
    assert np.abs(g1["dQ"]).max() > 0 and np.abs(g0["dqbar"]).max() > 0   # the routing path carries gradient
    eps = 1e-6
    for name in ("Q", "K", "V", "qbar"):
        args = dict(Q=Q, K=K, V=V, qbar=qbar)
        u = rng.standard_normal(args[name].shape)
        lp = dict(args); lp[name] = args[name] + eps * u
        lm = dict(args); lm[name] = args[name] - eps * u
        fp, _, rp = _chain(lp["Q"], lp["K"], lp["V"], lp["qbar"], dO, B, alpha, gamma, sigma, causal)
        fm, _, rm = _chain(lm["Q"], lm["K"], lm["V"], lm["qbar"], dO, B, alpha, gamma, sigma, causal)
        assert np.array_equal(rp["support"], rt["support"]) and np.array_equal(rm["support"], rt["support"])
        fd = (fp - fm) / (2 * eps)
        an = float((grads[name] * u).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_route_backward_zero_at_infinite_sigma():
    """σ = inf makes the bias identically zero: no gradient reaches the routing."""
    w = _small(n=64, seed=4)
    Q = np.asarray(w.Q, np.float64)
    kb = O.stage0_summaries(w.K, w.qbar, 16)
    rows = np.arange(64)
    rng = np.random.default_rng(2)
    db = rng.standard_normal((2, 2, 64, 4))
    g = O.route_backward(Q, rows[None], kb, 16, 1.5, 2.0, np.inf, True, 64, db)
    assert np.all(g["dQ"] == 0) and np.all(g["dkbar"] == 0)
