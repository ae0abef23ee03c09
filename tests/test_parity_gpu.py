"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Small shapes span several query tiles, chunks and a ragged tail so the oracle checks
every row; the five reference workloads run at full size with the launch
configuration the benchmark uses and are checked on sampled rows.
"""
import numpy as np
import pytest
import torch

from long_context_amd import inputs

pytestmark = pytest.mark.gpu

def _gu():
    from tests import gpu_util
    return gpu_util


@pytest.fixture(autouse=True)
def _need_gpu(gpu_lib):
    yield


def _log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------------------------
# Stage 0
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d,B,n", [("f32", 64, 64, 1024), ("bf16", 128, 64, 1000),
                                         ("bf16", 64, 16, 200), ("f32", 128, 128, 640),
                                         ("bf16", 128, 32, 96), ("f32", 64, 48, 480),
                                         ("bf16", 128, 256, 1024)])
def test_summaries_match_oracle(dtype, d, B, n):
    G = _gu()
    from oracle import dash_oracle as O
    w = inputs.make_prefill(b=2, h_q=4, h_kv=2, d=d, n=n, B=B, dtype=dtype, seed=1)
    K = G.to_dev(w.K, dtype)
    kbar = torch.full((2, 2, n // B + 3, d), float("nan"), device="cuda")
    from long_context_amd import dash
    dash.dash_summarize(K, torch.from_numpy(w.qbar).cuda(), kbar, B)
    torch.cuda.synchronize()
    ref = O.stage0_summaries(w.K, w.qbar, B)
    got = kbar[:, :, :n // B].cpu().numpy()
    assert np.abs(got - ref).max() <= G.TOL_KBAR
    assert torch.isnan(kbar[:, :, n // B:]).all()          # rows beyond the range untouched


def test_summary_of_chunk_range_and_zero_query():
    G = _gu()
    from oracle import dash_oracle as O
    from long_context_amd import dash
    w = inputs.make_prefill(b=1, h_q=2, h_kv=2, d=128, n=512, B=64, dtype="bf16", seed=2)
    K = G.to_dev(w.K, "bf16")
    kbar = torch.zeros((1, 2, 8, 128), device="cuda")
    dash.dash_summarize(K, torch.zeros((2, 128), device="cuda"), kbar, 64, 3, 6)
    torch.cuda.synchronize()
    got = kbar.cpu().numpy()
    mean = w.K.astype(np.float64).reshape(1, 2, 8, 64, 128).mean(3)
    assert np.abs(got[:, :, 3:6] - mean[:, :, 3:6]).max() <= 1e-5
    assert np.all(got[:, :, :3] == 0) and np.all(got[:, :, 6:] == 0)


# ------------------------------------------------------------------------------------
# Prefill: routing and attention on small shapes (all rows checked)
# ------------------------------------------------------------------------------------

SMALL = [
    # dtype, b, h_q, h_kv, d, n, B, alpha, gamma, sigma, causal
    ("f32", 1, 1, 1, 64, 1024, 64, 1.5, 1.0, 1.0, True),        # the fp32 workload's shape
    ("f32", 1, 1, 1, 64, 1024, 64, 1.5, 30.0, 1.0, True),       # sparse fp32 routing
    ("bf16", 2, 16, 2, 128, 1000, 64, 1.5, 8.0, 1.0, True),     # GQA 8, ragged tail
    ("bf16", 1, 32, 2, 128, 768, 64, 2.0, 3.0, 1.0, True),      # GQA 16, sparsemax
    ("bf16", 1, 32, 2, 128, 640, 64, 1.25, 4.0, 1.0, True),     # α = 1.25
    ("bf16", 1, 8, 2, 128, 512, 64, 1.75, 6.0, 1.0, True),      # non-integer exponent
    ("bf16", 2, 4, 2, 64, 600, 32, 1.5, 6.0, 0.5, True),        # B = 32, d = 64, σ = 0.5
    ("bf16", 1, 4, 1, 128, 700, 128, 1.5, 6.0, float("inf"), True),   # B = 128, σ = inf
    ("bf16", 1, 8, 2, 128, 520, 64, 1.5, 6.0, 1.0, False),      # non-causal with a tail
    ("f32", 1, 2, 1, 128, 300, 32, 1.5, 5.0, 1.0, True),        # fp32, d = 128
    ("bf16", 1, 16, 8, 128, 48, 64, 1.5, 5.0, 1.0, True),       # n < B: no routable chunk
    ("bf16", 1, 32, 2, 128, 900, 64, 1.0, 3.0, 1.0, True),      # α = 1: softmax routing
    ("f32", 1, 4, 2, 64, 700, 32, 1.0, 8.0, 0.5, True),         # softmax routing, fp32
]


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}-g{c[2] // c[3]}-d{c[4]}-n{c[5]}-B{c[6]}-a{c[7]}-s{c[9]}-c{int(c[10])}" for c in SMALL])
def test_prefill_small_matches_oracle(case):
    G = _gu()
    dtype, b, h_q, h_kv, d, n, B, alpha, gamma, sigma, causal = case
    w = inputs.make_prefill(b=b, h_q=h_q, h_kv=h_kv, d=d, n=n, B=B, alphas=(alpha,), gamma=gamma,
                            sigma=sigma, causal=causal, dtype=dtype, seed=3)
    _log(f"prefill case {case}")
    g = G.gpu_prefill(w)
    rows = np.arange(n)
    kb, rt, Oref = G.oracle_prefill_rows(w, rows)
    if n // B > 0:
        assert np.abs(g["kbar"][:, :, :n // B].cpu().numpy() - kb).max() <= G.TOL_KBAR
    nex, tot = G.compare_route(g, rt, rows, n // B)
    err = G.compare_out(g["O"].cpu().numpy(), Oref, rt["margin"] <= G.MARGIN, h_q // h_kv, dtype)
    _log(f"  exempt rows {nex}/{tot}, output error {err:.3e}")


def test_prefill_bf16_output_dtype():
    G = _gu()
    w = inputs.make_prefill(b=1, h_q=16, h_kv=2, d=128, n=512, B=64, gamma=6.0, dtype="bf16", seed=4)
    g32 = G.gpu_prefill(w)
    g16 = G.gpu_prefill(w, out_dtype=torch.bfloat16)
    ref = g32["O"].to(torch.bfloat16).float()
    assert torch.equal(g16["O"].float(), ref)


def test_prefill_is_deterministic():
    G = _gu()
    w = inputs.make_prefill(b=1, h_q=32, h_kv=2, d=128, n=1024, B=64, gamma=3.0, dtype="bf16", seed=5)
    a = G.gpu_prefill(w)
    b = G.gpu_prefill(w)
    for k in ("kbar", "cnt", "w", "O"):
        assert torch.equal(a[k], b[k]), k
    listed = torch.arange(a["idx"].shape[-1], device="cuda") < a["cnt"][..., None]
    assert torch.equal(a["idx"][listed], b["idx"][listed])
    assert torch.equal(a["bias"][listed], b["bias"][listed])


# ------------------------------------------------------------------------------------
# Decode on small shapes
# ------------------------------------------------------------------------------------

def gpu_decode(w, seq_len, kbar=None, with_lists=True, top_k=0):
    G = _gu()
    from long_context_amd import dash
    Q, K, V = G.to_dev(w.Q, w.dtype), G.to_dev(w.K, w.dtype), G.to_dev(w.V, w.dtype)
    b, h_q, _, d = w.Q.shape
    L_cap = w.K.shape[2]
    T = L_cap // w.B
    if kbar is None:
        kbar = dash.alloc_kbar(b, w.h_kv, T, d)
        dash.dash_summarize(K, torch.from_numpy(w.qbar).cuda(), kbar, w.B)
    sl = torch.from_numpy(np.asarray(seq_len, np.int32)).cuda()
    ws = dash.alloc_decode_ws(b, h_q, w.h_kv, L_cap, d, w.B)
    Oo = torch.empty((b, h_q, 1, d), device="cuda")
    cap = max((L_cap - 1) // w.B, 1)
    idx = torch.full((b, w.h_kv, cap), -1, dtype=torch.int32, device="cuda")
    bias = torch.zeros((b, w.h_kv, cap), device="cuda")
    cnt = torch.zeros((b, w.h_kv), dtype=torch.int32, device="cuda")
    wo = torch.zeros((b, w.h_kv, kbar.shape[2]), device="cuda")
    if with_lists:
        dash.dash_attend_decode(Q, K, V, kbar, sl, w.B, w.alpha, w.gamma, w.sigma, Oo, ws,
                                idx, bias, cnt, wo, top_k=top_k)
    else:
        dash.dash_attend_decode(Q, K, V, kbar, sl, w.B, w.alpha, w.gamma, w.sigma, Oo, ws, top_k=top_k)
    torch.cuda.synchronize()
    return dict(O=Oo, idx=idx, bias=bias, cnt=cnt, w=wo, kbar=kbar)


def check_decode(w, seq_len, g, top_k=0):
    G = _gu()
    from oracle import dash_oracle as O
    kb = O.stage0_summaries(w.K, w.qbar, w.B)
    res = O.decode(w.Q, w.K, w.V, kb, seq_len, w.B, w.alpha, w.gamma, w.sigma, keep_heads=True, top_k=top_k)
    nex = 0
    errs = []
    worst = 0.0
    tols = []
    bias = g["bias"].cpu().numpy()
    for bi, rt in enumerate(res["routes"]):
        L = int(seq_len[bi])
        T = (L - 1) // w.B
        ex = G.exempt_rows(rt)[0, :, 0]                     # [h_kv]
        nex += int(ex.sum())
        tolb = G.bias_tolerance(w.Q[bi:bi + 1], kb[bi:bi + 1, :, :L // w.B], rt, w.alpha, w.gamma, w.sigma)
        if T > 0:
            dw = np.abs(g["w"][bi, :, :T].cpu().numpy() - rt["w"][0, :, 0, :T]).max()
            assert dw <= G.TOL_W, f"b={bi}: weights differ by {dw}"
        for r in range(w.h_kv):
            if ex[r]:
                continue
            ref = np.nonzero(rt["support"][0, r, 0])[0]
            c = int(g["cnt"][bi, r])
            assert c == ref.size, f"b={bi} r={r}: cnt {c} != {ref.size}"
            assert np.array_equal(g["idx"][bi, r, :c].cpu().numpy(), ref)
            worst = max(worst, G.compare_bias(bias[bi, r, :c], ref, rt["bias"][0, r, 0], tolb[0, r, 0],
                                              f"b={bi} r={r}"))
            tols.append(tolb[0, r, 0][ref])
        errs.append(G.compare_out(g["O"][bi:bi + 1].cpu().numpy(), res["O"][bi:bi + 1],
                                  ex[None, :, None], w.g, w.dtype))
    G.check_exempt_count(nex, len(res["routes"]) * w.h_kv)
    if tols and np.concatenate(tols).size:
        med = float(np.median(np.concatenate(tols)))
        _log(f"  bias: worst |Δd|/bound {worst:.3e}, median bound {med:.2e}")
        assert med <= G.BIAS_MEDIAN_MAX, f"bias bound uninformative (median {med:.2e})"
    return nex, max(errs)


TOPK = [
    # dtype, b, h_q, h_kv, d, n, B, alpha, gamma, sigma, top_k
    ("bf16", 1, 32, 2, 128, 900, 64, 1.0, 3.0, 1.0, 4),          # softmax routing, budget 4
    ("bf16", 1, 16, 2, 128, 1000, 64, 1.5, 2.0, 1.0, 3),         # entmax routing cut to 3
    ("f32", 1, 4, 2, 64, 700, 32, 1.5, 2.0, float("inf"), 2),    # fp32, σ = inf
    ("bf16", 1, 16, 2, 128, 40000, 32, 1.0, 6.0, 1.0, 16),       # 1250 chunks (4 wavefronts per row)
]


@pytest.mark.parametrize("case", TOPK, ids=[f"{c[0]}-g{c[2] // c[3]}-n{c[5]}-a{c[7]}-k{c[10]}" for c in TOPK])
def test_prefill_topk_matches_oracle(case):
    G = _gu()
    dtype, b, h_q, h_kv, d, n, B, alpha, gamma, sigma, k = case
    w = inputs.make_prefill(b=b, h_q=h_q, h_kv=h_kv, d=d, n=n, B=B, alphas=(alpha,), gamma=gamma,
                            sigma=sigma, causal=True, dtype=dtype, seed=11)
    _log(f"top-k case {case}")
    g = G.gpu_prefill(w, top_k=k)
    rows = np.arange(n) if n <= 2048 else _sample_rows(n, B, 96, 5)
    kb, rt, Oref = G.oracle_prefill_rows(w, rows, top_k=k)
    nex, tot = G.compare_route(g, rt, rows, n // B)
    assert (g["cnt"].cpu().numpy() <= k).all()
    err = G.compare_out(g["O"][:, :, rows].cpu().numpy(), Oref, G.exempt_rows(rt), h_q // h_kv, dtype)
    _log(f"  exempt rows {nex}/{tot}, output error {err:.3e}")


def test_route_mask_matches_lists_and_oracle():
    """Bitpacked mask of the GPU's routed lists: equal to the lists packed on the host
    for every row, and to the oracle's support off the exempt rows."""
    G = _gu()
    from oracle import dash_oracle as O
    from long_context_amd import dash
    w = inputs.make_prefill(b=2, h_q=16, h_kv=2, d=128, n=2500, B=32, alphas=(1.5,), gamma=4.0,
                            sigma=1.0, causal=True, dtype="bf16", seed=21)
    _log("mask case bf16 g8 n2500 B32")
    g = G.gpu_prefill(w)
    T = 2500 // 32
    words = (T + 31) // 32
    mask = torch.zeros((2, 2, 2500, words), dtype=torch.int32, device="cuda")
    dash.dash_route_mask(g["idx"], g["cnt"], T, mask)
    got = mask.cpu().numpy().view(np.uint32)
    idx, cnt = g["idx"].cpu().numpy(), g["cnt"].cpu().numpy()
    sup = np.zeros((2, 2, 2500, T), bool)
    for ix in np.ndindex(*cnt.shape):
        sup[ix][idx[ix][:cnt[ix]]] = True
    assert np.array_equal(got, O.route_mask(sup, words))
    rows = _sample_rows(2500, 32, 64, 9)
    _, rt, _ = G.oracle_prefill_rows(w, rows)
    ref = O.route_mask(rt["support"], words)
    keep = ~G.exempt_rows(rt)
    assert np.array_equal(got[:, :, rows][keep], ref[keep])


DEC = [
    # dtype, b, h_q, h_kv, d, L, B, alpha, gamma, seq_len
    ("bf16", 3, 32, 2, 128, 4096, 64, 1.5, 1.0, [4096, 4000, 65]),
    ("bf16", 2, 16, 2, 128, 5000, 128, 1.5, 6.0, [5000, 4097]),
    ("bf16", 2, 8, 2, 64, 3000, 32, 2.0, 4.0, [3000, 33]),
    ("bf16", 2, 32, 2, 128, 2048, 64, 1.25, 2.0, [2048, 64]),
    ("f32", 2, 4, 2, 64, 1500, 64, 1.5, 3.0, [1500, 1]),
    ("bf16", 2, 32, 2, 128, 4096, 64, 1.0, 3.0, [4096, 700]),   # α = 1: softmax routing
]


@pytest.mark.parametrize("case", DEC, ids=[f"{c[0]}-g{c[2] // c[3]}-L{c[5]}-B{c[6]}-a{c[7]}" for c in DEC])
def test_decode_small_matches_oracle(case):
    dtype, b, h_q, h_kv, d, L, B, alpha, gamma, seq_len = case
    _log(f"decode case {case}")
    w = inputs.make_decode(b=b, h_q=h_q, h_kv=h_kv, d=d, L=L, B=B, alphas=(alpha,), gamma=gamma,
                           dtype=dtype, seed=6, seq_len=seq_len)
    g = gpu_decode(w, seq_len)
    nex, err = check_decode(w, np.asarray(seq_len), g)
    _log(f"  exempt groups {nex}, output error {err:.3e}")
    g2 = gpu_decode(w, seq_len, kbar=g["kbar"], with_lists=False)
    assert torch.equal(g["O"], g2["O"])


DEC_GROUP = [
    # beyond 1024 chunks with bf16 queries the group router routes (one workgroup per
    # group); dtype, b, h_q, h_kv, d, L, B, alpha, gamma, seq_len
    ("bf16", 3, 32, 2, 64, 36000, 32, 1.75, 3.0, [36000, 33000, 40]),    # d = 64, p non-integer, a short row
    ("bf16", 2, 16, 2, 128, 70000, 64, 1.25, 2.0, [70000, 65600]),       # g = 8, p = 4
    ("bf16", 2, 32, 2, 128, 40000, 32, 2.0, 4.0, [40000, 1]),            # sparsemax; L = 1 routes nothing
    ("bf16", 2, 32, 2, 128, 36000, 32, 1.0, 3.0, [36000, 35000]),        # softmax routing
]


@pytest.mark.parametrize("case", DEC_GROUP, ids=[f"g{c[2] // c[3]}-d{c[4]}-L{c[5]}-a{c[7]}" for c in DEC_GROUP])
def test_decode_group_router_matches_oracle(case):
    dtype, b, h_q, h_kv, d, L, B, alpha, gamma, seq_len = case
    _log(f"decode group-router case {case}")
    w = inputs.make_decode(b=b, h_q=h_q, h_kv=h_kv, d=d, L=L, B=B, alphas=(alpha,), gamma=gamma,
                           dtype=dtype, seed=62, seq_len=seq_len)
    assert (L - 1) // B > 1024
    g = gpu_decode(w, seq_len)
    nex, err = check_decode(w, np.asarray(seq_len), g)
    _log(f"  exempt groups {nex}, output error {err:.3e}, counts {g['cnt'].cpu().numpy().ravel().tolist()}")


DEC_TOPK = [
    # dtype, b, h_q, h_kv, d, L, B, alpha, gamma, seq_len, top_k
    ("bf16", 3, 32, 2, 128, 4096, 64, 1.0, 3.0, [4096, 3000, 700], 8),     # softmax routing: exactly 8
    ("bf16", 2, 16, 2, 128, 5000, 64, 1.5, 1.0, [5000, 2100], 5),          # entmax support cut to 5
    ("bf16", 2, 32, 2, 128, 40000, 32, 1.5, 0.5, [40000, 39000], 64),      # 1249 chunks, budget 64
]


@pytest.mark.parametrize("case", DEC_TOPK, ids=[f"g{c[2] // c[3]}-L{c[5]}-a{c[7]}-k{c[10]}" for c in DEC_TOPK])
def test_decode_topk_matches_oracle(case):
    """A fixed routing budget in decode: each group keeps its top_k largest weights
    (the oracle's route(..., top_k)); lists, biases and outputs as in the other decode
    checks, exempting groups whose log-weight gap at the cut is within 1e-5."""
    dtype, b, h_q, h_kv, d, L, B, alpha, gamma, seq_len, k = case
    _log(f"decode top-k case {case}")
    w = inputs.make_decode(b=b, h_q=h_q, h_kv=h_kv, d=d, L=L, B=B, alphas=(alpha,), gamma=gamma,
                           dtype=dtype, seed=61, seq_len=seq_len)
    g = gpu_decode(w, seq_len, top_k=k)
    assert (g["cnt"].cpu().numpy() <= k).all()
    nex, err = check_decode(w, np.asarray(seq_len), g, top_k=k)
    _log(f"  exempt groups {nex}, output error {err:.3e}, counts {g['cnt'].cpu().numpy().ravel().tolist()}")


def test_decode_equals_last_prefill_row():
    G = _gu()
    w = inputs.make_prefill(b=1, h_q=16, h_kv=2, d=128, n=1000, B=64, gamma=4.0, dtype="bf16", seed=7)
    pre = G.gpu_prefill(w)
    wd = inputs.make_decode(b=1, h_q=16, h_kv=2, d=128, L=1000, B=64, gamma=4.0, dtype="bf16", seed=7)
    wd.Q = np.ascontiguousarray(w.Q[:, :, -1:])
    wd.K, wd.V, wd.qbar = w.K, w.V, w.qbar
    dec = gpu_decode(wd, [1000], kbar=pre["kbar"])
    r = pre["cnt"][0, :, -1]
    assert torch.equal(dec["cnt"][0], r)
    for kv in range(2):                                   # each group's list up to its own count
        c = int(r[kv])
        assert torch.equal(dec["idx"][0, kv, :c], pre["idx"][0, kv, -1, :c]), f"group {kv}: lists differ"
    # both paths round P to bf16 (in different tile orders), so they agree to the
    # bf16 output tolerance rather than bit for bit
    o1 = pre["O"][:, :, -1:].cpu().numpy().astype(np.float64)
    o2 = dec["O"].cpu().numpy().astype(np.float64)
    rel = np.abs(o1 - o2).max(-1) / np.sqrt((o1 ** 2).mean(-1))
    assert rel.max() <= 2e-2


# ------------------------------------------------------------------------------------
# Rows longer than one router wavefront holds (512 chunks): the chunks of a row are
# split over 2 or 4 cooperating wavefronts (prefill) / more values per lane (decode)
# ------------------------------------------------------------------------------------

LONG = [
    # dtype, b, h_q, h_kv, d, n, B, alpha, gamma, sigma
    ("bf16", 1, 32, 2, 128, 20032, 32, 1.5, 4.0, 1.0),     # 626 chunks: 2 wavefronts per row group
    ("bf16", 1, 16, 2, 128, 40000, 32, 1.5, 6.0, 1.0),     # 1250 chunks: 4 wavefronts
    ("f32", 1, 4, 2, 64, 24000, 32, 2.0, 5.0, 1.0),        # 750 chunks, fp32 queries: 2 wavefronts
    ("bf16", 1, 2, 2, 64, 35200, 32, 1.5, 4.0, 1.0),       # g = 1, 1100 chunks: 16 rows x 4 wavefronts
    # 129-512 chunks in one wavefront per row group (four-wavefront workgroups), g < 16:
    # fewer DPP levels in the group average and several rows per group of 16 pairs
    ("bf16", 1, 16, 2, 128, 12000, 32, 1.5, 4.0, 1.0),     # g = 8, 375 chunks, 2 rows per group
    ("bf16", 1, 8, 2, 64, 10000, 64, 1.25, 3.0, 1.0),      # g = 4, 156 chunks, 4 rows per group
    ("bf16", 1, 4, 4, 64, 9000, 32, 2.0, 5.0, 1.0),        # g = 1, 281 chunks, 16 rows: workgroup of two groups
    ("bf16", 1, 16, 2, 128, 10000, 32, 1.0, 3.0, 1.0),     # α = 1 (softmax routing), g = 8, 312 chunks
]


@pytest.mark.parametrize("case", LONG, ids=[f"{c[0]}-g{c[2] // c[3]}-n{c[5]}-B{c[6]}" for c in LONG])
def test_prefill_long_rows(case):
    G = _gu()
    dtype, b, h_q, h_kv, d, n, B, alpha, gamma, sigma = case
    w = inputs.make_prefill(b=b, h_q=h_q, h_kv=h_kv, d=d, n=n, B=B, alphas=(alpha,), gamma=gamma,
                            sigma=sigma, causal=True, dtype=dtype, seed=5)
    _log(f"long prefill case {case}")
    g = G.gpu_prefill(w)
    rows = _sample_rows(w.n, w.B, 40, 9)
    kb, rt, Oref = G.oracle_prefill_rows(w, rows)
    nex, tot = G.compare_route(g, rt, rows, w.n // w.B)
    err = G.compare_out(g["O"][:, :, rows].cpu().numpy(), Oref, rt["margin"] <= G.MARGIN, w.g, dtype)
    _log(f"long prefill {case}: exempt {nex}/{tot}, output error {err:.3e}")


@pytest.mark.parametrize("L", [40000, 35232])
def test_decode_long_rows(L):
    seq = [L, L - 1000]
    w = inputs.make_decode(b=2, h_q=32, h_kv=2, d=128, L=L, B=32, alphas=(1.5,), gamma=3.0,
                           sigma=1.0, dtype="bf16", seed=6, seq_len=seq)
    _log(f"long decode L={L} seq={seq}")
    g = gpu_decode(w, seq)
    nex, err = check_decode(w, seq, g)
    _log(f"long decode L={L}: exempt {nex}, output error {err:.3e}")


# ------------------------------------------------------------------------------------
# The five reference workloads at full size (sampled rows)
# ------------------------------------------------------------------------------------

def _sample_rows(n, B, k, seed):
    rng = np.random.default_rng(seed)
    fixed = np.array([0, 1, B - 1, B, B + 1, 2 * B - 1, n // 2, n - B - 1, n - B, n - 2, n - 1])
    return np.unique(np.concatenate([fixed, rng.choice(n, size=k, replace=False)]))


def test_workload_prefill_1k_fp32_all_rows():
    G = _gu()
    w = inputs.prefill_1k_fp32()
    g = G.gpu_prefill(w)
    rows = np.arange(w.n)
    kb, rt, Oref = G.oracle_prefill_rows(w, rows)
    nex, tot = G.compare_route(g, rt, rows, w.n // w.B)
    err = G.compare_out(g["O"].cpu().numpy(), Oref, rt["margin"] <= G.MARGIN, 1, "f32")
    _log(f"prefill_1k_fp32: exempt {nex}/{tot}, max |dO| {err:.3e}")


def test_workload_prefill_8k_needles():
    G = _gu()
    w = inputs.prefill_8k_gqa8_needles()
    g = G.gpu_prefill(w)
    rows = _sample_rows(w.n, w.B, 600, 11)
    kb, rt, Oref = G.oracle_prefill_rows(w, rows)
    assert np.abs(g["kbar"].cpu().numpy() - kb).max() <= G.TOL_KBAR
    nex, tot = G.compare_route(g, rt, rows, w.n // w.B)
    err = G.compare_out(g["O"][:, :, rows].cpu().numpy(), Oref, rt["margin"] <= G.MARGIN, w.g, "bf16")
    _log(f"prefill_8k_gqa8_needles: exempt {nex}/{tot}, row error {err:.3e}")


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_workload_prefill_32k_clusters(alpha):
    G = _gu()
    w = _cached_32k()
    g = G.gpu_prefill(w, alpha=alpha)
    rows = _sample_rows(w.n, w.B, 150, 12)
    kb, rt, Oref = G.oracle_prefill_rows(w, rows, kbar_or=_cached_32k_kbar(), alpha=alpha)
    nex, tot = G.compare_route(g, rt, rows, w.n // w.B)
    err = G.compare_out(g["O"][:, :, rows].cpu().numpy(), Oref, rt["margin"] <= G.MARGIN, w.g, "bf16")
    _log(f"prefill_32k_clusters alpha={alpha}: exempt {nex}/{tot}, row error {err:.3e}")


_C32 = {}


def _cached_32k():
    if "w" not in _C32:
        _C32["w"] = inputs.prefill_32k_clusters()
    return _C32["w"]


def _cached_32k_kbar():
    from oracle import dash_oracle as O
    if "kb" not in _C32:
        w = _cached_32k()
        _C32["kb"] = O.stage0_summaries(w.K, w.qbar, w.B)
    return _C32["kb"]


@pytest.mark.parametrize("name", ["decode_32k_b16", "decode_128k_b4"])
def test_workload_decode(name):
    w = inputs.make(name)
    g = gpu_decode(w, w.seq_len)
    nex, err = check_decode(w, w.seq_len, g)
    _log(f"{name}: exempt groups {nex}, row error {err:.3e}, routed {g['cnt'].cpu().numpy().ravel().tolist()}")


# ------------------------------------------------------------------------------------
# Paged KV cache and an incremental decode loop
# ------------------------------------------------------------------------------------

def _to_pages(Kc, B, perm):
    """[b, h_kv, L_cap, d] -> pages [P, h_kv, B, d] with chunk c of sequence b in page
    perm[b * pps + c]; unused pages hold noise."""
    b, h_kv, L_cap, d = Kc.shape
    pps = L_cap // B
    P = perm.max() + 1 + 3
    pages = torch.randn((P, h_kv, B, d), device=Kc.device).to(Kc.dtype)
    src = Kc.reshape(b, h_kv, pps, B, d).permute(0, 2, 1, 3, 4).reshape(b * pps, h_kv, B, d)
    pages[torch.from_numpy(perm).to(Kc.device).long()] = src
    return pages


def test_paged_decode_equals_contiguous():
    """Pages of one chunk each in a shuffled order: summaries and decode outputs equal
    the contiguous cache's bit for bit (same kernels, other addresses)."""
    G = _gu()
    from long_context_amd import dash
    b, h_q, h_kv, d, B, L_cap = 3, 16, 2, 128, 64, 2048
    seq_len = [2048, 1500, 65]
    w = inputs.make_decode(b=b, h_q=h_q, h_kv=h_kv, d=d, L=L_cap, B=B, alphas=(1.5,), gamma=3.0,
                           dtype="bf16", seed=31, seq_len=seq_len)
    _log("paged decode bf16 g8 L2048 B64")
    ref = gpu_decode(w, seq_len)
    pps = L_cap // B
    perm = np.random.default_rng(2).permutation(b * pps + 5)[:b * pps].astype(np.int32)
    K, V = G.to_dev(w.K, "bf16"), G.to_dev(w.V, "bf16")
    Kp, Vp = _to_pages(K, B, perm), _to_pages(V, B, perm)
    table = torch.from_numpy(perm.reshape(b, pps)).cuda()
    kbar = dash.alloc_kbar(b, h_kv, pps, d)
    dash.dash_summarize_paged(Kp, torch.from_numpy(w.qbar).cuda(), kbar, table, B, 0, pps)
    torch.cuda.synchronize()
    assert torch.equal(kbar[:, :, :pps], ref["kbar"][:, :, :pps])
    Q = G.to_dev(w.Q, "bf16")
    sl = torch.from_numpy(np.asarray(seq_len, np.int32)).cuda()
    ws = dash.alloc_decode_ws(b, h_q, h_kv, L_cap, d, B)
    O = torch.empty((b, h_q, 1, d), device="cuda")
    dash.dash_attend_decode_paged(Q, Kp, Vp, kbar, sl, table, B, w.alpha, w.gamma, w.sigma, O, ws)
    torch.cuda.synchronize()
    assert torch.equal(O, ref["O"])


def test_incremental_decode_loop_matches_oracle():
    """A serving loop on a paged cache: one token per step across three chunk
    boundaries, each chunk summarised once when it completes; every step's output
    matches the oracle's decode of the same prefix."""
    G = _gu()
    from long_context_amd import dash
    from oracle import dash_oracle as O
    b, h_q, h_kv, d, B, L_cap = 2, 8, 2, 64, 32, 256
    w = inputs.make_decode(b=b, h_q=h_q, h_kv=h_kv, d=d, L=L_cap, B=B, alphas=(1.5,), gamma=4.0,
                           dtype="bf16", seed=41, seq_len=[L_cap, L_cap])
    _log("incremental decode loop bf16 g4 B32")
    pps = L_cap // B
    perm = np.random.default_rng(3).permutation(b * pps).astype(np.int32)
    K, V = G.to_dev(w.K, "bf16"), G.to_dev(w.V, "bf16")
    Kp, Vp = _to_pages(K, B, perm), _to_pages(V, B, perm)
    table = torch.from_numpy(perm.reshape(b, pps)).cuda()
    qbar = torch.from_numpy(w.qbar).cuda()
    kbar = dash.alloc_kbar(b, h_kv, pps, d)
    ws = dash.alloc_decode_ws(b, h_q, h_kv, L_cap, d, B)
    kb_ref = O.stage0_summaries(w.K, w.qbar, B)
    done = 0
    worst = 0.0
    for L in range(2 * B - 3, 4 * B + 4):                 # crosses the ends of chunks 1, 2, 3
        while done < (L - 1) // B:                         # chunks complete before the query
            dash.dash_summarize_paged(Kp, qbar, kbar, table, B, done, done + 1)
            done += 1
        sl = torch.full((b,), L, dtype=torch.int32, device="cuda")
        Qs = torch.from_numpy(w.Q).to("cuda", torch.bfloat16)
        Og = torch.empty((b, h_q, 1, d), device="cuda")
        dash.dash_attend_decode_paged(Qs, Kp, Vp, kbar, sl, table, B, w.alpha, w.gamma, w.sigma, Og, ws)
        torch.cuda.synchronize()
        res = O.decode(w.Q, w.K, w.V, kb_ref, np.full(b, L), B, w.alpha, w.gamma, w.sigma)
        for bi in range(b):
            ex = G.exempt_rows(res["routes"][bi])[0, :, 0]
            worst = max(worst, G.compare_out(Og[bi:bi + 1].cpu().numpy(), res["O"][bi:bi + 1],
                                             ex[None, :, None], h_q // h_kv, "bf16"))
    assert done == (4 * B + 3 - 1) // B
    _log(f"  worst per-row relative error {worst:.3e}")


def test_decode_graph_replay_matches_eager():
    """A decode step captured in a HIP graph (a serving loop's form): the entry point
    records no memset or allocation, so each replay, with new query values copied into
    the captured buffer and eager decode work and synchronisation in between, equals
    the eager step on the same inputs bit for bit."""
    from long_context_amd import dash
    seq_len = [4096, 3000, 700]
    w = inputs.make_decode(b=3, h_q=16, h_kv=2, d=128, L=4096, B=64, alphas=(1.5,), gamma=4.0, dtype="bf16",
                           seed=17, seq_len=seq_len)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.bfloat16)
    Q, K, V = dev(w.Q), dev(w.K), dev(w.V)
    kbar = dash.alloc_kbar(3, 2, w.n // w.B, 128)
    dash.dash_summarize(K, torch.from_numpy(w.qbar).cuda(), kbar, w.B)
    sl = torch.tensor(seq_len, dtype=torch.int32, device="cuda")
    ws = dash.alloc_decode_ws(3, 16, 2, w.n, 128, w.B)
    ws_eager = dash.alloc_decode_ws(3, 16, 2, w.n, 128, w.B)
    O = torch.empty((3, 16, 1, 128), device="cuda")
    O_eager = torch.empty_like(O)
    step = lambda out, wsp: dash.dash_attend_decode(Q, K, V, kbar, sl, w.B, 1.5, 4.0, 1.0, out, wsp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step(O, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(O, ws)
    rng = np.random.default_rng(18)
    for k in range(4):
        Q.copy_(dev(inputs.round_bf16(rng.standard_normal(Q.shape).astype(np.float32))))
        O.zero_()
        graph.replay()
        torch.cuda.synchronize()
        step(O_eager, ws_eager)                      # eager work between replays
        torch.cuda.synchronize()
        _log(f"graph replay {k}: max |diff| {float((O - O_eager).abs().max()):.3e}")
        assert torch.equal(O, O_eager), f"replay {k} differs from the eager step"


# ------------------------------------------------------------------------------------
# The pages' efficiency operating points (paper review section 六, 6.2 efficiency
# table): 96K-token prefill and decode at batch 24, B = 64, 32 query / 2 KV heads,
# γ calibrated to the stated group sparsity; the benchmark's launch, sampled rows.
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("sparsity", [0.75, 0.9375])
def test_efficiency_prefill_96k_sampled_rows(sparsity):
    """1536 chunks per row group: the router splits every row over four wavefronts."""
    G = _gu()
    w = inputs.efficiency_prefill(96 * 1024, sparsity)
    _log(f"efficiency prefill 96K sparsity {sparsity} gamma {w.gamma}")
    g = G.gpu_prefill(w)
    rows = _sample_rows(w.n, w.B, 30, 13)
    kb, rt, Oref = G.oracle_prefill_rows(w, rows)
    assert np.abs(g["kbar"].cpu().numpy() - kb).max() <= G.TOL_KBAR
    nex, tot = G.compare_route(g, rt, rows, w.n // w.B)
    err = G.compare_out(g["O"][:, :, rows].cpu().numpy(), Oref, rt["margin"] <= G.MARGIN, w.g, "bf16")
    from oracle import dash_oracle as O
    _log(f"efficiency prefill 96K: exempt {nex}/{tot}, row error {err:.3e}, "
         f"sampled-row group sparsity {O.group_sparsity(rt):.3f}")


@pytest.mark.parametrize("sparsity", [0.75, 0.9375])
def test_efficiency_decode_96k_b24(sparsity):
    w = inputs.efficiency_decode(sparsity)
    _log(f"efficiency decode 96K b24 sparsity {sparsity} gamma {w.gamma}")
    g = gpu_decode(w, w.seq_len)
    nex, err = check_decode(w, w.seq_len, g)
    cnt = g["cnt"].cpu().numpy()
    vis = (w.seq_len - 1) // w.B
    _log(f"efficiency decode 96K: exempt groups {nex}, row error {err:.3e}, "
         f"group sparsity {1.0 - cnt.sum() / (vis[:, None] * np.ones_like(cnt)).sum():.3f}")


def test_prefill_stage2_beyond_4k_chunks():
    """Stage 2 over 4097 chunks (d = 128, 64-token tiles): the tile tables no longer fit
    LDS beside two groups of two tiles, so the kernel takes one tile per barrier. The
    router stops at 2048 chunks, so the lists are made here (the first, middle and
    last visible chunk of each row, random biases) and the oracle's attention
    (Prop. 4.1 form) runs on the same lists for sampled rows."""
    from long_context_amd import dash
    from oracle import dash_oracle as O
    G = _gu()
    B, d, T = 64, 128, 4097
    n = T * B
    _log(f"stage-2 case n={n} T={T} (one tile per barrier)")
    rng = np.random.default_rng(21)
    Qh = rng.standard_normal((1, 1, n, d), dtype=np.float32)
    Kh = rng.standard_normal((1, 1, n, d), dtype=np.float32)
    Vh = rng.standard_normal((1, 1, n, d), dtype=np.float32)
    Q, K, V = (G.to_dev(x, "bf16") for x in (Qh, Kh, Vh))
    Qr, Kr, Vr = (x.float().cpu().numpy() for x in (Q, K, V))      # the bf16 values both sides use
    vis = np.arange(n) // B
    cnt = np.minimum(vis, 3).astype(np.int32)
    idx = np.zeros((n, 3), np.int32)
    idx[:, 1] = np.where(cnt == 3, vis // 2, np.maximum(vis - 1, 0))
    idx[:, 2] = np.maximum(vis - 1, 0)
    bias = rng.uniform(-1.0, 1.0, (n, 3)).astype(np.float32)
    # the lists are sized for every visible chunk (list_cap >= T); only the first three
    # entries of a row are filled
    idx_d = torch.zeros((1, 1, n, T), dtype=torch.int32, device="cuda")
    bias_d = torch.zeros((1, 1, n, T), device="cuda")
    idx_d[0, 0, :, :3] = torch.from_numpy(idx).cuda()
    bias_d[0, 0, :, :3] = torch.from_numpy(bias).cuda()
    O_gpu = torch.full((1, 1, n, d), float("nan"), device="cuda")
    dash.dash_attend_prefill(Q, K, V, idx_d, bias_d, torch.from_numpy(cnt[None, None]).cuda(), O_gpu, B, True)
    torch.cuda.synchronize()
    rows = _sample_rows(n, B, 24, 5)
    rows = np.unique(np.concatenate([rows, [2 * B, 3 * B + 5]]))
    R = rows.size
    support = np.zeros((1, 1, R, T), bool)
    bmat = np.zeros((1, 1, R, T))
    for k, i in enumerate(rows):
        for e in range(cnt[i]):
            support[0, 0, k, idx[i, e]] = True
            bmat[0, 0, k, idx[i, e]] = bias[i, e]
    rt = dict(support=support, bias=bmat)
    ref = O.attend(Qr[:, :, rows], rows[None], Kr, Vr, rt, B, True, n)
    got = O_gpu[0, 0, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    err = np.abs(got - ref[0, 0]).max(-1) / np.sqrt((ref[0, 0] ** 2).mean(-1))
    _log(f"  rows {R}, worst per-row relative error {err.max():.2e}")
    assert np.isfinite(got).all()
    assert err.max() <= G.TOL_BF16_ROW
