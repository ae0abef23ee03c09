"""GPU parity of ragged prefill batches (the *_varlen entry points) against the CPU
oracle run on each sequence alone.

DashAttention's stages are defined per sequence (paper review section 三: Eq. 4 over
a sequence's complete chunks, Eq. 6 over the chunks a row may see, Eq. 10 over its
routed chunks and diagonal branch), so a batch of sequences of different lengths
padded to one n must give, for every sequence, what the oracle gives on that
sequence's first seq_len[b] rows. The padding of Q, K and V is filled with NaN on
the device: a single read of it would surface in the compared outputs. Rows at or
past seq_len[b] must get empty lists and leave O, lse and k̄ untouched.
"""
import dataclasses

import numpy as np
import pytest
import torch

from long_context_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(gpu_lib):
    yield


def _gu():
    from tests import gpu_util
    return gpu_util


def _nan_padded(x, lengths, dtype):
    """Device copy of x [b, h, n, d] with rows at or past lengths[b] set to NaN."""
    t = _gu().to_dev(x, dtype)
    for bi, L in enumerate(lengths):
        t[bi, :, max(L, 0):] = float("nan")
    return t


def gpu_varlen(w, lengths, causal=None, top_k=0, out_dtype=torch.float32):
    from long_context_amd import dash
    causal = w.causal if causal is None else causal
    b, h_q, n, d = w.Q.shape
    T = n // w.B
    Q = _nan_padded(w.Q, lengths, w.dtype)
    K = _nan_padded(w.K, lengths, w.dtype)
    V = _nan_padded(w.V, lengths, w.dtype)
    sl = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    qbar = torch.from_numpy(w.qbar).cuda()
    kbar = torch.full((b, w.h_kv, T, d), float("nan"), device="cuda")
    dash.dash_summarize_varlen(K, qbar, kbar, sl, w.B)
    idx, bias, cnt, wo = dash.alloc_route(b, w.h_kv, n, T, with_w=True)
    cnt.fill_(-7)
    wo.fill_(float("nan"))
    dash.dash_route_varlen(Q, kbar, sl, w.B, w.alpha, w.gamma, w.sigma, causal, idx, bias, cnt, wo, top_k=top_k)
    Oo = torch.full((b, h_q, n, d), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((b, h_q, n), float("nan"), device="cuda")
    dash.dash_attend_prefill_varlen(Q, K, V, sl, idx, bias, cnt, Oo, w.B, causal, lse=lse)
    torch.cuda.synchronize()
    return dict(kbar=kbar, idx=idx, bias=bias, cnt=cnt, w=wo, O=Oo, lse=lse)


def check_varlen(w, lengths, causal=None, top_k=0):
    G = _gu()
    causal = w.causal if causal is None else causal
    g = gpu_varlen(w, lengths, causal, top_k)
    n = w.n
    T = n // w.B
    gq = w.h_q // w.h_kv
    for bi, L0 in enumerate(lengths):
        L = min(max(L0, 0), n)
        Tb = L // w.B
        print(f"  sequence {bi}: {L} tokens, {Tb} chunks", flush=True)
        # padding: empty lists, untouched outputs and summaries
        assert (g["cnt"][bi, :, L:] == 0).all(), "padding rows must get empty lists"
        assert torch.isnan(g["O"][bi, :, L:]).all(), "padding rows of O were written"
        assert torch.isnan(g["lse"][bi, :, L:]).all(), "padding rows of lse were written"
        assert torch.isnan(g["kbar"][bi, :, Tb:]).all(), "summaries past the sequence were written"
        if L == 0:
            continue
        ws = dataclasses.replace(w, b=1, n=L, Q=w.Q[bi:bi + 1, :, :L], K=w.K[bi:bi + 1, :, :L],
                                 V=w.V[bi:bi + 1, :, :L])
        rows = np.arange(L)
        kb, rt, Oref = G.oracle_prefill_rows(ws, rows, causal=causal, top_k=top_k)
        if Tb > 0:
            assert np.abs(g["kbar"][bi:bi + 1, :, :Tb].cpu().numpy() - kb).max() <= G.TOL_KBAR
            assert (g["w"][bi, :, :L, Tb:] == 0).all(), "weights of chunks past the sequence must be 0"
        gs = {k: g[k][bi:bi + 1] for k in ("idx", "bias", "cnt", "w")}
        nex, tot = G.compare_route(gs, rt, rows, Tb)
        err = G.compare_out(g["O"][bi:bi + 1, :, :L].cpu().numpy(), Oref, G.exempt_rows(rt), gq, w.dtype)
        lse = g["lse"][bi, :, :L].cpu().numpy()
        assert np.isfinite(lse).all()
        print(f"  exempt rows {nex}/{tot}, output error {err:.3e}", flush=True)
    return g


VARLEN = [
    # dtype, b, h_q, h_kv, d, n, B, alpha, gamma, causal, lengths
    ("bf16", 3, 16, 2, 128, 1000, 64, 1.5, 8.0, True, [1000, 700, 130]),
    ("bf16", 4, 8, 2, 128, 520, 64, 1.5, 6.0, False, [520, 300, 40, 0]),
    ("bf16", 2, 32, 2, 128, 900, 64, 1.0, 3.0, True, [900, 333]),
    ("bf16", 2, 4, 2, 64, 600, 32, 2.0, 6.0, True, [77, 600]),
    ("f32", 2, 1, 1, 64, 1024, 64, 1.5, 1.0, True, [1024, 577]),
    ("f32", 3, 2, 1, 128, 300, 32, 1.5, 5.0, False, [300, 161, 31]),
]


@pytest.mark.parametrize("case", VARLEN,
                         ids=[f"{c[0]}-g{c[2] // c[3]}-d{c[4]}-n{c[5]}-a{c[7]}-c{int(c[9])}-L{'_'.join(map(str, c[10]))}"
                              for c in VARLEN])
def test_varlen_prefill_matches_per_sequence_oracle(case):
    dtype, b, h_q, h_kv, d, n, B, alpha, gamma, causal, lengths = case
    print(f"varlen case {case}", flush=True)
    w = inputs.make_prefill(b=b, h_q=h_q, h_kv=h_kv, d=d, n=n, B=B, alphas=(alpha,), gamma=gamma,
                            causal=causal, dtype=dtype, seed=11)
    check_varlen(w, lengths)


def test_varlen_topk_matches_per_sequence_oracle():
    w = inputs.make_prefill(b=2, h_q=16, h_kv=2, d=128, n=960, B=64, alphas=(1.5,), gamma=4.0,
                            dtype="bf16", seed=12)
    check_varlen(w, [960, 450], top_k=3)


def test_varlen_lengths_are_clamped():
    """Lengths beyond n act as n, negative lengths as 0."""
    w = inputs.make_prefill(b=2, h_q=8, h_kv=2, d=128, n=384, B=64, alphas=(1.5,), gamma=6.0,
                            dtype="bf16", seed=13)
    check_varlen(w, [384 + 50, -3])


def test_varlen_full_lengths_equal_the_dense_entry_points():
    """seq_len = n everywhere gives bit for bit what the plain entry points give."""
    G = _gu()
    for case in [("bf16", 16, 2, 128, 1000, True), ("bf16", 8, 2, 128, 520, False), ("f32", 2, 1, 64, 640, True)]:
        dtype, h_q, h_kv, d, n, causal = case
        print(f"full-length case {case}", flush=True)
        w = inputs.make_prefill(b=2, h_q=h_q, h_kv=h_kv, d=d, n=n, B=64, alphas=(1.5,), gamma=6.0,
                                causal=causal, dtype=dtype, seed=14)
        a = G.gpu_prefill(w)
        v = gpu_varlen(w, [n, n])
        assert torch.equal(a["kbar"], v["kbar"])
        assert torch.equal(a["cnt"], v["cnt"])
        assert torch.equal(a["w"], v["w"])
        assert torch.equal(a["O"], v["O"])
        listed = torch.arange(a["idx"].shape[-1], device="cuda") < a["cnt"][..., None]
        assert torch.equal(a["idx"][listed], v["idx"][listed])
        assert torch.equal(a["bias"][listed], v["bias"][listed])


# ------------------------------------------------------------------------------------
# Paged K/V in prefill (the serving layout of dash_attend_decode_paged)
# ------------------------------------------------------------------------------------

def _pages_of(X, B, perm, fill=float("nan")):
    """[b, h_kv, n, d] -> [P, h_kv, B, d] with chunk c of sequence b in page
    perm[b * pps + c] (pps = ceil(n / B)); rows past n and unused pages hold NaN."""
    b, h_kv, n, d = X.shape
    pps = (n + B - 1) // B
    Xp = torch.full((b, h_kv, pps * B, d), fill, device=X.device).to(X.dtype)
    Xp[:, :, :n] = X
    P = int(perm.max()) + 1 + 2
    pages = torch.full((P, h_kv, B, d), fill, device=X.device).to(X.dtype)
    src = Xp.reshape(b, h_kv, pps, B, d).permute(0, 2, 1, 3, 4).reshape(b * pps, h_kv, B, d)
    pages[torch.from_numpy(perm).to(X.device).long()] = src
    return pages


PAGED = [
    # dtype, b, h_q, h_kv, d, n, B, causal, lengths (None: all n)
    ("bf16", 2, 16, 2, 128, 1000, 64, True, None),
    ("bf16", 2, 8, 2, 128, 520, 64, False, None),
    ("bf16", 3, 16, 2, 128, 900, 128, True, [900, 517, 33]),
    ("f32", 2, 2, 1, 64, 700, 32, True, [700, 301]),
    ("bf16", 1, 32, 2, 128, 4096, 32, True, None),
]


@pytest.mark.parametrize("case", PAGED, ids=[f"{c[0]}-g{c[2] // c[3]}-n{c[5]}-B{c[6]}-c{int(c[7])}-{'ragged' if c[8] else 'full'}"
                                             for c in PAGED])
def test_paged_prefill_equals_contiguous(case):
    """Stage 2 reading K and V through a page table (pages in random order, NaN in
    every row outside the sequences) gives the contiguous entry points' O and lse bit
    for bit; the summaries of dash_summarize_paged equal dash_summarize's."""
    from long_context_amd import dash
    G = _gu()
    dtype, b, h_q, h_kv, d, n, B, causal, lengths = case
    print(f"paged prefill case {case}", flush=True)
    w = inputs.make_prefill(b=b, h_q=h_q, h_kv=h_kv, d=d, n=n, B=B, alphas=(1.5,), gamma=6.0,
                            causal=causal, dtype=dtype, seed=31)
    Q, K, V = G.to_dev(w.Q, dtype), G.to_dev(w.K, dtype), G.to_dev(w.V, dtype)
    T = n // B
    pps = (n + B - 1) // B
    perm = np.random.default_rng(5).permutation(b * pps + 3)[:b * pps].astype(np.int32)
    Kp, Vp = _pages_of(K, B, perm), _pages_of(V, B, perm)
    pages = torch.from_numpy(perm.reshape(b, pps)).cuda()
    qbar = torch.from_numpy(w.qbar).cuda()
    kbar = dash.alloc_kbar(b, h_kv, T, d)
    dash.dash_summarize(K, qbar, kbar, B)
    if T > 0:
        kbp = torch.full_like(kbar, float("nan"))
        dash.dash_summarize_paged(Kp, qbar, kbp, pages, B, 0, T)
        assert torch.equal(kbp, kbar)
    idx, bias, cnt, _ = dash.alloc_route(b, h_kv, n, T)
    sl = None if lengths is None else torch.tensor(lengths, dtype=torch.int32, device="cuda")
    if sl is None:
        dash.dash_route(Q, kbar, B, w.alpha, w.gamma, w.sigma, causal, idx, bias, cnt)
    else:
        dash.dash_route_varlen(Q, kbar, sl, B, w.alpha, w.gamma, w.sigma, causal, idx, bias, cnt)
    O1 = torch.full((b, h_q, n, d), float("nan"), device="cuda")
    O2 = torch.full_like(O1, float("nan"))
    l1 = torch.full((b, h_q, n), float("nan"), device="cuda")
    l2 = torch.full_like(l1, float("nan"))
    if sl is None:
        dash.dash_attend_prefill_lse(Q, K, V, idx, bias, cnt, O1, l1, B, causal)
    else:
        dash.dash_attend_prefill_varlen(Q, K, V, sl, idx, bias, cnt, O1, B, causal, lse=l1)
    dash.dash_attend_prefill_paged(Q, Kp, Vp, pages, idx, bias, cnt, O2, B, causal, seq_len=sl, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(O1, nan=7.0), torch.nan_to_num(O2, nan=7.0))
    assert torch.equal(torch.nan_to_num(l1, nan=7.0), torch.nan_to_num(l2, nan=7.0))
    valid = torch.ones((b, n), dtype=torch.bool, device="cuda")
    if lengths is not None:
        for bi, L in enumerate(lengths):
            valid[bi, L:] = False
    assert torch.isfinite(O2.permute(0, 2, 1, 3)[valid]).all()
