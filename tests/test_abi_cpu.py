"""The C ABI without a GPU: exported symbols and host-side validation.

Every call here fails validation on the host, which returns before any HIP call,
so nothing is launched. Fake non-null pointers are never dereferenced.
"""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "long_context_amd", "libdash.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libdash.so not built")


@pytest.fixture(scope="module")
def dash():
    from long_context_amd import dash as d
    return d


P = ctypes.c_void_p(4096)        # a non-null pointer that validation never touches
NUL = None


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "dash.h")).read()
    return sorted(set(re.findall(r"\b(dash_[a-z_]+)\s*\(", text)))


def test_header_symbols_are_exported(dash):
    syms = declared_symbols()
    assert set(syms) == set(dash.SYMBOLS)
    for s in syms:
        assert hasattr(dash.lib, s), s


def test_status_strings(dash):
    assert dash.dash_status_string(0) == "ok"
    assert dash.dash_status_string(5) == "workspace too small"
    assert dash.dash_status_string(99) == "unknown status"


def _route(dash, **kw):
    a = dict(Q=P, qdt=1, kbar=P, b=1, h_q=4, h_kv=2, n=256, cap=4, d=128, B=64, alpha=1.5,
             gamma=1.0, sigma=1.0, causal=1, idx=P, bias=P, cnt=P, list_cap=4, w=NUL)
    a.update(kw)
    return dash.lib.dash_route(a["Q"], a["qdt"], a["kbar"], a["b"], a["h_q"], a["h_kv"], a["n"],
                               a["cap"], a["d"], a["B"], a["alpha"], a["gamma"], a["sigma"],
                               a["causal"], a["idx"], a["bias"], a["cnt"], a["list_cap"], a["w"],
                               NUL, 0, NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(Q=NUL), 1), (dict(idx=NUL), 1), (dict(cnt=NUL), 1),
    (dict(h_q=3), 2), (dict(b=0), 2), (dict(n=-1), 2), (dict(cap=3), 2), (dict(list_cap=2), 2),
    (dict(alpha=0.99), 3), (dict(alpha=float("nan")), 3), (dict(gamma=0.0), 3),
    (dict(gamma=float("inf")), 3), (dict(sigma=0.0), 3), (dict(sigma=float("nan")), 3),
    (dict(qdt=7), 3), (dict(causal=2), 3),
    (dict(d=96), 4), (dict(B=24), 4), (dict(h_q=64, h_kv=2), 4), (dict(h_q=6, h_kv=2), 4),
    (dict(n=129 * 1024, cap=2064, list_cap=2064), 4),
    # one query head per KV head, 2048 chunks: fits LDS (split rows stage no summaries
    # there), so validation goes on to the missing bf16 workspace
    (dict(h_q=2, h_kv=2, n=2048 * 64, cap=2048, list_cap=2048), 5),
])
def test_route_validation(dash, kw, status):
    assert _route(dash, **kw) == status
    assert dash.lib.dash_last_error().decode() != ""


def _route_topk(dash, top_k, **kw):
    a = dict(Q=P, qdt=1, kbar=P, b=1, h_q=4, h_kv=2, n=256, cap=4, d=128, B=64, alpha=1.5,
             gamma=1.0, sigma=1.0, causal=1, idx=P, bias=P, cnt=P, list_cap=4, w=NUL)
    a.update(kw)
    return dash.lib.dash_route_topk(a["Q"], a["qdt"], a["kbar"], a["b"], a["h_q"], a["h_kv"], a["n"],
                                    a["cap"], a["d"], a["B"], a["alpha"], a["gamma"], a["sigma"],
                                    a["causal"], a["idx"], a["bias"], a["cnt"], a["list_cap"], a["w"],
                                    top_k, NUL, 0, NUL)


def test_route_topk_validation(dash):
    assert _route_topk(dash, -1) == dash.DASH_ERR_PARAM
    assert "top_k" in dash.lib.dash_last_error().decode()
    assert _route_topk(dash, 2, Q=NUL) == dash.DASH_ERR_NULL
    assert _route_topk(dash, 2, alpha=0.5) == dash.DASH_ERR_PARAM
    assert _route_topk(dash, 2) == dash.DASH_ERR_WORKSPACE        # valid up to the workspace


def test_route_mask_validation(dash):
    m = dash.lib.dash_route_mask
    assert m(NUL, P, 1, 2, 64, 4, 4, P, 1, NUL) == dash.DASH_ERR_NULL
    assert m(P, P, 0, 2, 64, 4, 4, P, 1, NUL) == dash.DASH_ERR_SHAPE
    assert m(P, P, 1, 2, 64, 40, 40, P, 1, NUL) == dash.DASH_ERR_SHAPE      # 40 chunks need 2 words
    assert m(P, P, 1, 2, 64, 4, 4, P, 65, NUL) == dash.DASH_ERR_SHAPE       # at most 64 words
    assert m(P, P, 1, 2, 64, 2, 4, P, 1, NUL) == dash.DASH_ERR_SHAPE        # list_cap < T_c
    assert m(P, P, 1, 2, 64, 4096, 4096, P, 64, NUL) == dash.DASH_ERR_UNSUPPORTED
    assert m(P, P, 1, 2, 64, 0, 0, P, 0, NUL) == dash.DASH_OK                # nothing to write


def test_paged_entry_points_validation(dash):
    sp = dash.lib.dash_summarize_paged
    assert sp(P, 1, P, P, NUL, 4, 8, 1, 2, 4, 128, 64, 0, 1, NUL) == dash.DASH_ERR_NULL
    assert sp(P, 1, P, P, P, 0, 8, 1, 2, 4, 128, 64, 0, 1, NUL) == dash.DASH_ERR_SHAPE
    assert sp(P, 1, P, P, P, 4, 8, 1, 2, 4, 128, 64, 0, 5, NUL) == dash.DASH_ERR_SHAPE   # chunk_end > pages
    assert sp(P, 1, P, P, P, 4, 8, 1, 2, 4, 96, 64, 0, 1, NUL) == dash.DASH_ERR_UNSUPPORTED
    dp = dash.lib.dash_attend_decode_paged
    args = [P, P, P, 1, P, P, P, 4, 8, 1, 4, 2, 4, 128, 64, 1.5, 1.0, 1.0, P, 0, NUL, NUL, NUL, NUL, 0]
    assert dp(*args, NUL, 0, NUL) == dash.DASH_ERR_WORKSPACE
    bad = list(args)
    bad[6] = NUL
    assert dp(*bad, NUL, 0, NUL) == dash.DASH_ERR_NULL
    bad = list(args)
    bad[8] = 0
    assert dp(*bad, NUL, 0, NUL) == dash.DASH_ERR_SHAPE


def test_route_accepts_alpha_one(dash):
    # α = 1 (softmax routing) passes parameter validation; the missing workspace of
    # this bf16 call is what fails next
    assert _route(dash, alpha=1.0) == dash.DASH_ERR_WORKSPACE


def test_route_bf16_needs_workspace(dash):
    # valid bf16 routing with no workspace: the split summaries have nowhere to go
    assert _route(dash) == dash.DASH_ERR_WORKSPACE
    assert "workspace" in dash.lib.dash_last_error().decode()


def test_route_accepts_infinite_sigma_in_validation(dash):
    # sigma = +inf passes validation; a NULL Q then still fails with DASH_ERR_NULL first
    assert _route(dash, Q=NUL, sigma=math.inf) == 1


def _summ(dash, **kw):
    a = dict(K=P, kdt=1, qbar=P, kbar=P, b=1, h_kv=2, n=256, cap=4, d=128, B=64, c0=0, c1=4)
    a.update(kw)
    return dash.lib.dash_summarize(a["K"], a["kdt"], a["qbar"], a["kbar"], a["b"], a["h_kv"],
                                   a["n"], a["cap"], a["d"], a["B"], a["c0"], a["c1"], NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(K=NUL), 1), (dict(kbar=NUL), 1), (dict(kdt=2), 3), (dict(c1=5), 2),
    (dict(c0=3, c1=2), 2), (dict(cap=3), 2), (dict(c0=-1), 2), (dict(d=32), 4), (dict(B=8), 4),
])
def test_summarize_validation(dash, kw, status):
    assert _summ(dash, **kw) == status


def _prefill(dash, **kw):
    a = dict(Q=P, K=P, V=P, dt=1, idx=P, bias=P, cnt=P, cap=4, O=P, odt=0, b=1, h_q=4, h_kv=2,
             n=256, d=128, B=64, causal=1)
    a.update(kw)
    return dash.lib.dash_attend_prefill(a["Q"], a["K"], a["V"], a["dt"], a["idx"], a["bias"],
                                        a["cnt"], a["cap"], a["O"], a["odt"], a["b"], a["h_q"],
                                        a["h_kv"], a["n"], a["d"], a["B"], a["causal"], NUL, 0, NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(O=NUL), 1), (dict(V=NUL), 1), (dict(odt=3), 3), (dict(cap=3), 2), (dict(B=48), 4),
    (dict(h_q=5, h_kv=2), 2),
])
def test_prefill_validation(dash, kw, status):
    assert _prefill(dash, **kw) == status


def test_prefill_bf16_needs_workspace(dash):
    need = dash.dash_workspace_bytes(dash.DASH_OP_PREFILL, 1, 4, 2, 256, 128, 64)
    args = (P, P, P, 1, P, P, P, 4, P, 0, 1, 4, 2, 256, 128, 64, 1)
    assert dash.lib.dash_attend_prefill(*args, NUL, need, NUL) == dash.DASH_ERR_WORKSPACE
    assert dash.lib.dash_attend_prefill(*args, P, need - 1, NUL) == dash.DASH_ERR_WORKSPACE


def _decode(dash, ws_bytes, **kw):
    a = dict(Q=P, Kc=P, Vc=P, dt=1, kbar=P, sl=P, b=4, h_q=32, h_kv=2, L=131072, cap=1024,
             d=128, B=128, alpha=1.5, gamma=1.0, sigma=1.0, O=P, odt=0, idx=NUL, bias=NUL,
             cnt=NUL, w=NUL, list_cap=0, ws=P)
    a.update(kw)
    return dash.lib.dash_attend_decode(a["Q"], a["Kc"], a["Vc"], a["dt"], a["kbar"], a["sl"],
                                       a["b"], a["h_q"], a["h_kv"], a["L"], a["cap"], a["d"],
                                       a["B"], a["alpha"], a["gamma"], a["sigma"], a["O"],
                                       a["odt"], a["idx"], a["bias"], a["cnt"], a["w"],
                                       a["list_cap"], a["ws"], ws_bytes, NUL)


def test_decode_workspace_checks(dash):
    need = dash.dash_workspace_bytes(dash.DASH_OP_DECODE, 4, 32, 2, 131072, 128, 128)
    assert 0 < need < (1 << 30)
    assert _decode(dash, need - 1) == dash.DASH_ERR_WORKSPACE
    assert _decode(dash, need, ws=NUL) == dash.DASH_ERR_WORKSPACE
    assert _decode(dash, need, idx=P) == dash.DASH_ERR_NULL          # partial list outputs
    assert _decode(dash, need, idx=P, bias=P, cnt=P, list_cap=10) == dash.DASH_ERR_SHAPE
    assert _decode(dash, need, alpha=0.5) == dash.DASH_ERR_PARAM
    assert _decode(dash, need, B=48) == dash.DASH_ERR_UNSUPPORTED
    assert _decode(dash, need, L=300000) == dash.DASH_ERR_UNSUPPORTED      # 2343 chunks > 2048


def test_decode_topk_rejects_negative_budget(dash):
    need = dash.dash_workspace_bytes(dash.DASH_OP_DECODE, 4, 32, 2, 131072, 128, 128)
    st = dash.lib.dash_attend_decode_topk(P, P, P, dash.DASH_BF16, P, P, 4, 32, 2, 131072, 1023, 128, 128,
                                          1.5, 1.0, 1.0, P, dash.DASH_BF16, NUL, NUL, NUL, NUL, 0, -1,
                                          P, need, NUL)
    assert st == dash.DASH_ERR_PARAM


def test_decode_noalloc_rejects_shapes_beyond_its_scratch(dash):
    """The entry point without a workspace refuses, before touching any device, a
    shape whose decode workspace exceeds the library's scratch (32 MiB)."""
    b, h_q, h_kv, d, L, B = 512, 32, 2, 128, 131072, 128
    assert dash.dash_workspace_bytes(dash.DASH_OP_DECODE, b, h_q, h_kv, L, d, B) > (32 << 20)
    st = dash.lib.dash_attend_decode_noalloc(P, P, P, dash.DASH_BF16, P, P, b, h_q, h_kv, L, L // B, d, B,
                                             1.5, 1.0, 1.0, P, dash.DASH_BF16, NUL, NUL, NUL, NUL, 0, NUL)
    assert st == dash.DASH_ERR_WORKSPACE
    assert b"scratch" in dash.lib.dash_last_error()


def test_workspace_sizes(dash):
    # route: split summaries, b * h_kv * (T_c rounded up to 32) * 3 * d * 2 bytes
    assert dash.dash_workspace_bytes(dash.DASH_OP_ROUTE, 1, 32, 2, 32768, 128, 64) == 2 * 512 * 3 * 128 * 2
    assert dash.dash_workspace_bytes(dash.DASH_OP_ROUTE, 1, 4, 2, 100, 64, 32) == 2 * 32 * 3 * 64 * 2
    assert dash.dash_workspace_bytes(dash.DASH_OP_PREFILL, 1, 32, 2, 32768, 128, 64) == 2 * 128 * 32768 * 2
    assert dash.dash_workspace_bytes(dash.DASH_OP_PREFILL, 1, 4, 2, 100, 64, 32) == 2 * 64 * 128 * 2
    big = dash.dash_workspace_bytes(dash.DASH_OP_DECODE, 16, 32, 2, 32768, 128, 64)
    small = dash.dash_workspace_bytes(dash.DASH_OP_DECODE, 16, 32, 2, 4096, 128, 64)
    assert big > small > 0
    assert dash.dash_workspace_bytes(9, 1, 1, 1, 1, 64, 64) == 2 ** 64 - 1
    assert dash.dash_workspace_bytes(0, 1, 3, 2, 1, 64, 64) == 2 ** 64 - 1


def _backward(dash, ws_bytes=None, **kw):
    a = dict(Q=P, K=P, V=P, dt=1, idx=P, bias=P, cnt=P, cap=4, O=P, dO=P, odt=1, lse=P, dQ=P, dK=P,
             dV=P, dbias=P, b=1, h_q=16, h_kv=2, n=256, d=128, B=64, causal=1, ws=P)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = dash.dash_workspace_bytes(dash.DASH_OP_PREFILL_BWD, a["b"], a["h_q"], a["h_kv"], a["n"],
                                             a["d"], a["B"])
    return dash.lib.dash_attend_prefill_backward(
        a["Q"], a["K"], a["V"], a["dt"], a["idx"], a["bias"], a["cnt"], a["cap"], a["O"], a["dO"],
        a["odt"], a["lse"], a["dQ"], a["dK"], a["dV"], a["dbias"], a["b"], a["h_q"], a["h_kv"], a["n"],
        a["d"], a["B"], a["causal"], a["ws"], ws_bytes, NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(lse=NUL), 1), (dict(dO=NUL), 1), (dict(dbias=NUL), 1), (dict(dK=NUL), 1),
    (dict(odt=2), 3), (dict(causal=2), 3), (dict(cap=3), 2), (dict(h_q=15), 2),
    (dict(dt=0), 4),                        # fp32 Q/K/V
    (dict(B=48, cap=8), 4),                 # B % 32 != 0
    (dict(h_q=64), 4),                      # g = 32
    (dict(ws=NUL), 5),
])
def test_backward_validation(dash, kw, status):
    assert _backward(dash, **kw) == status


def test_backward_workspace(dash):
    need = dash.dash_workspace_bytes(dash.DASH_OP_PREFILL_BWD, 1, 16, 2, 256, 128, 64)
    assert _backward(dash, ws_bytes=need - 1) == dash.DASH_ERR_WORKSPACE
    up = lambda x: (x + 255) // 256 * 256
    b, hq, hkv, n, d, B = 1, 16, 2, 256, 128, 64
    T, nblk = n // B, (n + 63) // 64
    seg = 8192 // (hq // hkv)
    items = hkv * ((T + 1) + -(-(n * T + n + B) // seg))
    expect = (up(hkv * d * 256 * 2) + up(hq * n * d * 2) + up(hq * n * 4) + up(hkv * T * nblk * 4)
              + up(hkv * (T + 1) * 4) + 2 * up(hkv * n * T * 4) + up(items * 16) + 256)
    assert need == expect
    # 32-token chunks: one (half used) 64-token dK/dV tile per chunk
    B = 32
    T = n // B
    items32 = hkv * ((T + 1) + -(-(n * T + n + B) // seg))
    expect32 = (up(hkv * d * 256 * 2) + up(hq * n * d * 2) + up(hq * n * 4) + up(hkv * T * nblk * 4)
                + up(hkv * (T + 1) * 4) + 2 * up(hkv * n * T * 4) + up(items32 * 16) + 256)
    assert dash.dash_workspace_bytes(dash.DASH_OP_PREFILL_BWD, 1, hq, hkv, n, d, B) == expect32
    # n * floor(n/B) must stay below 2^31 (inverted list offsets are int32)
    assert _backward(dash, n=1 << 20, B=64, cap=1 << 14, ws_bytes=1 << 62) == dash.DASH_ERR_UNSUPPORTED


def test_prefill_lse_validation(dash):
    args = (P, P, P, 1, P, P, P, 4, P, 0, P, 1, 4, 2, 256, 128, 64, 1)
    assert dash.lib.dash_attend_prefill_lse(*args, NUL, 0, NUL) == dash.DASH_ERR_WORKSPACE
    args = (P, P, P, 1, P, P, P, 3, P, 0, NUL, 1, 4, 2, 256, 128, 64, 1)
    assert dash.lib.dash_attend_prefill_lse(*args, P, 1 << 30, NUL) == dash.DASH_ERR_SHAPE


def _route_bwd(dash, **kw):
    a = dict(Q=P, qdt=1, kbar=P, kcap=4, idx=P, cnt=P, dbias=P, cap=4, stats=P, b=1, h_q=16, h_kv=2, n=256,
             d=128, B=64, alpha=1.5, gamma=1.0, sigma=1.0, dQ=P, dkbar=P, ws=P, ws_bytes=1 << 30)
    a.update(kw)
    return dash.lib.dash_route_backward(a["Q"], a["qdt"], a["kbar"], a["kcap"], a["idx"], a["cnt"], a["dbias"],
                                        a["cap"], a["stats"], a["b"], a["h_q"], a["h_kv"], a["n"], a["d"],
                                        a["B"], a["alpha"], a["gamma"], a["sigma"], a["dQ"], a["dkbar"],
                                        a["ws"], a["ws_bytes"], NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(stats=NUL), 1), (dict(dbias=NUL), 1), (dict(dkbar=NUL), 1), (dict(dQ=NUL), 1),
    (dict(qdt=5), 3), (dict(alpha=0.5), 3), (dict(gamma=0.0), 3), (dict(sigma=-1.0), 3),
    (dict(kcap=3), 2), (dict(cap=3), 2), (dict(n=-1), 2), (dict(h_q=15), 2),
    (dict(h_q=64), 4), (dict(d=96), 4),
    (dict(ws=NUL), 5), (dict(ws_bytes=1024), 5),            # bf16 queries need the split summaries
    (dict(n=2049 * 16, B=16, kcap=2049, cap=2049), 4),       # more chunks than the router takes
])
def test_route_backward_validation(dash, kw, status):
    assert _route_bwd(dash, **kw) == status
    assert dash.lib.dash_last_error().decode() != ""


def _sum_bwd(dash, **kw):
    a = dict(K=P, kdt=1, qbar=P, dkbar=P, b=1, h_kv=2, n=256, kcap=4, d=128, B=64, dK=P, dqbar=P)
    a.update(kw)
    return dash.lib.dash_summarize_backward(a["K"], a["kdt"], a["qbar"], a["dkbar"], a["b"], a["h_kv"], a["n"],
                                            a["kcap"], a["d"], a["B"], a["dK"], a["dqbar"], NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(K=NUL), 1), (dict(dkbar=NUL), 1), (dict(dqbar=NUL), 1), (dict(kdt=7), 3),
    (dict(kcap=3), 2), (dict(n=-5), 2), (dict(b=0), 2), (dict(d=80), 4), (dict(B=24), 4),
])
def test_summarize_backward_validation(dash, kw, status):
    assert _sum_bwd(dash, **kw) == status


def test_route_backward_workspace(dash):
    need = dash.dash_workspace_bytes(dash.DASH_OP_ROUTE, 1, 16, 2, 256, 128, 64)
    assert _route_bwd(dash, ws_bytes=need - 1) == dash.DASH_ERR_WORKSPACE
    # fp32 queries need no workspace; validation then fails only on the shape given
    assert _route_bwd(dash, qdt=0, ws=NUL, ws_bytes=0, kcap=3) == dash.DASH_ERR_SHAPE


def test_route_stats_needs_stats(dash):
    args = (P, 0, P, 1, 8, 2, 256, 4, 64, 64, 1.5, 1.0, 1.0, 1, P, P, P, 4, NUL)
    assert dash.lib.dash_route_stats(*args, NUL, NUL, 0, NUL) == dash.DASH_ERR_NULL


def test_varlen_entry_points_validation(dash):
    """The ragged-batch entry points need seq_len and otherwise validate as their
    dense counterparts (the checks come before any launch)."""
    L = dash.lib
    s = L.dash_summarize_varlen
    assert s(P, 1, P, P, NUL, 1, 2, 256, 4, 128, 64, 0, 4, NUL) == dash.DASH_ERR_NULL
    assert "seq_len" in L.dash_last_error().decode()
    assert s(P, 1, P, P, P, 1, 2, 256, 4, 128, 64, 0, 5, NUL) == dash.DASH_ERR_SHAPE
    assert s(P, 1, P, P, P, 1, 2, 256, 4, 128, 8, 0, 4, NUL) == dash.DASH_ERR_UNSUPPORTED
    r = L.dash_route_varlen
    args = [P, 1, P, P, 1, 4, 2, 256, 4, 128, 64, 1.5, 1.0, 1.0, 1, P, P, P, 4, NUL, 0]
    assert r(*args, NUL, 0, NUL) == dash.DASH_ERR_WORKSPACE          # valid up to the workspace
    bad = list(args)
    bad[3] = NUL
    assert r(*bad, NUL, 0, NUL) == dash.DASH_ERR_NULL
    bad = list(args)
    bad[20] = -1
    assert r(*bad, NUL, 0, NUL) == dash.DASH_ERR_PARAM              # negative budget
    p = L.dash_attend_prefill_varlen
    args = [P, P, P, 1, P, P, P, P, 4, P, 0, NUL, 1, 4, 2, 256, 128, 64, 1]
    assert p(*args, NUL, 0, NUL) == dash.DASH_ERR_WORKSPACE
    bad = list(args)
    bad[4] = NUL
    assert p(*bad, NUL, 0, NUL) == dash.DASH_ERR_NULL
    bad = list(args)
    bad[17] = 48
    assert p(*bad, NUL, 0, NUL) == dash.DASH_ERR_UNSUPPORTED        # B % 32 != 0


def test_paged_prefill_validation(dash):
    p = dash.lib.dash_attend_prefill_paged
    args = [P, P, P, 1, P, 16, 40, NUL, P, P, P, 16, P, 0, NUL, 1, 4, 2, 1024, 128, 64, 1]
    assert p(*args, NUL, 0, NUL) == dash.DASH_ERR_WORKSPACE          # valid up to the workspace
    bad = list(args)
    bad[4] = NUL
    assert p(*bad, NUL, 0, NUL) == dash.DASH_ERR_NULL               # no page table
    bad = list(args)
    bad[5] = 15
    assert p(*bad, NUL, 0, NUL) == dash.DASH_ERR_SHAPE              # 15 pages of 64 < 1024 tokens
    bad = list(args)
    bad[6] = 0
    assert p(*bad, NUL, 0, NUL) == dash.DASH_ERR_SHAPE


def test_empty_sequence_is_a_no_op(dash):
    """n = 0 (a batch of empty sequences) is a valid call of every prefill-side entry
    point: validation passes and nothing is launched (there is no GPU here, so any
    launch would come back as DASH_ERR_LAUNCH)."""
    assert _summ(dash, n=0, cap=1, c0=0, c1=0) == dash.DASH_OK
    assert _route(dash, n=0, cap=1, list_cap=1) == dash.DASH_OK
    assert _prefill(dash, n=0) == dash.DASH_OK
    assert _prefill(dash, n=0, dt=1, odt=1) == dash.DASH_OK
    assert _backward(dash, n=0, ws_bytes=0) == dash.DASH_OK
    assert _route_bwd(dash, n=0, ws_bytes=0) == dash.DASH_OK
