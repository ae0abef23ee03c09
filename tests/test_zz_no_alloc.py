"""The decode entry point that allocates nothing (dash_attend_decode_noalloc, for
callers that cannot allocate) against dash_attend_decode with a caller workspace:
two calls in a row on the library's per-GPU scratch, the second with a smaller
input, each equal to the workspace entry point's output and routed lists (same
kernels, so bit for bit, within the decode parity bar a fortiori)."""
import numpy as np
import pytest
import torch

from long_context_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(gpu_lib):
    yield


def _case(b, h_q, h_kv, d, L, B, seq_len, seed):
    from long_context_amd import dash
    w = inputs.make_decode(b=b, h_q=h_q, h_kv=h_kv, d=d, L=L, B=B, alphas=(1.5,), gamma=4.0, dtype="bf16",
                           seed=seed, seq_len=seq_len)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.bfloat16)
    Q, K, V = dev(w.Q), dev(w.K), dev(w.V)
    T = L // B
    kbar = dash.alloc_kbar(b, h_kv, T, d)
    dash.dash_summarize(K, torch.from_numpy(w.qbar).cuda(), kbar, B)
    sl = torch.tensor(seq_len, dtype=torch.int32, device="cuda")
    cap = max((L - 1) // B, 1)

    def outputs():
        O = torch.full((b, h_q, 1, d), float("nan"), device="cuda")
        idx = torch.full((b, h_kv, cap), -1, dtype=torch.int32, device="cuda")
        bias = torch.zeros((b, h_kv, cap), device="cuda")
        cnt = torch.zeros((b, h_kv), dtype=torch.int32, device="cuda")
        return O, idx, bias, cnt

    ref = outputs()
    ws = dash.alloc_decode_ws(b, h_q, h_kv, L, d, B)
    dash.dash_attend_decode(Q, K, V, kbar, sl, B, 1.5, 4.0, 1.0, ref[0], ws, *ref[1:])
    got = outputs()
    dash.dash_attend_decode_noalloc(Q, K, V, kbar, sl, B, 1.5, 4.0, 1.0, got[0], *got[1:])
    torch.cuda.synchronize()
    print(f"no-alloc decode b={b} L={L} seq={seq_len}: max |dO| {float((got[0] - ref[0]).abs().max()):.3e}", flush=True)
    assert torch.isfinite(got[0]).all()
    assert torch.equal(got[0], ref[0])
    assert torch.equal(got[3], ref[3])
    live = torch.arange(cap, device="cuda") < ref[3][..., None]
    assert torch.equal(got[1][live], ref[1][live])
    assert torch.equal(got[2][live], ref[2][live])


def test_noalloc_decode_matches_workspace_entry_point_twice():
    _case(3, 32, 2, 128, 8192, 64, [8192, 5000, 700], seed=51)     # first call
    _case(2, 16, 2, 128, 2048, 128, [2048, 1500], seed=52)         # second, smaller
