"""Benchmark of the DashAttention forward pass on one MI355X.

One step = one pass of the whole hot path over synthetic inputs:
  * prefill of the 32K clustered workload (b=1, 32 query / 2 KV heads, d=128,
    n=32768, B=64, γ=1): Stage 0 summaries, Stage 1 routing, Stage 2 attention;
  * one decode step of the 128K workload (b=4, 32 / 2 heads, d=128, L=131072,
    B=128): routing against the cached summaries and split-KV attention.
`value` is the prefill throughput in tokens/s at α=1.5; the decode latency, the
α sweep {1.25, 1.5, 2.0}, per-stage times, the dense (0%-sparsity) baseline and
the roofline fractions ride along in the same JSON line.

Timing: HIP events recorded on the stream the kernels are launched on (torch's
current stream, which the binding passes to every entry point), W untimed warm-up
steps, then exactly K timed steps bracketed by device synchronisation.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DashAttention fwd: prefill tok/s @32k, decode µs/step @128k; % of roofline"
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0              # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--alpha", type=float, default=1.5)
    ap.add_argument("--no-sweep", action="store_true", help="skip the alpha sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense baseline")
    ap.add_argument("--cpu-rows", type=int, default=3072, help="query rows of the oracle sample")
    ap.add_argument("--only", choices=["prefill", "decode", "both", "decode128k", "decode32k"], default="both",
                    help="decode128k / decode32k: time one decode workload alone (no prefill)")
    ap.add_argument("--flushed-only", action="store_true",
                    help="decode: time only the Infinity-Cache-flushed steps (one kernel mix per trace)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (HBM counter calibration)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (Stages 2, 1 and 0) at the 32K workload instead of the forward")
    ap.add_argument("--efficiency", action="store_true",
                    help="only run the replicas of the pages' efficiency operating points")
    return ap.parse_args()


# Counter summaries (profiles/): an HBM traffic figure measured with hardware
# counters is reported only while the sources of the kernels it covers are unchanged.
COMMON_SOURCES = ["long_context_amd/csrc/attn_common.h", "long_context_amd/csrc/common.h"]
STAGE2_SOURCES = ["long_context_amd/csrc/attend_prefill_bf16.hip", "long_context_amd/csrc/prefill_common.h"] + COMMON_SOURCES
DECODE_SOURCES = ["long_context_amd/csrc/decode.hip"] + COMMON_SOURCES
TRAFFIC_FILE = "profiles/sparse_prior_attn_bf16_kernel_prefill_32k_traffic.txt"
DECODE_TRAFFIC_FILE = "profiles/decode_128k_b4_traffic.txt"


def kernel_source_hash(files=STAGE2_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(path=TRAFFIC_FILE, sources=STAGE2_SOURCES, key="traffic_bytes_per_launch"):
    """HBM bytes per launch (or step) from a committed counter summary (FETCH_SIZE +
    WRITE_SIZE scaled by a plain copy's readings), or None when the summary is missing
    or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, path)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != kernel_source_hash(sources):
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch):
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)


class Prefill:
    """Device buffers of the 32K prefill and the three ABI calls of one pass."""

    def __init__(self, w, torch, dash):
        self.w, self.torch, self.dash = w, torch, dash
        self.Q = torch.from_numpy(w.Q).to("cuda", torch.bfloat16)
        self.K = torch.from_numpy(w.K).to("cuda", torch.bfloat16)
        self.V = torch.from_numpy(w.V).to("cuda", torch.bfloat16)
        self.qbar = torch.from_numpy(w.qbar).cuda()
        b, h_q, n, d = w.Q.shape
        self.T = n // w.B
        self.kbar = dash.alloc_kbar(b, w.h_kv, self.T, d)
        self.idx, self.bias, self.cnt, _ = dash.alloc_route(b, w.h_kv, n, self.T)
        self.O = torch.empty((b, h_q, n, d), dtype=torch.bfloat16, device="cuda")
        self.ws = dash.alloc_prefill_ws(b, h_q, w.h_kv, n, d, w.B)
        self.rws = dash.alloc_route_ws(b, h_q, w.h_kv, n, d, w.B)

    def run(self, alpha, ev=None):
        d, w = self.dash, self.w
        if ev: ev[0].record()
        d.dash_summarize(self.K, self.qbar, self.kbar, w.B)
        if ev: ev[1].record()
        d.dash_route(self.Q, self.kbar, w.B, alpha, w.gamma, w.sigma, True, self.idx, self.bias,
                     self.cnt, ws=self.rws)
        if ev: ev[2].record()
        d.dash_attend_prefill(self.Q, self.K, self.V, self.idx, self.bias, self.cnt, self.O, w.B, True,
                              ws=self.ws)
        if ev: ev[3].record()

    def route_bytes(self):
        """Algorithmic HBM bytes of the last routing: Q, summaries, lists written, counts."""
        w = self.w
        sup = int(self.cnt.to(self.torch.int64).sum().item())
        return (w.Q.size * 2 + w.b * w.h_kv * self.T * w.d * 4 + sup * 8 + w.b * w.h_kv * w.n * 4)

    def group_sparsity(self):
        """Group sparsity of the last routing (rows with at least one visible chunk)."""
        torch, w = self.torch, self.w
        pos = torch.arange(w.n, device="cuda")
        vis = torch.clamp(pos // w.B, max=self.T)
        sup = self.cnt.to(torch.int64).sum().item()
        return 1.0 - sup / max((vis.sum() * w.h_kv * w.b).item(), 1)

    def stats(self):
        """Work of the last routing (bookkeeping outside the timed region).

        flops_row:  per-row algorithmic Stage-2 flops, 4 d g (B |S_i| + |D_i|) summed
                    over rows and KV groups (what the method must compute);
        flops_wave: flops the MFMAs execute: a wavefront (32 (row, head) pairs =
                    32/g rows) runs a chunk when any of its rows routes it, and the
                    diagonal in 64-token tiles;
        flops_tile: the same at workgroup-tile granularity (256 pairs = 256/g rows).
        """
        torch, w = self.torch, self.w
        n, B, d, g = w.n, w.B, w.d, w.g
        cnt = self.cnt.to(torch.int64)                     # [b, h_kv, n]
        pos = torch.arange(n, device="cuda")
        vis = torch.clamp(pos // B, max=self.T)
        diag = pos - (pos // B) * B + 1
        rows_sup = cnt.sum().item()
        rows_vis = (vis.sum() * w.h_kv * w.b).item()
        diag_tok = (diag.sum() * w.h_kv * w.b).item()
        flops_row = 4.0 * d * g * (B * rows_sup + diag_tok)

        def union_and_diag(rows_per_group):
            uni = 0
            for r in range(w.h_kv):
                for i0 in range(0, n, 2048):
                    c = cnt[0, r, i0:i0 + 2048]
                    ids = self.idx[0, r, i0:i0 + 2048, :self.T].to(torch.int64)
                    valid = torch.arange(self.T, device="cuda")[None, :] < c[:, None]
                    mask = torch.zeros((ids.shape[0], self.T), dtype=torch.bool, device="cuda")
                    mask.scatter_(1, torch.where(valid, ids, torch.zeros_like(ids)), valid)
                    uni += mask.view(-1, rows_per_group, self.T).any(1).sum().item()
            dt = 0
            for t0 in range(0, n, rows_per_group):
                last = min(t0 + rows_per_group, n) - 1
                dt += ((last - (t0 // B) * B) // 64 + 1) * 64
            return uni, dt * w.h_kv * w.b

        uw, dw = union_and_diag(max(32 // g, 1))
        ut, dtk = union_and_diag(max(256 // g, 1))
        flops_wave = 4.0 * d * 32 * (B * uw + dw)
        flops_tile = 4.0 * d * 256 * (B * ut + dtk)
        return dict(flops_row=flops_row, flops_wave=flops_wave, flops_tile=flops_tile,
                    sparsity=1.0 - rows_sup / max(rows_vis, 1),
                    inflation_wave=flops_wave / flops_row, inflation_tile=flops_tile / flops_row)


class Decode:
    def __init__(self, w, torch, dash):
        self.w, self.torch, self.dash = w, torch, dash
        self.Q = torch.from_numpy(w.Q).to("cuda", torch.bfloat16)
        self.K = torch.from_numpy(w.K).to("cuda", torch.bfloat16)
        self.V = torch.from_numpy(w.V).to("cuda", torch.bfloat16)
        b, h_q, _, d = w.Q.shape
        self.T = w.n // w.B
        self.kbar = dash.alloc_kbar(b, w.h_kv, self.T, d)
        dash.dash_summarize(self.K, torch.from_numpy(w.qbar).cuda(), self.kbar, w.B)
        self.sl = torch.from_numpy(w.seq_len).cuda()
        self.ws = dash.alloc_decode_ws(b, h_q, w.h_kv, w.n, d, w.B)
        cap = (w.n - 1) // w.B
        self.idx = torch.empty((b, w.h_kv, cap), dtype=torch.int32, device="cuda")
        self.bias = torch.empty((b, w.h_kv, cap), device="cuda")
        self.cnt = torch.empty((b, w.h_kv), dtype=torch.int32, device="cuda")
        self.O = torch.empty((b, h_q, 1, d), dtype=torch.bfloat16, device="cuda")

    def run(self, ev=None):
        w = self.w
        if ev: ev[0].record()
        self.dash.dash_attend_decode(self.Q, self.K, self.V, self.kbar, self.sl, w.B, w.alpha,
                                     w.gamma, w.sigma, self.O, self.ws, self.idx, self.bias,
                                     self.cnt)
        if ev: ev[1].record()

    def bytes_per_step(self):
        w = self.w
        cnt = self.cnt.cpu().numpy().astype(np.int64)
        L = w.seq_len.astype(np.int64)
        vis = (L - 1) // w.B
        diag = L - vis * w.B
        total = 0
        for bi in range(w.b):
            for r in range(w.h_kv):
                total += vis[bi] * w.d * 4                                  # summaries
                total += (w.B * cnt[bi, r] + diag[bi]) * w.d * 2 * 2        # K + V bf16
        total += w.Q.size * 2 + w.Q.size * 2 + cnt.size * 4 + cnt.sum() * 8
        return int(total), cnt


def dense_lists(pre, torch):
    """Full routed lists (every visible chunk, bias 0): dense causal attention."""
    w = pre.w
    T = pre.T
    pos = torch.arange(w.n, device="cuda")
    idx = torch.arange(T, dtype=torch.int32, device="cuda").expand(w.b, w.h_kv, w.n, T).contiguous()
    cnt = torch.clamp(pos // w.B, max=T).to(torch.int32).expand(w.b, w.h_kv, w.n).contiguous()
    bias = torch.zeros((w.b, w.h_kv, w.n, T), device="cuda")
    return idx, bias, cnt


def time_events(torch, fn, nev, steps, warmup):
    for _ in range(warmup):
        fn(None)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        fn(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    seg = np.array([[evs[k][j].elapsed_time(evs[k][j + 1]) for j in range(nev - 1)]
                    for k in range(steps)])
    return seg, wall


def cpu_baseline(w, rows_n):
    from oracle import dash_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    rows = np.unique(np.linspace(0, w.n - 1, rows_n).astype(np.int64))
    t0 = time.perf_counter()
    O.prefill(w.Q, w.K, w.V, w.qbar, w.B, 1.5, w.gamma, w.sigma, True, rows=rows)
    dt = time.perf_counter() - t0
    return {"value": rows.size / dt, "unit": "tok/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows.size} evenly spaced query rows (all 32 heads) of the 32K prefill at "
                      f"alpha=1.5, Stage 0 over the whole K; {dt:.1f} s on {os.cpu_count()} host "
                      f"CPUs; tok/s = rows / time"}


# Speedups over dense FlashAttention printed at these operating points (paper
# review section 六, 6.2 efficiency benchmarks table; other hardware, context only).
PAGES_SPEEDUP = {("prefill", 16, 0.75): 1.34, ("prefill", 96, 0.9375): 3.09,
                 ("decode", 96, 0.75): 1.96, ("decode", 96, 0.9375): 3.36}


def sdpa_time(torch, q, k, v, causal, steps):
    """Median ms of torch's fused dense attention (flash / memory-efficient kernels
    only, bf16), the dense baseline of the efficiency table; None if neither fused
    kernel takes these shapes."""
    import torch.nn.functional as F
    from torch.nn.attention import sdpa_kernel, SDPBackend
    fused = [SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]

    def call():
        with sdpa_kernel(fused):
            return F.scaled_dot_product_attention(q, k, v, is_causal=causal)
    try:
        call()
    except RuntimeError as e:
        print(f"[bench] fused SDPA unavailable: {e}", file=sys.stderr, flush=True)
        return None
    fn = lambda ev: (ev and ev[0].record(), call(), ev and ev[1].record())
    return float(np.median(time_events(torch, fn, 2, steps, 1)[0]))


def efficiency(torch, dash, inputs, steps):
    """DashAttention at the efficiency operating points (prefill 16K / 96K at b=1,
    decode 96K at b=24, B=64, group sparsity set through γ) against two dense
    baselines: torch's fused attention, and these kernels with every chunk routed
    (prefill: full lists, no routing; decode: γ≈0, routing included)."""
    rows = []
    for n in (16 * 1024, 96 * 1024):
        targets = [t for t in inputs.EFFICIENCY_SPARSITY
                   if (f"prefill_{n // 1024}k", t) in inputs.GAMMA_EFFICIENCY]
        w = inputs.efficiency_prefill(n)
        pre = Prefill(w, torch, dash)
        di, db, dc = dense_lists(pre, torch)
        Od = torch.empty_like(pre.O)
        fn = lambda ev: (ev and ev[0].record(),
                         dash.dash_attend_prefill(pre.Q, pre.K, pre.V, di, db, dc, Od, w.B, True, ws=pre.ws),
                         ev and ev[1].record())
        td = float(np.median(time_events(torch, fn, 2, steps, 1)[0]))
        del di, db, dc, Od
        g = w.h_q // w.h_kv                  # query head h reads KV head h // g
        tf = sdpa_time(torch, pre.Q, pre.K.repeat_interleave(g, 1), pre.V.repeat_interleave(g, 1),
                       True, steps)
        torch.cuda.empty_cache()
        for t in targets:
            w.gamma = inputs.GAMMA_EFFICIENCY[(f"prefill_{n // 1024}k", t)]
            seg, _ = time_events(torch, lambda ev: pre.run(1.5, ev), 4, steps, 1)
            ts = float(np.median(seg.sum(1)))
            st = pre.stats() if n <= 16 * 1024 else None
            sp = st["sparsity"] if st else pre.group_sparsity()
            rows.append(dict(mode="prefill", context=f"{n // 1024}K", batch=1, target_sparsity=t,
                             sparsity=sp, gamma=w.gamma, ms=ts, stage1_ms=float(np.median(seg[:, 1])),
                             stage2_ms=float(np.median(seg[:, 2])), dense_self_ms=td, dense_sdpa_ms=tf,
                             speedup_vs_self=td / ts, speedup_vs_sdpa=tf / ts if tf else None,
                             pages_speedup=PAGES_SPEEDUP.get(("prefill", n // 1024, t))))
            print(f"[bench] efficiency {rows[-1]}", file=sys.stderr, flush=True)
        del pre
        torch.cuda.empty_cache()
    w = inputs.efficiency_decode()
    dd = Decode(w, torch, dash)
    w.gamma = 1e-3                          # near-uniform weights: every chunk routed, d = 0
    td = float(np.median(time_events(torch, dd.run, 2, steps, 1)[0]))
    dense_cnt = dd.bytes_per_step()[1]
    g = w.h_q // w.h_kv                      # a decode query sees every key: the g heads of
    qg = dd.Q.view(w.b, w.h_kv, g, w.d)      # a group become g query rows of one KV head
    tf = sdpa_time(torch, qg, dd.K, dd.V, False, steps)
    for t in inputs.EFFICIENCY_SPARSITY:
        key = (f"decode_{w.n // 1024}k_b{w.b}", t)
        if key not in inputs.GAMMA_EFFICIENCY:
            continue
        w.gamma = inputs.GAMMA_EFFICIENCY[key]
        tt = float(np.median(time_events(torch, dd.run, 2, steps, 1)[0]))
        cnt = dd.bytes_per_step()[1]
        vis = (w.seq_len - 1) // w.B
        sp = 1.0 - cnt.sum() / (vis[:, None] * np.ones_like(cnt)).sum()
        rows.append(dict(mode="decode", context=f"{w.n // 1024}K", batch=w.b, target_sparsity=t,
                         sparsity=float(sp), gamma=w.gamma, us=tt * 1e3, dense_self_us=td * 1e3,
                         dense_self_routed=int(dense_cnt.sum()),
                         dense_sdpa_us=tf * 1e3 if tf else None,
                         speedup_vs_self=td / tt, speedup_vs_sdpa=tf / tt if tf else None,
                         pages_speedup=PAGES_SPEEDUP.get(("decode", w.n // 1024, t))))
        print(f"[bench] efficiency {rows[-1]}", file=sys.stderr, flush=True)
    return rows


def backward(torch, dash, inputs, alpha, steps, warmup, no_dense=False):
    """The backward of the whole 32K prefill at α: the routed lists and router
    statistics of the forward, the forward's O and lse, an N(0,1) upstream gradient;
    timed per stage: Stage 2 (Δ and transposes, list inversion, dQ/d(bias) kernel,
    dK/dV kernel), Stage 1 (routing backward adding to dQ, into dk̄) and Stage 0
    (summary backward adding to dK, into dq̄). The Stage-2 kernels on the dense lists
    (every visible chunk, bias 0) are the 0%-sparsity baseline: dense attention has
    no routing to differentiate. Algorithmic flops of Stage 2: the five products of a
    softmax-attention backward (S, dP, dQ, dK, dV) over the pairs each row sees,
    2.5x the forward's."""
    wp = inputs.prefill_32k_clusters()
    pre = Prefill(wp, torch, dash)
    pre.run(alpha)
    b, h_q, n, d = wp.Q.shape
    B, hkv = wp.B, wp.h_kv
    stats = torch.empty((b, h_q, n, 2), device="cuda")
    dash.dash_route_stats(pre.Q, pre.kbar, B, alpha, wp.gamma, wp.sigma, True, pre.idx, pre.bias, pre.cnt,
                          stats, ws=pre.rws)
    torch.cuda.synchronize()
    st = pre.stats()
    lse = torch.empty((b, h_q, n), device="cuda")
    dO = torch.from_numpy(inputs.upstream_grad((b, h_q, n, d), seed=1, dtype="bf16")).to("cuda", torch.bfloat16)
    dQ = torch.empty((b, h_q, n, d), device="cuda")
    dK = torch.empty((b, hkv, n, d), device="cuda")
    dV = torch.empty((b, hkv, n, d), device="cuda")
    dkb = torch.empty((b, hkv, pre.T, d), device="cuda")
    dqb = torch.empty((hkv, d), device="cuda")
    ws = dash.alloc_backward_ws(b, h_q, hkv, n, d, B)

    def timed(idx, bias, cnt, chain):
        db = torch.empty(idx.shape, device="cuda")
        dash.dash_attend_prefill_lse(pre.Q, pre.K, pre.V, idx, bias, cnt, pre.O, lse, B, True, ws=pre.ws)

        def fn(ev):
            if ev: ev[0].record()
            dash.dash_attend_prefill_backward(pre.Q, pre.K, pre.V, idx, bias, cnt, pre.O, dO, lse,
                                              dQ, dK, dV, db, B, True, ws=ws)
            if ev: ev[1].record()
            if chain:
                dkb.zero_()
                dash.dash_route_backward(pre.Q, pre.kbar, idx, cnt, db, stats, B, alpha, wp.gamma, wp.sigma,
                                         dQ, dkb, ws=pre.rws)
                if ev: ev[2].record()
                dqb.zero_()
                dash.dash_summarize_backward(pre.K, pre.qbar, dkb, B, dK, dqb)
                if ev: ev[3].record()
        seg, _ = time_events(torch, fn, 4 if chain else 2, steps, warmup)
        return seg.mean(0)

    t2, t1, t0 = (float(x) for x in timed(pre.idx, pre.bias, pre.cnt, True))
    t = t2 + t1 + t0
    flops = 2.5 * st["flops_row"]
    out = dict(ms=t, stage2_ms=t2, stage1_ms=t1, stage0_ms=t0,
               stage2_tflops=flops / (t2 * 1e-3) / 1e12, stage2_frac=flops / (t2 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
               sparsity=st["sparsity"], stage2_algorithmic_tflop=flops / 1e12)
    print(f"[bench] backward alpha={alpha}: {out}", file=sys.stderr, flush=True)
    if no_dense:
        return out
    di, dbias, dc = dense_lists(pre, torch)
    td = float(timed(di, dbias, dc, False)[0])
    dense_flops = 2.5 * 4.0 * d * h_q * (n * (n + 1) / 2)
    out["dense"] = dict(ms=td, tflops=dense_flops / (td * 1e-3) / 1e12)
    out["speedup_vs_dense"] = td / t
    out["stage2_speedup_vs_dense"] = td / t2
    return out


def time_decode(torch, dd, scrub, args):
    """Median µs of a decode step with the 256 MiB Infinity Cache evicted before each
    step by reading a 512 MiB buffer (a read leaves no dirty lines to write back
    during the step; it sits outside the events), and unflushed for context."""
    sfl, _ = time_events(torch, lambda ev: (scrub.max(), dd.run(ev)), 2, args.steps, args.warmup)
    nbytes, cnt = dd.bytes_per_step()
    tfl = float(np.median(sfl))
    out = dict(us_per_step=tfl * 1e3, us_min=float(sfl.min()) * 1e3, us_max=float(sfl.max()) * 1e3,
               gbs=nbytes / (tfl * 1e-3) / 1e9, hbm_frac=nbytes / (tfl * 1e-3) / 1e9 / PEAK_HBM_GBS,
               bytes=nbytes, routed=cnt.ravel().tolist())
    if not args.flushed_only:
        sun, _ = time_events(torch, dd.run, 2, args.steps, args.warmup)
        out["us_per_step_unflushed"] = float(np.median(sun)) * 1e3
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1 (sharding across GPUs is not implemented)"}))
        sys.exit(2)
    import torch
    from long_context_amd import dash, inputs
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.efficiency:
        rows = efficiency(torch, dash, inputs, max(args.steps // 2, 3))
        print(json.dumps({"metric": "DashAttention speedup over dense at the efficiency operating points",
                          "n_gpus": 1, "data": "synthetic", "dtype": "bf16", "efficiency": rows}), flush=True)
        return

    if args.backward:
        res = backward(torch, dash, inputs, args.alpha, args.steps, args.warmup, args.no_dense)
        print(json.dumps({"metric": "backward time at the 32K prefill workload", "unit": "ms",
                          "value": res["ms"], "higher_is_better": False, "n_gpus": 1, "steps": args.steps,
                          "warmup": args.warmup, "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": "prefill_32k_clusters", "alpha": args.alpha},
                          "backward": res}), flush=True)
        return

    if args.only in ("decode128k", "decode32k"):
        w = inputs.decode_128k_b4() if args.only == "decode128k" else inputs.decode_32k_b16()
        scrub = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
        dec = time_decode(torch, Decode(w, torch, dash), scrub, args)
        print(json.dumps({"metric": f"decode µs/step, {w.name}", "unit": "us", "value": dec["us_per_step"],
                          "higher_is_better": False, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "dtype": "bf16", "data": "synthetic", "config": {"workload": w.name},
                          "decode": dec}), flush=True)
        return

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic"}
    print(f"[bench] generating workloads", file=sys.stderr, flush=True)
    wp = inputs.prefill_32k_clusters()
    pre = Prefill(wp, torch, dash)
    res = {}

    # --- prefill at the headline α, timed per stage ------------------------------
    seg, wall = time_events(torch, lambda ev: pre.run(args.alpha, ev), 4, args.steps, args.warmup)
    st = pre.stats()
    t_sum, t_route, t_att = (float(np.mean(seg[:, j])) for j in range(3))
    t_pre = t_sum + t_route + t_att
    tot = seg.sum(1)
    route_bytes = pre.route_bytes()
    res["prefill"] = dict(ms=t_pre, stage0_ms=t_sum, stage1_ms=t_route, stage2_ms=t_att,
                          tok_s=wp.n / (t_pre * 1e-3), sparsity=st["sparsity"],
                          stage2_row_tflops=st["flops_row"] / (t_att * 1e-3) / 1e12,
                          stage2_wave_tflops=st["flops_wave"] / (t_att * 1e-3) / 1e12,
                          stage2_tile_tflops=st["flops_tile"] / (t_att * 1e-3) / 1e12,
                          inflation_wave=st["inflation_wave"], inflation_tile=st["inflation_tile"],
                          ms_median=float(np.median(tot)), ms_min=float(tot.min()), ms_max=float(tot.max()),
                          stage1_gbs=route_bytes / (t_route * 1e-3) / 1e9,
                          wall_s=wall)
    print(f"[bench] prefill alpha={args.alpha}: {res['prefill']}", file=sys.stderr, flush=True)

    sweep = {}
    if not args.no_sweep:
        for a in (1.25, 1.5, 2.0):
            s2, _ = time_events(torch, lambda ev: pre.run(a, ev), 4, max(3, args.steps // 2), 1)
            sta = pre.stats()
            tt = float(s2.sum(1).mean())
            sweep[str(a)] = dict(tok_s=wp.n / (tt * 1e-3), ms=tt, sparsity=sta["sparsity"],
                                 stage2_ms=float(s2[:, 2].mean()),
                                 stage2_row_tflops=sta["flops_row"] / (float(s2[:, 2].mean()) * 1e-3) / 1e12)
            print(f"[bench] sweep alpha={a}: {sweep[str(a)]}", file=sys.stderr, flush=True)
        pre.run(args.alpha)
        torch.cuda.synchronize()

    # --- dense (0% sparsity) baseline of the same Stage-2 kernel ------------------
    dense = None
    if not args.no_dense:
        di, db, dc = dense_lists(pre, torch)
        Od = torch.empty_like(pre.O)
        fn = lambda ev: (ev and ev[0].record(),
                         dash.dash_attend_prefill(pre.Q, pre.K, pre.V, di, db, dc, Od, wp.B, True, ws=pre.ws),
                         ev and ev[1].record())
        sd, _ = time_events(torch, fn, 2, max(3, args.steps // 2), 1)
        td = float(sd.mean())
        dense_flops = 4.0 * wp.d * wp.h_q * (wp.n * (wp.n + 1) / 2)
        dense = dict(stage2_ms=td, tflops=dense_flops / (td * 1e-3) / 1e12,
                     speedup_vs_dense=td / t_pre)
        del di, db, dc, Od
        print(f"[bench] dense: {dense}", file=sys.stderr, flush=True)

    # --- decode at 128K (and 32K x 16) ----------------------------------------------
    dec = dec32 = None
    if args.only in ("decode", "both"):
        scrub = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
        dd = Decode(inputs.decode_128k_b4(), torch, dash)
        dec = time_decode(torch, dd, scrub, args)
        print(f"[bench] decode 128k: {dec}", file=sys.stderr, flush=True)
        del dd
        dd = Decode(inputs.decode_32k_b16(), torch, dash)
        dec32 = time_decode(torch, dd, scrub, args)
        dec32.pop("routed")
        print(f"[bench] decode 32k x16: {dec32}", file=sys.stderr, flush=True)
        del dd, scrub

    t_step = t_pre + (dec["us_per_step"] * 1e-3 if dec else 0.0)
    out.update({"value": res["prefill"]["tok_s"], "unit": "tok/s", "ms_per_step": t_step,
                "config": {"workload": "prefill_32k_clusters + decode_128k_b4",
                           "prefill": "b=1 h_q=32 h_kv=2 d=128 n=32768 B=64 gamma=1 sigma=1 "
                                      f"alpha={args.alpha}, 32 clusters x 4 chunks per KV head",
                           "decode": "b=4 h_q=32 h_kv=2 d=128 L=131072 B=128 alpha=1.5, "
                                     "4 flat + 4 sharp groups, 8 needles per group"}})
    att = res["prefill"]
    out["roofline"] = {"bound": "mfma", "kernel": "sparse_prior_attn_bf16_kernel",
                       "achieved": att["stage2_row_tflops"], "peak": PEAK_BF16_TFLOPS,
                       "unit": "TFLOP/s", "frac": att["stage2_row_tflops"] / PEAK_BF16_TFLOPS,
                       "traffic": measured_traffic(),
                       "routed_block_tflops": att["stage2_wave_tflops"],
                       "routed_block_frac": att["stage2_wave_tflops"] / PEAK_BF16_TFLOPS}
    out["prefill"] = att
    out["alpha_sweep"] = sweep
    out["dense_baseline"] = dense
    if dec:
        out["decode"] = dec
        out["decode_32k_b16"] = dec32
        out["decode_roofline"] = {"bound": "hbm", "kernel": "decode (route + split-KV + combine)",
                                  "achieved": dec["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": dec["hbm_frac"],
                                  "traffic": measured_traffic(DECODE_TRAFFIC_FILE, DECODE_SOURCES,
                                                              "traffic_bytes_per_step")}
    del pre
    torch.cuda.empty_cache()
    if not args.no_cpu:
        print(f"[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wp, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
