"""Python binding of libdash (the C ABI in include/dash.h).

Argument marshalling only: each function takes torch tensors that already live on
the GPU, checks they are contiguous, reads their sizes, and passes raw device
pointers and the current HIP stream to the C entry point of the same name. Every
step of the computation runs in the library's HIP kernels. PyTorch provides device
memory and streams.

Loading fails loudly (ImportError) when libdash.so has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdash.so")

DASH_OK, DASH_ERR_NULL, DASH_ERR_SHAPE, DASH_ERR_PARAM = 0, 1, 2, 3
DASH_ERR_UNSUPPORTED, DASH_ERR_WORKSPACE, DASH_ERR_LAUNCH = 4, 5, 6
DASH_F32, DASH_BF16 = 0, 1
DASH_OP_ROUTE, DASH_OP_PREFILL, DASH_OP_DECODE, DASH_OP_PREFILL_BWD = 0, 1, 2, 3


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m long_context_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.dash_summarize.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.dash_summarize.restype = i32
    lib.dash_summarize_varlen.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.dash_summarize_varlen.restype = i32
    lib.dash_route.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, i32, i32, f32, f32, f32, i32,
                               vp, vp, vp, i32, vp, vp, sz, vp]
    lib.dash_route.restype = i32
    lib.dash_route_topk.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, i32, i32, f32, f32, f32, i32,
                                    vp, vp, vp, i32, vp, i32, vp, sz, vp]
    lib.dash_route_topk.restype = i32
    lib.dash_route_varlen.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, f32, f32, i32,
                                      vp, vp, vp, i32, vp, i32, vp, sz, vp]
    lib.dash_route_varlen.restype = i32
    lib.dash_route_stats.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, i32, i32, f32, f32, f32, i32,
                                     vp, vp, vp, i32, vp, vp, vp, sz, vp]
    lib.dash_route_stats.restype = i32
    lib.dash_route_backward.argtypes = [vp, i32, vp, i32, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32,
                                        f32, f32, f32, vp, vp, vp, sz, vp]
    lib.dash_route_backward.restype = i32
    lib.dash_summarize_backward.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.dash_summarize_backward.restype = i32
    lib.dash_route_mask.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, i32, vp]
    lib.dash_route_mask.restype = i32
    lib.dash_attend_prefill.argtypes = [vp, vp, vp, i32, vp, vp, vp, i32, vp, i32,
                                        i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.dash_attend_prefill.restype = i32
    lib.dash_attend_prefill_lse.argtypes = [vp, vp, vp, i32, vp, vp, vp, i32, vp, i32, vp,
                                            i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.dash_attend_prefill_lse.restype = i32
    lib.dash_attend_prefill_varlen.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, i32, vp, i32, vp,
                                               i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.dash_attend_prefill_varlen.restype = i32
    lib.dash_attend_prefill_paged.argtypes = [vp, vp, vp, i32, vp, i32, i32, vp, vp, vp, vp, i32, vp, i32, vp,
                                              i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.dash_attend_prefill_paged.restype = i32
    lib.dash_attend_prefill_backward.argtypes = [vp, vp, vp, i32, vp, vp, vp, i32, vp, vp, i32, vp,
                                                 vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                                 vp, sz, vp]
    lib.dash_attend_prefill_backward.restype = i32
    lib.dash_attend_decode.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                       f32, f32, f32, vp, i32, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.dash_attend_decode.restype = i32
    lib.dash_attend_decode_topk.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                            f32, f32, f32, vp, i32, vp, vp, vp, vp, i32, i32, vp, sz, vp]
    lib.dash_attend_decode_topk.restype = i32
    lib.dash_attend_decode_noalloc.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                               f32, f32, f32, vp, i32, vp, vp, vp, vp, i32, vp]
    lib.dash_attend_decode_noalloc.restype = i32
    lib.dash_summarize_paged.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.dash_summarize_paged.restype = i32
    lib.dash_attend_decode_paged.argtypes = [vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                             i32, f32, f32, f32, vp, i32, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.dash_attend_decode_paged.restype = i32
    lib.dash_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.dash_workspace_bytes.restype = sz
    lib.dash_status_string.argtypes = [i32]
    lib.dash_status_string.restype = ctypes.c_char_p
    lib.dash_last_error.argtypes = []
    lib.dash_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()

SYMBOLS = ("dash_summarize", "dash_summarize_varlen", "dash_summarize_paged", "dash_summarize_backward",
           "dash_route", "dash_route_topk", "dash_route_varlen", "dash_route_stats", "dash_route_backward",
           "dash_route_mask", "dash_attend_prefill", "dash_attend_prefill_lse", "dash_attend_prefill_varlen",
           "dash_attend_prefill_paged",
           "dash_attend_prefill_backward",
           "dash_attend_decode", "dash_attend_decode_topk", "dash_attend_decode_noalloc", "dash_attend_decode_paged",
           "dash_workspace_bytes", "dash_status_string", "dash_last_error")


class DashError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{lib.dash_status_string(status).decode()} ({status}): {detail}")


def _check(status: int) -> None:
    if status != DASH_OK:
        raise DashError(status, lib.dash_last_error().decode())


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DASH_F32
    if t.dtype == torch.bfloat16:
        return DASH_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def dash_status_string(status: int) -> str:
    return lib.dash_status_string(status).decode()


def dash_workspace_bytes(op: int, b: int, h_q: int, h_kv: int, n_or_Lcap: int, d: int, B: int) -> int:
    return int(lib.dash_workspace_bytes(op, b, h_q, h_kv, n_or_Lcap, d, B))


def dash_summarize(K, qbar, kbar, B, chunk_begin=0, chunk_end=None, stream=None):
    """Stage 0 summaries of chunks [chunk_begin, chunk_end) of K [b,h_kv,n,d] into kbar."""
    b, h_kv, n, d = K.shape
    if chunk_end is None:
        chunk_end = n // B
    _check(lib.dash_summarize(_ptr(K), _dtype(K), _ptr(qbar), _ptr(kbar), b, h_kv, n,
                              kbar.shape[2], d, B, chunk_begin, chunk_end, _stream(stream)))


def dash_summarize_varlen(K, qbar, kbar, seq_len, B, chunk_begin=0, chunk_end=None, stream=None):
    """dash_summarize over a ragged batch: only chunks below seq_len[b] // B of each sequence."""
    b, h_kv, n, d = K.shape
    if chunk_end is None:
        chunk_end = min(n // B, kbar.shape[2])
    _check(lib.dash_summarize_varlen(_ptr(K), _dtype(K), _ptr(qbar), _ptr(kbar), _ptr(seq_len), b, h_kv, n,
                                     kbar.shape[2], d, B, chunk_begin, chunk_end, _stream(stream)))


def dash_route_varlen(Q, kbar, seq_len, B, alpha, gamma, sigma, causal, idx, bias, cnt, w_out=None,
                      ws=None, stream=None, top_k=0):
    """dash_route over a ragged batch (seq_len [b] int32): padding rows get cnt 0."""
    b, h_q, n, d = Q.shape
    h_kv = kbar.shape[1]
    if ws is None and Q.dtype == torch.bfloat16:
        ws = alloc_route_ws(b, h_q, h_kv, n, d, B, device=Q.device)
    _check(lib.dash_route_varlen(_ptr(Q), _dtype(Q), _ptr(kbar), _ptr(seq_len), b, h_q, h_kv, n, kbar.shape[2], d,
                                 B, float(alpha), float(gamma), float(sigma), int(causal),
                                 _ptr(idx), _ptr(bias), _ptr(cnt), idx.shape[-1], _ptr(w_out), int(top_k),
                                 _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def dash_route(Q, kbar, B, alpha, gamma, sigma, causal, idx, bias, cnt, w_out=None,
               ws=None, stream=None, top_k=0):
    """Stage 1 of a prefill: routed chunk lists idx/bias [b,h_kv,n,cap] and cnt [b,h_kv,n].

    bf16 queries need a workspace (alloc_route_ws); one is allocated when ws is None.
    top_k > 0 calls dash_route_topk (a fixed budget of routed chunks per row)."""
    b, h_q, n, d = Q.shape
    h_kv = kbar.shape[1]
    if ws is None and Q.dtype == torch.bfloat16:
        ws = alloc_route_ws(b, h_q, h_kv, n, d, B, device=Q.device)
    args = (_ptr(Q), _dtype(Q), _ptr(kbar), b, h_q, h_kv, n, kbar.shape[2], d, B,
            float(alpha), float(gamma), float(sigma), int(causal),
            _ptr(idx), _ptr(bias), _ptr(cnt), idx.shape[-1], _ptr(w_out))
    tail = (_ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    if top_k:
        _check(lib.dash_route_topk(*args, int(top_k), *tail))
    else:
        _check(lib.dash_route(*args, *tail))


def dash_route_stats(Q, kbar, B, alpha, gamma, sigma, causal, idx, bias, cnt, stats, w_out=None,
                     ws=None, stream=None):
    """dash_route that also writes stats [b,h_q,n,2] (max raw logit, threshold)."""
    b, h_q, n, d = Q.shape
    h_kv = kbar.shape[1]
    if ws is None and Q.dtype == torch.bfloat16:
        ws = alloc_route_ws(b, h_q, h_kv, n, d, B, device=Q.device)
    _check(lib.dash_route_stats(_ptr(Q), _dtype(Q), _ptr(kbar), b, h_q, h_kv, n, kbar.shape[2], d, B,
                                float(alpha), float(gamma), float(sigma), int(causal),
                                _ptr(idx), _ptr(bias), _ptr(cnt), idx.shape[-1], _ptr(w_out), _ptr(stats),
                                _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def dash_route_backward(Q, kbar, idx, cnt, dbias, stats, B, alpha, gamma, sigma, dQ, dkbar, ws=None, stream=None):
    """Stage-1 backward: adds the routing path's gradients to dQ [b,h_q,n,d] and dkbar."""
    b, h_q, n, d = Q.shape
    h_kv = kbar.shape[1]
    if ws is None and Q.dtype == torch.bfloat16:
        ws = alloc_route_ws(b, h_q, h_kv, n, d, B, device=Q.device)
    _check(lib.dash_route_backward(_ptr(Q), _dtype(Q), _ptr(kbar), kbar.shape[2], _ptr(idx), _ptr(cnt),
                                   _ptr(dbias), idx.shape[-1], _ptr(stats), b, h_q, h_kv, n, d, B,
                                   float(alpha), float(gamma), float(sigma), _ptr(dQ), _ptr(dkbar),
                                   _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                   _stream(stream)))


def dash_summarize_backward(K, qbar, dkbar, B, dK, dqbar, stream=None):
    """Stage-0 backward: adds to dK [b,h_kv,n,d] and dqbar [h_kv,d] for dkbar."""
    b, h_kv, n, d = K.shape
    _check(lib.dash_summarize_backward(_ptr(K), _dtype(K), _ptr(qbar), _ptr(dkbar), b, h_kv, n, dkbar.shape[2],
                                       d, B, _ptr(dK), _ptr(dqbar), _stream(stream)))


def dash_route_mask(idx, cnt, T_c, mask, stream=None):
    """Bitpacked mask [b,h_kv,n,words] (int32 storage of uint32 words) of routed lists."""
    b, h_kv, n, cap = idx.shape
    _check(lib.dash_route_mask(_ptr(idx), _ptr(cnt), b, h_kv, n, cap, int(T_c), _ptr(mask),
                               mask.shape[-1], _stream(stream)))


def dash_attend_prefill(Q, K, V, idx, bias, cnt, O, B, causal, ws=None, stream=None):
    """Stage 2 of a prefill into O [b,h_q,n,d] (fp32 or bf16).

    bf16 inputs need a workspace (alloc_prefill_ws); one is allocated when ws is None."""
    b, h_q, n, d = Q.shape
    h_kv = K.shape[1]
    if ws is None and Q.dtype == torch.bfloat16:
        ws = alloc_prefill_ws(b, h_q, h_kv, n, d, B, device=Q.device)
    _check(lib.dash_attend_prefill(_ptr(Q), _ptr(K), _ptr(V), _dtype(Q), _ptr(idx), _ptr(bias),
                                   _ptr(cnt), idx.shape[-1], _ptr(O), _dtype(O), b, h_q, h_kv, n,
                                   d, B, int(causal), _ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(),
                                   _stream(stream)))


def dash_attend_prefill_lse(Q, K, V, idx, bias, cnt, O, lse, B, causal, ws=None, stream=None):
    """dash_attend_prefill that also writes the log-sum-exp lse [b,h_q,n] (fp32)."""
    b, h_q, n, d = Q.shape
    h_kv = K.shape[1]
    if ws is None and Q.dtype == torch.bfloat16:
        ws = alloc_prefill_ws(b, h_q, h_kv, n, d, B, device=Q.device)
    _check(lib.dash_attend_prefill_lse(_ptr(Q), _ptr(K), _ptr(V), _dtype(Q), _ptr(idx), _ptr(bias),
                                       _ptr(cnt), idx.shape[-1], _ptr(O), _dtype(O), _ptr(lse), b, h_q,
                                       h_kv, n, d, B, int(causal), _ptr(ws),
                                       0 if ws is None else ws.numel() * ws.element_size(),
                                       _stream(stream)))


def dash_attend_prefill_varlen(Q, K, V, seq_len, idx, bias, cnt, O, B, causal, lse=None, ws=None, stream=None):
    """dash_attend_prefill over a ragged batch: rows at or past seq_len[b] are not written."""
    b, h_q, n, d = Q.shape
    h_kv = K.shape[1]
    if ws is None and Q.dtype == torch.bfloat16:
        ws = alloc_prefill_ws(b, h_q, h_kv, n, d, B, device=Q.device)
    _check(lib.dash_attend_prefill_varlen(_ptr(Q), _ptr(K), _ptr(V), _dtype(Q), _ptr(seq_len), _ptr(idx),
                                          _ptr(bias), _ptr(cnt), idx.shape[-1], _ptr(O), _dtype(O), _ptr(lse),
                                          b, h_q, h_kv, n, d, B, int(causal), _ptr(ws),
                                          0 if ws is None else ws.numel() * ws.element_size(),
                                          _stream(stream)))


def dash_attend_prefill_paged(Q, Kp, Vp, pages, idx, bias, cnt, O, B, causal, n=None, seq_len=None, lse=None,
                              ws=None, stream=None):
    """Stage 2 of a prefill over a paged cache Kp, Vp [num_pages, h_kv, B, d]; pages
    [b, pages_per_seq] int32; seq_len (optional) for a ragged batch."""
    b, h_q, nq, d = Q.shape
    n = nq if n is None else n
    h_kv = Kp.shape[1]
    if ws is None and Q.dtype == torch.bfloat16:
        ws = alloc_prefill_ws(b, h_q, h_kv, n, d, B, device=Q.device)
    _check(lib.dash_attend_prefill_paged(_ptr(Q), _ptr(Kp), _ptr(Vp), _dtype(Q), _ptr(pages), pages.shape[1],
                                         Kp.shape[0], _ptr(seq_len), _ptr(idx), _ptr(bias), _ptr(cnt),
                                         idx.shape[-1], _ptr(O), _dtype(O), _ptr(lse), b, h_q, h_kv, n, d, B,
                                         int(causal), _ptr(ws),
                                         0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def dash_attend_prefill_backward(Q, K, V, idx, bias, cnt, O, dO, lse, dQ, dK, dV, dbias, B, causal,
                                 ws=None, stream=None):
    """Stage-2 gradients dQ [b,h_q,n,d], dK/dV [b,h_kv,n,d] and dbias [b,h_kv,n,cap] (fp32).

    A workspace (alloc_backward_ws) is allocated when ws is None."""
    b, h_q, n, d = Q.shape
    h_kv = K.shape[1]
    if ws is None:
        ws = alloc_backward_ws(b, h_q, h_kv, n, d, B, device=Q.device)
    if O.dtype != dO.dtype:
        raise TypeError("O and dO must share a dtype")
    _check(lib.dash_attend_prefill_backward(_ptr(Q), _ptr(K), _ptr(V), _dtype(Q), _ptr(idx), _ptr(bias),
                                            _ptr(cnt), idx.shape[-1], _ptr(O), _ptr(dO), _dtype(O), _ptr(lse),
                                            _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dbias), b, h_q, h_kv, n, d, B,
                                            int(causal), _ptr(ws),
                                            0 if ws is None else ws.numel() * ws.element_size(),
                                            _stream(stream)))


def dash_attend_decode(Q, Kc, Vc, kbar, seq_len, B, alpha, gamma, sigma, O, ws,
                       idx_out=None, bias_out=None, cnt_out=None, w_out=None, stream=None, top_k=0):
    """One decode step: Q [b,h_q,1,d] against the KV cache Kc/Vc [b,h_kv,L_cap,d].
    top_k > 0 calls dash_attend_decode_topk (a fixed budget of routed chunks per group)."""
    b, h_q, _, d = Q.shape
    _, h_kv, L_cap, _ = Kc.shape
    list_cap = idx_out.shape[-1] if idx_out is not None else 0
    args = (_ptr(Q), _ptr(Kc), _ptr(Vc), _dtype(Q), _ptr(kbar), _ptr(seq_len), b, h_q, h_kv, L_cap,
            kbar.shape[2], d, B, float(alpha), float(gamma), float(sigma), _ptr(O), _dtype(O),
            _ptr(idx_out), _ptr(bias_out), _ptr(cnt_out), _ptr(w_out), list_cap)
    tail = (_ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if top_k:
        _check(lib.dash_attend_decode_topk(*args, int(top_k), *tail))
    else:
        _check(lib.dash_attend_decode(*args, *tail))


def dash_attend_decode_noalloc(Q, Kc, Vc, kbar, seq_len, B, alpha, gamma, sigma, O,
                               idx_out=None, bias_out=None, cnt_out=None, w_out=None, stream=None):
    """dash_attend_decode without a workspace: the library's per-GPU device scratch."""
    b, h_q, _, d = Q.shape
    _, h_kv, L_cap, _ = Kc.shape
    list_cap = idx_out.shape[-1] if idx_out is not None else 0
    _check(lib.dash_attend_decode_noalloc(_ptr(Q), _ptr(Kc), _ptr(Vc), _dtype(Q), _ptr(kbar),
                                          _ptr(seq_len), b, h_q, h_kv, L_cap, kbar.shape[2], d, B,
                                          float(alpha), float(gamma), float(sigma), _ptr(O), _dtype(O),
                                          _ptr(idx_out), _ptr(bias_out), _ptr(cnt_out), _ptr(w_out),
                                          list_cap, _stream(stream)))


def dash_summarize_paged(Kp, qbar, kbar, pages, B, chunk_begin, chunk_end, stream=None):
    """Stage 0 of chunks [chunk_begin, chunk_end) from a paged cache Kp [P,h_kv,B,d]."""
    P, h_kv, _, d = Kp.shape
    b, pps = pages.shape
    _check(lib.dash_summarize_paged(_ptr(Kp), _dtype(Kp), _ptr(qbar), _ptr(kbar), _ptr(pages), pps, P,
                                    b, h_kv, kbar.shape[2], d, B, chunk_begin, chunk_end, _stream(stream)))


def dash_attend_decode_paged(Q, Kp, Vp, kbar, seq_len, pages, B, alpha, gamma, sigma, O, ws,
                             idx_out=None, bias_out=None, cnt_out=None, w_out=None, stream=None):
    """One decode step against a paged cache Kp/Vp [P,h_kv,B,d] with page table [b, pages_per_seq]."""
    b, h_q, _, d = Q.shape
    P, h_kv, _, _ = Kp.shape
    pps = pages.shape[1]
    list_cap = idx_out.shape[-1] if idx_out is not None else 0
    _check(lib.dash_attend_decode_paged(_ptr(Q), _ptr(Kp), _ptr(Vp), _dtype(Q), _ptr(kbar), _ptr(seq_len),
                                        _ptr(pages), pps, P, b, h_q, h_kv, kbar.shape[2], d, B,
                                        float(alpha), float(gamma), float(sigma), _ptr(O), _dtype(O),
                                        _ptr(idx_out), _ptr(bias_out), _ptr(cnt_out), _ptr(w_out),
                                        list_cap, _ptr(ws), ws.numel() * ws.element_size(),
                                        _stream(stream)))


# ----------------------------------------------------------------------------------
# Allocation helpers (device memory only; no computation).
# ----------------------------------------------------------------------------------

def alloc_kbar(b, h_kv, T, d, device="cuda"):
    return torch.empty((b, h_kv, max(T, 1), d), dtype=torch.float32, device=device)


def alloc_route(b, h_kv, n, T, device="cuda", with_w=False):
    cap = max(T, 1)
    idx = torch.empty((b, h_kv, n, cap), dtype=torch.int32, device=device)
    bias = torch.empty((b, h_kv, n, cap), dtype=torch.float32, device=device)
    cnt = torch.empty((b, h_kv, n), dtype=torch.int32, device=device)
    w = torch.empty((b, h_kv, n, cap), dtype=torch.float32, device=device) if with_w else None
    return idx, bias, cnt, w


def alloc_route_ws(b, h_q, h_kv, n, d, B, device="cuda"):
    nbytes = dash_workspace_bytes(DASH_OP_ROUTE, b, h_q, h_kv, n, d, B)
    return torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=device)


def alloc_prefill_ws(b, h_q, h_kv, n, d, B, device="cuda"):
    nbytes = dash_workspace_bytes(DASH_OP_PREFILL, b, h_q, h_kv, n, d, B)
    return torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=device)


def alloc_backward_ws(b, h_q, h_kv, n, d, B, device="cuda"):
    nbytes = dash_workspace_bytes(DASH_OP_PREFILL_BWD, b, h_q, h_kv, n, d, B)
    return torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=device)


def alloc_decode_ws(b, h_q, h_kv, L_cap, d, B, device="cuda"):
    nbytes = dash_workspace_bytes(DASH_OP_DECODE, b, h_q, h_kv, L_cap, d, B)
    return torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=device)
