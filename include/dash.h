/*
 * dash.h -- C ABI of the DashAttention forward pass on MI355X (gfx950).
 *
 * The method is the one of "DashAttention: Differentiable and Adaptive Sparse
 * Hierarchical Attention" as summarised on the xllm-io paper review, section 三
 * (technical architecture):
 *   Stage 0 (Eq. 4)   chunk summaries k̄_c = local SDPA of the learned query q̄
 *                      over the keys of chunk c (keys are also the values);
 *   Stage 1 (Eq. 6)   chunk logits z̄ = <q, k̄>/sqrt(d), per-head α-entmax of γz̄,
 *                      GQA average w within each KV group, support = union;
 *   Stage 2 (Eq. 9-12 via Prop. 4.1)  softmax over the routed chunks' tokens and
 *                      the query's own diagonal chunk, with the additive bias
 *                      d = (log w - μ)/σ on routed tokens (μ = mean of log w over
 *                      the support) and 0 on the diagonal.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     keeps no pointer after returning and allocates no device memory (scratch
 *     memory comes in through the workspace arguments).
 *   - Tensors are contiguous, batch-head-sequence-dim (BHSD):
 *       Q [b, h_q, n, d], K and V [b, h_kv, n, d], q̄ [h_kv, d] (fp32),
 *       k̄ [b, h_kv, kbar_cap, d] (fp32).
 *   - Query head h belongs to KV group r = floor(h / g) with g = h_q / h_kv.
 *   - Chunk c holds tokens [c*B, (c+1)*B). Only complete chunks have a summary
 *     (T_c = floor(n / B)).
 *   - Causal routing: the query at position p may route to chunks c < floor(p/B);
 *     its own chunk (tokens floor(p/B)*B .. p) is the diagonal branch and is
 *     always attended with bias 0. Non-causal: every complete chunk is routable
 *     and the trailing n mod B tokens form the diagonal branch.
 *   - Routed lists are ascending chunk ids per (b, r, query row), with the bias
 *     of each listed chunk alongside.
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue
 *     work; they never synchronise.
 *   - n = 0 (empty sequences) is a valid call of the prefill-side entry points: the
 *     arguments are validated as usual (pointers non-null) and nothing is launched.
 *   - Every argument is validated on the host before anything is enqueued; on
 *     error nothing is launched, outputs are untouched, and a detail string is
 *     available from dash_last_error() (per thread). The library never aborts.
 *     Device faults surface at the caller's next synchronisation.
 *   - Supported: d in {64, 128}; B a multiple of 16 (the prefill attention
 *     kernel needs B a multiple of 32); g = h_q/h_kv a power of two <= 16;
 *     Q/K/V both fp32 or all bf16; α >= 1, γ > 0, σ > 0 (σ = +inf allowed);
 *     at most 2048 routable chunks per row (e.g. 128K tokens at B = 64).
 *   - α = 1 routes with softmax instead of entmax (the α -> 1 limit of the
 *     entmax family, a dense-routing ablation): ŵ = softmax(γ z̄) per head,
 *     every visible chunk is routed, and w, μ and d are formed as for α > 1.
 */
#ifndef DASH_H
#define DASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DASH_OK = 0,
    DASH_ERR_NULL = 1,         /* a required pointer is NULL                    */
    DASH_ERR_SHAPE = 2,        /* inconsistent or non-positive sizes            */
    DASH_ERR_PARAM = 3,        /* α, γ, σ out of range, bad dtype or flag       */
    DASH_ERR_UNSUPPORTED = 4,  /* valid but outside the supported set above     */
    DASH_ERR_WORKSPACE = 5,    /* workspace missing or smaller than required    */
    DASH_ERR_LAUNCH = 6        /* the HIP runtime refused a launch              */
} dash_status;

typedef enum { DASH_F32 = 0, DASH_BF16 = 1 } dash_dtype;

typedef enum { DASH_OP_ROUTE = 0, DASH_OP_PREFILL = 1, DASH_OP_DECODE = 2, DASH_OP_PREFILL_BWD = 3 } dash_op;

/*
 * Stage 0 (Eq. 4): for every (b, r) and every chunk c in [chunk_begin, chunk_end):
 *   k̄[b,r,c,:] = sum_{t in chunk c} softmax_t(<q̄[r], K[b,r,t]>/sqrt(d)) K[b,r,t,:].
 * K: [b, h_kv, n_kv, d] of k_dtype; qbar: [h_kv, d] fp32; kbar: [b, h_kv, kbar_cap, d]
 * fp32 (only rows chunk_begin..chunk_end-1 are written). Requires
 * 0 <= chunk_begin <= chunk_end <= min(floor(n_kv/B), kbar_cap). During decode,
 * call it for a chunk once the chunk is complete (the summary is then fixed).
 */
dash_status dash_summarize(const void* K, int k_dtype, const float* qbar, float* kbar,
                           int b, int h_kv, int n_kv, int kbar_cap, int d, int B,
                           int chunk_begin, int chunk_end, void* stream);

/*
 * Ragged batches (sequences of different lengths padded to one n): seq_len [b]
 * (device int32) gives the tokens of each sequence, clamped to [0, n]. The pages
 * define every stage per sequence (Eq. 4, Eq. 6 and Eq. 10 see only the
 * sequence's own tokens), so a ragged batch is the per-sequence computation on
 * each sequence's first seq_len[b] rows, with T_b = floor(seq_len[b]/B) complete
 * chunks. Padding rows of Q, K and V are never read and may hold anything.
 *
 * dash_summarize_varlen: dash_summarize restricted to chunks c < T_b of each
 * sequence (the chunk range still applies); k̄ rows of later chunks are not
 * written. seq_len == NULL returns DASH_ERR_NULL (use dash_summarize).
 */
dash_status dash_summarize_varlen(const void* K, int k_dtype, const float* qbar, float* kbar,
                                  const int32_t* seq_len, int b, int h_kv, int n_kv, int kbar_cap, int d, int B,
                                  int chunk_begin, int chunk_end, void* stream);

/*
 * Stage 1 for a prefill (Eq. 6, the GQA paragraph, Prop. 4.1's μ and d): every
 * query row i (position i) of Q [b, h_q, n, d] (q_dtype) is routed against
 * k̄ [b, h_kv, kbar_cap, d] (chunks 0..floor(n/B)-1 must be summarised).
 * Outputs per (b, r, i):
 *   cnt [b, h_kv, n] int32      number of routed chunks |S_i|
 *   idx [b, h_kv, n, list_cap]  int32 ascending routed chunk ids (first cnt valid)
 *   bias[b, h_kv, n, list_cap]  fp32  d = (ln w - μ)/σ of each listed chunk
 *   w_out (nullable) [b, h_kv, n, kbar_cap] fp32 dense group weights w (0 off
 *          the visible set); meant for verification.
 * list_cap >= floor(n/B) and kbar_cap >= floor(n/B). bf16 queries need a device
 * workspace of at least dash_workspace_bytes(DASH_OP_ROUTE, ...) bytes (the
 * summaries split into three bf16 terms, b * h_kv * (floor(n/B) rounded up to 32)
 * * 3 * d * 2 bytes); fp32 queries need none (ws may be NULL). Calls that share one
 * workspace must not overlap. Shapes whose working set does not fit a compute
 * unit's LDS (many chunks with few query heads per KV head) return
 * DASH_ERR_UNSUPPORTED.
 */
dash_status dash_route(const void* Q, int q_dtype, const float* kbar,
                       int b, int h_q, int h_kv, int n, int kbar_cap, int d, int B,
                       float alpha, float gamma, float sigma, int causal,
                       int32_t* idx, float* bias, int32_t* cnt, int list_cap,
                       float* w_out, void* ws, size_t ws_bytes, void* stream);

/*
 * dash_route with a fixed routing budget, for ablations against the top-k block
 * selection the pages compare with (paper review section 二, the hierarchical
 * sparse attention background): after the group weights w are formed, each row
 * keeps only the top_k largest w among its routed chunks (all of them when it has
 * at most top_k; equal weights go to the lower chunk id first), and μ and d are
 * taken over the kept chunks. top_k = 0 is dash_route. With α = 1 (softmax
 * routing, every visible chunk has w > 0) each row routes exactly
 * min(top_k, visible chunks). top_k < 0 returns DASH_ERR_PARAM; everything else
 * as dash_route.
 */
dash_status dash_route_topk(const void* Q, int q_dtype, const float* kbar,
                            int b, int h_q, int h_kv, int n, int kbar_cap, int d, int B,
                            float alpha, float gamma, float sigma, int causal,
                            int32_t* idx, float* bias, int32_t* cnt, int list_cap,
                            float* w_out, int top_k, void* ws, size_t ws_bytes, void* stream);

/*
 * dash_route_topk over a ragged batch (seq_len as for dash_summarize_varlen): row i
 * < seq_len[b] of sequence b is routed against that sequence's chunks c < T_b only
 * (causal: c < min(floor(i/B), T_b)); k̄ rows of later chunks are not read. Padding
 * rows i >= seq_len[b] get cnt = 0, and their idx, bias and w_out rows are not
 * written. w_out of a routed row is 0 for chunks >= T_b. Everything else,
 * including the workspace (sized by n), as dash_route_topk.
 */
dash_status dash_route_varlen(const void* Q, int q_dtype, const float* kbar, const int32_t* seq_len,
                              int b, int h_q, int h_kv, int n, int kbar_cap, int d, int B,
                              float alpha, float gamma, float sigma, int causal,
                              int32_t* idx, float* bias, int32_t* cnt, int list_cap,
                              float* w_out, int top_k, void* ws, size_t ws_bytes, void* stream);

/*
 * dash_route with the forward statistics the routing backward needs: stats
 * [b, h_q, n, 2] (device fp32) gets, for every (query head, row) with a visible
 * chunk, the largest raw logit <q, k̄_c> and the threshold of its weights (α > 1: τ of
 * ŵ = [y - τ]_+^{1/(α-1)}; α = 1: log2 Σ_c 2^y), with y = cs (<q, k̄_c> - max) and
 * cs = (α-1)γ/sqrt(d) (α = 1: γ log2(e)/sqrt(d)). Other arguments as dash_route.
 */
dash_status dash_route_stats(const void* Q, int q_dtype, const float* kbar,
                             int b, int h_q, int h_kv, int n, int kbar_cap, int d, int B,
                             float alpha, float gamma, float sigma, int causal,
                             int32_t* idx, float* bias, int32_t* cnt, int list_cap,
                             float* w_out, float* stats, void* ws, size_t ws_bytes, void* stream);

/*
 * Stage-1 backward (paper review section 三: Eq. 6 routing, the GQA average and the
 * Prop. 4.1 bias; the support held fixed): for the gradient dbias of the routed bias
 * entries [b, h_kv, n, list_cap] (device fp32, as dash_attend_prefill_backward
 * writes it) and the lists and statistics of dash_route_stats, ADDS to dQ
 * [b, h_q, n, d] the routing path's query gradient and to dkbar [b, h_kv, kbar_cap, d]
 * the summaries' gradient (both device fp32; dkbar by atomic adds, so its last bits
 * may vary between runs). Per row: g_c = (db_c - mean db)/σ, ∂ŵ_c = g_c/Σ_h ŵ_hc,
 * the α-entmax Jacobian diag(s) - s sᵀ/Σs with s = ŵ^(2-α) (α = 1: s = ŵ), and the
 * chain through <q_h, k̄_c>·γ/sqrt(d). σ = +inf: no-op. floor(n/B) ≤ 2048 chunks (as
 * for the router). List entries outside [0, floor(n/B)) are skipped. Lists of a fixed top-k budget are not supported (their
 * kept set drops chunks the entmax normalisation couples). The weights are rebuilt
 * with the router's own arithmetic, so the support seen here is the forward's. bf16
 * queries need a device workspace of at least dash_workspace_bytes(DASH_OP_ROUTE, ...)
 * bytes (k̄ split into bf16 terms); fp32 queries need none (ws may be NULL). Calls
 * that share one workspace must not overlap.
 */
dash_status dash_route_backward(const void* Q, int q_dtype, const float* kbar, int kbar_cap,
                                const int32_t* idx, const int32_t* cnt, const float* dbias, int list_cap,
                                const float* stats, int b, int h_q, int h_kv, int n, int d, int B,
                                float alpha, float gamma, float sigma, float* dQ, float* dkbar,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * Stage-0 backward (Eq. 4: k̄_c = Σ_j π_j k_j, π = softmax_j(<q̄, k_j>/sqrt(d))): for
 * dkbar [b, h_kv, kbar_cap, d] ADDS to dK [b, h_kv, n, d] (tokens of complete chunks)
 * and to dqbar [h_kv, d] (device fp32; dqbar by atomic adds). K in k_dtype, q̄
 * [h_kv, d] fp32.
 */
dash_status dash_summarize_backward(const void* K, int k_dtype, const float* qbar, const float* dkbar,
                                    int b, int h_kv, int n, int kbar_cap, int d, int B,
                                    float* dK, float* dqbar, void* stream);

/*
 * Bitpacked block mask of routed lists (the form of the routing decision in the
 * pages' GPU kernel table: M_i in {0,1}^{T_c}, 32 chunks per 32-bit word): for every
 * (b, r, row) of idx [b, h_kv, n, list_cap] / cnt [b, h_kv, n] (device int32, as
 * dash_route writes them), mask [b, h_kv, n, words] (device uint32) gets bit c % 32
 * of word c / 32 set iff chunk c (0 <= c < T_c) is listed; all other bits are zero.
 * Requires list_cap >= T_c, T_c <= 2048 and ceil(T_c/32) <= words <= 64. List
 * entries outside [0, T_c) and counts outside [0, list_cap] are clamped away.
 */
dash_status dash_route_mask(const int32_t* idx, const int32_t* cnt, int b, int h_kv, int n, int list_cap,
                            int T_c, uint32_t* mask, int words, void* stream);

/*
 * Stage 2 for a prefill (Eq. 10 in the bias form of Prop. 4.1): for every query
 * head and row, softmax over the tokens of the routed chunks (logit
 * <q,k>/sqrt(d) + bias of the chunk) and of the diagonal branch (bias 0, causal
 * mask inside the own chunk), times V. Q, K, V share in_dtype; O
 * [b, h_q, n, d] is written in out_dtype. idx/bias/cnt are dash_route's outputs
 * (same list_cap). Requires B % 32 == 0. bf16 inputs need a device workspace of at
 * least dash_workspace_bytes(DASH_OP_PREFILL, ...) bytes (V transposed to
 * [b, h_kv, d, n rounded up to 64]); fp32 inputs need none (ws may be NULL). Calls
 * that share one workspace must not overlap.
 */
dash_status dash_attend_prefill(const void* Q, const void* K, const void* V, int in_dtype,
                                const int32_t* idx, const float* bias, const int32_t* cnt,
                                int list_cap, void* O, int out_dtype,
                                int b, int h_q, int h_kv, int n, int d, int B, int causal,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * dash_attend_prefill that also writes lse [b, h_q, n] (device fp32): the natural
 * log of the softmax denominator of each (head, row), i.e. log sum_j exp(z_ij + d_ij)
 * over the row's routed and diagonal tokens; -inf for a row that sees no token.
 * lse == NULL behaves as dash_attend_prefill. This is the statistic the backward
 * (dash_attend_prefill_backward) reuses instead of a second softmax pass.
 */
dash_status dash_attend_prefill_lse(const void* Q, const void* K, const void* V, int in_dtype,
                                    const int32_t* idx, const float* bias, const int32_t* cnt,
                                    int list_cap, void* O, int out_dtype, float* lse,
                                    int b, int h_q, int h_kv, int n, int d, int B, int causal,
                                    void* ws, size_t ws_bytes, void* stream);

/*
 * dash_attend_prefill_lse over a ragged batch (seq_len as for dash_summarize_varlen;
 * idx/bias/cnt as dash_route_varlen writes them): row i < seq_len[b] attends to its
 * routed chunks and to its diagonal branch inside the sequence (causal: its own
 * chunk up to i; non-causal: the sequence's tokens from T_b*B on), never to a
 * token >= seq_len[b]. Rows i >= seq_len[b] of O and lse (nullable) are not
 * written. The Stage-2 backward has no ragged form. Workspace as
 * dash_attend_prefill (sized by n).
 */
dash_status dash_attend_prefill_varlen(const void* Q, const void* K, const void* V, int in_dtype,
                                       const int32_t* seq_len, const int32_t* idx, const float* bias,
                                       const int32_t* cnt, int list_cap, void* O, int out_dtype, float* lse,
                                       int b, int h_q, int h_kv, int n, int d, int B, int causal,
                                       void* ws, size_t ws_bytes, void* stream);

/*
 * Stage 2 of a prefill (Eq. 9-12 via Prop. 4.1, as dash_attend_prefill) whose K and
 * V live in a paged KV cache, so that prefill and incremental decoding (the
 * gist.science summary, "Efficient GPU Implementation") share one cache. Layout of
 * dash_attend_decode_paged: Kp, Vp [num_pages, h_kv, B, d], chunk c of sequence b in page
 * pages[b * pages_per_seq + c] (device int32 [b, pages_per_seq]); Q stays contiguous
 * [b, h_q, n, d]. seq_len (nullable) gives a ragged batch as for
 * dash_attend_prefill_varlen; otherwise every sequence holds n tokens. Requires
 * pages_per_seq * B >= n and a cache of fewer than 2^31 rows. Page ids outside
 * [0, num_pages) are clamped (wrong output, never a stray read). The summaries come
 * from dash_summarize_paged, the lists from dash_route or dash_route_varlen. Output,
 * lse (nullable) and workspace as dash_attend_prefill_lse; the result equals the
 * contiguous entry point's on the same tokens.
 */
dash_status dash_attend_prefill_paged(const void* Q, const void* Kp, const void* Vp, int in_dtype,
                                      const int32_t* pages, int pages_per_seq, int num_pages,
                                      const int32_t* seq_len, const int32_t* idx, const float* bias,
                                      const int32_t* cnt, int list_cap, void* O, int out_dtype, float* lse,
                                      int b, int h_q, int h_kv, int n, int d, int B, int causal,
                                      void* ws, size_t ws_bytes, void* stream);

/*
 * Stage-2 backward (the support and the per-chunk bias of Prop. 4.1 held fixed: the
 * gradient of a softmax attention with an additive bias). Inputs: the forward's
 * Q, K, V (in_dtype, bf16 only), idx/bias/cnt (same list_cap), its output O and the
 * upstream gradient dO [b, h_q, n, d] (both o_dtype) and lse from
 * dash_attend_prefill_lse. Outputs, all device fp32:
 *   dQ [b, h_q, n, d], dK and dV [b, h_kv, n, d];
 *   dbias [b, h_kv, n, list_cap]: entry e of a row is the gradient of bias entry e,
 *   the sum of dZ over the tokens of chunk idx[e] and the group's g query heads;
 *   entries at or past cnt, or naming a chunk the row cannot see, are zero.
 * Requires B % 32 == 0 (a 32-token chunk takes a 64-token tile of the dK/dV pass,
 * half of it computed and discarded), g = h_q/h_kv <= 16, d in {64, 128}, n*floor(n/B) < 2^31
 * and a device workspace of dash_workspace_bytes(DASH_OP_PREFILL_BWD, ...) bytes
 * (grows with n^2/B: the routed lists inverted per chunk are sized for dense
 * routing). dK and dV sum several partials with atomic adds, so their last bits
 * may differ between runs; dQ and dbias are reproducible. Calls that share a
 * workspace must not overlap.
 */
dash_status dash_attend_prefill_backward(const void* Q, const void* K, const void* V, int in_dtype,
                                         const int32_t* idx, const float* bias, const int32_t* cnt, int list_cap,
                                         const void* O, const void* dO, int o_dtype, const float* lse,
                                         float* dQ, float* dK, float* dV, float* dbias,
                                         int b, int h_q, int h_kv, int n, int d, int B, int causal,
                                         void* ws, size_t ws_bytes, void* stream);

/*
 * One decode step (Stages 1-2 for one new query per sequence, split-KV Stage 2):
 *   Q [b, h_q, 1, d]; Kc, Vc [b, h_kv, L_cap, d] hold the KV cache including the
 *   new token; seq_len [b] (device int32) = KV length L incl. the new token, so
 *   the query sits at position L-1; kbar [b, h_kv, kbar_cap, d] must hold the
 *   summaries of chunks 0..floor((L-1)/B)-1. Device-side lengths are clamped to
 *   [1, L_cap] and the routable chunks to kbar_cap.
 *   O [b, h_q, 1, d] in out_dtype.
 *   Optional outputs (NULL to skip): idx_out/bias_out [b, h_kv, list_cap],
 *   cnt_out [b, h_kv], w_out [b, h_kv, kbar_cap] dense group weights.
 * ws: at least dash_workspace_bytes(DASH_OP_DECODE, b, h_q, h_kv, L_cap, d, B)
 * bytes of device memory (scores, routed lists, per-group counters and split-KV
 * partials); no initial contents are needed (the kernels clear what they count).
 * Calls that share one workspace must not overlap.
 */
dash_status dash_attend_decode(const void* Q, const void* Kc, const void* Vc, int in_dtype,
                               const float* kbar, const int32_t* seq_len,
                               int b, int h_q, int h_kv, int L_cap, int kbar_cap, int d, int B,
                               float alpha, float gamma, float sigma,
                               void* O, int out_dtype,
                               int32_t* idx_out, float* bias_out, int32_t* cnt_out,
                               float* w_out, int list_cap,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * Decode with a fixed routing budget (an ablation of the adaptive support; the
 * decode counterpart of dash_route_topk): each group keeps only the top_k largest
 * group weights w among its routed chunks (all of them when it has at most top_k;
 * equal weights go to the lower chunk id first), and μ and the bias d of
 * Proposition 4.1 are taken over the kept chunks. top_k = 0 is dash_attend_decode;
 * top_k < 0 returns DASH_ERR_PARAM. Everything else as in dash_attend_decode.
 */
dash_status dash_attend_decode_topk(const void* Q, const void* Kc, const void* Vc, int in_dtype,
                                    const float* kbar, const int32_t* seq_len,
                                    int b, int h_q, int h_kv, int L_cap, int kbar_cap, int d, int B,
                                    float alpha, float gamma, float sigma,
                                    void* O, int out_dtype,
                                    int32_t* idx_out, float* bias_out, int32_t* cnt_out,
                                    float* w_out, int list_cap, int top_k,
                                    void* ws, size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): dash_attend_decode without a workspace
 * argument. The kernels' scratch (scores, routed lists, counters, split-KV
 * partials) lives in a library-owned device array of DASH_NOALLOC_SCRATCH_BYTES
 * that each GPU the library runs on holds until the process ends; the call makes
 * no allocation of any kind. Shapes whose decode workspace
 * (dash_workspace_bytes(DASH_OP_DECODE, ...)) exceeds it return DASH_ERR_WORKSPACE
 * before anything is enqueued. Every call on one GPU shares that GPU's array and
 * leaves its contents behind (the kernels clear what they count), so calls that
 * overlap on one GPU (other streams, other threads) race. Arguments and outputs are
 * otherwise those of dash_attend_decode.
 */
#define DASH_NOALLOC_SCRATCH_BYTES (32u << 20)
dash_status dash_attend_decode_noalloc(const void* Q, const void* Kc, const void* Vc, int in_dtype,
                                       const float* kbar, const int32_t* seq_len,
                                       int b, int h_q, int h_kv, int L_cap, int kbar_cap, int d, int B,
                                       float alpha, float gamma, float sigma,
                                       void* O, int out_dtype,
                                       int32_t* idx_out, float* bias_out, int32_t* cnt_out,
                                       float* w_out, int list_cap, void* stream);

/*
 * Paged KV cache (serving): pages of one chunk each. Kp, Vp are
 * [num_pages, h_kv, B, d]; chunk c of sequence b (tokens cB .. cB+B-1) lives in
 * page pages[b * pages_per_seq + c] (device int32 table [b, pages_per_seq]), so a
 * sequence holds at most L_cap = pages_per_seq * B tokens. Everything else is as in
 * dash_summarize / dash_attend_decode with that L_cap (the workspace is
 * dash_workspace_bytes(DASH_OP_DECODE, b, h_q, h_kv, pages_per_seq * B, d, B)).
 * Page ids outside [0, num_pages) are clamped (wrong output, never a stray read).
 */
dash_status dash_summarize_paged(const void* Kp, int k_dtype, const float* qbar, float* kbar,
                                 const int32_t* pages, int pages_per_seq, int num_pages,
                                 int b, int h_kv, int kbar_cap, int d, int B,
                                 int chunk_begin, int chunk_end, void* stream);
dash_status dash_attend_decode_paged(const void* Q, const void* Kp, const void* Vp, int in_dtype,
                                     const float* kbar, const int32_t* seq_len,
                                     const int32_t* pages, int pages_per_seq, int num_pages,
                                     int b, int h_q, int h_kv, int kbar_cap, int d, int B,
                                     float alpha, float gamma, float sigma,
                                     void* O, int out_dtype,
                                     int32_t* idx_out, float* bias_out, int32_t* cnt_out,
                                     float* w_out, int list_cap,
                                     void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes an operation needs (n_or_Lcap: n for prefill ops, L_cap for
 * decode; DASH_OP_ROUTE and DASH_OP_PREFILL give the size for bf16 inputs, which
 * fp32 inputs do not need; DASH_OP_PREFILL_BWD is the Stage-2 backward's). Returns 0 when no
 * workspace is needed, (size_t)-1 on invalid sizes. */
size_t dash_workspace_bytes(int op, int b, int h_q, int h_kv, int n_or_Lcap, int d, int B);

/* Static English name of a status code. */
const char* dash_status_string(int status);

/* Detail of the last failed call on this thread ("" if none). */
const char* dash_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DASH_H */
