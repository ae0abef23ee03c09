// Internal launchers of the DashAttention kernels (called by the C ABI layer).
// Each returns hipSuccess or the launch error; arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dash {

struct SummaryArgs {
    const void* K; bool k_bf16; const float* qbar; float* kbar;
    int b, h_kv, n_kv, kbar_cap, d, B, chunk_begin, chunk_end;
    // paged cache (pages != nullptr): K is [num_pages, h_kv, B, d] and chunk c of
    // sequence b lives in page pages[b * pages_per_seq + c]
    const int32_t* pages = nullptr;
    int pages_per_seq = 0, num_pages = 0;
    // ragged batch (nullable): sequence b holds seq_len[b] tokens; chunks past its
    // last complete one are skipped
    const int32_t* seq_len = nullptr;
};
hipError_t launch_summary(const SummaryArgs& a, hipStream_t s);

struct RouteArgs {
    const void* Q; bool q_bf16; const float* kbar;
    int b, h_q, h_kv, n, kbar_cap, d, B, causal, list_cap;
    float alpha, gamma, sigma;
    int32_t* idx; float* bias; int32_t* cnt; float* w_out;
    void* ws;            // bf16 queries: split summaries, route_workspace_bytes
    int top_k;           // > 0: fixed budget of routed chunks per row
    float* stats = nullptr;  // optional [b, h_q, n, 2]: max raw logit, threshold
    const int32_t* seq_len = nullptr;  // ragged batch (nullable): rows of sequence b past
                                       // seq_len[b] get an empty list
};
hipError_t launch_route(const RouteArgs& a, hipStream_t s);
// Routed lists -> bitpacked mask [rows][words] (bit c%32 of word c/32 = chunk c routed).
hipError_t launch_lists_to_mask(const int32_t* idx, const int32_t* cnt, size_t rows, int list_cap, int T_c,
                                uint32_t* mask, int words, hipStream_t s);
// Scale of the routing logits: (α-1)γ/sqrt(d) for entmax, γ log2(e)/sqrt(d) for α = 1.
float route_scale(float alpha, float gamma, int d);
int pmode_of(float alpha);
// k̄ split into three bf16 terms in the routing kernel's staged layout (route.hip),
// written to ws (route_workspace_bytes bytes).
hipError_t launch_kbar_split(const float* kbar, void* ws, int b, int h_kv, int kbar_cap, int T_c, int d,
                             hipStream_t s);
// Workspace of a bf16-query routing: the summaries split into three bf16 terms,
// b * h_kv * (T_c rounded up to 32) * 3 * d * 2 bytes.
size_t route_workspace_bytes(int b, int h_kv, int T_c, int d);
// LDS bytes the routing kernel needs for group size g, chunk size B, T_c chunks
// (the host rejects shapes beyond what a compute unit holds).
size_t route_lds_bytes(int g, int B, int T_c, int d, bool q_bf16);
constexpr size_t kRouteLdsLimit = 159 * 1024;   // 160 KiB less room for static LDS
// Number of 16-chunk tiles the routing kernels keep in registers per row group
// for T chunks (0 if T is beyond the supported range of 2048 chunks).
int route_tiles_bucket(int T);

struct PrefillArgs {
    const void* Q; const void* K; const void* V; bool in_bf16;
    const int32_t* idx; const float* bias; const int32_t* cnt; int list_cap;
    void* O; bool out_bf16;
    int b, h_q, h_kv, n, d, B, causal;
    void* ws;            // bf16 inputs: V transposed, prefill_workspace_bytes
    float* lse = nullptr;  // optional [b, h_q, n] log-sum-exp of each row's logits
    const int32_t* seq_len = nullptr;  // ragged batch (nullable): sequence b holds
                                       // seq_len[b] tokens; later rows are not written
    // paged K/V (nullable): K and V are [num_pages, h_kv, B, d], chunk c of sequence b
    // in page pages[b * pages_per_seq + c]
    const int32_t* pages = nullptr;
    int pages_per_seq = 0, num_pages = 0;
};
hipError_t launch_attend_prefill(const PrefillArgs& a, hipStream_t s);

// Stage-2 backward for bf16 inputs (attend_backward_bf16.hip).
struct PrefillBwdArgs {
    const void* Q; const void* K; const void* V;
    const int32_t* idx; const float* bias; const int32_t* cnt; int list_cap;
    const void* O; const void* dO; bool o_bf16; const float* lse;
    float* dQ; float* dK; float* dV; float* dbias;
    int b, h_q, h_kv, n, d, B, causal;
    void* ws;            // K transposed, prefill_workspace_bytes
};
hipError_t launch_attend_prefill_backward(const PrefillBwdArgs& a, hipStream_t s);
// Backward of Stage 1 (route_backward.hip): dQ and dkbar accumulate (+=).
struct RouteBwdArgs {
    const void* Q; bool q_bf16; const float* kbar; int kbar_cap;
    const int32_t* idx; const int32_t* cnt; const float* dbias; int list_cap; const float* stats;
    int b, h_q, h_kv, n, d, B;
    float alpha, gamma, sigma;
    float* dQ; float* dkbar;
    void* ws;           // bf16 queries: the split summaries (route_workspace_bytes)
};
hipError_t launch_route_backward(const RouteBwdArgs& a, hipStream_t s);
// Backward of Stage 0 (route_backward.hip): dK and dqbar accumulate (+=).
struct SumBwdArgs {
    const void* K; bool k_bf16; const float* qbar; const float* dkbar;
    int b, h_kv, n, kbar_cap, d, B;
    float* dK; float* dqbar;
};
hipError_t launch_summary_backward(const SumBwdArgs& a, hipStream_t s);

// Rows per backward query tile for group size g at T_c chunks (0: unsupported).
int backward_tile_rows(int g, int B, int T_c, int d);
// Workspace of the backward: K^T per KV head, a bf16 dO, Δ and the inverted routed
// lists (sized for every row routing every visible chunk).
size_t backward_workspace_bytes(int b, int h_q, int h_kv, int n, int d, int B);
// V or K [b*h_kv][n][d] bf16 -> [b*h_kv][d][n_pad] (zero tokens n .. n_pad-1).
hipError_t launch_transpose_rows(const uint16_t* src, uint16_t* dst, int bh, int n, int n_pad, int d, hipStream_t s);
// Workspace of a bf16 prefill: V transposed per (b, KV head) as [d][n_pad] bf16 with
// n_pad = n rounded up to 64 (the pad is zero-filled).
int prefill_n_pad(int n);
size_t prefill_workspace_bytes(int b, int h_kv, int n, int d);
// Rows per query tile and dynamic LDS bytes of the prefill attention kernel
// (rows = 0 when the shape is not supported).
void prefill_tiling(int g, int B, int T_c, int d, bool bf16, int* rows, size_t* lds_bytes);

struct DecodeArgs {
    const void* Q; const void* Kc; const void* Vc; bool in_bf16;
    const float* kbar; const int32_t* seq_len;
    int b, h_q, h_kv, L_cap, kbar_cap, d, B;
    float alpha, gamma, sigma;
    void* O; bool out_bf16;
    int32_t* idx; float* bias; int32_t* cnt; float* w_out; int list_cap;
    float* scores;       // [b, h_q, T_route] workspace
    int32_t* counters;   // [3, b, h_kv] workspace: arrival counters (cleared by the
                         // kernels), then each group's first and last partial slot
    float* part_ml;      // [g, decode_partial_slots, 2] workspace
    float* part_o;       // [g, decode_partial_slots, d] workspace
    int T_route;         // routable chunk capacity: min(floor((L_cap-1)/B), kbar_cap)
    int top_k = 0;       // > 0: a fixed budget of routed chunks per group
    // paged cache (pages != nullptr): Kc/Vc are [num_pages, h_kv, B, d], chunk c of
    // sequence b lives in page pages[b * pages_per_seq + c], L_cap = pages_per_seq * B
    const int32_t* pages = nullptr;
    int pages_per_seq = 0, num_pages = 0;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// Partial-result slots of the split-KV decode: one per (attention wavefront, group it
// touches), at most the wavefront count bound plus b * h_kv.
int decode_partial_slots(int b, int h_kv);

}  // namespace dash
