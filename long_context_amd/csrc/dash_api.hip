// C ABI of the DashAttention forward pass (declared in include/dash.h).
// Every entry point validates all of its arguments on the host before it enqueues
// anything; on error it returns a status, leaves the outputs untouched and records
// a detail string for dash_last_error(). Nothing here synchronises the stream.
#include "../../include/dash.h"
#include "kernels.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

namespace {

thread_local char g_err[512] = "";

dash_status fail(dash_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

dash_status ok() {
    g_err[0] = '\0';
    return DASH_OK;
}

dash_status from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(DASH_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
bool valid_dtype(int t) { return t == DASH_F32 || t == DASH_BF16; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

dash_status check_common(int b, int h_q, int h_kv, int d, int B) {
    if (b < 1 || h_q < 1 || h_kv < 1) return fail(DASH_ERR_SHAPE, "b, h_q, h_kv must be >= 1");
    if (h_q % h_kv != 0) return fail(DASH_ERR_SHAPE, "h_q (%d) must be a multiple of h_kv (%d)", h_q, h_kv);
    if (d != 64 && d != 128) return fail(DASH_ERR_UNSUPPORTED, "head dim %d not in {64, 128}", d);
    if (B < 16 || B % 16 != 0) return fail(DASH_ERR_UNSUPPORTED, "chunk size %d must be a positive multiple of 16", B);
    const int g = h_q / h_kv;
    if (!is_pow2(g) || g > 16) return fail(DASH_ERR_UNSUPPORTED, "GQA group size %d must be a power of two <= 16", g);
    return DASH_OK;
}

dash_status check_params(float alpha, float gamma, float sigma) {
    if (!(alpha >= 1.0f) || isinf(alpha)) return fail(DASH_ERR_PARAM, "alpha must be finite and >= 1 (got %g)", alpha);
    if (!(gamma > 0.0f) || isinf(gamma)) return fail(DASH_ERR_PARAM, "gamma must be finite and > 0 (got %g)", gamma);
    if (!(sigma > 0.0f)) return fail(DASH_ERR_PARAM, "sigma must be > 0 or +inf (got %g)", sigma);
    return DASH_OK;
}

struct DecodeLayout {
    int T_ws, T_route;
    size_t off_scores, off_idx, off_bias, off_cnt, off_counters, off_ml, off_o, total;
};

DecodeLayout decode_layout(int b, int h_q, int h_kv, int L_cap, int kbar_cap, int d, int B) {
    DecodeLayout L;
    const int g = h_q / h_kv;
    L.T_ws = (L_cap - 1) / B;                       // upper bound of the routable chunks
    L.T_route = kbar_cap < L.T_ws ? kbar_cap : L.T_ws;
    const size_t nT = (size_t)(L.T_ws > 0 ? L.T_ws : 1);
    const size_t slots = (size_t)dash::decode_partial_slots(b, h_kv);
    L.off_scores = 0;
    L.off_idx = align256(L.off_scores + (size_t)b * h_q * nT * 4);
    L.off_bias = align256(L.off_idx + (size_t)b * h_kv * nT * 4);
    L.off_cnt = align256(L.off_bias + (size_t)b * h_kv * nT * 4);
    L.off_counters = align256(L.off_cnt + (size_t)b * h_kv * 4);
    L.off_ml = align256(L.off_counters + (size_t)3 * b * h_kv * 4);
    L.off_o = align256(L.off_ml + (size_t)g * slots * 2 * 4);
    L.total = align256(L.off_o + (size_t)g * slots * d * 4);
    return L;
}

// Device scratch of dash_attend_decode_noalloc: a file-scope array that every GPU the
// library runs on holds until the process ends. Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): it asks each
// device once for the array's address there and keeps that pointer per device.
static __device__ __align__(256) unsigned char scratch[DASH_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

dash_status scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DASH_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(DASH_ERR_UNSUPPORTED, "device %d beyond the scratch table", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(DASH_ERR_LAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return DASH_OK;
}

}  // namespace

extern "C" {

const char* dash_status_string(int status) {
    switch (status) {
        case DASH_OK: return "ok";
        case DASH_ERR_NULL: return "null pointer";
        case DASH_ERR_SHAPE: return "invalid shape";
        case DASH_ERR_PARAM: return "invalid parameter";
        case DASH_ERR_UNSUPPORTED: return "unsupported configuration";
        case DASH_ERR_WORKSPACE: return "workspace too small";
        case DASH_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

const char* dash_last_error(void) { return g_err; }

dash_status dash_summarize(const void* K, int k_dtype, const float* qbar, float* kbar,
                           int b, int h_kv, int n_kv, int kbar_cap, int d, int B,
                           int chunk_begin, int chunk_end, void* stream) {
    if (!K || !qbar || !kbar) return fail(DASH_ERR_NULL, "K, qbar and kbar must be non-null");
    if (!valid_dtype(k_dtype)) return fail(DASH_ERR_PARAM, "bad K dtype %d", k_dtype);
    dash_status st = check_common(b, h_kv, h_kv, d, B);
    if (st != DASH_OK) return st;
    if (n_kv < 0 || kbar_cap < 0) return fail(DASH_ERR_SHAPE, "n_kv and kbar_cap must be >= 0");
    const int T = n_kv / B;
    const int lim = T < kbar_cap ? T : kbar_cap;
    if (chunk_begin < 0 || chunk_begin > chunk_end || chunk_end > lim)
        return fail(DASH_ERR_SHAPE, "chunk range [%d, %d) outside [0, %d]", chunk_begin, chunk_end, lim);
    dash::SummaryArgs a{K, k_dtype == DASH_BF16, qbar, kbar, b, h_kv, n_kv, kbar_cap, d, B,
                        chunk_begin, chunk_end};
    return from_hip(dash::launch_summary(a, (hipStream_t)stream), "chunk_summary_kernel");
}

dash_status dash_summarize_varlen(const void* K, int k_dtype, const float* qbar, float* kbar,
                                  const int32_t* seq_len, int b, int h_kv, int n_kv, int kbar_cap, int d, int B,
                                  int chunk_begin, int chunk_end, void* stream) {
    if (!seq_len) return fail(DASH_ERR_NULL, "seq_len must be non-null");
    if (!K || !qbar || !kbar) return fail(DASH_ERR_NULL, "K, qbar and kbar must be non-null");
    if (!valid_dtype(k_dtype)) return fail(DASH_ERR_PARAM, "bad K dtype %d", k_dtype);
    dash_status st = check_common(b, h_kv, h_kv, d, B);
    if (st != DASH_OK) return st;
    if (n_kv < 0 || kbar_cap < 0) return fail(DASH_ERR_SHAPE, "n_kv and kbar_cap must be >= 0");
    const int T = n_kv / B;
    const int lim = T < kbar_cap ? T : kbar_cap;
    if (chunk_begin < 0 || chunk_begin > chunk_end || chunk_end > lim)
        return fail(DASH_ERR_SHAPE, "chunk range [%d, %d) outside [0, %d]", chunk_begin, chunk_end, lim);
    dash::SummaryArgs a{K, k_dtype == DASH_BF16, qbar, kbar, b, h_kv, n_kv, kbar_cap, d, B,
                        chunk_begin, chunk_end};
    a.seq_len = seq_len;
    return from_hip(dash::launch_summary(a, (hipStream_t)stream), "chunk_summary_kernel");
}

dash_status dash_summarize_paged(const void* Kp, int k_dtype, const float* qbar, float* kbar,
                                 const int32_t* pages, int pages_per_seq, int num_pages,
                                 int b, int h_kv, int kbar_cap, int d, int B,
                                 int chunk_begin, int chunk_end, void* stream) {
    if (!Kp || !qbar || !kbar || !pages) return fail(DASH_ERR_NULL, "Kp, qbar, kbar and pages must be non-null");
    if (!valid_dtype(k_dtype)) return fail(DASH_ERR_PARAM, "bad K dtype %d", k_dtype);
    dash_status st = check_common(b, h_kv, h_kv, d, B);
    if (st != DASH_OK) return st;
    if (pages_per_seq < 1 || num_pages < 1 || kbar_cap < 0)
        return fail(DASH_ERR_SHAPE, "pages_per_seq and num_pages must be >= 1 and kbar_cap >= 0");
    const int lim = pages_per_seq < kbar_cap ? pages_per_seq : kbar_cap;
    if (chunk_begin < 0 || chunk_begin > chunk_end || chunk_end > lim)
        return fail(DASH_ERR_SHAPE, "chunk range [%d, %d) outside [0, %d]", chunk_begin, chunk_end, lim);
    dash::SummaryArgs a{Kp, k_dtype == DASH_BF16, qbar, kbar, b, h_kv, pages_per_seq * B, kbar_cap, d, B,
                        chunk_begin, chunk_end, pages, pages_per_seq, num_pages};
    return from_hip(dash::launch_summary(a, (hipStream_t)stream), "chunk_summary_kernel");
}

static dash_status route_impl(const void* Q, int q_dtype, const float* kbar,
                              int b, int h_q, int h_kv, int n, int kbar_cap, int d, int B,
                              float alpha, float gamma, float sigma, int causal,
                              int32_t* idx, float* bias, int32_t* cnt, int list_cap,
                              float* w_out, int top_k, float* stats, void* ws, size_t ws_bytes, void* stream,
                              const int32_t* seq_len = nullptr) {
    if (!Q || !kbar || !idx || !bias || !cnt) return fail(DASH_ERR_NULL, "Q, kbar, idx, bias and cnt must be non-null");
    if (!valid_dtype(q_dtype)) return fail(DASH_ERR_PARAM, "bad Q dtype %d", q_dtype);
    if (causal != 0 && causal != 1) return fail(DASH_ERR_PARAM, "causal must be 0 or 1");
    if (top_k < 0) return fail(DASH_ERR_PARAM, "top_k must be >= 0 (got %d)", top_k);
    dash_status st = check_common(b, h_q, h_kv, d, B);
    if (st != DASH_OK) return st;
    if ((st = check_params(alpha, gamma, sigma)) != DASH_OK) return st;
    if (n < 0) return fail(DASH_ERR_SHAPE, "n must be >= 0");
    const int T = n / B;
    if (kbar_cap < T) return fail(DASH_ERR_SHAPE, "kbar_cap %d < floor(n/B) = %d", kbar_cap, T);
    if (list_cap < T) return fail(DASH_ERR_SHAPE, "list_cap %d < floor(n/B) = %d", list_cap, T);
    if (dash::route_tiles_bucket(T) == 0) return fail(DASH_ERR_UNSUPPORTED, "%d chunks exceed the router's 2048", T);
    const size_t lds = dash::route_lds_bytes(h_q / h_kv, B, T, d, q_dtype == DASH_BF16);
    if (lds > dash::kRouteLdsLimit)
        return fail(DASH_ERR_UNSUPPORTED, "routing %d chunks at g = %d needs %zu bytes of LDS (limit %zu)", T, h_q / h_kv,
                    lds, dash::kRouteLdsLimit);
    if (q_dtype == DASH_BF16 && T > 0) {
        const size_t need = dash::route_workspace_bytes(b, h_kv, T, d);
        if (!ws || ws_bytes < need)
            return fail(DASH_ERR_WORKSPACE, "bf16 routing needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : (size_t)0);
    }
    dash::RouteArgs a{Q, q_dtype == DASH_BF16, kbar, b, h_q, h_kv, n, kbar_cap, d, B, causal, list_cap,
                      alpha, gamma, sigma, idx, bias, cnt, w_out, ws, top_k, stats, seq_len};
    return from_hip(dash::launch_route(a, (hipStream_t)stream), "entmax_route_kernel");
}

dash_status dash_route_topk(const void* Q, int q_dtype, const float* kbar,
                            int b, int h_q, int h_kv, int n, int kbar_cap, int d, int B,
                            float alpha, float gamma, float sigma, int causal,
                            int32_t* idx, float* bias, int32_t* cnt, int list_cap,
                            float* w_out, int top_k, void* ws, size_t ws_bytes, void* stream) {
    return route_impl(Q, q_dtype, kbar, b, h_q, h_kv, n, kbar_cap, d, B, alpha, gamma, sigma, causal, idx, bias, cnt,
                      list_cap, w_out, top_k, nullptr, ws, ws_bytes, stream);
}

dash_status dash_route_varlen(const void* Q, int q_dtype, const float* kbar, const int32_t* seq_len,
                              int b, int h_q, int h_kv, int n, int kbar_cap, int d, int B,
                              float alpha, float gamma, float sigma, int causal,
                              int32_t* idx, float* bias, int32_t* cnt, int list_cap,
                              float* w_out, int top_k, void* ws, size_t ws_bytes, void* stream) {
    if (!seq_len) return fail(DASH_ERR_NULL, "seq_len must be non-null");
    return route_impl(Q, q_dtype, kbar, b, h_q, h_kv, n, kbar_cap, d, B, alpha, gamma, sigma, causal, idx, bias, cnt,
                      list_cap, w_out, top_k, nullptr, ws, ws_bytes, stream, seq_len);
}

dash_status dash_route_stats(const void* Q, int q_dtype, const float* kbar,
                             int b, int h_q, int h_kv, int n, int kbar_cap, int d, int B,
                             float alpha, float gamma, float sigma, int causal,
                             int32_t* idx, float* bias, int32_t* cnt, int list_cap,
                             float* w_out, float* stats, void* ws, size_t ws_bytes, void* stream) {
    if (!stats) return fail(DASH_ERR_NULL, "stats must be non-null");
    return route_impl(Q, q_dtype, kbar, b, h_q, h_kv, n, kbar_cap, d, B, alpha, gamma, sigma, causal, idx, bias, cnt,
                      list_cap, w_out, 0, stats, ws, ws_bytes, stream);
}

dash_status dash_route(const void* Q, int q_dtype, const float* kbar,
                       int b, int h_q, int h_kv, int n, int kbar_cap, int d, int B,
                       float alpha, float gamma, float sigma, int causal,
                       int32_t* idx, float* bias, int32_t* cnt, int list_cap,
                       float* w_out, void* ws, size_t ws_bytes, void* stream) {
    return dash_route_topk(Q, q_dtype, kbar, b, h_q, h_kv, n, kbar_cap, d, B, alpha, gamma, sigma, causal, idx,
                           bias, cnt, list_cap, w_out, 0, ws, ws_bytes, stream);
}

dash_status dash_route_backward(const void* Q, int q_dtype, const float* kbar, int kbar_cap,
                                const int32_t* idx, const int32_t* cnt, const float* dbias, int list_cap,
                                const float* stats, int b, int h_q, int h_kv, int n, int d, int B,
                                float alpha, float gamma, float sigma, float* dQ, float* dkbar,
                                void* ws, size_t ws_bytes, void* stream) {
    if (!Q || !kbar || !idx || !cnt || !dbias || !stats || !dQ || !dkbar)
        return fail(DASH_ERR_NULL, "every tensor argument of the routing backward must be non-null");
    if (!valid_dtype(q_dtype)) return fail(DASH_ERR_PARAM, "bad Q dtype %d", q_dtype);
    dash_status st = check_common(b, h_q, h_kv, d, B);
    if (st != DASH_OK) return st;
    if ((st = check_params(alpha, gamma, sigma)) != DASH_OK) return st;
    if (n < 0) return fail(DASH_ERR_SHAPE, "n must be >= 0");
    const int T = n / B;
    if (kbar_cap < T) return fail(DASH_ERR_SHAPE, "kbar_cap %d < floor(n/B) = %d", kbar_cap, T);
    if (list_cap < T) return fail(DASH_ERR_SHAPE, "list_cap %d < floor(n/B) = %d", list_cap, T);
    if (dash::route_tiles_bucket(T) == 0) return fail(DASH_ERR_UNSUPPORTED, "%d chunks exceed the router's 2048", T);
    if (q_dtype == DASH_BF16 && T > 0) {
        const size_t need = dash::route_workspace_bytes(b, h_kv, T, d);
        if (!ws || ws_bytes < need)
            return fail(DASH_ERR_WORKSPACE, "bf16 routing backward needs %zu workspace bytes, got %zu", need,
                        ws ? ws_bytes : (size_t)0);
    }
    dash::RouteBwdArgs a{Q, q_dtype == DASH_BF16, kbar, kbar_cap, idx, cnt, dbias, list_cap, stats,
                         b, h_q, h_kv, n, d, B, alpha, gamma, sigma, dQ, dkbar, ws};
    return from_hip(dash::launch_route_backward(a, (hipStream_t)stream), "route_backward_lds_kernel");
}

dash_status dash_summarize_backward(const void* K, int k_dtype, const float* qbar, const float* dkbar,
                                    int b, int h_kv, int n, int kbar_cap, int d, int B,
                                    float* dK, float* dqbar, void* stream) {
    if (!K || !qbar || !dkbar || !dK || !dqbar)
        return fail(DASH_ERR_NULL, "K, qbar, dkbar, dK and dqbar must be non-null");
    if (!valid_dtype(k_dtype)) return fail(DASH_ERR_PARAM, "bad K dtype %d", k_dtype);
    dash_status st = check_common(b, h_kv, h_kv, d, B);
    if (st != DASH_OK) return st;
    if (n < 0) return fail(DASH_ERR_SHAPE, "n must be >= 0");
    if (kbar_cap < n / B) return fail(DASH_ERR_SHAPE, "kbar_cap %d < floor(n/B) = %d", kbar_cap, n / B);
    dash::SumBwdArgs a{K, k_dtype == DASH_BF16, qbar, dkbar, b, h_kv, n, kbar_cap, d, B, dK, dqbar};
    return from_hip(dash::launch_summary_backward(a, (hipStream_t)stream), "summary_backward_kernel");
}

dash_status dash_route_mask(const int32_t* idx, const int32_t* cnt, int b, int h_kv, int n, int list_cap,
                            int T_c, uint32_t* mask, int words, void* stream) {
    if (!idx || !cnt || !mask) return fail(DASH_ERR_NULL, "idx, cnt and mask must be non-null");
    if (b < 1 || h_kv < 1 || n < 0) return fail(DASH_ERR_SHAPE, "need b >= 1, h_kv >= 1, n >= 0");
    if (T_c < 0 || T_c > 2048) return fail(DASH_ERR_UNSUPPORTED, "T_c must be in [0, 2048] (got %d)", T_c);
    if (list_cap < T_c) return fail(DASH_ERR_SHAPE, "list_cap %d < T_c %d", list_cap, T_c);
    if (words < (T_c + 31) / 32 || words > 64)
        return fail(DASH_ERR_SHAPE, "words must be in [ceil(T_c/32), 64] (got %d for T_c %d)", words, T_c);
    if (words == 0) return DASH_OK;
    return from_hip(dash::launch_lists_to_mask(idx, cnt, (size_t)b * h_kv * n, list_cap, T_c, mask, words,
                                               (hipStream_t)stream),
                    "lists_to_mask_kernel");
}

static dash_status attend_prefill(const void* Q, const void* K, const void* V, int in_dtype,
                                  const int32_t* idx, const float* bias, const int32_t* cnt,
                                  int list_cap, void* O, int out_dtype, float* lse,
                                  int b, int h_q, int h_kv, int n, int d, int B, int causal,
                                  void* ws, size_t ws_bytes, void* stream, const int32_t* seq_len,
                                  const int32_t* pages = nullptr, int pages_per_seq = 0, int num_pages = 0) {
    if (!Q || !K || !V || !idx || !bias || !cnt || !O) return fail(DASH_ERR_NULL, "Q, K, V, idx, bias, cnt and O must be non-null");
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return fail(DASH_ERR_PARAM, "bad dtype");
    if (causal != 0 && causal != 1) return fail(DASH_ERR_PARAM, "causal must be 0 or 1");
    dash_status st = check_common(b, h_q, h_kv, d, B);
    if (st != DASH_OK) return st;
    if (B % 32 != 0) return fail(DASH_ERR_UNSUPPORTED, "prefill attention needs B %% 32 == 0 (B = %d)", B);
    if (n < 0) return fail(DASH_ERR_SHAPE, "n must be >= 0");
    const int T = n / B;
    if (list_cap < T) return fail(DASH_ERR_SHAPE, "list_cap %d < floor(n/B) = %d", list_cap, T);
    int rows = 0;
    size_t lds = 0;
    dash::prefill_tiling(h_q / h_kv, B, T, d, in_dtype == DASH_BF16, &rows, &lds);
    if (rows == 0) return fail(DASH_ERR_UNSUPPORTED, "no query tiling fits LDS (g=%d, B=%d, T_c=%d)", h_q / h_kv, B, T);
    if (in_dtype == DASH_BF16 && n > 0) {
        const size_t need = dash::prefill_workspace_bytes(b, h_kv, n, d);
        if (!ws || ws_bytes < need)
            return fail(DASH_ERR_WORKSPACE, "bf16 prefill needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : (size_t)0);
    }
    dash::PrefillArgs a{Q, K, V, in_dtype == DASH_BF16, idx, bias, cnt, list_cap, O, out_dtype == DASH_BF16,
                        b, h_q, h_kv, n, d, B, causal, ws, lse, seq_len};
    a.pages = pages; a.pages_per_seq = pages_per_seq; a.num_pages = num_pages;
    return from_hip(dash::launch_attend_prefill(a, (hipStream_t)stream), "sparse_prior_attn_kernel");
}

dash_status dash_attend_prefill_lse(const void* Q, const void* K, const void* V, int in_dtype,
                                    const int32_t* idx, const float* bias, const int32_t* cnt,
                                    int list_cap, void* O, int out_dtype, float* lse,
                                    int b, int h_q, int h_kv, int n, int d, int B, int causal,
                                    void* ws, size_t ws_bytes, void* stream) {
    return attend_prefill(Q, K, V, in_dtype, idx, bias, cnt, list_cap, O, out_dtype, lse, b, h_q, h_kv, n, d, B,
                          causal, ws, ws_bytes, stream, nullptr);
}

dash_status dash_attend_prefill_paged(const void* Q, const void* Kp, const void* Vp, int in_dtype,
                                      const int32_t* pages, int pages_per_seq, int num_pages,
                                      const int32_t* seq_len, const int32_t* idx, const float* bias,
                                      const int32_t* cnt, int list_cap, void* O, int out_dtype, float* lse,
                                      int b, int h_q, int h_kv, int n, int d, int B, int causal,
                                      void* ws, size_t ws_bytes, void* stream) {
    if (!pages) return fail(DASH_ERR_NULL, "pages must be non-null");
    if (pages_per_seq < 1 || num_pages < 1)
        return fail(DASH_ERR_SHAPE, "pages_per_seq and num_pages must be >= 1");
    if (n > 0 && (long long)pages_per_seq * B < n)
        return fail(DASH_ERR_SHAPE, "pages_per_seq * B = %lld < n = %d", (long long)pages_per_seq * B, n);
    if ((long long)num_pages * h_kv * B > 0x7fffffffLL)
        return fail(DASH_ERR_UNSUPPORTED, "the cache holds more than 2^31 rows");
    return attend_prefill(Q, Kp, Vp, in_dtype, idx, bias, cnt, list_cap, O, out_dtype, lse, b, h_q, h_kv, n, d, B,
                          causal, ws, ws_bytes, stream, seq_len, pages, pages_per_seq, num_pages);
}

dash_status dash_attend_prefill_varlen(const void* Q, const void* K, const void* V, int in_dtype,
                                       const int32_t* seq_len, const int32_t* idx, const float* bias,
                                       const int32_t* cnt, int list_cap, void* O, int out_dtype, float* lse,
                                       int b, int h_q, int h_kv, int n, int d, int B, int causal,
                                       void* ws, size_t ws_bytes, void* stream) {
    if (!seq_len) return fail(DASH_ERR_NULL, "seq_len must be non-null");
    return attend_prefill(Q, K, V, in_dtype, idx, bias, cnt, list_cap, O, out_dtype, lse, b, h_q, h_kv, n, d, B,
                          causal, ws, ws_bytes, stream, seq_len);
}

dash_status dash_attend_prefill(const void* Q, const void* K, const void* V, int in_dtype,
                                const int32_t* idx, const float* bias, const int32_t* cnt,
                                int list_cap, void* O, int out_dtype,
                                int b, int h_q, int h_kv, int n, int d, int B, int causal,
                                void* ws, size_t ws_bytes, void* stream) {
    return dash_attend_prefill_lse(Q, K, V, in_dtype, idx, bias, cnt, list_cap, O, out_dtype, nullptr, b, h_q, h_kv,
                                   n, d, B, causal, ws, ws_bytes, stream);
}

dash_status dash_attend_prefill_backward(const void* Q, const void* K, const void* V, int in_dtype,
                                         const int32_t* idx, const float* bias, const int32_t* cnt, int list_cap,
                                         const void* O, const void* dO, int o_dtype, const float* lse,
                                         float* dQ, float* dK, float* dV, float* dbias,
                                         int b, int h_q, int h_kv, int n, int d, int B, int causal,
                                         void* ws, size_t ws_bytes, void* stream) {
    if (!Q || !K || !V || !idx || !bias || !cnt || !O || !dO || !lse || !dQ || !dK || !dV || !dbias)
        return fail(DASH_ERR_NULL, "every tensor argument of the backward must be non-null");
    if (!valid_dtype(in_dtype) || !valid_dtype(o_dtype)) return fail(DASH_ERR_PARAM, "bad dtype");
    if (causal != 0 && causal != 1) return fail(DASH_ERR_PARAM, "causal must be 0 or 1");
    dash_status st = check_common(b, h_q, h_kv, d, B);
    if (st != DASH_OK) return st;
    if (in_dtype != DASH_BF16) return fail(DASH_ERR_UNSUPPORTED, "the Stage-2 backward takes bf16 Q, K, V");
    if (B % 32 != 0) return fail(DASH_ERR_UNSUPPORTED, "the Stage-2 backward needs B %% 32 == 0 (B = %d)", B);
    if (n < 0) return fail(DASH_ERR_SHAPE, "n must be >= 0");
    const int T = n / B;
    if (list_cap < T) return fail(DASH_ERR_SHAPE, "list_cap %d < floor(n/B) = %d", list_cap, T);
    if (dash::backward_tile_rows(h_q / h_kv, B, T, d) == 0)
        return fail(DASH_ERR_UNSUPPORTED, "no backward query tiling fits LDS (g=%d, B=%d, T_c=%d)", h_q / h_kv, B, T);
    if ((int64_t)n * T >= ((int64_t)1 << 31))
        return fail(DASH_ERR_UNSUPPORTED, "the backward needs n * floor(n/B) < 2^31 (n = %d, B = %d)", n, B);
    if (n > 0) {
        const size_t need = dash::backward_workspace_bytes(b, h_q, h_kv, n, d, B);
        if (!ws || ws_bytes < need)
            return fail(DASH_ERR_WORKSPACE, "the backward needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : (size_t)0);
    }
    dash::PrefillBwdArgs a{Q, K, V, idx, bias, cnt, list_cap, O, dO, o_dtype == DASH_BF16, lse,
                           dQ, dK, dV, dbias, b, h_q, h_kv, n, d, B, causal, ws};
    return from_hip(dash::launch_attend_prefill_backward(a, (hipStream_t)stream), "sparse_prior_attn_bwd_kernel");
}

size_t dash_workspace_bytes(int op, int b, int h_q, int h_kv, int n_or_Lcap, int d, int B) {
    if (b < 1 || h_q < 1 || h_kv < 1 || h_q % h_kv != 0 || n_or_Lcap < 0 || d < 1 || B < 1) return (size_t)-1;
    switch (op) {
        case DASH_OP_ROUTE: return dash::route_workspace_bytes(b, h_kv, n_or_Lcap / B, d);
        case DASH_OP_PREFILL: return dash::prefill_workspace_bytes(b, h_kv, n_or_Lcap, d);
        case DASH_OP_PREFILL_BWD: return dash::backward_workspace_bytes(b, h_q, h_kv, n_or_Lcap, d, B);
        case DASH_OP_DECODE: {
            if (n_or_Lcap < 1) return (size_t)-1;
            return decode_layout(b, h_q, h_kv, n_or_Lcap, 1 << 30, d, B).total;
        }
        default: return (size_t)-1;
    }
}

static dash_status attend_decode(const void* Q, const void* Kc, const void* Vc, int in_dtype,
                                 const float* kbar, const int32_t* seq_len,
                                 int b, int h_q, int h_kv, int L_cap, int kbar_cap, int d, int B,
                                 float alpha, float gamma, float sigma,
                                 void* O, int out_dtype,
                                 int32_t* idx_out, float* bias_out, int32_t* cnt_out,
                                 float* w_out, int list_cap,
                                 void* ws, size_t ws_bytes, void* stream,
                                 const int32_t* pages, int pages_per_seq, int num_pages, int top_k = 0) {
    if (!Q || !Kc || !Vc || !kbar || !seq_len || !O) return fail(DASH_ERR_NULL, "Q, Kc, Vc, kbar, seq_len and O must be non-null");
    if (top_k < 0) return fail(DASH_ERR_PARAM, "top_k must be >= 0 (got %d)", top_k);
    const int given = (idx_out != nullptr) + (bias_out != nullptr) + (cnt_out != nullptr);
    if (given != 0 && given != 3) return fail(DASH_ERR_NULL, "idx_out, bias_out and cnt_out must be all NULL or all non-null");
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return fail(DASH_ERR_PARAM, "bad dtype");
    dash_status st = check_common(b, h_q, h_kv, d, B);
    if (st != DASH_OK) return st;
    if ((st = check_params(alpha, gamma, sigma)) != DASH_OK) return st;
    if (B % 32 != 0) return fail(DASH_ERR_UNSUPPORTED, "decode attention needs B %% 32 == 0 (B = %d)", B);
    if (L_cap < 1 || kbar_cap < 0) return fail(DASH_ERR_SHAPE, "L_cap must be >= 1 and kbar_cap >= 0");
    const DecodeLayout Lo = decode_layout(b, h_q, h_kv, L_cap, kbar_cap, d, B);
    if (Lo.T_ws > 2048) return fail(DASH_ERR_UNSUPPORTED, "%d routable chunks exceed the decode router's 2048", Lo.T_ws);
    if (given == 3 && list_cap < Lo.T_route) return fail(DASH_ERR_SHAPE, "list_cap %d < routable chunks %d", list_cap, Lo.T_route);
    if (!ws || ws_bytes < Lo.total) return fail(DASH_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", Lo.total, ws ? ws_bytes : (size_t)0);
    char* w = static_cast<char*>(ws);
    dash::DecodeArgs a;
    a.Q = Q; a.Kc = Kc; a.Vc = Vc; a.in_bf16 = in_dtype == DASH_BF16; a.kbar = kbar; a.seq_len = seq_len;
    a.b = b; a.h_q = h_q; a.h_kv = h_kv; a.L_cap = L_cap; a.kbar_cap = kbar_cap; a.d = d; a.B = B;
    a.alpha = alpha; a.gamma = gamma; a.sigma = sigma; a.O = O; a.out_bf16 = out_dtype == DASH_BF16;
    if (given == 3) {
        a.idx = idx_out; a.bias = bias_out; a.cnt = cnt_out; a.list_cap = list_cap;
    } else {
        a.idx = reinterpret_cast<int32_t*>(w + Lo.off_idx);
        a.bias = reinterpret_cast<float*>(w + Lo.off_bias);
        a.cnt = reinterpret_cast<int32_t*>(w + Lo.off_cnt);
        a.list_cap = Lo.T_ws > 0 ? Lo.T_ws : 1;
    }
    a.w_out = w_out;
    a.scores = reinterpret_cast<float*>(w + Lo.off_scores);
    a.counters = reinterpret_cast<int32_t*>(w + Lo.off_counters);
    a.part_ml = reinterpret_cast<float*>(w + Lo.off_ml);
    a.part_o = reinterpret_cast<float*>(w + Lo.off_o);
    a.T_route = Lo.T_route;
    a.pages = pages; a.pages_per_seq = pages_per_seq; a.num_pages = num_pages;
    a.top_k = top_k;
    return from_hip(dash::launch_decode(a, (hipStream_t)stream), "decode kernels");
}

dash_status dash_attend_decode(const void* Q, const void* Kc, const void* Vc, int in_dtype,
                               const float* kbar, const int32_t* seq_len,
                               int b, int h_q, int h_kv, int L_cap, int kbar_cap, int d, int B,
                               float alpha, float gamma, float sigma,
                               void* O, int out_dtype,
                               int32_t* idx_out, float* bias_out, int32_t* cnt_out,
                               float* w_out, int list_cap,
                               void* ws, size_t ws_bytes, void* stream) {
    return attend_decode(Q, Kc, Vc, in_dtype, kbar, seq_len, b, h_q, h_kv, L_cap, kbar_cap, d, B, alpha, gamma,
                         sigma, O, out_dtype, idx_out, bias_out, cnt_out, w_out, list_cap, ws, ws_bytes, stream,
                         nullptr, 0, 0);
}

dash_status dash_attend_decode_topk(const void* Q, const void* Kc, const void* Vc, int in_dtype,
                                    const float* kbar, const int32_t* seq_len,
                                    int b, int h_q, int h_kv, int L_cap, int kbar_cap, int d, int B,
                                    float alpha, float gamma, float sigma,
                                    void* O, int out_dtype,
                                    int32_t* idx_out, float* bias_out, int32_t* cnt_out,
                                    float* w_out, int list_cap, int top_k,
                                    void* ws, size_t ws_bytes, void* stream) {
    return attend_decode(Q, Kc, Vc, in_dtype, kbar, seq_len, b, h_q, h_kv, L_cap, kbar_cap, d, B, alpha, gamma,
                         sigma, O, out_dtype, idx_out, bias_out, cnt_out, w_out, list_cap, ws, ws_bytes, stream,
                         nullptr, 0, 0, top_k);
}

dash_status dash_attend_decode_noalloc(const void* Q, const void* Kc, const void* Vc, int in_dtype,
                                       const float* kbar, const int32_t* seq_len,
                                       int b, int h_q, int h_kv, int L_cap, int kbar_cap, int d, int B,
                                       float alpha, float gamma, float sigma,
                                       void* O, int out_dtype,
                                       int32_t* idx_out, float* bias_out, int32_t* cnt_out,
                                       float* w_out, int list_cap, void* stream) {
    if (b >= 1 && h_kv >= 1 && h_q >= h_kv && h_q % h_kv == 0 && L_cap >= 1 && B >= 1 && d >= 1) {
        const size_t need = decode_layout(b, h_q, h_kv, L_cap, kbar_cap < 0 ? 0 : kbar_cap, d, B).total;
        if (need > DASH_NOALLOC_SCRATCH_BYTES)
            return fail(DASH_ERR_WORKSPACE, "decode needs %zu scratch bytes; the no-allocation scratch holds %zu",
                        need, (size_t)DASH_NOALLOC_SCRATCH_BYTES);
    }
    void* ws = nullptr;
    const dash_status st = scratch_of_current_device(&ws);
    if (st != DASH_OK) return st;
    return attend_decode(Q, Kc, Vc, in_dtype, kbar, seq_len, b, h_q, h_kv, L_cap, kbar_cap, d, B, alpha, gamma,
                         sigma, O, out_dtype, idx_out, bias_out, cnt_out, w_out, list_cap, ws,
                         DASH_NOALLOC_SCRATCH_BYTES, stream, nullptr, 0, 0);
}

dash_status dash_attend_decode_paged(const void* Q, const void* Kp, const void* Vp, int in_dtype,
                                     const float* kbar, const int32_t* seq_len,
                                     const int32_t* pages, int pages_per_seq, int num_pages,
                                     int b, int h_q, int h_kv, int kbar_cap, int d, int B,
                                     float alpha, float gamma, float sigma,
                                     void* O, int out_dtype,
                                     int32_t* idx_out, float* bias_out, int32_t* cnt_out,
                                     float* w_out, int list_cap,
                                     void* ws, size_t ws_bytes, void* stream) {
    if (!pages) return fail(DASH_ERR_NULL, "pages must be non-null");
    if (pages_per_seq < 1 || num_pages < 1) return fail(DASH_ERR_SHAPE, "pages_per_seq and num_pages must be >= 1");
    return attend_decode(Q, Kp, Vp, in_dtype, kbar, seq_len, b, h_q, h_kv, pages_per_seq * B, kbar_cap, d, B, alpha,
                         gamma, sigma, O, out_dtype, idx_out, bias_out, cnt_out, w_out, list_cap, ws, ws_bytes,
                         stream, pages, pages_per_seq, num_pages);
}

}  // extern "C"
