// Dispatch of the prefill routing kernel (the kernel itself is in route_impl.h and
// is instantiated per query dtype and head dimension in route_*.hip).
#include "route_impl.h"

namespace dash {

int route_tiles_bucket(int T) {
    if (T <= 32) return 2;
    if (T <= 128) return 8;
    if (T <= 512) return 32;
    if (T <= 1024) return 64;        // 32 tiles x 2 wavefronts per row group
    if (T <= 2048) return 128;       // 32 tiles x 4 wavefronts per row group
    return 0;
}

float route_scale(float alpha, float gamma, int d) {
    if (alpha == 1.0f) return (float)(1.4426950408889634 * (double)gamma / sqrt((double)d));
    return (float)(((double)alpha - 1.0) * (double)gamma / sqrt((double)d));
}

size_t route_workspace_bytes(int b, int h_kv, int T_c, int d) {
    const size_t T_pad = (size_t)(T_c + 31) / 32 * 32;
    return (size_t)b * h_kv * T_pad * 3 * d * sizeof(uint16_t);
}

template <typename T, int D>
static size_t route_lds_d(int R, int B, int T_c) {
    size_t lds = 0;
    switch (route_tiles_bucket(T_c)) {
        case 2: route_groups_per_block<T, D, 2, 1>(R, B, &lds); break;
        case 8: route_groups_per_block<T, D, 8, 1>(R, B, &lds); break;
        case 32: route_groups_per_block<T, D, 32, 1>(R, B, &lds); break;
        case 64: route_groups_per_block<T, D, 32, 2>(R, B, &lds); break;
        default: route_groups_per_block<T, D, 32, 4>(R, B, &lds); break;
    }
    return lds;
}

size_t route_lds_bytes(int g, int B, int T_c, int d, bool q_bf16) {
    const int R = 16 / g;
    if (q_bf16) return d == 64 ? route_lds_d<uint16_t, 64>(R, B, T_c) : route_lds_d<uint16_t, 128>(R, B, T_c);
    return d == 64 ? route_lds_d<float, 64>(R, B, T_c) : route_lds_d<float, 128>(R, B, T_c);
}

template <int D>
static hipError_t launch_ksplit(const RouteParams& p, int b, hipStream_t s) {
    const int pieces = p.T_pad * (D / 8);
    hipLaunchKernelGGL((ksplit_kernel<D>), dim3((pieces + 255) / 256, p.h_kv, b), dim3(256), 0, s,
                       p.kbar, const_cast<uint8_t*>(p.ksplit), p.kbar_cap, p.T_c, p.T_pad);
    return hipGetLastError();
}

hipError_t launch_kbar_split(const float* kbar, void* ws, int b, int h_kv, int kbar_cap, int T_c, int d,
                             hipStream_t s) {
    if (T_c <= 0) return hipSuccess;
    RouteParams p;
    p.kbar = kbar;
    p.ksplit = static_cast<const uint8_t*>(ws);
    p.h_kv = h_kv; p.kbar_cap = kbar_cap; p.T_c = T_c;
    p.T_pad = (T_c + 31) / 32 * 32;
    return d == 64 ? launch_ksplit<64>(p, b, s) : launch_ksplit<128>(p, b, s);
}

int pmode_of(float alpha) {
    if (alpha == 1.0f) return kSoftmaxRouting;
    const double pe = 1.0 / ((double)alpha - 1.0);
    if (pe == 1.0) return 1;
    if (pe == 2.0) return 2;
    if (pe == 4.0) return 4;
    return 0;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
    RouteParams p;
    p.Q = a.Q; p.kbar = a.kbar; p.idx = a.idx; p.bias = a.bias; p.cnt = a.cnt; p.w_out = a.w_out;
    p.h_q = a.h_q; p.h_kv = a.h_kv; p.n = a.n; p.kbar_cap = a.kbar_cap; p.list_cap = a.list_cap;
    p.B = a.B; p.T_c = a.n / a.B; p.g = a.h_q / a.h_kv;
    p.seq_len = a.seq_len;
    p.log2g = 0;
    while ((1 << p.log2g) < p.g) ++p.log2g;
    p.causal = a.causal;
    p.cs = route_scale(a.alpha, a.gamma, a.d);
    p.pexp = (float)(1.0 / ((double)a.alpha - 1.0));
    p.pmode = pmode_of(a.alpha);
    p.inv_sigma = isinf(a.sigma) ? 0.f : (float)(1.0 / (double)a.sigma);
    p.ksplit = static_cast<const uint8_t*>(a.ws);
    p.top_k = a.top_k;
    p.stats = a.stats;
    p.T_pad = (p.T_c + 31) / 32 * 32;
    if (a.n == 0) return hipSuccess;
    if (a.q_bf16) {
        if (p.T_c > 0) {
            const hipError_t e = a.d == 64 ? launch_ksplit<64>(p, a.b, s) : launch_ksplit<128>(p, a.b, s);
            if (e != hipSuccess) return e;
        }
        return a.d == 64 ? launch_route_bf16_64(p, a.b, s) : launch_route_bf16_128(p, a.b, s);
    }
    return a.d == 64 ? launch_route_f32_64(p, a.b, s) : launch_route_f32_128(p, a.b, s);
}

}  // namespace dash
