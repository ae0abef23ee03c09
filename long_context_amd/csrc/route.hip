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

int pmode_of(float alpha) {
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
    p.log2g = 0;
    while ((1 << p.log2g) < p.g) ++p.log2g;
    p.causal = a.causal;
    p.cs = (float)(((double)a.alpha - 1.0) * (double)a.gamma / sqrt((double)a.d));
    p.pexp = (float)(1.0 / ((double)a.alpha - 1.0));
    p.pmode = pmode_of(a.alpha);
    p.inv_sigma = isinf(a.sigma) ? 0.f : (float)(1.0 / (double)a.sigma);
    if (a.n == 0) return hipSuccess;
    if (a.q_bf16) return a.d == 64 ? launch_route_bf16_64(p, a.b, s) : launch_route_bf16_128(p, a.b, s);
    return a.d == 64 ? launch_route_f32_64(p, a.b, s) : launch_route_f32_128(p, a.b, s);
}

}  // namespace dash
