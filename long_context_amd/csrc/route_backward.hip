// Backward of Stage 1 and Stage 0 (the support of each row held fixed).
//
// Stage 1 (paper review section 三: Eq. 6 routing, the GQA average and the bias of
// Proposition 4.1). For one row of one KV group with routed list S and the gradient
// db of its bias entries:
//   g_c  = (db_c - mean over S of db) / σ            (the bias is (log w - μ)/σ)
//   ∂ŵ_c = g_c / (g w_c)                             (w = (1/g) Σ_h ŵ_h, all heads)
//   for every head h: s_c = ŵ_hc^(2-α) on the head's support (α = 1: s = ŵ),
//   ∂x_hc = s_c (∂ŵ_c - Σ s ∂ŵ / Σ s)                (the α-entmax Jacobian)
//   dz_hc = γ ∂x_hc / sqrt(d)                        (x = γ <q_h, k̄_c>/sqrt(d))
//   dq_h += Σ_c dz_hc k̄_c,   dk̄_c += Σ_h dz_hc q_h.
// The head's weights are rebuilt on S from the forward's statistics: ŵ = [y - τ]_+^p
// (α = 1: 2^(y - lse)) with y = cs (<q_h, k̄_c> - max logit) exactly as the router
// forms it. A chunk of S outside a head's support has ŵ = 0 and takes no gradient,
// and the support of every head lies inside S, so the list carries the whole
// Jacobian.
//
// Stage 0 (Eq. 4): k̄_c = Σ_j π_j k_j with π = softmax_j(<q̄, k_j>/sqrt(d)):
//   ∂a_j = π_j (<dk̄_c, k_j> - Σ_l π_l <dk̄_c, k_l>),
//   dk_j += π_j dk̄_c + ∂a_j q̄/sqrt(d),   dq̄ += Σ_j ∂a_j k_j/sqrt(d).
#include "kernels.h"
#include "common.h"

#include <math.h>

namespace dash {

struct RouteBwdParams {
    const void* Q; const float* kbar; const int32_t* idx; const int32_t* cnt; const float* dbias;
    const float* stats;
    float* dQ; float* dkbar;
    int h_q, h_kv, n, kbar_cap, list_cap, g, soft, T;
    float cs;           // scale of y: (α-1)γ/sqrt(d), or γ log2(e)/sqrt(d) when soft
    float pexp;         // 1/(α-1)
    float two_m_alpha;  // 2 - α
    float inv_sigma, dz_scale;   // 1/σ and γ/sqrt(d)
};

// max_g heads per group; entries handled 64 at a time (one per lane).
constexpr int kMaxG = 16;

template <typename T>
__device__ __forceinline__ float load_f(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_f<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_f<uint16_t>(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }

// One wavefront per (b, KV head, row); 4 wavefronts per workgroup. LDS per
// wavefront: the group's query rows [g][D] fp32 and dz [g][64].
template <typename T, int D>
__global__ __launch_bounds__(256) void route_backward_kernel(RouteBwdParams p, int rows_total) {
    __shared__ float qs[4][kMaxG][D];
    __shared__ float dzs[4][kMaxG][64];
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + wid;
    if (item >= rows_total) return;                  // wavefront-uniform; no barrier below
    const int row = item % p.n;
    const size_t bh = (size_t)(item / p.n);          // b * h_kv + r
    const int bi = (int)(bh / p.h_kv), r = (int)(bh % p.h_kv);
    const int g = p.g;
    const size_t rb = bh * p.n + row;
    const int cn = min(p.cnt[rb], p.list_cap);
    if (cn <= 0) return;
    const int32_t* li = p.idx + rb * p.list_cap;
    const float* ldb = p.dbias + rb * p.list_cap;
    const T* Q = static_cast<const T*>(p.Q);
    const float* kb = p.kbar + bh * (size_t)p.kbar_cap * D;

    // the group's query rows into LDS (fp32) and the heads' statistics
    for (int x = lane; x < g * D; x += 64) {
        const int h = x / D, dd = x % D;
        qs[wid][h][dd] = load_f<T>(Q, (((size_t)bi * p.h_q + r * g + h) * p.n + row) * D + dd);
    }
    float smax[kMaxG], thr[kMaxG];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
        if (h < g) {
            const float* st = p.stats + 2 * (((size_t)bi * p.h_q + r * g + h) * p.n + row);
            smax[h] = st[0];
            thr[h] = st[1];
        }
    }
    __builtin_amdgcn_wave_barrier();

    // mean of the bias gradient over the list
    float dsum = 0.f;
    for (int e = lane; e < cn; e += 64) dsum += ldb[e];
    const float dmean = wave_sum(dsum) / (float)cn;

    // per head: Σ_c s ∂ŵ and Σ_c s over the list (first pass)
    float A[kMaxG], Bs[kMaxG];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) { A[h] = 0.f; Bs[h] = 0.f; }
    auto weights = [&](int e, float (&wh)[kMaxG], float& dwhat) {
        const int c = li[e];
        if ((unsigned)c >= (unsigned)p.T) {          // not a chunk: no weight, no gradient
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) wh[h] = 0.f;
            dwhat = 0.f;
            return;
        }
        const float* kr = kb + (size_t)c * D;
        float z[kMaxG];
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) z[h] = 0.f;
        for (int d0 = 0; d0 < D; d0 += 4) {
            const f32x4 kv = *reinterpret_cast<const f32x4*>(kr + d0);
#pragma unroll
            for (int h = 0; h < kMaxG; ++h)
                if (h < g)
                    z[h] = fmaf(kv[0], qs[wid][h][d0], fmaf(kv[1], qs[wid][h][d0 + 1],
                           fmaf(kv[2], qs[wid][h][d0 + 2], fmaf(kv[3], qs[wid][h][d0 + 3], z[h]))));
        }
        float wsum = 0.f;
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
            if (h < g) {
                const float y = p.cs * (z[h] - smax[h]);
                float v;
                if (p.soft) v = exp2f(y - thr[h]);
                else {
                    const float t = fmaxf(y - thr[h], 0.f);
                    v = t > 0.f ? powf(t, p.pexp) : 0.f;
                }
                wh[h] = v;
                wsum += v;
            } else {
                wh[h] = 0.f;
            }
        }
        // ∂L/∂ŵ, the same for every head: g_c / (g w_c) = g_c / Σ_h ŵ_hc
        const float gc = (ldb[e] - dmean) * p.inv_sigma;
        dwhat = wsum > 0.f ? gc / wsum : 0.f;
    };
    auto s_of = [&](float v) {
        return v > 0.f ? (p.soft ? v : powf(v, p.two_m_alpha)) : 0.f;
    };
    for (int e0 = 0; e0 < cn; e0 += 64) {
        const int e = e0 + lane;
        float wh[kMaxG], dwh = 0.f;
        if (e < cn) weights(e, wh, dwh);
        else {
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) wh[h] = 0.f;
        }
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
            const float s = s_of(wh[h]);
            A[h] += s * dwh;
            Bs[h] += s;
        }
    }
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
        if (h < g) {
            A[h] = wave_sum(A[h]);
            Bs[h] = wave_sum(Bs[h]);
        }
    }

    // second pass: dz per (head, entry), then dq (lanes over d) and dk̄ (atomics)
    float dq[kMaxG][D / 64];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h)
#pragma unroll
        for (int u = 0; u < D / 64; ++u) dq[h][u] = 0.f;
    for (int e0 = 0; e0 < cn; e0 += 64) {
        const int e = e0 + lane;
        float wh[kMaxG], dwh = 0.f;
        if (e < cn) weights(e, wh, dwh);
        else {
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) wh[h] = 0.f;
        }
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
            if (h < g) {
                const float s = s_of(wh[h]);
                const float dx = Bs[h] > 0.f ? s * (dwh - A[h] / Bs[h]) : 0.f;
                dzs[wid][h][lane] = e < cn ? dx * p.dz_scale : 0.f;
            }
        }
        __builtin_amdgcn_wave_barrier();
        const int ne = min(64, cn - e0);
        for (int k = 0; k < ne; ++k) {
            const int c = li[e0 + k];
            if ((unsigned)c >= (unsigned)p.T) continue;   // wavefront-uniform
            const float* kr = kb + (size_t)c * D;
            float gk[D / 64];
#pragma unroll
            for (int u = 0; u < D / 64; ++u) gk[u] = 0.f;
#pragma unroll
            for (int u = 0; u < D / 64; ++u) {
                const int dd = lane + 64 * u;
                const float kv = kr[dd];
#pragma unroll
                for (int h = 0; h < kMaxG; ++h) {
                    if (h < g) {
                        const float dz = dzs[wid][h][k];
                        dq[h][u] = fmaf(dz, kv, dq[h][u]);
                        gk[u] = fmaf(dz, qs[wid][h][dd], gk[u]);
                    }
                }
            }
            float* dkr = p.dkbar + (bh * (size_t)p.kbar_cap + c) * D;
#pragma unroll
            for (int u = 0; u < D / 64; ++u) unsafeAtomicAdd(dkr + lane + 64 * u, gk[u]);
        }
        __builtin_amdgcn_wave_barrier();
    }
    // dQ: each (head, row) belongs to this wavefront alone
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
        if (h < g) {
            float* out = p.dQ + (((size_t)bi * p.h_q + r * g + h) * p.n + row) * D;
#pragma unroll
            for (int u = 0; u < D / 64; ++u) out[lane + 64 * u] += dq[h][u];
        }
    }
}

struct SumBwdParams {
    const void* K; const float* qbar; const float* dkbar;
    float* dK; float* dqbar;
    int h_kv, n, kbar_cap, B, T;
    float inv_sqrt_d;
};

// One wavefront per (b, KV head, chunk); lanes over d (D/64 columns each).
template <typename T, int D>
__global__ __launch_bounds__(64) void summary_backward_kernel(SumBwdParams p) {
    extern __shared__ float sb[];                    // a[B], dp[B]
    float* as = sb;
    float* dps = sb + p.B;
    const int lane = threadIdx.x;
    const int c = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int r = (int)(bh % p.h_kv);
    const T* K = static_cast<const T*>(p.K) + (bh * p.n + (size_t)c * p.B) * D;
    constexpr int U = D / 64;
    float qb[U], dk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        qb[u] = p.qbar[(size_t)r * D + lane + 64 * u];
        dk[u] = p.dkbar[(bh * p.kbar_cap + c) * D + lane + 64 * u];
    }
    // logits and <dk̄, k_j> per token
    float amax = -INFINITY;
    for (int j = 0; j < p.B; ++j) {
        float a = 0.f, dp = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float kv = load_f<T>(K, (size_t)j * D + lane + 64 * u);
            a = fmaf(qb[u], kv, a);
            dp = fmaf(dk[u], kv, dp);
        }
        a = wave_sum(a) * p.inv_sqrt_d;
        dp = wave_sum(dp);
        if (lane == 0) { as[j] = a; dps[j] = dp; }
        amax = fmaxf(amax, a);
    }
    __builtin_amdgcn_wave_barrier();
    float esum = 0.f, edp = 0.f;
    for (int j = 0; j < p.B; ++j) {
        const float e = expf(as[j] - amax);
        esum += e;
        edp += e * dps[j];
    }
    const float inv = 1.f / esum;
    const float mdp = edp * inv;                     // Σ_l π_l <dk̄, k_l>
    float dqb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) dqb[u] = 0.f;
    float* dK = p.dK + (bh * p.n + (size_t)c * p.B) * D;
    for (int j = 0; j < p.B; ++j) {
        const float pi = expf(as[j] - amax) * inv;
        const float da = pi * (dps[j] - mdp);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t o = (size_t)j * D + lane + 64 * u;
            const float kv = load_f<T>(K, o);
            dK[o] += pi * dk[u] + da * qb[u] * p.inv_sqrt_d;
            dqb[u] = fmaf(da, kv, dqb[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) unsafeAtomicAdd(p.dqbar + (size_t)r * D + lane + 64 * u, dqb[u] * p.inv_sqrt_d);
}

hipError_t launch_route_backward(const RouteBwdArgs& a, hipStream_t s) {
    if (a.n == 0 || isinf(a.sigma)) return hipSuccess;
    RouteBwdParams p;
    p.Q = a.Q; p.kbar = a.kbar; p.idx = a.idx; p.cnt = a.cnt; p.dbias = a.dbias; p.stats = a.stats;
    p.dQ = a.dQ; p.dkbar = a.dkbar;
    p.h_q = a.h_q; p.h_kv = a.h_kv; p.n = a.n; p.kbar_cap = a.kbar_cap; p.list_cap = a.list_cap;
    p.g = a.h_q / a.h_kv;
    p.T = a.n / a.B;
    p.soft = a.alpha == 1.0f;
    p.cs = route_scale(a.alpha, a.gamma, a.d);
    p.pexp = p.soft ? 1.f : 1.f / (a.alpha - 1.f);
    p.two_m_alpha = 2.f - a.alpha;
    p.inv_sigma = 1.f / a.sigma;
    p.dz_scale = (float)(a.gamma / sqrt((double)a.d));
    const int rows = a.b * a.h_kv * a.n;
    const dim3 grid((rows + 3) / 4);
    if (a.q_bf16) {
        if (a.d == 64) hipLaunchKernelGGL((route_backward_kernel<uint16_t, 64>), grid, dim3(256), 0, s, p, rows);
        else hipLaunchKernelGGL((route_backward_kernel<uint16_t, 128>), grid, dim3(256), 0, s, p, rows);
    } else {
        if (a.d == 64) hipLaunchKernelGGL((route_backward_kernel<float, 64>), grid, dim3(256), 0, s, p, rows);
        else hipLaunchKernelGGL((route_backward_kernel<float, 128>), grid, dim3(256), 0, s, p, rows);
    }
    return hipGetLastError();
}

hipError_t launch_summary_backward(const SumBwdArgs& a, hipStream_t s) {
    const int T = a.n / a.B;
    if (T == 0) return hipSuccess;
    SumBwdParams p;
    p.K = a.K; p.qbar = a.qbar; p.dkbar = a.dkbar; p.dK = a.dK; p.dqbar = a.dqbar;
    p.h_kv = a.h_kv; p.n = a.n; p.kbar_cap = a.kbar_cap; p.B = a.B; p.T = T;
    p.inv_sqrt_d = (float)(1.0 / sqrt((double)a.d));
    const dim3 grid(T, a.b * a.h_kv);
    const size_t lds = (size_t)2 * a.B * sizeof(float);
    if (a.k_bf16) {
        if (a.d == 64) hipLaunchKernelGGL((summary_backward_kernel<uint16_t, 64>), grid, dim3(64), lds, s, p);
        else hipLaunchKernelGGL((summary_backward_kernel<uint16_t, 128>), grid, dim3(64), lds, s, p);
    } else {
        if (a.d == 64) hipLaunchKernelGGL((summary_backward_kernel<float, 64>), grid, dim3(64), lds, s, p);
        else hipLaunchKernelGGL((summary_backward_kernel<float, 128>), grid, dim3(64), lds, s, p);
    }
    return hipGetLastError();
}

}  // namespace dash
