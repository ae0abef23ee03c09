// Stage 1 of DashAttention for a prefill (paper review section 三, Eq. 6 and the
// GQA paragraph; μ and d from Proposition 4.1):
//   z̄_{i,c} = <q_i^(h), k̄_c^(r)>/sqrt(d) over the visible chunks c < floor(i/B),
//   ŵ^(h) = α-entmax(γ z̄^(h)) = [(α-1)γz̄ - τ]_+^{1/(α-1)},
//   w^(r) = mean over the g heads of group r of ŵ^(h), S = {c : w_c > 0},
//   μ = mean_{c in S} ln w_c, bias d_c = (ln w_c - μ)/σ.
//
// entmax_route_kernel: one wavefront handles 16 (row, head) pairs = 16/g rows x all
// g heads of one KV group, so the GQA average is a reduction across lanes.
//  * Logits: fp32 MFMA 16x16x4 with A = k̄ tile (16 chunks x d) and B = q (d x 16
//    pairs); lane (kg, n) ends with chunks 16t+4kg+i of pair n, all visible chunks of
//    a row stay in registers (the row is short: T_c = floor(n/B)).
//  * Threshold: work on y = (α-1)γ(z̄ - max z̄) <= 0 (exact shift by the row maximum)
//    so τ lies in [-1, 0). Newton's method on g(τ) = ||[y - τ]_+||_p - 1 with
//    p = 1/(α-1), started at τ = -1 where g >= 0: g is convex and decreasing, so the
//    iterates increase monotonically to the root; uniform rows converge in one step.
//    Exponents p in {1, 2, 4} (α in {2, 1.5, 1.25}) use plain products, other α
//    use exp2/log2.
//  * GQA average with DPP row permutations (within 16-lane rows), then the group
//    weights go to LDS and each row is compacted with a ballot/prefix count into an
//    ascending chunk list with its bias.
#pragma once

#include "common.h"
#include "kernels.h"

#include <math.h>

namespace dash {

struct RouteParams {
    const void* Q; const float* kbar;
    int32_t* idx; float* bias; int32_t* cnt; float* w_out;
    int h_q, h_kv, n, kbar_cap, list_cap, B, T_c, g, log2g, causal;
    float cs;           // (α-1) γ / sqrt(d)
    float pexp;         // 1/(α-1)
    int pmode;          // 1, 2, 4 for integer exponents, 0 otherwise
    float inv_sigma;    // 1/σ (0 for σ = inf)
};

// Sum over the lanes of a 16-lane row whose index differs only in the low `steps` bits.
__device__ __forceinline__ float row_group_sum(float v, int steps) {
    if (steps > 0) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)); // xor 1
    if (steps > 1) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)); // xor 2
    if (steps > 2) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)); // half-row mirror
    if (steps > 3) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)); // row mirror
    return v;
}

// Exponent-specific accumulation for one Newton step: a0 = sum t^{p-1}, a1 = sum t^p.
template <int PM>
__device__ __forceinline__ void accum_pow(float t, float pexp, float& a0, float& a1) {
    if (PM == 1) { a0 += (t > 0.f) ? 1.f : 0.f; a1 += t; }
    else if (PM == 2) { a0 += t; a1 = fmaf(t, t, a1); }
    else if (PM == 4) { float t2 = t * t; a0 = fmaf(t2, t, a0); a1 = fmaf(t2, t2, a1); }
    else {
        if (t > 0.f) {
            float lt = fast_log2(t);
            a0 += fast_exp2((pexp - 1.f) * lt);
            a1 += fast_exp2(pexp * lt);
        }
    }
}
template <int PM>
__device__ __forceinline__ float pow_p(float t, float pexp) {
    if (PM == 1) return t;
    if (PM == 2) return t * t;
    if (PM == 4) { float t2 = t * t; return t2 * t2; }
    return t > 0.f ? fast_exp2(pexp * fast_log2(t)) : 0.f;
}

// Newton iterations on the wave's 16 pairs; sv holds y (-inf on invalid chunks).
template <int NT, int PM>
__device__ __forceinline__ float solve_tau(float (&sv)[NT][4], int nt, float pexp, bool active) {
    float tau = -1.f;
    bool done = !active;
    for (int it = 0; it < 100; ++it) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < nt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) accum_pow<PM>(fmaxf(sv[t][i] - tau, 0.f), pexp, a0, a1);
            }
        }
        a0 += shfl_xor(a0, 16); a1 += shfl_xor(a1, 16);
        a0 += shfl_xor(a0, 32); a1 += shfl_xor(a1, 32);
        float delta;
        if (PM == 1) {
            delta = (a1 - 1.f) / a0;               // f = sum t - 1, f' = -|{t > 0}|
        } else {
            float nrm = (PM == 2) ? sqrtf(a1) : (PM == 4) ? sqrtf(sqrtf(a1)) : fast_exp2(fast_log2(a1) / pexp);
            delta = (nrm - 1.f) * (a1 / nrm) / a0;  // g/|g'| with g = ||t||_p - 1
        }
        if (!(a0 > 0.f)) delta = 0.f;
        if (!done) tau += delta;
        done = done || !(fabsf(delta) > 1e-6f);
        if (ballot(!done) == 0) break;
    }
    return tau;
}

// Load 4 consecutive elements of a row as fp32.
__device__ __forceinline__ void load4(const float* p, float* o) {
    f32x4 v = *reinterpret_cast<const f32x4*>(p);
    o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
}
__device__ __forceinline__ void load4(const uint16_t* p, float* o) {
    u32x2 v = *reinterpret_cast<const u32x2*>(p);
    o[0] = __uint_as_float(v[0] << 16); o[1] = __uint_as_float(v[0] & 0xFFFF0000u);
    o[2] = __uint_as_float(v[1] << 16); o[3] = __uint_as_float(v[1] & 0xFFFF0000u);
}

template <typename T, int D, int NT, int PM>
__global__ __launch_bounds__(256) void entmax_route_kernel(RouteParams p) {
    constexpr int WS = NT * 16;                       // LDS floats per row of weights
    extern __shared__ float wl_all[];
    const int wid = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n16 = lane & 15, kg = lane >> 4;
    const int g = p.g, lg = p.log2g;
    const int R = 16 >> lg;                           // rows per wave
    const int r = blockIdx.y, bi = blockIdx.z;
    const int row0 = (blockIdx.x * (blockDim.x >> 6) + wid) * R;
    if (row0 >= p.n) return;                          // wave-uniform
    float* wl = wl_all + wid * R * WS;
    const int nvis = p.causal ? min(row0 / p.B, p.T_c) : p.T_c;
    const int my_row = row0 + (n16 >> lg);
    const int my_head = r * g + (n16 & (g - 1));
    const bool row_ok = my_row < p.n;
    const int nt = (nvis + 15) >> 4;

    float sv[NT][4];
    if (nvis > 0) {
        // q fragment: the MFMA k-slot kg of step (s, j) carries dimension 16s + 4kg + j,
        // for both operands, so every dimension is summed exactly once.
        float qv[D / 4];
        {
            const T* qrow = static_cast<const T*>(p.Q) +
                (((size_t)bi * p.h_q + my_head) * p.n + (row_ok ? my_row : 0)) * D + 4 * kg;
#pragma unroll
            for (int s = 0; s < D / 16; ++s) load4(qrow + 16 * s, &qv[4 * s]);
            if (!row_ok) {
#pragma unroll
                for (int e = 0; e < D / 4; ++e) qv[e] = 0.f;
            }
        }
        const float* kb = p.kbar + ((size_t)bi * p.h_kv + r) * (size_t)p.kbar_cap * D + 4 * kg;
        float smax = -INFINITY;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < nt) {
                const int c = min(t * 16 + n16, nvis - 1);   // A row = chunk
                const float* krow = kb + (size_t)c * D;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < D / 16; ++s) {
                    float a[4];
                    load4(krow + 16 * s, a);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], qv[4 * s + j], acc, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ch = t * 16 + 4 * kg + i;
                    sv[t][i] = (ch < nvis) ? acc[i] : -INFINITY;
                    smax = fmaxf(smax, sv[t][i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[t][i] = -INFINITY;
            }
        }
        smax = fmaxf(smax, shfl_xor(smax, 16));
        smax = fmaxf(smax, shfl_xor(smax, 32));
        // thresholded argument shifted by the row maximum: y = (α-1)γ(z̄ - max z̄) <= 0
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[t][i] = p.cs * (sv[t][i] - smax);

        const float tau = solve_tau<NT, PM>(sv, nt, p.pexp, row_ok);
        // per-head weights, then the group average across the g lanes of each row
        const float inv_g = 1.f / (float)g;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float wv = (t < nt && row_ok) ? pow_p<PM>(fmaxf(sv[t][i] - tau, 0.f), p.pexp) : 0.f;
                sv[t][i] = row_group_sum(wv, lg) * inv_g;
            }
    } else {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[t][i] = 0.f;
    }
    // group weights to LDS: the first lane of each row writes its chunks
    if ((n16 & (g - 1)) == 0) {
        float* wr = wl + (n16 >> lg) * WS;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) wr[t * 16 + 4 * kg + i] = sv[t][i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // compaction: ascending chunk ids of the support, with d = (ln w - μ)/σ
    const size_t rowbase = ((size_t)bi * p.h_kv + r) * p.n;
    for (int j = 0; j < R; ++j) {
        const int row = row0 + j;
        if (row >= p.n) break;
        const float* wr = wl + j * WS;
        float sl = 0.f, sc = 0.f;
        for (int c = lane; c < nvis; c += 64) {
            const float v = wr[c];
            if (v > 0.f) { sl += fast_log2(v); sc += 1.f; }
        }
        sl = wave_sum(sl);
        sc = wave_sum(sc);
        const float mu2 = sc > 0.f ? sl / sc : 0.f;            // μ in log2 units
        const float bscale = kLn2 * p.inv_sigma;
        int32_t* idx = p.idx + (rowbase + row) * (size_t)p.list_cap;
        float* bias = p.bias + (rowbase + row) * (size_t)p.list_cap;
        float* wo = p.w_out ? p.w_out + (rowbase + row) * (size_t)p.kbar_cap : nullptr;
        int base = 0;
        for (int c0 = 0; c0 < p.T_c; c0 += 64) {
            const int c = c0 + lane;
            const float v = (c < nvis) ? wr[c] : 0.f;
            const bool in = v > 0.f;
            const uint64_t m = ballot(in);
            const int pre = __builtin_popcountll(m & ((1ull << lane) - 1ull));
            if (in) {
                idx[base + pre] = c;
                bias[base + pre] = p.inv_sigma == 0.f ? 0.f : bscale * (fast_log2(v) - mu2);
            }
            if (wo && c < p.T_c) wo[c] = v;
            base += __builtin_popcountll(m);
        }
        if (lane == 0) p.cnt[rowbase + row] = base;
    }
}

// Waves per workgroup: 4, fewer when a wave's LDS rows would exceed 64 KiB in total.
inline int route_waves_per_block(int R, int NT) {
    const int per_wave = R * NT * 16 * 4;
    int w = 65536 / per_wave;
    return w >= 4 ? 4 : (w < 1 ? 1 : w);
}

template <typename T, int D, int NT>
static hipError_t launch_route_nt(const RouteParams& p, int b, hipStream_t s) {
    const int R = 16 / p.g;
    const int W = route_waves_per_block(R, NT);
    const int waves = (p.n + R - 1) / R;
    dim3 grid((waves + W - 1) / W, p.h_kv, b), block(64 * W);
    const size_t lds = (size_t)W * R * NT * 16 * sizeof(float);
    switch (p.pmode) {
        case 1: hipLaunchKernelGGL((entmax_route_kernel<T, D, NT, 1>), grid, block, lds, s, p); break;
        case 2: hipLaunchKernelGGL((entmax_route_kernel<T, D, NT, 2>), grid, block, lds, s, p); break;
        case 4: hipLaunchKernelGGL((entmax_route_kernel<T, D, NT, 4>), grid, block, lds, s, p); break;
        default: hipLaunchKernelGGL((entmax_route_kernel<T, D, NT, 0>), grid, block, lds, s, p); break;
    }
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_route_d(const RouteParams& p, int b, hipStream_t s) {
    switch (route_tiles_bucket(p.T_c)) {
        case 2: return launch_route_nt<T, D, 2>(p, b, s);
        case 8: return launch_route_nt<T, D, 8>(p, b, s);
        case 32: return launch_route_nt<T, D, 32>(p, b, s);
        default: return launch_route_nt<T, D, 64>(p, b, s);
    }
}

hipError_t launch_route_f32_64(const RouteParams& p, int b, hipStream_t s);
hipError_t launch_route_f32_128(const RouteParams& p, int b, hipStream_t s);
hipError_t launch_route_bf16_64(const RouteParams& p, int b, hipStream_t s);
hipError_t launch_route_bf16_128(const RouteParams& p, int b, hipStream_t s);

}  // namespace dash
