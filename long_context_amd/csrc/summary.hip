// Stage 0 of DashAttention (paper review section 三, Eq. 4): the summary of chunk c
// is local attention of the learned query q̄ over the chunk's keys, with the keys
// also used as the values:  k̄_c = sum_t softmax_t(<q̄, k_t>/sqrt(d)) k_t.
//
// chunk_summary_kernel: one wavefront per (b, r, c). Each lane reads 16 bytes of a
// key row per iteration (a wave reads 1 KiB contiguous), the row's dot product
// with q̄ is reduced across the lanes that share the row, and an online softmax
// (log2 domain, fp32) accumulates the weighted keys. The row groups are merged at
// the end and the fp32 summary is written once. HBM-bound: the K chunk is read
// exactly once.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace dash {

template <typename T> struct Vec16;
template <> struct Vec16<float> {
    static constexpr int N = 4;
    __device__ __forceinline__ static void load(const float* p, float* o) {
        f32x4 v = *reinterpret_cast<const f32x4*>(p);
        o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
    }
};
template <> struct Vec16<uint16_t> {
    static constexpr int N = 8;
    __device__ __forceinline__ static void load(const uint16_t* p, float* o) {
        u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(v[i] << 16);
            o[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
        }
    }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void chunk_summary_kernel(
    const T* __restrict__ K, const float* __restrict__ qbar, float* __restrict__ kbar,
    int h_kv, int n_kv, int kbar_cap, int B, int chunk_begin, int nsel, int total,
    float scale, const int32_t* __restrict__ pages, int pages_per_seq, int num_pages) {
    constexpr int VEC = Vec16<T>::N;
    constexpr int LPR = D / VEC;        // lanes sharing one key row
    constexpr int RPI = 64 / LPR;       // key rows per wave iteration
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wave >= total) return;
    const int lane = threadIdx.x & 63;
    const int c = chunk_begin + wave % nsel;
    const int br = wave / nsel;         // b * h_kv + r
    const int r = br % h_kv;
    const int rr = lane / LPR;
    const int col = (lane % LPR) * VEC;

    float q[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) q[v] = qbar[r * D + col + v];
    // contiguous: rows of (b, r) from c*B; paged: the chunk's page (out-of-range page
    // ids are clamped, so a bad table gives wrong summaries, never a stray read)
    const T* Kc;
    if (pages) {
        const int pg = min(max(pages[(size_t)(br / h_kv) * pages_per_seq + c], 0), num_pages - 1);
        Kc = K + (((size_t)pg * h_kv + r) * B) * D + col;
    } else {
        Kc = K + ((size_t)br * n_kv + (size_t)c * B) * D + col;
    }

    float m = -INFINITY, l = 0.f, acc[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.f;

    for (int t0 = 0; t0 < B; t0 += RPI) {
        float k[VEC];
        Vec16<T>::load(Kc + (size_t)(t0 + rr) * D, k);
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < VEC; ++v) s = fmaf(q[v], k[v], s);
#pragma unroll
        for (int o = LPR / 2; o >= 1; o >>= 1) s += shfl_xor(s, o);
        s *= scale;
        const float mn = fmaxf(m, s);
        const float corr = fast_exp2(m - mn);
        const float p = fast_exp2(s - mn);
        l = fmaf(l, corr, p);
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = fmaf(acc[v], corr, p * k[v]);
        m = mn;
    }
    // merge the RPI row groups of the wave
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
        const float mo = shfl_xor(m, o);
        const float lo = shfl_xor(l, o);
        const float mn = fmaxf(m, mo);
        const float a = fast_exp2(m - mn), bsc = fast_exp2(mo - mn);
        l = l * a + lo * bsc;
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = acc[v] * a + shfl_xor(acc[v], o) * bsc;
        m = mn;
    }
    if (lane < LPR) {
        const float inv = 1.f / l;
        float* out = kbar + ((size_t)br * kbar_cap + c) * D + col;
#pragma unroll
        for (int v = 0; v < VEC; ++v) out[v] = acc[v] * inv;
    }
}

template <typename T, int D>
static hipError_t launch_summary_t(const SummaryArgs& a, hipStream_t s) {
    const int nsel = a.chunk_end - a.chunk_begin;
    const int total = a.b * a.h_kv * nsel;
    if (total == 0) return hipSuccess;
    dim3 grid((total + 3) / 4), block(256);
    hipLaunchKernelGGL((chunk_summary_kernel<T, D>), grid, block, 0, s,
                       static_cast<const T*>(a.K), a.qbar, a.kbar, a.h_kv, a.n_kv, a.kbar_cap,
                       a.B, a.chunk_begin, nsel, total,
                       (float)(1.4426950408889634 / sqrt((double)D)), a.pages, a.pages_per_seq, a.num_pages);
    return hipGetLastError();
}

hipError_t launch_summary(const SummaryArgs& a, hipStream_t s) {
    if (a.k_bf16) {
        return a.d == 64 ? launch_summary_t<uint16_t, 64>(a, s) : launch_summary_t<uint16_t, 128>(a, s);
    }
    return a.d == 64 ? launch_summary_t<float, 64>(a, s) : launch_summary_t<float, 128>(a, s);
}

}  // namespace dash
