// Stage 0 of DashAttention (paper review section 三, Eq. 4): the summary of chunk c
// is local attention of the learned query q̄ over the chunk's keys, with the keys
// also used as the values:  k̄_c = sum_t softmax_t(<q̄, k_t>/sqrt(d)) k_t.
//
// chunk_summary_kernel: one workgroup of four wavefronts per (b, r, c); batches of 16
// key rows go round-robin to the wavefronts. Each lane reads 16 bytes of a key row
// (a wavefront reads 1 KiB contiguous per load, a whole batch in flight), the rows'
// dot products with q̄ are reduced across the lanes that share a row (DPP), and a
// softmax in the log2 domain (fp32) accumulates the weighted keys. The row groups of
// a wavefront, then the four wavefronts (through LDS, in a fixed order), are merged
// and the fp32 summary is written once. HBM-bound: the K chunk is read exactly once.
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

// Sum over aligned groups of LPR lanes (8, 16 or 32), the same result in every lane of
// a group: DPP xor 1, xor 2, the 8-lane mirror and the 16-lane mirror with a symmetric
// combine, then the swap of 16-lane rows.
template <int LPR>
__device__ __forceinline__ float lane_group_sum(float v) {
    v += dpp_partner<0xB1>(v);
    v += dpp_partner<0x4E>(v);
    v += dpp_partner<0x141>(v);
    if constexpr (LPR >= 16) v += dpp_partner<0x140>(v);
    if constexpr (LPR >= 32) v = pair16_sum(v);
    return v;
}

constexpr int kSumWaves = 4;            // wavefronts per chunk

template <typename T, int D>
__global__ __launch_bounds__(64 * kSumWaves) void chunk_summary_kernel(
    const T* __restrict__ K, const float* __restrict__ qbar, float* __restrict__ kbar,
    int h_kv, int n_kv, int kbar_cap, int B, int chunk_begin, int nsel, int total,
    float scale, const int32_t* __restrict__ pages, int pages_per_seq, int num_pages,
    const int32_t* __restrict__ seq_len) {
    constexpr int VEC = Vec16<T>::N;
    constexpr int LPR = D / VEC;        // lanes sharing one key row
    constexpr int RPI = 64 / LPR;       // key rows per wave iteration
    constexpr int UNR = 16 / RPI;       // row groups per batch: 16 rows
    constexpr int ROWS = RPI * UNR;
    __shared__ float s_m[kSumWaves], s_l[kSumWaves], s_acc[kSumWaves][D];
    const int item = blockIdx.x;        // one chunk per workgroup
    if (item >= total) return;
    const int ws = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int c = chunk_begin + item % nsel;
    const int br = item / nsel;         // b * h_kv + r
    const int r = br % h_kv;
    // ragged batch: only the complete chunks of the sequence's own tokens
    // (workgroup-uniform, before the barrier)
    if (seq_len && c >= min(max(seq_len[br / h_kv], 0), n_kv) / B) return;
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

    // batches of 16 rows go round-robin to the wavefronts of the workgroup. The rows of
    // a batch (UNR row groups) are loaded before any is used; their UNR logits are
    // independent (row sums by DPP within the lanes of a row), and the batch enters
    // the wavefront's running softmax once
    for (int b0 = ws * ROWS; b0 < B; b0 += kSumWaves * ROWS) {
        float kk[UNR][VEC];
        // rows past the chunk (a batch longer than B) re-read its last row: no branch, so
        // all UNR loads are in flight together; those rows are skipped below
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int t = min(b0 + u * RPI + rr, B - 1);
            Vec16<T>::load(Kc + (size_t)t * D, kk[u]);
        }
        float sc[UNR];
        float bm = -INFINITY;
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            sc[u] = -INFINITY;
            if (b0 + u * RPI < B) {                  // wave-uniform: B is a multiple of RPI
                float sd = 0.f;
#pragma unroll
                for (int v = 0; v < VEC; ++v) sd = fmaf(q[v], kk[u][v], sd);
                sc[u] = lane_group_sum<LPR>(sd) * scale;
                bm = fmaxf(bm, sc[u]);
            }
        }
        const float mn = fmaxf(m, bm);
        const float corr = fast_exp2(m - mn);
        l *= corr;
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] *= corr;
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            if (b0 + u * RPI < B) {
                const float pu = fast_exp2(sc[u] - mn);
                l += pu;
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[v] = fmaf(pu, kk[u][v], acc[v]);
            }
        }
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
    // merge the wavefronts that have rows (the first nw; B is a multiple of 16, so
    // each of them has whole batches) in a fixed order
    const int nw = min(kSumWaves, B / ROWS);
    if (ws < nw && lane < LPR) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) s_acc[ws][col + v] = acc[v];
        if (lane == 0) { s_m[ws] = m; s_l[ws] = l; }
    }
    __syncthreads();
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float mt = s_m[0];
        for (int w = 1; w < nw; ++w) mt = fmaxf(mt, s_m[w]);
        float lt = 0.f, at = 0.f;
        for (int w = 0; w < nw; ++w) {
            const float f = fast_exp2(s_m[w] - mt);
            lt = fmaf(s_l[w], f, lt);
            at = fmaf(s_acc[w][d], f, at);
        }
        kbar[((size_t)br * kbar_cap + c) * D + d] = at / lt;
    }
}

template <typename T, int D>
static hipError_t launch_summary_t(const SummaryArgs& a, hipStream_t s) {
    const int nsel = a.chunk_end - a.chunk_begin;
    const int total = a.b * a.h_kv * nsel;
    if (total == 0) return hipSuccess;
    dim3 grid(total), block(64 * kSumWaves);
    hipLaunchKernelGGL((chunk_summary_kernel<T, D>), grid, block, 0, s,
                       static_cast<const T*>(a.K), a.qbar, a.kbar, a.h_kv, a.n_kv, a.kbar_cap,
                       a.B, a.chunk_begin, nsel, total,
                       (float)(1.4426950408889634 / sqrt((double)D)), a.pages, a.pages_per_seq, a.num_pages,
                       a.seq_len);
    return hipGetLastError();
}

hipError_t launch_summary(const SummaryArgs& a, hipStream_t s) {
    if (a.k_bf16) {
        return a.d == 64 ? launch_summary_t<uint16_t, 64>(a, s) : launch_summary_t<uint16_t, 128>(a, s);
    }
    return a.d == 64 ? launch_summary_t<float, 64>(a, s) : launch_summary_t<float, 128>(a, s);
}

}  // namespace dash
