// One DashAttention decode step (paper review section 三: Eq. 6 routing against the
// cached chunk summaries, Prop. 4.1 bias, and the split-KV Stage-2 variant of the
// kernel table), for one new query per sequence at position p = L-1.
//
//   decode_scores_kernel   z̄ for every (b, head, visible chunk): fp32 MFMA 16x16x4,
//                          one wavefront per 16 chunks x the g heads of a group, all
//                          summary loads issued before the first product. It also
//                          clears the per-group arrival counters of the router.
//   decode_route_kernel    one workgroup per (b, query head): the entmax threshold of
//                          the head over all its visible chunks (Newton on the
//                          p-norm form, as in the prefill router, with workgroup-wide
//                          sums), the head's weights written back over its scores.
//                          The last head of a group to finish (an arrival counter)
//                          takes the group average in a fixed head order, μ, the
//                          bias and a workgroup ballot compaction. The heads of a
//                          group are placed on one XCD (one L2).
//   decode_group_route_kernel  instead of the two above, for bf16 queries over more
//                          than 1024 chunks: one workgroup per group computes the g
//                          heads' logits (k̄ split into three bf16 terms on load),
//                          one wavefront per head solves τ, and the group step reads
//                          the heads' weights from LDS.
//   decode_attn_kernel     split-KV Stage 2 as a balanced token stream: every group
//                          contributes its routed chunks, then its diagonal chunk up
//                          to the query, in 32-token units; the units of all groups
//                          form one sequence, cut into equal contiguous ranges, one
//                          per wavefront (no empty workgroups, whatever the routed
//                          counts). A wavefront copies the K and V rows of its units
//                          into its own LDS ring (asynchronous global->LDS copies,
//                          stages ahead of the compute), runs S^T = K Q^T and
//                          O^T = V^T P^T on MFMA with an online softmax over the g
//                          heads of the group, and writes one unnormalised partial
//                          (max, sum, output) per group it touches. HBM-bound.
//   decode_combine_kernel  merges the partials of each (b, head) with the usual
//                          max-rescaled sum and normalises; the partials of one head
//                          are contiguous, so the merge reads them as one stream (one
//                          wavefront per (b, head, quarter of d) when there are many
//                          groups, eight when a few groups own many partials each).
#include "attn_common.h"
#include "kernels.h"

#include <math.h>

namespace dash {

constexpr int kDecUnit = 32;          // tokens per stream unit (one 32x32 S^T block)
constexpr int kDecSoftmax = -1;       // pmode of α = 1 (softmax routing)
constexpr int kRouteThreads = 256;    // workgroup of the per-head router
constexpr int kMaxStreams = 1024;     // upper bound of the attention wavefronts
constexpr int kCombThreads = 512;     // combine workgroup when groups are few
// Attention wavefronts per compute unit: more streams add in-flight copies but also
// partial results, which the next kernel must read back.
constexpr int kDecStreamsPerCU = 2;

struct DecodeParams {
    const void* Q; const void* Kc; const void* Vc;
    const float* kbar; const int32_t* seq_len;
    int b, h_q, h_kv, L_cap, kbar_cap, B, g, log2g, T_route, list_cap, streams;
    float cs, pexp, inv_sigma, scale_log2;
    int pmode, out_bf16;
    int top_k;           // > 0: keep only the top_k largest group weights of the group
    void* O;
    int32_t* idx; float* bias; int32_t* cnt; float* w_out;
    float* scores;       // [b, h_q, T_route]: raw logits, then each head's weights
    int32_t* counters;   // [b * h_kv]: head workgroups of a group that have finished
    int32_t* ranges;     // [b * h_kv][2]: first and last partial slot of each group
    float* part_ml;      // [g][slots][2]: running max and sum of a stream segment
    float* part_o;       // [g][slots][D]: its unnormalised output
    int slots;           // kMaxStreams + b * h_kv
    const int32_t* pages; int pages_per_seq, num_pages;    // paged cache (nullable)
};

__device__ __forceinline__ int seq_len_of(const DecodeParams& p, int bi) {
    return min(max(p.seq_len[bi], 1), p.L_cap);
}
__device__ __forceinline__ int visible_of(const DecodeParams& p, int L) {
    return min((L - 1) / p.B, p.T_route);
}

// ---------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_scores_kernel(DecodeParams p, const void* Qv, bool q_bf16) {
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n16 = lane & 15, kg = lane >> 4;
    const int r = blockIdx.y, bi = blockIdx.z;
    // the router's arrival counters start every call at zero (this kernel runs first)
    if (blockIdx.x == 0 && threadIdx.x == 0) p.counters[bi * p.h_kv + r] = 0;
    const int c0 = (blockIdx.x * 4 + wid) * 16;
    const int nvis = visible_of(p, seq_len_of(p, bi));
    if (c0 >= nvis) return;
    const bool head_ok = n16 < p.g;
    const int hh = r * p.g + (head_ok ? n16 : 0);
    // every load of the wavefront is issued before the first product
    const int c = min(c0 + n16, nvis - 1);
    const float* krow = p.kbar + (((size_t)bi * p.h_kv + r) * p.kbar_cap + c) * D + 4 * kg;
    f32x4 a[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) a[s] = *reinterpret_cast<const f32x4*>(krow + 16 * s);
    float qv[D / 4];
    const size_t qoff = ((size_t)bi * p.h_q + hh) * D + 4 * kg;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        float x[4];
        if (q_bf16) {
            const u32x2 v = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(Qv) + qoff + 16 * s);
            x[0] = __uint_as_float(v[0] << 16); x[1] = __uint_as_float(v[0] & 0xFFFF0000u);
            x[2] = __uint_as_float(v[1] << 16); x[3] = __uint_as_float(v[1] & 0xFFFF0000u);
        } else {
            const f32x4 v = *reinterpret_cast<const f32x4*>(static_cast<const float*>(Qv) + qoff + 16 * s);
            x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) qv[4 * s + j] = head_ok ? x[j] : 0.f;
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s][j], qv[4 * s + j], acc, 0, 0, 0);
    if (head_ok) {
        float* out = p.scores + ((size_t)bi * p.h_q + hh) * p.T_route;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ch = c0 + 4 * kg + i;
            if (ch < nvis) out[ch] = acc[i];
        }
    }
}

// ---------------------------------------------------------------------------------
// The Newton terms below take [y - τ]_+ as a clamp of y - τ to [0, 1]: y <= 0 and
// τ >= -1 (the iterates rise from -1), so y - τ <= 1 and the clamp folds into the
// subtraction.
template <int PM>
__device__ __forceinline__ void dec_accum(float t, float pexp, float& a0, float& a1) {
    if (PM == 1) { a0 += (t > 0.f) ? 1.f : 0.f; a1 += t; }
    else if (PM == 2) { a0 += t; a1 = fmaf(t, t, a1); }
    else if (PM == 4) { float t2 = t * t; a0 = fmaf(t2, t, a0); a1 = fmaf(t2, t2, a1); }
    else if (t > 0.f) {
        float lt = fast_log2(t);
        a0 += fast_exp2((pexp - 1.f) * lt);
        a1 += fast_exp2(pexp * lt);
    }
}
template <int PM>
__device__ __forceinline__ float dec_pow(float t, float pexp) {
    if (PM == 1) return t;
    if (PM == 2) return t * t;
    if (PM == 4) { float t2 = t * t; return t2 * t2; }
    return t > 0.f ? fast_exp2(pexp * fast_log2(t)) : 0.f;
}

// Inclusive prefix sum and total of one int per lane over the wavefront.
__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(v, o);
        if (lane >= o) v += y;
    }
    return v;
}
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Workgroup sum / max of one value per thread (4 wavefronts), the same result in every
// thread; `buf` holds 4 floats and is reused after a barrier.
__device__ __forceinline__ float block4_sum(float v, float* buf) {
    v = wave_sum(v);
    const int wid = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) buf[wid] = v;
    __syncthreads();
    const float r = (buf[0] + buf[1]) + (buf[2] + buf[3]);
    __syncthreads();
    return r;
}
__device__ __forceinline__ float block4_max(float v, float* buf) {
    v = wave_max(v);
    const int wid = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) buf[wid] = v;
    __syncthreads();
    const float r = fmaxf(fmaxf(buf[0], buf[1]), fmaxf(buf[2], buf[3]));
    __syncthreads();
    return r;
}

// Integer workgroup sum and exclusive prefix (4 wavefronts); `buf` holds 4 ints.
__device__ __forceinline__ int block4_sum_int(int v, int* buf) {
    v = wave_sum_int(v);
    if ((threadIdx.x & 63) == 0) buf[threadIdx.x >> 6] = v;
    __syncthreads();
    const int r = (buf[0] + buf[1]) + (buf[2] + buf[3]);
    __syncthreads();
    return r;
}
__device__ __forceinline__ int block4_excl_scan(int v, int* buf) {
    const int incl = wave_incl_scan(v);
    const int wid = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 63) buf[wid] = incl;
    __syncthreads();
    int pre = incl - v;
    for (int w = 0; w < wid; ++w) pre += buf[w];
    __syncthreads();
    return pre;
}
// Order-preserving map of a float to an unsigned key (larger float, larger key).
__device__ __forceinline__ uint32_t dec_float_key(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Hand-off between workgroups of one launch without an agent-scope release fence (on
// gfx950 it writes back the whole L2, and those write-backs serialise across
// workgroups): the data goes out through agent-scope relaxed atomic stores, which
// write through the non-coherent caches (sc1), and the arrival on a counter comes
// after every store of the workgroup has completed.
__device__ __forceinline__ void store_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// All threads call it; returns (through *last, in LDS) whether this workgroup is the
// n-th and last to arrive on the counter. The last one then invalidates its caches
// (an agent-scope acquire: no write-back), so plain loads see what the others stored.
__device__ __forceinline__ void arrive_last(int32_t* counter, int n, int* last) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");      // this thread's stores are done
    __syncthreads();                                      // ... and every thread's
    if (threadIdx.x == 0)
        *last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n - 1;
    __syncthreads();
    if (*last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Workgroups of the router are numbered so that the g heads of a group get ids of
// equal residue mod 8: consecutive workgroup ids go round-robin to the 8 XCDs, so the
// heads of a group share an L2 (the summaries they read, the weights the last one
// gathers).
__device__ __forceinline__ void route_block_of(int id, int g, int& grp, int& h) {
    const int x = id & 7, j = id >> 3;
    grp = (j / g) * 8 + x;
    h = j % g;
}

template <int VPT, int PM>
__global__ __launch_bounds__(kRouteThreads) void decode_route_kernel(DecodeParams p, int ngroups) {
    constexpr bool SOFT = PM == kDecSoftmax;
    __shared__ float red[4];
    __shared__ float nsum[2][4][2];                 // Newton partial sums, by step parity
    __shared__ int s_last, wcnt[4];
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    int grp, h;
    route_block_of(blockIdx.x, p.g, grp, h);
    if (grp >= ngroups) return;
    const int g = p.g;
    const int bi = grp / p.h_kv, r = grp % p.h_kv;
    const int nvis = visible_of(p, seq_len_of(p, bi));
    float* row = p.scores + ((size_t)bi * p.h_q + r * g + h) * p.T_route;

    if (nvis > 0) {                                   // workgroup-uniform
        float y[VPT];
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int c = VPT * tid + k;
            y[k] = c < nvis ? row[c] : -INFINITY;
            mx = fmaxf(mx, y[k]);
        }
        mx = block4_max(mx, red);
#pragma unroll
        for (int k = 0; k < VPT; ++k) y[k] = p.cs * (y[k] - mx);
        if constexpr (SOFT) {
            // α = 1: per-head softmax, kept as log2 ŵ = y - log2 Σ 2^y
            float se = 0.f;
#pragma unroll
            for (int k = 0; k < VPT; ++k) se += fast_exp2(y[k]);
            const float lse = fast_log2(block4_sum(se, red));
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int c = VPT * tid + k;
                if (c < nvis) store_coherent(row + c, y[k] - lse);
            }
        } else {
            // Newton from τ = -1 (every thread takes the same steps: the partial sums
            // of the 4 wavefronts are added in a fixed order)
            float tau = -1.f;
            for (int it = 0; it < 100; ++it) {
                float a0 = 0.f, a1 = 0.f;
#pragma unroll
                for (int k = 0; k < VPT; ++k)
                    dec_accum<PM>(__builtin_amdgcn_fmed3f(y[k] - tau, 0.f, 1.f), p.pexp, a0, a1);
                a0 = wave_sum(a0);
                a1 = wave_sum(a1);
                if (lane == 0) { nsum[it & 1][wid][0] = a0; nsum[it & 1][wid][1] = a1; }
                __syncthreads();
                a0 = (nsum[it & 1][0][0] + nsum[it & 1][1][0]) + (nsum[it & 1][2][0] + nsum[it & 1][3][0]);
                a1 = (nsum[it & 1][0][1] + nsum[it & 1][1][1]) + (nsum[it & 1][2][1] + nsum[it & 1][3][1]);
                float delta;
                if (PM == 1) delta = (a1 - 1.f) / a0;
                else {
                    const float nrm = (PM == 2) ? sqrtf(a1) : (PM == 4) ? sqrtf(sqrtf(a1)) : fast_exp2(fast_log2(a1) / p.pexp);
                    delta = (nrm - 1.f) * (a1 / nrm) / a0;
                }
                if (!(a0 > 0.f)) delta = 0.f;
                tau += delta;
                if (!(fabsf(delta) > 1e-6f)) break;
            }
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int c = VPT * tid + k;
                if (c < nvis) store_coherent(row + c, dec_pow<PM>(__builtin_amdgcn_fmed3f(y[k] - tau, 0.f, 1.f), p.pexp));
            }
        }
    }
    // publish this head's weights; the last head of the group to arrive goes on
    arrive_last(&p.counters[grp], g, &s_last);
    if (!s_last) return;

    // group average in a fixed head order (α = 1: log2 w = log2((1/g) Σ_h ŵ_h), taken
    // stably, and every visible chunk is in the support), then μ over the support.
    // Every head's weights are loaded before any is used (g <= 16 slots, unrolled).
    const float* rows = p.scores + ((size_t)bi * p.h_q + r * g) * p.T_route;
    const float inv_g = 1.f / (float)g;
    float hv[VPT][16];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int c = min(VPT * tid + k, max(nvis - 1, 0));
#pragma unroll
        for (int hh = 0; hh < 16; ++hh) hv[k][hh] = hh < g ? rows[(size_t)hh * p.T_route + c] : (SOFT ? -INFINITY : 0.f);
    }
    float wv[VPT];
    bool in[VPT];
    int ncand = 0;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int c = VPT * tid + k;
        float w = SOFT ? -INFINITY : 0.f;
        if (c < nvis) {
            if (SOFT) {
                float m = -INFINITY;
#pragma unroll
                for (int hh = 0; hh < 16; ++hh) m = fmaxf(m, hv[k][hh]);
                float sm = 0.f;
#pragma unroll
                for (int hh = 0; hh < 16; ++hh) sm += hh < g ? fast_exp2(hv[k][hh] - m) : 0.f;
                w = m + fast_log2(sm) - fast_log2((float)g);
            } else {
#pragma unroll
                for (int hh = 0; hh < 16; ++hh) w += hv[k][hh];
                w *= inv_g;
            }
        }
        wv[k] = w;
        in[k] = c < nvis && (SOFT || w > 0.f);
        ncand += in[k] ? 1 : 0;
    }
    // fixed budget: keep the top_k largest weights (equal weights to the lower chunk):
    // the top_k-th largest key by bisection on the key bits, counted over the workgroup
    if (p.top_k > 0 && block4_sum_int(ncand, wcnt) > p.top_k) {     // workgroup-uniform
        uint32_t key[VPT];
#pragma unroll
        for (int k = 0; k < VPT; ++k) key[k] = in[k] ? dec_float_key(wv[k]) : 0u;
        uint32_t kstar = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t trial = kstar | (1u << bit);
            int ge = 0;
#pragma unroll
            for (int k = 0; k < VPT; ++k) ge += key[k] >= trial ? 1 : 0;
            if (block4_sum_int(ge, wcnt) >= p.top_k) kstar = trial;
        }
        int gt = 0, eq = 0;
#pragma unroll
        for (int k = 0; k < VPT; ++k) { gt += key[k] > kstar ? 1 : 0; eq += (in[k] && key[k] == kstar) ? 1 : 0; }
        const int need_eq = p.top_k - block4_sum_int(gt, wcnt);
        int rank = block4_excl_scan(eq, wcnt);           // equal keys of lower chunks
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            if (in[k] && key[k] == kstar) in[k] = rank++ < need_eq;
            else in[k] = in[k] && key[k] > kstar;
        }
    }
    float sl = 0.f, scn = 0.f;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
        if (in[k]) { sl += SOFT ? wv[k] : fast_log2(wv[k]); scn += 1.f; }
    const float tsl = block4_sum(sl, red);
    const float tsc = block4_sum(scn, red);
    const float mu2 = tsc > 0.f ? tsl / tsc : 0.f;
    const float bscale = kLn2 * p.inv_sigma;
    int32_t* idx = p.idx + (size_t)grp * p.list_cap;
    float* bias = p.bias + (size_t)grp * p.list_cap;
    // compaction: thread tid holds chunks VPT*tid .. VPT*tid+VPT-1, so a chunk's list
    // position is the workgroup's exclusive prefix of the per-thread counts plus its
    // rank inside the thread
    int mine = 0;
#pragma unroll
    for (int k = 0; k < VPT; ++k) mine += in[k] ? 1 : 0;
    const int incl = wave_incl_scan(mine);
    if (lane == 63) wcnt[wid] = incl;
    __syncthreads();
    int pos = incl - mine;
    for (int w = 0; w < wid; ++w) pos += wcnt[w];
    const int base = (wcnt[0] + wcnt[1]) + (wcnt[2] + wcnt[3]);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int c = VPT * tid + k;
        if (in[k]) {
            idx[pos] = c;
            bias[pos] = p.inv_sigma == 0.f ? 0.f : bscale * ((SOFT ? wv[k] : fast_log2(wv[k])) - mu2);
            ++pos;
        }
        if (p.w_out && c < p.T_route) p.w_out[(size_t)grp * p.kbar_cap + c] = SOFT ? fast_exp2(wv[k]) : wv[k];
    }
    if (tid == 0) p.cnt[grp] = base;
}

// ---------------------------------------------------------------------------------
// Routing of a whole group in one workgroup (bf16 queries): decode_group_route_kernel
// computes the g heads' logits itself, so no score buffer, arrival counter or second
// kernel is involved, and the group average reads the heads' weights from LDS.
//  * Logits: 16-chunk tiles over the 8 wavefronts; each k̄ row is split on load into
//    three bf16 terms (hi + mid + lo reproduces the fp32 value), so three 16x16x32
//    bf16 MFMA chains against the exact bf16 q give the fp32 products; lane (kg, n)
//    ends with chunks 16t + 4kg + i of head n (the prefill router's arithmetic).
//  * Threshold: one wavefront per head, Newton from τ = -1 with wavefront sums only.
//  * Group step as in decode_route_kernel, with the workgroup's 8 wavefronts.
constexpr int kGroupThreads = 512;
constexpr int kGroupWaves = kGroupThreads / 64;

__device__ __forceinline__ float blockg_sum(float v, float* buf) {
    v = wave_sum(v);
    const int wid = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) buf[wid] = v;
    __syncthreads();
    float r = 0.f;
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) r += buf[w];
    __syncthreads();
    return r;
}
__device__ __forceinline__ int blockg_sum_int(int v, int* buf) {
    v = wave_sum_int(v);
    if ((threadIdx.x & 63) == 0) buf[threadIdx.x >> 6] = v;
    __syncthreads();
    int r = 0;
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) r += buf[w];
    __syncthreads();
    return r;
}
__device__ __forceinline__ int blockg_excl_scan(int v, int* buf) {
    const int incl = wave_incl_scan(v);
    const int wid = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 63) buf[wid] = incl;
    __syncthreads();
    int pre = incl - v;
    for (int w = 0; w < wid; ++w) pre += buf[w];
    __syncthreads();
    return pre;
}

// LDS of the group router: 16 head rows of NV * 64 floats.
template <int NV> constexpr size_t dec_group_lds() { return (size_t)16 * NV * 64 * sizeof(float); }

template <int D, int PM, int NV>
__global__ __launch_bounds__(kGroupThreads) void decode_group_route_kernel(DecodeParams p, const uint16_t* Q,
                                                                           int ngroups) {
    constexpr bool SOFT = PM == kDecSoftmax;
    constexpr int VPT = NV * 64 / kGroupThreads;      // chunks per thread in the group step
    typedef __bf16 b8 __attribute__((ext_vector_type(8)));
    extern __shared__ __attribute__((aligned(16))) float hw[];    // [16][TS]
    __shared__ float red[kGroupWaves];
    __shared__ int ired[kGroupWaves];
    const int grp = blockIdx.x;
    if (grp >= ngroups) return;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    const int n16 = lane & 15, kg = lane >> 4;
    const int g = p.g;
    const int bi = grp / p.h_kv, r = grp % p.h_kv;
    const int nvis = visible_of(p, seq_len_of(p, bi));
    constexpr int TS = NV * 64;

    if (nvis > 0) {                                   // workgroup-uniform
        // logits of 16-chunk tiles; wavefront w takes tiles w, w + 8, ..., four at a time
        const bool head_ok = n16 < g;
        b8 qb[D / 32];
        {
            const uint16_t* qrow = Q + ((size_t)bi * p.h_q + r * g + (head_ok ? n16 : 0)) * D + 8 * kg;
#pragma unroll
            for (int s = 0; s < D / 32; ++s) {
                qb[s] = *reinterpret_cast<const b8*>(qrow + 32 * s);
                if (!head_ok) qb[s] = b8{};
            }
        }
        const float* kb = p.kbar + (size_t)grp * p.kbar_cap * D + 8 * kg;
        const int ntile = (nvis + 15) / 16;
        constexpr int TPR = 4;                        // tiles of a wavefront in flight
        for (int t0 = wid; t0 < ntile; t0 += kGroupWaves * TPR) {
            f32x4 raw[TPR][D / 32][2];
#pragma unroll
            for (int u = 0; u < TPR; ++u) {
                const int t = min(t0 + u * kGroupWaves, ntile - 1);
                const float* krow = kb + (size_t)min(16 * t + n16, nvis - 1) * D;
#pragma unroll
                for (int s = 0; s < D / 32; ++s) {
                    raw[u][s][0] = *reinterpret_cast<const f32x4*>(krow + 32 * s);
                    raw[u][s][1] = *reinterpret_cast<const f32x4*>(krow + 32 * s + 4);
                }
            }
#pragma unroll
            for (int u = 0; u < TPR; ++u) {
                const int t = t0 + u * kGroupWaves;
                if (t < ntile) {                      // wavefront-uniform
                    f32x4 acc[3];
#pragma unroll
                    for (int h = 0; h < 3; ++h) acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < D / 32; ++s) {
                        b8 hv, mv, lv;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float x = raw[u][s][e >> 2][e & 3];
                            const __bf16 hb = (__bf16)x;
                            const float r1 = x - (float)hb;
                            const __bf16 mb = (__bf16)r1;
                            hv[e] = hb; mv[e] = mb; lv[e] = (__bf16)(r1 - (float)mb);
                        }
                        acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hv, qb[s], acc[0], 0, 0, 0);
                        acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mv, qb[s], acc[1], 0, 0, 0);
                        acc[2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lv, qb[s], acc[2], 0, 0, 0);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int ch = 16 * t + 4 * kg + i;
                        if (head_ok && ch < nvis) hw[n16 * TS + ch] = acc[0][i] + (acc[1][i] + acc[2][i]);
                    }
                }
            }
        }
    }
    __syncthreads();
    if (nvis > 0) {
        // per head: y = cs (z - max z) <= 0, then τ (α > 1) or log2 Σ 2^y (α = 1); the
        // head's weights replace its logits
        for (int h = wid; h < g; h += kGroupWaves) {
            float* row = hw + h * TS;
            float y[NV];
            float mx = -INFINITY;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int c = 64 * k + lane;
                y[k] = c < nvis ? row[c] : -INFINITY;
                mx = fmaxf(mx, y[k]);
            }
            mx = wave_max(mx);
#pragma unroll
            for (int k = 0; k < NV; ++k) y[k] = p.cs * (y[k] - mx);
            if constexpr (SOFT) {
                float se = 0.f;
#pragma unroll
                for (int k = 0; k < NV; ++k) se += fast_exp2(y[k]);
                const float lse = fast_log2(wave_sum(se));
#pragma unroll
                for (int k = 0; k < NV; ++k) {
                    const int c = 64 * k + lane;
                    if (c < nvis) row[c] = y[k] - lse;
                }
            } else {
                float tau = -1.f;
                for (int it = 0; it < 100; ++it) {
                    float a0 = 0.f, a1 = 0.f;
#pragma unroll
                    for (int k = 0; k < NV; ++k)
                        dec_accum<PM>(__builtin_amdgcn_fmed3f(y[k] - tau, 0.f, 1.f), p.pexp, a0, a1);
                    a0 = wave_sum(a0);
                    a1 = wave_sum(a1);
                    float delta;
                    if (PM == 1) delta = (a1 - 1.f) / a0;
                    else {
                        const float nrm = (PM == 2) ? sqrtf(a1) : (PM == 4) ? sqrtf(sqrtf(a1)) : fast_exp2(fast_log2(a1) / p.pexp);
                        delta = (nrm - 1.f) * (a1 / nrm) / a0;
                    }
                    if (!(a0 > 0.f)) delta = 0.f;
                    tau += delta;
                    if (!(fabsf(delta) > 1e-6f)) break;
                }
#pragma unroll
                for (int k = 0; k < NV; ++k) {
                    const int c = 64 * k + lane;
                    if (c < nvis) row[c] = dec_pow<PM>(__builtin_amdgcn_fmed3f(y[k] - tau, 0.f, 1.f), p.pexp);
                }
            }
        }
    }
    __syncthreads();

    // group average in a fixed head order, then the fixed budget, μ and the compaction
    // (thread tid holds chunks VPT*tid .. VPT*tid+VPT-1)
    const float inv_g = 1.f / (float)g;
    float wv[VPT];
    bool in[VPT];
    int ncand = 0;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int c = VPT * tid + k;
        float w = SOFT ? -INFINITY : 0.f;
        if (c < nvis) {
            if (SOFT) {
                float m = -INFINITY;
                for (int h = 0; h < g; ++h) m = fmaxf(m, hw[h * TS + c]);
                float sm = 0.f;
                for (int h = 0; h < g; ++h) sm += fast_exp2(hw[h * TS + c] - m);
                w = m + fast_log2(sm) - fast_log2((float)g);
            } else {
                for (int h = 0; h < g; ++h) w += hw[h * TS + c];
                w *= inv_g;
            }
        }
        wv[k] = w;
        in[k] = c < nvis && (SOFT || w > 0.f);
        ncand += in[k] ? 1 : 0;
    }
    if (p.top_k > 0 && blockg_sum_int(ncand, ired) > p.top_k) {     // workgroup-uniform
        uint32_t key[VPT];
#pragma unroll
        for (int k = 0; k < VPT; ++k) key[k] = in[k] ? dec_float_key(wv[k]) : 0u;
        uint32_t kstar = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t trial = kstar | (1u << bit);
            int ge = 0;
#pragma unroll
            for (int k = 0; k < VPT; ++k) ge += key[k] >= trial ? 1 : 0;
            if (blockg_sum_int(ge, ired) >= p.top_k) kstar = trial;
        }
        int gt = 0, eq = 0;
#pragma unroll
        for (int k = 0; k < VPT; ++k) { gt += key[k] > kstar ? 1 : 0; eq += (in[k] && key[k] == kstar) ? 1 : 0; }
        const int need_eq = p.top_k - blockg_sum_int(gt, ired);
        int rank = blockg_excl_scan(eq, ired);
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            if (in[k] && key[k] == kstar) in[k] = rank++ < need_eq;
            else in[k] = in[k] && key[k] > kstar;
        }
    }
    float sl = 0.f, scn = 0.f;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
        if (in[k]) { sl += SOFT ? wv[k] : fast_log2(wv[k]); scn += 1.f; }
    const float tsl = blockg_sum(sl, red);
    const float tsc = blockg_sum(scn, red);
    const float mu2 = tsc > 0.f ? tsl / tsc : 0.f;
    const float bscale = kLn2 * p.inv_sigma;
    int32_t* idx = p.idx + (size_t)grp * p.list_cap;
    float* bias = p.bias + (size_t)grp * p.list_cap;
    int mine = 0;
#pragma unroll
    for (int k = 0; k < VPT; ++k) mine += in[k] ? 1 : 0;
    int pos = blockg_excl_scan(mine, ired);
    const int base = blockg_sum_int(mine, ired);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int c = VPT * tid + k;
        if (in[k]) {
            idx[pos] = c;
            bias[pos] = p.inv_sigma == 0.f ? 0.f : bscale * ((SOFT ? wv[k] : fast_log2(wv[k])) - mu2);
            ++pos;
        }
        if (p.w_out && c < p.T_route) p.w_out[(size_t)grp * p.kbar_cap + c] = SOFT ? fast_exp2(wv[k]) : wv[k];
    }
    if (tid == 0) p.cnt[grp] = base;
}

// ---------------------------------------------------------------------------------
// The decode token stream. Group grp = b * h_kv + r contributes units_of(grp) units
// of 32 tokens: cnt * B/32 for its routed chunks, then the diagonal chunk up to the
// query. The units of all groups, in group order, form one sequence of W units; the
// P = min(streams, W) wavefronts take the ranges [blk*W/P, (blk+1)*W/P).
__device__ __forceinline__ int units_of(const DecodeParams& p, int grp) {
    const int pos = seq_len_of(p, grp / p.h_kv) - 1;
    return p.cnt[grp] * (p.B / kDecUnit) + (pos % p.B) / kDecUnit + 1;
}
__device__ __forceinline__ int first_unit_of(long long blk, long long W, long long P) {
    return (int)(blk * W / P);
}
// the range that holds unit x
__device__ __forceinline__ int range_of(long long x, long long W, long long P) {
    return (int)(((x + 1) * P + W - 1) / W) - 1;
}
__device__ __forceinline__ int stream_units(const DecodeParams& p, int ngroups) {
    int W = 0;
    for (int base = 0; base < ngroups; base += 64) {
        const int grp = base + (threadIdx.x & 63);
        W += wave_sum_int(grp < ngroups ? units_of(p, grp) : 0);
    }
    return W;
}

template <int CPW>
__device__ __forceinline__ void wait_copies_behind(int n) {
    // at most n units' copies (CPW instructions each) still in flight
    if (n <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (n == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CPW) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * CPW) : "memory");
}

template <typename T, int D, int NST>
__global__ __launch_bounds__(64) void decode_attn_kernel(DecodeParams p, int ngroups) {
    typedef SwzTile<T, D, kDecUnit> S;
    typedef TileCopier<T, D, kDecUnit, 1> CP;
    typedef Mfma<T> MM;
    typedef typename MM::Op Op;
    static_assert(NST >= 2 && NST <= 3, "two or three ring stages");
    static_assert(CP::CPW * (NST - 1) < 64, "vmcnt range");
    extern __shared__ __attribute__((aligned(16))) char ring[];   // NST stages of K, V
    const int lane = threadIdx.x & 63, l32 = lane & 31, hl = lane >> 5;
    const int blk = blockIdx.x;
    const int W = stream_units(p, ngroups);
    const int P = min(p.streams, W);
    if (blk >= P) return;
    const int u_begin = first_unit_of(blk, W, P), u_end = first_unit_of(blk + 1, W, P);
    const int upc = p.B / kDecUnit;                   // units per chunk
    const int g = p.g;
    const bool paged = p.pages != nullptr;
    CP cp;
    cp.init(0, lane);

    int S0 = 0;                                       // first unit of the current round's groups
    for (int base = 0; base < ngroups && S0 < u_end; base += 64) {
        const int mg = base + lane;
        const int mu = mg < ngroups ? units_of(p, mg) : 0;
        const int incl = wave_incl_scan(mu);
        const int mstart = S0 + incl - mu;
        uint64_t hit = ballot(mg < ngroups && mstart < u_end && mstart + mu > u_begin);
        S0 += __shfl(incl, 63);
        while (hit) {
            const int k = __builtin_ctzll(hit);
            hit &= hit - 1;
            // ---- one segment: the units [s0, s1) of group grp (relative to the group)
            const int grp = base + k;
            const int gS = __shfl(mstart, k), gU = __shfl(mu, k);
            const int s0 = max(u_begin, gS) - gS, s1 = min(u_end, gS + gU) - gS;
            const int bi = grp / p.h_kv, r = grp % p.h_kv;
            const int pos = seq_len_of(p, bi) - 1;
            const int cq = pos / p.B;
            const int cnt = p.cnt[grp];
            const bool pair_ok = l32 < g;
            if (s0 == 0 && lane == 0) {           // this wavefront holds the group's first unit
                p.ranges[2 * grp] = blk + grp;
                p.ranges[2 * grp + 1] = range_of(gS + gU - 1, W, P) + grp;
            }
            Op qf[D / 16];
            {
                const int hh = r * g + (pair_ok ? l32 : 0);
                const T* qrow = static_cast<const T*>(p.Q) + ((size_t)bi * p.h_q + hh) * D + 8 * hl;
#pragma unroll
                for (int s = 0; s < D / 16; ++s) qf[s] = pair_ok ? MM::load(qrow + 16 * s) : MM::zero();
            }
            float m_run = -INFINITY, l_run = 0.f;
            f32x16 o_acc[D / 32];
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o_acc[db][i] = 0.f;

            for (int w0 = s0; w0 < s1;) {
                // ---- a window of up to 64 list entries (chunks): lane e holds the first
                // cache row of entry e_lo + e, its last valid row and its bias
                const int e_lo = w0 / upc;
                const int e_hi = min((s1 - 1) / upc, e_lo + 63);
                const int w1 = min(s1, (e_hi + 1) * upc);
                int row0 = 0, rowmax = 0;
                float bias2 = 0.f;
                {
                    const int e = e_lo + lane;
                    if (e <= e_hi) {
                        const bool routed = e < cnt;
                        // a routed chunk is one of the query's visible chunks (< cq)
                        const int c = routed ? min(max(p.idx[(size_t)grp * p.list_cap + e], 0), max(cq - 1, 0)) : cq;
                        bias2 = routed ? p.bias[(size_t)grp * p.list_cap + e] * kLog2e : 0.f;
                        if (paged) {
                            const int pg = min(max(p.pages[(size_t)bi * p.pages_per_seq + c], 0), p.num_pages - 1);
                            row0 = (pg * p.h_kv + r) * p.B;
                        } else {
                            row0 = (grp * p.L_cap) + c * p.B;
                        }
                        // the diagonal chunk: rows past the query are never read
                        rowmax = row0 + (routed ? p.B - 1 : pos % p.B);
                    }
                }
                const int nu = w1 - w0;
                auto issue = [&](int j) {                // unit w0 + j into its stage
                    const int u = w0 + j;
                    const int e = u / upc - e_lo;
                    const int tb = __builtin_amdgcn_readlane(row0, e) + (u % upc) * kDecUnit;
                    const int nmax = __builtin_amdgcn_readlane(rowmax, e);
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // stage reads done
                    cp.issue(ring + (j % NST) * S::STAGE, static_cast<const T*>(p.Kc),
                             static_cast<const T*>(p.Vc), tb, nmax, 0);
                };
#pragma unroll
                for (int j = 0; j < NST - 1; ++j)
                    if (j < nu) issue(j);
                for (int j = 0; j < nu; ++j) {
                    if (j + NST - 1 < nu) issue(j + NST - 1);
                    wait_copies_behind<CP::CPW>(min(nu - 1 - j, NST - 1));
                    const char* kt = ring + (j % NST) * S::STAGE;
                    const char* vt = kt + S::BYTES;
                    const int u = w0 + j;
                    const int e = u / upc - e_lo;
                    const float b2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bias2), e));
                    const int lim = __builtin_amdgcn_readlane(rowmax, e) - __builtin_amdgcn_readlane(row0, e);
                    const int toff0 = (u % upc) * kDecUnit;       // token offset of the unit in its chunk
                    // S^T = K Q^T for the unit's 32 tokens
                    Op ka[D / 16];
#pragma unroll
                    for (int s = 0; s < D / 16; ++s) ka[s] = load_k_op<T, D, kDecUnit>(kt, l32, 16 * s + 8 * hl);
                    f32x16 sacc;
#pragma unroll
                    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
                    for (int s = 0; s < D / 16; ++s) sacc = MM::mma(ka[s], qf[s], sacc);
                    float mx = -INFINITY;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int toff = toff0 + 8 * (i >> 2) + 4 * hl + (i & 3);
                        const float v = fmaf(sacc[i], p.scale_log2, b2);
                        sacc[i] = toff > lim ? -INFINITY : v;
                        mx = fmaxf(mx, sacc[i]);
                    }
                    mx = pair32_max(mx);
                    // lazy rescaling: the reference maximum moves only when the unit's
                    // maximum exceeds it by more than 8 (probabilities stay <= 2^8)
                    const bool grow = mx > m_run + 8.f;
                    const float alpha = grow ? fast_exp2(m_run - mx) : 1.f;
                    m_run = grow ? mx : m_run;
                    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
                    float ps = 0.f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float pv = fast_exp2(sacc[i] - m_use);
                        sacc[i] = pv;
                    }
                    Op pb[2];
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        float pv8[8];
#pragma unroll
                        for (int e8 = 0; e8 < 8; ++e8) pv8[e8] = sacc[8 * s2 + e8];
                        pb[s2] = MM::pack(pv8);
                        ps = MM::sum(pb[s2], pv8, ps);            // the denominator sums what the MFMA sees
                    }
                    l_run = fmaf(l_run, alpha, ps);
                    if (ballot(grow) != 0) {
#pragma unroll
                        for (int db = 0; db < D / 32; ++db)
#pragma unroll
                            for (int i = 0; i < 16; ++i) o_acc[db][i] *= alpha;
                    }
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        Op va[D / 32];
#pragma unroll
                        for (int db = 0; db < D / 32; ++db) va[db] = load_vt_op<T, D, kDecUnit>(vt, s2, db, lane);
#pragma unroll
                        for (int db = 0; db < D / 32; ++db) o_acc[db] = MM::mma(va[db], pb[s2], o_acc[db]);
                    }
                }
                w0 = w1;
            }
            // ---- the segment's partial, per head: running max, sum, unnormalised output
            const float l_tot = pair32_sum(l_run);
            if (pair_ok) {
                const size_t slot = (size_t)blk + grp;
                if (hl == 0) {
                    float* ml = p.part_ml + ((size_t)l32 * p.slots + slot) * 2;
                    ml[0] = m_run;
                    ml[1] = l_tot;
                }
                float* po = p.part_o + ((size_t)l32 * p.slots + slot) * D;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        f32x4 o;
                        o[0] = o_acc[db][4 * a]; o[1] = o_acc[db][4 * a + 1];
                        o[2] = o_acc[db][4 * a + 2]; o[3] = o_acc[db][4 * a + 3];
                        *reinterpret_cast<f32x4*>(po + 32 * db + 8 * a + 4 * hl) = o;
                    }
            }
        }
    }
}

// ---------------------------------------------------------------------------------
// One workgroup per (b, query head, quarter of d): the partial slots of the head's
// group (first .. last, written by the attention kernel) sit contiguously in part_o
// for one head, D floats apart. Threads split them into slot lanes x column quads;
// each thread merges its slots with a running maximum (its loads of a batch issued
// together), then the slot lanes are merged in LDS.
constexpr int kCombParts = 4;
template <int D, int NT>
__global__ __launch_bounds__(NT) void decode_combine_kernel(DecodeParams p) {
    constexpr int DQ = D / 4 / kCombParts;         // column quads of this workgroup
    constexpr int SL = NT / DQ;                    // slot lanes
    constexpr int NB = 8;                          // slots per thread and batch
    const int tid = threadIdx.x;
    const int hh = blockIdx.x, bi = blockIdx.y, part = blockIdx.z;
    const int g = p.g, r = hh / g, pr = hh % g;
    const int grp = bi * p.h_kv + r;
    const int first = p.ranges[2 * grp], n = p.ranges[2 * grp + 1] - first + 1;
    const int sl = tid / DQ, dq = tid % DQ;
    const int d0 = part * (D / kCombParts) + 4 * dq;
    const float* ml = p.part_ml + ((size_t)pr * p.slots + first) * 2;
    const float* po = p.part_o + ((size_t)pr * p.slots + first) * D + d0;
    float m_t = -INFINITY, l_t = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = sl; j0 < n; j0 += NB * SL) {
        f32x4 v[NB];
        float mj[NB], lj[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int j = j0 + u * SL;
            const bool ok = j < n;
            v[u] = ok ? *reinterpret_cast<const f32x4*>(po + (size_t)j * D) : f32x4{0.f, 0.f, 0.f, 0.f};
            mj[u] = ok ? ml[2 * j] : -INFINITY;
            lj[u] = ok ? ml[2 * j + 1] : 0.f;
        }
        float mb = m_t;
#pragma unroll
        for (int u = 0; u < NB; ++u) mb = fmaxf(mb, mj[u]);
        const float sc = m_t == -INFINITY ? 0.f : fast_exp2(m_t - mb);
        acc *= sc;
        l_t *= sc;
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const float f = mj[u] == -INFINITY ? 0.f : fast_exp2(mj[u] - mb);
            acc[0] = fmaf(f, v[u][0], acc[0]); acc[1] = fmaf(f, v[u][1], acc[1]);
            acc[2] = fmaf(f, v[u][2], acc[2]); acc[3] = fmaf(f, v[u][3], acc[3]);
            l_t = fmaf(f, lj[u], l_t);
        }
        m_t = mb;
    }
    // merge the slot lanes pairwise in a fixed order: within the wavefront by a
    // butterfly over the slot bits of the lane (both lanes of a pair combine the same
    // operands in the same order), across wavefronts through LDS
#pragma unroll
    for (int o = DQ; o < 64 && o < NT; o <<= 1) {
        const float mo = shfl_xor(m_t, o), lo = shfl_xor(l_t, o);
        f32x4 ao;
#pragma unroll
        for (int e = 0; e < 4; ++e) ao[e] = shfl_xor(acc[e], o);
        const bool lower = (tid & o) == 0;
        const float ma = lower ? m_t : mo, mb2 = lower ? mo : m_t;
        const float la = lower ? l_t : lo, lb = lower ? lo : l_t;
        const f32x4 aa = lower ? acc : ao, ab = lower ? ao : acc;
        const float M = fmaxf(ma, mb2);
        const float fa = ma == -INFINITY ? 0.f : fast_exp2(ma - M);
        const float fb = mb2 == -INFINITY ? 0.f : fast_exp2(mb2 - M);
        m_t = M;
        l_t = fa * la + fb * lb;
        acc = fa * aa + fb * ab;
    }
    if constexpr (NT > 64) {
        constexpr int NW = NT / 64;
        __shared__ float s_m[NW][DQ], s_l[NW][DQ];
        __shared__ f32x4 s_acc[NW][DQ];
        const int wid = tid >> 6;
        if ((tid & 63) < DQ) {
            s_m[wid][dq] = m_t;
            s_l[wid][dq] = l_t;
            s_acc[wid][dq] = acc;
        }
        __syncthreads();
        if (tid < DQ) {
            for (int w = 1; w < NW; ++w) {
                const float mb2 = s_m[w][dq];
                const float M = fmaxf(m_t, mb2);
                const float fa = m_t == -INFINITY ? 0.f : fast_exp2(m_t - M);
                const float fb = mb2 == -INFINITY ? 0.f : fast_exp2(mb2 - M);
                m_t = M;
                l_t = fa * l_t + fb * s_l[w][dq];
                acc = fa * acc + fb * s_acc[w][dq];
            }
        }
    }
    if (tid < DQ) {
        const float inv = 1.f / l_t;
        const size_t oi = ((size_t)bi * p.h_q + hh) * D + part * (D / kCombParts) + 4 * tid;
        if (p.out_bf16) {
            u32x2 ob;
            ob[0] = (uint32_t)f32_to_bf16_bits(acc[0] * inv) | ((uint32_t)f32_to_bf16_bits(acc[1] * inv) << 16);
            ob[1] = (uint32_t)f32_to_bf16_bits(acc[2] * inv) | ((uint32_t)f32_to_bf16_bits(acc[3] * inv) << 16);
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.O) + oi) = ob;
        } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(p.O) + oi) = acc * inv;
        }
    }
}

// ---------------------------------------------------------------------------------
int decode_partial_slots(int b, int h_kv) { return kMaxStreams + b * h_kv; }

int pmode_of(float alpha);

template <int VPT, int PM>
static hipError_t launch_dec_route_pm(const DecodeParams& p, int ngroups, hipStream_t s) {
    const int nblk = (ngroups + 7) / 8 * 8 * p.g;
    hipLaunchKernelGGL((decode_route_kernel<VPT, PM>), dim3(nblk), dim3(kRouteThreads), 0, s, p, ngroups);
    return hipSuccess;
}

template <int VPT>
static hipError_t launch_dec_route(const DecodeParams& p, int ngroups, hipStream_t s) {
    switch (p.pmode) {
        case kDecSoftmax: return launch_dec_route_pm<VPT, kDecSoftmax>(p, ngroups, s);
        case 1: return launch_dec_route_pm<VPT, 1>(p, ngroups, s);
        case 2: return launch_dec_route_pm<VPT, 2>(p, ngroups, s);
        case 4: return launch_dec_route_pm<VPT, 4>(p, ngroups, s);
        default: return launch_dec_route_pm<VPT, 0>(p, ngroups, s);
    }
}

template <int D, int PM, int NV>
static hipError_t launch_dec_group_pm(const DecodeParams& p, const void* Q, int ngroups, hipStream_t s) {
    auto kern = decode_group_route_kernel<D, PM, NV>;
    static hipError_t configured = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024);
    if (configured != hipSuccess) return configured;
    hipLaunchKernelGGL(kern, dim3(ngroups), dim3(kGroupThreads), dec_group_lds<NV>(), s, p,
                       static_cast<const uint16_t*>(Q), ngroups);
    return hipGetLastError();
}

template <int D, int NV>
static hipError_t launch_dec_group_nv(const DecodeParams& p, const void* Q, int ngroups, hipStream_t s) {
    switch (p.pmode) {
        case kDecSoftmax: return launch_dec_group_pm<D, kDecSoftmax, NV>(p, Q, ngroups, s);
        case 1: return launch_dec_group_pm<D, 1, NV>(p, Q, ngroups, s);
        case 2: return launch_dec_group_pm<D, 2, NV>(p, Q, ngroups, s);
        case 4: return launch_dec_group_pm<D, 4, NV>(p, Q, ngroups, s);
        default: return launch_dec_group_pm<D, 0, NV>(p, Q, ngroups, s);
    }
}

// bf16 queries: the whole routing in decode_group_route_kernel (NV chunks of 64 per
// head row: the group step's threads hold NV/8 chunks each).
template <int D>
static hipError_t launch_dec_group(const DecodeParams& p, const void* Q, int ngroups, hipStream_t s) {
    if (p.T_route <= 512) return launch_dec_group_nv<D, 8>(p, Q, ngroups, s);
    if (p.T_route <= 1024) return launch_dec_group_nv<D, 16>(p, Q, ngroups, s);
    return launch_dec_group_nv<D, 32>(p, Q, ngroups, s);
}

// Ring stages and wavefronts resident per CU of the attention kernel.
template <typename T, int D> struct DecAttnCfg {
    static constexpr int NST = sizeof(T) == 2 ? 2 : 2;
    static constexpr size_t LDS = (size_t)NST * SwzTile<T, D, kDecUnit>::STAGE;
};

static int device_cus() {
    static int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess) return 256;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
        return n;
    }();
    return cus;
}

template <typename T, int D>
static hipError_t launch_decode_t(DecodeParams p, const DecodeArgs& a, hipStream_t s) {
    typedef DecAttnCfg<T, D> C;
    auto attn = decode_attn_kernel<T, D, C::NST>;
    static hipError_t configured = hipFuncSetAttribute(reinterpret_cast<const void*>(attn),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
    if (configured != hipSuccess) return configured;
    static int per_cu = [&] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(attn), 64, C::LDS) != hipSuccess || n < 1)
            return 1;
        return n;
    }();
    const int ngroups = a.b * a.h_kv;
    p.streams = min(kMaxStreams, device_cus() * min(per_cu, kDecStreamsPerCU));
    // bf16 queries over more than 1024 chunks: the whole routing in one workgroup per
    // group (at 96K with 48 groups the logits and per-head router take 15 + 48 µs, the
    // group router 37); otherwise logits over many workgroups, then the per-head router
    // (at 128K with 8 groups 6 + 11 µs, where eight group workgroups take longer)
    hipError_t er;
    if (a.in_bf16 && p.T_route > 1024) {
        er = launch_dec_group<D>(p, a.Q, ngroups, s);
    } else {
        dim3 g1(max((p.T_route + 63) / 64, 1), p.h_kv, a.b);
        hipLaunchKernelGGL((decode_scores_kernel<D>), g1, dim3(256), 0, s, p, a.Q, a.in_bf16);
        er = p.T_route <= 256 ? launch_dec_route<1>(p, ngroups, s)
           : p.T_route <= 512 ? launch_dec_route<2>(p, ngroups, s)
           : p.T_route <= 1024 ? launch_dec_route<4>(p, ngroups, s)
                               : launch_dec_route<8>(p, ngroups, s);
    }
    if (er != hipSuccess) return er;

    hipLaunchKernelGGL(attn, dim3(p.streams), dim3(64), C::LDS, s, p, ngroups);
    // few groups own many partials each (wide merge); many groups own few (one wavefront)
    if (ngroups >= 16)
        hipLaunchKernelGGL((decode_combine_kernel<D, 64>), dim3(p.h_q, a.b, kCombParts), dim3(64), 0, s, p);
    else
        hipLaunchKernelGGL((decode_combine_kernel<D, kCombThreads>), dim3(p.h_q, a.b, kCombParts),
                           dim3(kCombThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    DecodeParams p;
    p.Q = a.Q; p.Kc = a.Kc; p.Vc = a.Vc; p.kbar = a.kbar; p.seq_len = a.seq_len;
    p.b = a.b; p.h_q = a.h_q; p.h_kv = a.h_kv; p.L_cap = a.L_cap; p.kbar_cap = a.kbar_cap; p.B = a.B;
    p.g = a.h_q / a.h_kv;
    p.log2g = 0;
    while ((1 << p.log2g) < p.g) ++p.log2g;
    p.T_route = a.T_route; p.list_cap = a.list_cap;
    p.cs = route_scale(a.alpha, a.gamma, a.d);
    p.pexp = (float)(1.0 / ((double)a.alpha - 1.0));
    p.pmode = pmode_of(a.alpha);
    p.top_k = a.top_k;
    p.inv_sigma = isinf(a.sigma) ? 0.f : (float)(1.0 / (double)a.sigma);
    p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)a.d));
    p.out_bf16 = a.out_bf16;
    p.O = a.O; p.idx = a.idx; p.bias = a.bias; p.cnt = a.cnt; p.w_out = a.w_out;
    p.scores = a.scores; p.counters = a.counters; p.ranges = a.counters + a.b * a.h_kv; p.part_ml = a.part_ml; p.part_o = a.part_o;
    p.slots = decode_partial_slots(a.b, a.h_kv);
    p.streams = kMaxStreams;
    p.pages = a.pages; p.pages_per_seq = a.pages_per_seq; p.num_pages = a.num_pages;
    if (a.in_bf16) return a.d == 64 ? launch_decode_t<uint16_t, 64>(p, a, s) : launch_decode_t<uint16_t, 128>(p, a, s);
    return a.d == 64 ? launch_decode_t<float, 64>(p, a, s) : launch_decode_t<float, 128>(p, a, s);
}

}  // namespace dash
