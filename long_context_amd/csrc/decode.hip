// One DashAttention decode step (paper review section 三: Eq. 6 routing against the
// cached chunk summaries, Prop. 4.1 bias, and the split-KV Stage-2 variant of the
// kernel table), for one new query per sequence at position p = L-1.
//
//   decode_scores_kernel   z̄ for every (b, head, visible chunk): fp32 MFMA 16x16x4,
//                          one wavefront per 16 chunks x the g heads of a group;
//                          spread over many workgroups because this step is bound
//                          by reading the fp32 summaries.
//   decode_route_kernel    one workgroup per (b, KV group), up to 2048 chunks per
//                          row: wavefront h solves the
//                          entmax threshold of head h over all visible chunks
//                          (Newton on the p-norm form, as in the prefill router),
//                          the group average is taken in LDS in a fixed head order,
//                          then μ, the bias, and a block-wide ballot compaction.
//   decode_attn_kernel     split-KV Stage 2: the group's routed chunks followed by
//                          the diagonal chunk form one token stream; each workgroup
//                          takes a slice of it, its 4 wavefronts take 32 tokens of
//                          every 128-token tile (K/V staged in LDS, prefetched), and
//                          the workgroup writes one unnormalised partial
//                          (max, sum, output) per head. HBM-bound.
//   decode_combine_kernel  merges the partials of all slices with the usual
//                          max-rescaled sum and normalises.
#include "attn_common.h"
#include "kernels.h"

#include <math.h>

namespace dash {

constexpr int kDecTT = 64;           // tokens per decode tile (one 32-token block per wavefront)
constexpr int kDecWaves = kDecTT / 32;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecSlice = 512;        // stream tokens per workgroup
constexpr int kDecSoftmax = -1;       // pmode of α = 1 (softmax routing)

struct DecodeParams {
    const void* Q; const void* Kc; const void* Vc;
    const float* kbar; const int32_t* seq_len;
    int h_q, h_kv, L_cap, kbar_cap, B, g, log2g, T_route, list_cap, max_slices, slice_tokens;
    float cs, pexp, inv_sigma, scale_log2;
    int pmode, out_bf16;
    void* O;
    int32_t* idx; float* bias; int32_t* cnt; float* w_out;
    float* scores; float* partials;
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
    const int c0 = (blockIdx.x * 4 + wid) * 16;
    const int nvis = visible_of(p, seq_len_of(p, bi));
    if (c0 >= nvis) return;
    const bool head_ok = n16 < p.g;
    const int hh = r * p.g + (head_ok ? n16 : 0);
    float qv[D / 4];
    const size_t qoff = ((size_t)bi * p.h_q + hh) * D + 4 * kg;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        // 4 consecutive elements per lane and step: one 8-byte (bf16) or 16-byte load
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
    const int c = min(c0 + n16, nvis - 1);
    const float* krow = p.kbar + (((size_t)bi * p.h_kv + r) * p.kbar_cap + c) * D + 4 * kg;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(krow + 16 * s);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], qv[4 * s + j], acc, 0, 0, 0);
    }
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

template <int VPL, int PM>
__global__ __launch_bounds__(1024) void decode_route_kernel(DecodeParams p) {
    constexpr int TMAX = VPL * 64;
    extern __shared__ float dyn_wl[];                 // [16][TMAX] per-head weights
    auto wl = reinterpret_cast<float (*)[TMAX]>(dyn_wl);
    __shared__ float red[2][16];
    __shared__ int wcnt[16];
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    const int r = blockIdx.x, bi = blockIdx.y;
    const int g = p.g;
    const int nvis = visible_of(p, seq_len_of(p, bi));
    const size_t grp = (size_t)bi * p.h_kv + r;

    if (wid < g && nvis > 0) {
        const int hh = r * g + wid;
        const float* sc = p.scores + ((size_t)bi * p.h_q + hh) * p.T_route;
        float y[VPL];
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int c = lane + 64 * k;
            y[k] = c < nvis ? sc[c] : -INFINITY;
            mx = fmaxf(mx, y[k]);
        }
        mx = wave_max(mx);
#pragma unroll
        for (int k = 0; k < VPL; ++k) y[k] = p.cs * (y[k] - mx);
        if constexpr (PM == kDecSoftmax) {
            // α = 1: per-head softmax, kept as log2 ŵ = y - log2 Σ 2^y
            float se = 0.f;
#pragma unroll
            for (int k = 0; k < VPL; ++k) se += fast_exp2(y[k]);
            const float lse = fast_log2(wave_sum(se));
#pragma unroll
            for (int k = 0; k < VPL; ++k) wl[wid][lane + 64 * k] = y[k] - lse;
        } else {
        float tau = -1.f;
        for (int it = 0; it < 100; ++it) {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int k = 0; k < VPL; ++k) dec_accum<PM>(__builtin_amdgcn_fmed3f(y[k] - tau, 0.f, 1.f), p.pexp, a0, a1);
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
        for (int k = 0; k < VPL; ++k) wl[wid][lane + 64 * k] = dec_pow<PM>(__builtin_amdgcn_fmed3f(y[k] - tau, 0.f, 1.f), p.pexp);
        }
    }
    __syncthreads();
    // group average in a fixed head order, then μ over the support
    const float inv_g = 1.f / (float)g;
    float wv[TMAX / 1024 > 0 ? TMAX / 1024 : 1];
    constexpr int PER = TMAX / 1024 > 0 ? TMAX / 1024 : 1;
    // (α = 1: wv holds log2 w = log2((1/g) Σ_h ŵ_h), taken stably, and every visible
    // chunk is in the support)
    constexpr bool SOFT = PM == kDecSoftmax;
    float sl = 0.f, scn = 0.f;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int c = tid + 1024 * q;
        float w = SOFT ? -INFINITY : 0.f;
        if (c < nvis) {
            if (SOFT) {
                float m = -INFINITY;
                for (int h = 0; h < g; ++h) m = fmaxf(m, wl[h][c]);
                float sm = 0.f;
                for (int h = 0; h < g; ++h) sm += fast_exp2(wl[h][c] - m);
                w = m + fast_log2(sm) - fast_log2((float)g);
                sl += w; scn += 1.f;
            } else {
                for (int h = 0; h < g; ++h) w += wl[h][c];
                w *= inv_g;
            }
        }
        wv[q] = w;
        if (!SOFT && w > 0.f) { sl += fast_log2(w); scn += 1.f; }
    }
    sl = wave_sum(sl);
    scn = wave_sum(scn);
    if (lane == 0) { red[0][wid] = sl; red[1][wid] = scn; }
    __syncthreads();
    float tsl = 0.f, tsc = 0.f;
    for (int w = 0; w < 16; ++w) { tsl += red[0][w]; tsc += red[1][w]; }
    const float mu2 = tsc > 0.f ? tsl / tsc : 0.f;
    const float bscale = kLn2 * p.inv_sigma;
    int32_t* idx = p.idx + grp * p.list_cap;
    float* bias = p.bias + grp * p.list_cap;
    int base = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int c = tid + 1024 * q;
        const bool in = SOFT ? c < nvis : wv[q] > 0.f;
        const uint64_t m = ballot(in);
        if (lane == 0) wcnt[wid] = __builtin_popcountll(m);
        __syncthreads();
        int off = base;
        for (int w = 0; w < wid; ++w) off += wcnt[w];
        int tot = 0;
        for (int w = 0; w < 16; ++w) tot += wcnt[w];
        if (in) {
            const int pos = off + __builtin_popcountll(m & ((1ull << lane) - 1ull));
            idx[pos] = c;
            bias[pos] = p.inv_sigma == 0.f ? 0.f : bscale * ((SOFT ? wv[q] : fast_log2(wv[q])) - mu2);
        }
        if (p.w_out && c < p.T_route) p.w_out[grp * p.kbar_cap + c] = SOFT ? fast_exp2(wv[q]) : wv[q];
        base += tot;
        __syncthreads();
    }
    if (tid == 0) p.cnt[grp] = base;
}

// ---------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_attn_kernel(DecodeParams p) {
    typedef TileGeom<T, D, kDecTT> G;
    typedef Mfma<T> MM;
    typedef typename MM::Op Op;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    constexpr int MAXE = 64;                       // entry cache per slice
    int* s_chunk = reinterpret_cast<int*>(smem + G::BYTES);
    float* s_bias = reinterpret_cast<float*>(s_chunk + MAXE);
    int* s_row0 = reinterpret_cast<int*>(s_bias + MAXE);   // first cache row of each chunk

    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hl = lane >> 5;
    const int slice = blockIdx.x, r = blockIdx.y, bi = blockIdx.z;
    const int g = p.g, B = p.B;
    const size_t grp = (size_t)bi * p.h_kv + r;
    const int L = seq_len_of(p, bi);
    const int pos = L - 1;
    const int cq = pos / B;
    const int cnt = p.cnt[grp];
    const int E = cnt + 1;                          // routed chunks, then the diagonal
    const int ST = p.slice_tokens;
    const int t_begin = slice * ST;
    const int t_end = min(t_begin + ST, E * B);
    if (t_begin >= t_end) return;
    const int e_first = t_begin / B;
    const int e_last = (t_end - 1) / B;
    // contiguous cache: row of token t of chunk c = c*B + t in the (b, r) slab; paged
    // cache: ((page * h_kv + r) * B + t) in the page array (page ids clamped)
    const bool paged = p.pages != nullptr;
    for (int e = e_first + tid; e <= e_last; e += kDecThreads) {
        const bool routed = e < cnt;
        const int c = routed ? p.idx[grp * p.list_cap + e] : cq;
        s_chunk[e - e_first] = c;
        s_bias[e - e_first] = routed ? p.bias[grp * p.list_cap + e] * kLog2e : 0.f;
        if (paged) {
            const int pg = min(max(p.pages[(size_t)bi * p.pages_per_seq + c], 0), p.num_pages - 1);
            s_row0[e - e_first] = (pg * p.h_kv + r) * B;
        } else {
            s_row0[e - e_first] = c * B;
        }
    }
    __syncthreads();

    const bool pair_ok = l32 < g;
    const int hh = r * g + (pair_ok ? l32 : 0);
    Op qf[D / 16];
    {
        const T* qrow = static_cast<const T*>(p.Q) + ((size_t)bi * p.h_q + hh) * D + 8 * hl;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) qf[s] = pair_ok ? MM::load(qrow + 16 * s) : MM::zero();
    }
    const T* Kg = static_cast<const T*>(p.Kc) + (paged ? (size_t)0 : grp * (size_t)p.L_cap * D);
    const T* Vg = static_cast<const T*>(p.Vc) + (paged ? (size_t)0 : grp * (size_t)p.L_cap * D);

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o_acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o_acc[db][i] = 0.f;

    const int ntiles = (t_end - t_begin + kDecTT - 1) / kDecTT;
    // cache row of the first token of each 32-token group of a tile (a group never
    // straddles two chunks because B % 32 == 0); -1 past the slice end. Rows of the
    // diagonal chunk are clamped to the query's own row (later tokens are masked).
    auto group_base = [&](int tau) -> int {
        if (tau >= t_end) return -1;
        return s_row0[tau / B - e_first] + tau % B;
    };
    int rb[kDecWaves], rl[kDecWaves];
    auto set_bases = [&](int tt0) {
#pragma unroll
        for (int q = 0; q < kDecWaves; ++q) {
            const int tau = tt0 + 32 * q;
            rb[q] = group_base(tau);
            // the diagonal entry (the last one, index cnt) may hold rows past pos
            rl[q] = (tau < t_end && tau / B >= cnt) ? s_row0[tau / B - e_first] + pos % B : 0x7fffffff;
        }
    };
    auto row_of = [&](int t) -> int {
        const int base = rb[t >> 5];
        return base < 0 ? 0 : min(base + (t & 31), rl[t >> 5]);
    };
    TileRegs<T, D, kDecTT, kDecThreads> regs;
    set_bases(t_begin);
    regs.load(Kg, Vg, row_of, tid);
    for (int k = 0; k < ntiles; ++k) {
        const int tt0 = t_begin + k * kDecTT;
        __syncthreads();
        regs.store(smem, tid);
        __syncthreads();
        if (k + 1 < ntiles) {
            set_bases(tt0 + kDecTT);
            regs.load(Kg, Vg, row_of, tid);
        }
        const int wt0 = tt0 + 32 * wid;            // this wavefront's 32 stream tokens
        if (wt0 >= t_end) continue;
        const int e = wt0 / B;
        const bool diag = e >= cnt;
        const float bias2 = s_bias[e - e_first];
        const int kv0 = s_chunk[e - e_first] * B + wt0 % B;   // KV position of token 0
        f32x16 sacc1[1];
        score_blocks<T, D, 1, G::KROW>(sacc1, smem + (32 * wid + l32) * G::KROW + 8 * hl * G::ES, qf);
        f32x16 sacc = sacc1[0];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int toff = 8 * (i >> 2) + 4 * hl + (i & 3);
            float v = fmaf(sacc[i], p.scale_log2, bias2);
            if ((diag && kv0 + toff > pos) || wt0 + toff >= t_end) v = -INFINITY;
            sacc[i] = v;
            mx = fmaxf(mx, v);
        }
        mx = pair32_max(mx);
        // lazy rescaling: the reference maximum moves only when the tile maximum
        // exceeds it by more than 8 (probabilities stay <= 2^8 in between)
        const bool grow = mx > m_run + 8.f;
        const float alpha = grow ? fast_exp2(m_run - mx) : 1.f;
        m_run = grow ? mx : m_run;
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float pv = fast_exp2(sacc[i] - m_use);
            sacc[i] = pv;
            ps += pv;
        }
        l_run = fmaf(l_run, alpha, ps);
        if (ballot(grow) != 0) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o_acc[db][i] *= alpha;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float pv8[8];
#pragma unroll
            for (int e8 = 0; e8 < 8; ++e8) pv8[e8] = sacc[8 * s + e8];
            const Op pb = MM::pack(pv8);
            Op va[D / 32];
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                va[db] = MM::load(reinterpret_cast<const T*>(smem + G::KBYTES + (32 * db + l32) * G::VROW) + 32 * wid + 16 * s + 8 * hl);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o_acc[db] = MM::mma(va[db], pb, o_acc[db]);
        }
    }
    // merge the 4 wavefronts' partial softmax states in LDS
    __syncthreads();
    float* s_o = reinterpret_cast<float*>(smem);               // [4][32][D]
    float* s_m = s_o + kDecWaves * 32 * D;                     // [waves][32]
    float* s_l = s_m + kDecWaves * 32;                         // [waves][32]
    const float l_tot = pair32_sum(l_run);
    if (hl == 0) { s_m[wid * 32 + l32] = m_run; s_l[wid * 32 + l32] = l_tot; }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int d = 32 * db + 8 * (i >> 2) + 4 * hl + (i & 3);
            s_o[(wid * 32 + l32) * D + d] = o_acc[db][i];
        }
    __syncthreads();
    float* part = p.partials + ((grp * p.max_slices + slice) * (size_t)g) * (D + 2);
    for (int q = tid; q < g * D; q += kDecThreads) {
        const int pr = q / D, d = q % D;
        float mstar = -INFINITY;
        for (int w = 0; w < kDecWaves; ++w) mstar = fmaxf(mstar, s_m[w * 32 + pr]);
        const float mu = (mstar == -INFINITY) ? 0.f : mstar;
        float o = 0.f, l = 0.f;
        for (int w = 0; w < kDecWaves; ++w) {
            const float f = fast_exp2(s_m[w * 32 + pr] - mu);
            o += f * s_o[(w * 32 + pr) * D + d];
            l += f * s_l[w * 32 + pr];
        }
        float* pp = part + (size_t)pr * (D + 2);
        if (d == 0) { pp[0] = mstar; pp[1] = l; }
        pp[2 + d] = o;
    }
}

// ---------------------------------------------------------------------------------
// One workgroup of 1024 threads per (head, b): slice maxima and weighted sums by
// block reductions, then 1024/D thread groups each sum a share of the slices'
// outputs (the work is a few loads per thread; more threads shorten the chain).
constexpr int kCombThreads = 1024;
template <int D>
__global__ __launch_bounds__(kCombThreads) void decode_combine_kernel(DecodeParams p) {
    constexpr int NG = kCombThreads / D;            // thread groups splitting the slices
    constexpr int NW = kCombThreads / 64;
    extern __shared__ float s_f[];                  // [max_slices] slice factors
    __shared__ float red[2][NW];
    __shared__ float s_acc[NG][D];
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    const int hh = blockIdx.x, bi = blockIdx.y;
    const int g = p.g, r = hh / g, pr = hh % g;
    const size_t grp = (size_t)bi * p.h_kv + r;
    const int E = p.cnt[grp] + 1;
    const int nsl = (E * p.B + p.slice_tokens - 1) / p.slice_tokens;
    const float* base = p.partials + (grp * p.max_slices * (size_t)g + pr) * (D + 2);
    const size_t sstride = (size_t)g * (D + 2);
    float mx = -INFINITY;
    for (int s = tid; s < nsl; s += kCombThreads) mx = fmaxf(mx, base[s * sstride]);
    mx = wave_max(mx);
    if (lane == 0) red[0][wid] = mx;
    __syncthreads();
    float mstar = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mstar = fmaxf(mstar, red[0][w]);
    const float mu = (mstar == -INFINITY) ? 0.f : mstar;
    float ls = 0.f;
    for (int s = tid; s < nsl; s += kCombThreads) {
        const float f = fast_exp2(base[s * sstride] - mu);
        s_f[s] = f;
        ls += f * base[s * sstride + 1];
    }
    ls = wave_sum(ls);
    if (lane == 0) red[1][wid] = ls;
    __syncthreads();
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) l += red[1][w];
    const int gq = tid / D, d = tid % D;
    float acc = 0.f;
#pragma unroll 4
    for (int s = gq; s < nsl; s += NG) acc += s_f[s] * base[s * sstride + 2 + d];
    s_acc[gq][d] = acc;
    __syncthreads();
    if (gq == 0) {
        float o = 0.f;
#pragma unroll
        for (int k = 0; k < NG; ++k) o += s_acc[k][d];
        const float val = o / l;
        const size_t oi = ((size_t)bi * p.h_q + hh) * D + d;
        if (p.out_bf16) static_cast<uint16_t*>(p.O)[oi] = f32_to_bf16_bits(val);
        else static_cast<float*>(p.O)[oi] = val;
    }
}

// ---------------------------------------------------------------------------------
void decode_geometry(int L_cap, int kbar_cap, int B, int* T_route, int* slice_tokens,
                     int* max_slices) {
    const int tr = min((L_cap - 1) / B, kbar_cap);
    *T_route = tr;
    *slice_tokens = kDecSlice;
    *max_slices = ((tr + 1) * B + kDecSlice - 1) / kDecSlice;
}

int pmode_of(float alpha);

template <int VPL, int PM>
static hipError_t launch_dec_route_pm(const DecodeParams& p, int b, hipStream_t s) {
    constexpr size_t lds = (size_t)16 * VPL * 64 * sizeof(float);
    static hipError_t configured = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_route_kernel<VPL, PM>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (configured != hipSuccess) return configured;
    hipLaunchKernelGGL((decode_route_kernel<VPL, PM>), dim3(p.h_kv, b), dim3(1024), lds, s, p);
    return hipSuccess;
}

template <int VPL>
static hipError_t launch_dec_route(const DecodeParams& p, int b, hipStream_t s) {
    switch (p.pmode) {
        case kDecSoftmax: return launch_dec_route_pm<VPL, kDecSoftmax>(p, b, s);
        case 1: return launch_dec_route_pm<VPL, 1>(p, b, s);
        case 2: return launch_dec_route_pm<VPL, 2>(p, b, s);
        case 4: return launch_dec_route_pm<VPL, 4>(p, b, s);
        default: return launch_dec_route_pm<VPL, 0>(p, b, s);
    }
}

template <typename T, int D>
static hipError_t launch_decode_t(const DecodeParams& p, const DecodeArgs& a, hipStream_t s) {
    constexpr size_t lds = TileGeom<T, D, kDecTT>::BYTES + 64 * 12;   // + chunk, bias, first row
    static_assert(TileGeom<T, D, kDecTT>::BYTES >= kDecWaves * (32 * D + 64) * 4, "LDS merge space");
    static hipError_t configured = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_attn_kernel<T, D>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (configured != hipSuccess) return configured;
    if (p.T_route > 0) {
        dim3 g1((p.T_route + 63) / 64, p.h_kv, a.b);
        hipLaunchKernelGGL((decode_scores_kernel<D>), g1, dim3(256), 0, s, p, a.Q, a.in_bf16);
    }
    const hipError_t er = p.T_route <= 256 ? launch_dec_route<4>(p, a.b, s)
                        : p.T_route <= 1024 ? launch_dec_route<16>(p, a.b, s)
                                            : launch_dec_route<32>(p, a.b, s);
    if (er != hipSuccess) return er;
    hipLaunchKernelGGL((decode_attn_kernel<T, D>), dim3(p.max_slices, p.h_kv, a.b), dim3(kDecThreads), lds, s, p);
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(p.h_q, a.b), dim3(kCombThreads),
                       (size_t)p.max_slices * sizeof(float), s, p);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    DecodeParams p;
    p.Q = a.Q; p.Kc = a.Kc; p.Vc = a.Vc; p.kbar = a.kbar; p.seq_len = a.seq_len;
    p.h_q = a.h_q; p.h_kv = a.h_kv; p.L_cap = a.L_cap; p.kbar_cap = a.kbar_cap; p.B = a.B;
    p.g = a.h_q / a.h_kv;
    p.log2g = 0;
    while ((1 << p.log2g) < p.g) ++p.log2g;
    p.T_route = a.T_route; p.list_cap = a.list_cap; p.max_slices = a.max_slices;
    p.slice_tokens = a.slice_tokens;
    p.cs = route_scale(a.alpha, a.gamma, a.d);
    p.pexp = (float)(1.0 / ((double)a.alpha - 1.0));
    p.pmode = pmode_of(a.alpha);
    p.inv_sigma = isinf(a.sigma) ? 0.f : (float)(1.0 / (double)a.sigma);
    p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)a.d));
    p.out_bf16 = a.out_bf16;
    p.O = a.O; p.idx = a.idx; p.bias = a.bias; p.cnt = a.cnt; p.w_out = a.w_out;
    p.scores = a.scores; p.partials = a.partials;
    p.pages = a.pages; p.pages_per_seq = a.pages_per_seq; p.num_pages = a.num_pages;
    if (a.in_bf16) return a.d == 64 ? launch_decode_t<uint16_t, 64>(p, a, s) : launch_decode_t<uint16_t, 128>(p, a, s);
    return a.d == 64 ? launch_decode_t<float, 64>(p, a, s) : launch_decode_t<float, 128>(p, a, s);
}

}  // namespace dash
