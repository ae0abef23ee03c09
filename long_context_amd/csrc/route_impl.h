// Stage 1 of DashAttention for a prefill (paper review section 三, Eq. 6 and the
// GQA paragraph; μ and d from Proposition 4.1):
//   z̄_{i,c} = <q_i^(h), k̄_c^(r)>/sqrt(d) over the visible chunks c < floor(i/B),
//   ŵ^(h) = α-entmax(γ z̄^(h)) = [(α-1)γz̄ - τ]_+^{1/(α-1)},
//   w^(r) = mean over the g heads of group r of ŵ^(h), S = {c : w_c > 0},
//   μ = mean_{c in S} ln w_c, bias d_c = (ln w_c - μ)/σ.
//
// entmax_route_kernel: a group of CW wavefronts handles 16 (row, head) pairs = 16/g
// rows x all g heads of one KV group, so the GQA average is a reduction across lanes.
//  * Logits: MFMA with A = k̄ tile (16 chunks x d) and B = q (d x 16 pairs); lane
//    (kg, n) ends with chunks 16t+4kg+i of pair n. All visible chunks of a row stay in
//    registers: up to 512 per wavefront, rows with more chunks are split over CW = 2
//    or 4 wavefronts whose row maxima and Newton sums meet in LDS. The split is
//    interleaved by 16-chunk tile (wavefront cw takes tiles cw, cw + CW, ...). bf16
//    queries take the summaries from a buffer split into three bf16 terms: through an
//    LDS ring when one wavefront holds a row, straight from L2 when rows are split
//    (the ring's barriers across all wavefronts cost more than its sharing).
//  * Threshold: work on y = (α-1)γ(z̄ - max z̄) <= 0 (exact shift by the row maximum)
//    so τ lies in [-1, 0). Newton's method on g(τ) = ||[y - τ]_+||_p - 1 with
//    p = 1/(α-1), started at τ = -1 where g >= 0: g is convex and decreasing, so the
//    iterates increase monotonically to the root; uniform rows converge in one step.
//    Exponents p in {1, 2, 4} (α in {2, 1.5, 1.25}) use plain products, other α
//    use exp2/log2.
//  * GQA average with DPP row permutations (within 16-lane rows), then the group
//    weights go to LDS and each row is compacted with a ballot/prefix count into an
//    ascending chunk list with its bias.
//  * A wave64 VALU instruction takes four cycles on the 16-lane SIMD, and Newton and
//    the weights are bound by their instruction count: the row's tiles are visited in
//    groups of four with one uniform test per group, and the DPP levels of the group
//    average are tested once per level, not per value.
#pragma once

#include "common.h"
#include "kernels.h"

#include <math.h>

#include <algorithm>

namespace dash {

struct RouteParams {
    const void* Q; const float* kbar;
    const uint8_t* ksplit;  // bf16 queries: summaries split into bf16 (hi, mid, lo), staged layout
    int T_pad;              // chunks per (b, KV head) in ksplit: T_c rounded up to 32
    int32_t* idx; float* bias; int32_t* cnt; float* w_out;
    int h_q, h_kv, n, kbar_cap, list_cap, B, T_c, g, log2g, causal;
    float cs;           // (α-1) γ / sqrt(d)
    float pexp;         // 1/(α-1)
    int pmode;          // 1, 2, 4 for integer exponents, 0 otherwise, kSoftmaxRouting for α = 1
    float inv_sigma;    // 1/σ (0 for σ = inf)
    int top_k;          // > 0: keep only the top_k largest group weights of each row
    float* stats;       // nullable [b, h_q, n, 2]: max raw logit and the threshold
                        // (τ; α = 1: log2 Σ 2^y) of each (head, row)
    const int32_t* seq_len = nullptr;  // nullable: ragged batch, sequence b holds seq_len[b] rows
    int redo = 0;       // 1: route only the row groups the candidate kernel marked (cnt -1)
};

// Order-preserving map of a float to an unsigned key (larger float, larger key).
__device__ __forceinline__ uint32_t float_key(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Routing with α = 1: per-head softmax weights instead of entmax (every visible chunk
// is routed); p.cs then holds γ log2(e)/sqrt(d).
constexpr int kSoftmaxRouting = -1;

// Maximum over the lanes of a 16-lane row whose index differs only in the low `steps` bits.
__device__ __forceinline__ float row_group_max(float v, int steps) {
    if (steps > 0) v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    if (steps > 1) v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    if (steps > 2) v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
    if (steps > 3) v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
    return v;
}

// Sum over the lanes of a 16-lane row whose index differs only in the low `steps` bits.
__device__ __forceinline__ float row_group_sum(float v, int steps) {
    if (steps > 0) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)); // xor 1
    if (steps > 1) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)); // xor 2
    if (steps > 2) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)); // half-row mirror
    if (steps > 3) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)); // row mirror
    return v;
}

// [y - τ]_+ for y <= 0 and τ >= -1, where y - τ <= 1: a clamp to [0, 1], which the
// compiler folds into the subtraction (one instruction instead of two).
__device__ __forceinline__ float pos_part(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 1.f); }

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

// Tiles of a row are visited in groups of four, one uniform branch per group: a tile
// at or past nt holds y = -inf, so [y - τ]_+ = 0 and it adds exact zeros to every sum
// below. (One branch per tile made the compiler keep 32 loop-invariant conditions live
// across the Newton loop, spilling them and re-testing each through vector registers.)
template <int NT> constexpr int tile_group() { return NT < 4 ? NT : 4; }

// The (wavefront-uniform) tile count laundered through an empty asm statement, so that
// the group tests are evaluated where they stand instead of being hoisted out of the
// enclosing loop.
__device__ __forceinline__ int fresh_count(int nt) {
    nt = __builtin_amdgcn_readfirstlane(nt);
    asm volatile("" : "+s"(nt));
    return nt;
}

// Newton sums a0 = sum t^{p-1}, a1 = sum t^p over the lane's chunks, t = [y - τ]_+.
template <int NT, int PM>
__device__ __forceinline__ void newton_sums(const float (&sv)[NT][4], int nt, float tau, float pexp,
                                            float& a0, float& a1) {
    constexpr int TG = tile_group<NT>();
    const int ntl = fresh_count(nt);
#pragma unroll
    for (int t4 = 0; t4 < NT; t4 += TG) {
        if (t4 < ntl) {
#pragma unroll
            for (int t = t4; t < t4 + TG; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) accum_pow<PM>(pos_part(sv[t][i] - tau), pexp, a0, a1);
        }
    }
}

// Newton iterations on the wave's 16 pairs; sv holds y (-inf on invalid chunks).
template <int NT, int PM>
__device__ __forceinline__ float solve_tau(float (&sv)[NT][4], int nt, float pexp, bool active) {
    float tau = -1.f;
    bool done = !active;
    for (int it = 0; it < 100; ++it) {
        float a0 = 0.f, a1 = 0.f;
        newton_sums<NT, PM>(sv, nt, tau, pexp, a0, a1);
        a0 = pair32_sum(pair16_sum(a0));
        a1 = pair32_sum(pair16_sum(a1));
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

// Group weights w_c = (1/g) sum_h ŵ_hc of the lane's chunks in place of y: the per-head
// weights first, then the sum over the g = 2^lg lanes of each row one DPP level at a
// time over all chunks (the additions row_group_sum makes per value, in its order), so
// each level is tested once instead of once per value.
template <int CTRL, int NT>
__device__ __forceinline__ void dpp_level(float (&sv)[NT][4], int nt) {
    constexpr int TG = tile_group<NT>();
    const int ntl = fresh_count(nt);
#pragma unroll
    for (int t4 = 0; t4 < NT; t4 += TG) {
        if (t4 < ntl) {
#pragma unroll
            for (int t = t4; t < t4 + TG; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sv[t][i] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sv[t][i]), CTRL, 0xF, 0xF, false));
        }
    }
}
template <int NT, int PM>
__device__ __forceinline__ void group_weights(float (&sv)[NT][4], int nt, float tau, float pexp, bool row_ok,
                                              int lg, float inv_g) {
    constexpr int TG = tile_group<NT>();
    {
        const int ntl = fresh_count(nt);
#pragma unroll
        for (int t4 = 0; t4 < NT; t4 += TG) {
            if (t4 < ntl) {
#pragma unroll
                for (int t = t4; t < t4 + TG; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float wv = pow_p<PM>(pos_part(sv[t][i] - tau), pexp);
                        sv[t][i] = row_ok ? wv : 0.f;
                    }
            }
        }
    }
    if (lg > 0) dpp_level<0xB1>(sv, nt);     // xor 1
    if (lg > 1) dpp_level<0x4E>(sv, nt);     // xor 2
    if (lg > 2) dpp_level<0x141>(sv, nt);    // half-row mirror
    if (lg > 3) dpp_level<0x140>(sv, nt);    // row mirror
    const int ntl = fresh_count(nt);
#pragma unroll
    for (int t4 = 0; t4 < NT; t4 += TG) {
#pragma unroll
        for (int t = t4; t < t4 + TG; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[t][i] = t4 < ntl ? sv[t][i] * inv_g : 0.f;
    }
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

// Shared summaries of one stage (CH chunks) for bf16 queries: per chunk three rows
// (hi, mid, lo) of D bf16, i.e. 3*D/8 16-byte pieces; piece c of split h sits at
// h*(D/8) + (c ^ (chunk mod D/8)) so that the 16 lanes reading 16 consecutive chunks
// at one column hit distinct banks.
template <int D, int CH_>
struct KSplitStage {
    static constexpr int CH = CH_;                    // chunks per stage
    static constexpr int PPS = D / 8;                 // pieces per split row
    static constexpr int ROWB = 3 * D * 2;            // bytes per chunk
    static constexpr int BYTES = CH * ROWB;
    static constexpr int PIECES = CH * PPS;           // fp32 groups of 8 to split per stage
    __device__ __forceinline__ static int off(int c, int h, int piece) {
        return c * ROWB + (h * PPS + (piece ^ (c & (PPS - 1)))) * 16;
    }
};

// k̄ [b, h_kv, kbar_cap, D] fp32 -> ksplit [b, h_kv, T_pad] chunks of three bf16
// rows (hi, mid, lo; hi + mid + lo reproduces k̄ to the last bits of fp32) in the
// swizzled order of KSplitStage, so that a stage is one contiguous block that the
// routing kernel copies to LDS as is. Chunks T_c .. T_pad-1 are zero.
template <int D>
__global__ __launch_bounds__(256) void ksplit_kernel(const float* kbar, uint8_t* ksplit, int kbar_cap, int T_c,
                                                     int T_pad) {
    typedef KSplitStage<D, 32> KS;
    typedef __bf16 b8 __attribute__((ext_vector_type(8)));
    const int q = blockIdx.x * 256 + threadIdx.x;
    const int c = q / KS::PPS, pc = q % KS::PPS;
    if (c >= T_pad) return;
    const size_t bh = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
    f32x4 lo4 = {0.f, 0.f, 0.f, 0.f}, hi4 = {0.f, 0.f, 0.f, 0.f};
    if (c < T_c) {
        const f32x4* src = reinterpret_cast<const f32x4*>(kbar + (bh * kbar_cap + c) * D + pc * 8);
        lo4 = src[0];
        hi4 = src[1];
    }
    b8 hv, mv, lv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = e < 4 ? lo4[e] : hi4[e - 4];
        const __bf16 h = (__bf16)x;
        const float r1 = x - (float)h;
        const __bf16 m = (__bf16)r1;
        hv[e] = h; mv[e] = m; lv[e] = (__bf16)(r1 - (float)m);
    }
    uint8_t* dst = ksplit + bh * (size_t)T_pad * KS::ROWB;
    *reinterpret_cast<b8*>(dst + KS::off(c, 0, pc)) = hv;
    *reinterpret_cast<b8*>(dst + KS::off(c, 1, pc)) = mv;
    *reinterpret_cast<b8*>(dst + KS::off(c, 2, pc)) = lv;
}

// s_waitcnt vmcnt(n) for the counts the summary ring needs (larger counts wait for
// everything, which is always safe)
__device__ __forceinline__ void wait_vm_at_most(int n) {
    switch (n) {
        case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
        case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
        case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
        case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}

// Stages of the summary ring in LDS: three when a row can need many stages, so the
// copies run two stages ahead; two for rows of up to 512 chunks in one wavefront, whose
// workgroups are halved so that two share a compute unit (one streams summaries while
// the other solves τ; at 32K, 0.77 -> 0.72 ms against one workgroup with three stages).
template <int NT, int CW> constexpr int route_ring_stages() {
    return (NT >= 32 && CW == 1) ? 2 : NT * CW / 2 >= 4 ? 3 : 2;
}
template <typename T, int NT, int CW> constexpr int route_max_groups() {
    return (sizeof(T) == 2 && NT >= 32 && CW == 1) ? 4 : 8 / CW;
}
// bf16 queries stream the split summaries through an LDS ring when one wavefront
// holds a whole row; rows split over several wavefronts read them from L2.
template <typename T, int CW> constexpr bool route_uses_ring() { return sizeof(T) == 2 && CW == 1; }

// τ for rows whose chunks are split over CW cooperating wavefronts: every iteration
// each wavefront sums its own chunks, the CW partial sums meet in LDS (double
// buffered by iteration parity) and are added in a fixed order, so the CW wavefronts
// of a row group take identical steps. The loop runs until every row of the
// workgroup has converged (all wavefronts pass the same barriers).
template <int NT, int PM, int CW>
__device__ __forceinline__ float solve_tau_split(float (&sv)[NT][4], int nt, float pexp, bool active,
                                                 float* xsum, int G, int gid, int cw, int n16, int kg) {
    float tau = -1.f;
    bool done = !active;
    for (int it = 0; it < 100; ++it) {
        float a0 = 0.f, a1 = 0.f;
        newton_sums<NT, PM>(sv, nt, tau, pexp, a0, a1);
        a0 = pair32_sum(pair16_sum(a0));
        a1 = pair32_sum(pair16_sum(a1));
        float* buf = xsum + ((size_t)((it & 1) * G + gid) * CW) * 32;   // [CW][16][2]
        if (kg == 0) { buf[(cw * 16 + n16) * 2] = a0; buf[(cw * 16 + n16) * 2 + 1] = a1; }
        __syncthreads();
        a0 = 0.f; a1 = 0.f;
#pragma unroll
        for (int k = 0; k < CW; ++k) { a0 += buf[(k * 16 + n16) * 2]; a1 += buf[(k * 16 + n16) * 2 + 1]; }
        float delta;
        if (PM == 1) {
            delta = (a1 - 1.f) / a0;
        } else {
            float nrm = (PM == 2) ? sqrtf(a1) : (PM == 4) ? sqrtf(sqrtf(a1)) : fast_exp2(fast_log2(a1) / pexp);
            delta = (nrm - 1.f) * (a1 / nrm) / a0;
        }
        if (!(a0 > 0.f)) delta = 0.f;
        if (!done) tau += delta;
        done = done || !(fabsf(delta) > 1e-6f);
        if (!__syncthreads_or(!done)) break;
    }
    return tau;
}

// Chunk layout of a row over the CW wavefronts of its group: 16-chunk tile j of the
// row belongs to wavefront j % CW as its local tile j / CW.
template <int CW> struct RouteSplit {
    __device__ __forceinline__ static int tile_chunk(int t, int cw) { return 16 * (t * CW + cw); }
    // local tiles of wavefront cw that start below nvis
    __device__ __forceinline__ static int tiles_below(int nvis, int cw) {
        const int rest = (nvis + 15) / 16 - cw;
        return rest > 0 ? (rest + CW - 1) / CW : 0;
    }
};

// Compaction of the rows row0 .. row0+R-1 of one row group by one wavefront: the
// group weights of row j are wl[j * WS + c] (α = 1: log2 w) for the visible chunks
// c < nvis. Writes ascending chunk ids of the support with d = (ln w - μ)/σ, the
// counts and (optionally) the dense weights. With a top-k budget the support keeps
// its top_k largest weights (ties to the lower chunk): the k-th largest key is found
// by bisection on the key bits, counted with ballots over the row. NK >= WS/64.
template <bool SOFT, int NK>
__device__ __forceinline__ void route_compact(const RouteParams& p, const float* wl, int WS, int R, int row0, int nb,
                                              int nvis, int bi, int r, int lane) {
    const size_t rowbase = ((size_t)bi * p.h_kv + r) * p.n;
    for (int j = 0; j < R; ++j) {
        const int row = row0 + j;
        if (row >= p.n) break;
        if (row >= nb) {                              // a padding row of a ragged batch
            if (lane == 0) p.cnt[rowbase + row] = 0;
            continue;
        }
        const float* wr = wl + j * WS;
        auto cand = [&](int c, float v) { return c < nvis && (SOFT || v > 0.f); };
        bool limit = false;
        uint32_t kstar = 0;
        int need_eq = 0;
        if (p.top_k > 0) {
            uint32_t key[NK];
            int ncand = 0;
#pragma unroll
            for (int q = 0; q < NK; ++q) {
                const int c = lane + 64 * q;
                const float v = c < nvis ? wr[c] : 0.f;
                const bool in = cand(c, v);
                key[q] = in ? float_key(v) : 0u;
                ncand += __builtin_popcountll(ballot(in));
            }
            if (ncand > p.top_k) {                    // wavefront-uniform
                limit = true;
                uint32_t prefix = 0;
                for (int bit = 31; bit >= 0; --bit) {
                    const uint32_t trial = prefix | (1u << bit);
                    int cnt = 0;
#pragma unroll
                    for (int q = 0; q < NK; ++q) cnt += __builtin_popcountll(ballot(key[q] >= trial));
                    if (cnt >= p.top_k) prefix = trial;
                }
                kstar = prefix;
                int gt = 0;
#pragma unroll
                for (int q = 0; q < NK; ++q) gt += __builtin_popcountll(ballot(key[q] > kstar));
                need_eq = p.top_k - gt;
            }
        }
        // membership of chunk c (value v) given the running count of earlier ties
        auto selected = [&](int c, float v, int& eq_before) {
            const bool in = cand(c, v);
            if (!limit) return in;
            const uint32_t k = in ? float_key(v) : 0u;
            const uint64_t eq = ballot(in && k == kstar);
            const int rank = eq_before + __builtin_popcountll(eq & ((1ull << lane) - 1ull));
            eq_before += __builtin_popcountll(eq);
            return in && (k > kstar || (k == kstar && rank < need_eq));
        };
        float sl = 0.f, sc = 0.f;
        int eqb = 0;
        for (int c0 = 0; c0 < nvis; c0 += 64) {
            const int c = c0 + lane;
            const float v = c < nvis ? wr[c] : 0.f;
            if (selected(c, v, eqb)) { sl += SOFT ? v : fast_log2(v); sc += 1.f; }
        }
        sl = wave_sum(sl);
        sc = wave_sum(sc);
        const float mu2 = sc > 0.f ? sl / sc : 0.f;            // μ in log2 units
        const float bscale = kLn2 * p.inv_sigma;
        int32_t* idx = p.idx + (rowbase + row) * (size_t)p.list_cap;
        float* bias = p.bias + (rowbase + row) * (size_t)p.list_cap;
        float* wo = p.w_out ? p.w_out + (rowbase + row) * (size_t)p.kbar_cap : nullptr;
        int base = 0;
        eqb = 0;
        // chunks past the visible ones are never routed: walk them only to write the
        // dense weights
        const int cend = wo ? p.T_c : nvis;
        for (int c0 = 0; c0 < cend; c0 += 64) {
            const int c = c0 + lane;
            const float v = (c < nvis) ? wr[c] : (SOFT ? -INFINITY : 0.f);
            const bool in = selected(c, v, eqb);
            const uint64_t m = ballot(in);
            const int pre = __builtin_popcountll(m & ((1ull << lane) - 1ull));
            if (in) {
                idx[base + pre] = c;
                bias[base + pre] = p.inv_sigma == 0.f ? 0.f : bscale * ((SOFT ? v : fast_log2(v)) - mu2);
            }
            if (wo && c < p.T_c) wo[c] = SOFT ? fast_exp2(v) : v;
            base += __builtin_popcountll(m);
        }
        if (lane == 0) p.cnt[rowbase + row] = base;
    }
}

// One workgroup = G groups of 16 (row, head) pairs (16/g rows x the g heads of a
// group each) times CW wavefronts per group; each wavefront holds NT tiles of its
// rows' chunks in registers (CW > 1 for long rows).
template <typename T, int D, int NT, int PM, int CW>
__global__ __launch_bounds__(512) void entmax_route_kernel(RouteParams p) {
    constexpr int WSW = NT * 16;                      // chunks held by one wavefront
    constexpr int WS = CW * WSW;                      // LDS floats per row of weights
    typedef RouteSplit<CW> RS;
    typedef KSplitStage<D, 32> KS;
    typedef __bf16 b8 __attribute__((ext_vector_type(8)));
    extern __shared__ __attribute__((aligned(16))) char rsm[];
    const int W = blockDim.x >> 6;
    const int G = W / CW;
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int gid = wid / CW, cw = wid % CW;
    const int n16 = lane & 15, kg = lane >> 4;
    const int g = p.g, lg = p.log2g;
    const int R = 16 >> lg;                           // rows per group
    const int r = blockIdx.y, bi = blockIdx.z;
    // all rows of the workgroup lie in one chunk (G*R divides B): one visible range
    const int wg_row0 = blockIdx.x * G * R;
    const int row0 = wg_row0 + gid * R;
    // ragged batch: the sequence's own tokens and complete chunks
    const int nb = p.seq_len ? min(max(p.seq_len[bi], 0), p.n) : p.n;
    const int Tb = nb / p.B;
    // second pass after the candidate router: only the row groups it marked (count -1)
    // are routed here; a workgroup without one leaves at once (before any barrier)
    bool marked = true;
    if (p.redo) {
        marked = row0 < nb && p.cnt[((size_t)bi * p.h_kv + r) * p.n + row0] == -1;
        if (!__syncthreads_or(marked)) return;
    }
    const bool wave_live = row0 < p.n && marked;
    constexpr int RSTG = route_ring_stages<NT, CW>();
    constexpr bool RING = route_uses_ring<T, CW>();
    char* kstage = rsm;                                              // RSTG stages (ring only)
    float* wl_all = reinterpret_cast<float*>(rsm + (RING ? RSTG * KS::BYTES : 0));
    float* wl = wl_all + gid * R * WS;
    float* xred = wl_all + G * R * WS;                // [G][CW][16] row maxima of each wavefront
    float* xsum = xred + G * CW * 16;                 // [2][G][CW][16][2] Newton partial sums
    const int nvis = p.causal ? min(wg_row0 / p.B, Tb) : Tb;
    const int my_row = row0 + (n16 >> lg);
    const int my_head = r * g + (n16 & (g - 1));
    const bool row_ok = my_row < nb;
    const int nt = min(RS::tiles_below(nvis, cw), NT);   // tiles holding visible chunks

    float sv[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[t][i] = -INFINITY;
    if (nvis > 0) {                                   // workgroup-uniform
        float smax = -INFINITY;
        if constexpr (sizeof(T) == 2) {
            // bf16 queries are exact in bf16; k̄ = hi + mid + lo (three bf16 terms, exact up
            // to the last bits of fp32), so every product is exact in fp32 and three bf16
            // MFMAs 16x16x32 per k step reproduce the fp32 dot product; the three partial
            // sums are kept apart and added once. k-slot (kg, e) of step s carries
            // dimension 32s + 8kg + e for both operands.
            b8 qb[D / 32];
            {
                const T* qrow = static_cast<const T*>(p.Q) +
                    (((size_t)bi * p.h_q + my_head) * p.n + (row_ok ? my_row : 0)) * D + 8 * kg;
#pragma unroll
                for (int s = 0; s < D / 32; ++s) {
                    qb[s] = *reinterpret_cast<const b8*>(qrow + 32 * s);
                    if (!row_ok) qb[s] = b8{};
                }
            }
            // stages of 32 split summaries (chunks 32st .. 32st+31 = row tiles 2st and
            // 2st+1) reach LDS by asynchronous copies from the split buffer, RSTG-1
            // stages ahead; every wavefront issues the same number of copies per stage
            const int nst = (nvis + KS::CH - 1) / KS::CH;
            constexpr int CPI = KS::BYTES / 1024;    // 1 KiB copy instructions per stage
            const int cps = (CPI + W - 1) / W;         // per wavefront (some duplicated)
            const uint8_t* ksrc = p.ksplit + ((size_t)bi * p.h_kv + r) * (size_t)p.T_pad * KS::ROWB;
            auto issue = [&](int st) {                 // st may pass nst: a copy of the last
                char* dst = kstage + (st % RSTG) * KS::BYTES;   // stage into a free slot
                const uint8_t* src = ksrc + (size_t)min(st, nst - 1) * KS::BYTES + lane * 16;
                for (int i = 0; i < cps; ++i) {
                    int j = wid + i * W;
                    if (j >= CPI) j -= CPI;
                    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(src + j * 1024),
                                                     reinterpret_cast<uint32_t*>(dst + j * 1024), 16, 0, 0);
                }
            };
            // stage st is complete once at most the (RSTG-2) newer stages' copies are
            // outstanding; the barrier then also frees the slot of stage st-1, which
            // the copies of stage st+RSTG-1 fill
            auto enter_stage = [&](int st) {
                wait_vm_at_most((RSTG - 2) * cps);
                __syncthreads();
                issue(st + RSTG - 1);
            };
            // logits of local tile t (a compile-time index once inlined) from stage
            // tile tt: A = 16 summaries x D (three bf16 splits), B = the 16 pairs' q
            auto tile_logits = [&](const char* stg, int tt, int t) {
                const int cl = 16 * tt + n16;         // chunk inside the stage
                f32x4 acc[3];
#pragma unroll
                for (int h = 0; h < 3; ++h) {
                    acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < D / 32; ++s) {
                        const b8 a = *reinterpret_cast<const b8*>(stg + KS::off(cl, h, 4 * s + kg));
                        acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[s], acc[h], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ch = RS::tile_chunk(t, cw) + 4 * kg + i;
                    const float v = acc[0][i] + (acc[1][i] + acc[2][i]);
                    sv[t][i] = (ch < nvis) ? v : -INFINITY;
                    smax = fmaxf(smax, sv[t][i]);
                }
            };
            if constexpr (RING) {
#pragma unroll
                for (int j = 0; j < RSTG - 1; ++j) issue(j);
                // stage st holds local tiles 2st and 2st+1 of the single wavefront
#pragma unroll
                for (int st = 0; st < NT / 2; ++st) {
                    if (st < nst) {                   // workgroup-uniform
                        enter_stage(st);
                        const char* stg = kstage + (st % RSTG) * KS::BYTES;
#pragma unroll
                        for (int tt = 0; tt < 2; ++tt)
                            if (2 * st + tt < nt) tile_logits(stg, tt, 2 * st + tt);
                    }
                }
            } else {
                // rows split over CW wavefronts: each wavefront reads its own tiles of
                // the split buffer straight from L2 (a shared ring's per-stage barriers
                // across all wavefronts cost more than its sharing saves here)
                const char* kglob = reinterpret_cast<const char*>(ksrc);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    if (t < nt) {
                        const int c0 = RS::tile_chunk(t, cw);
                        tile_logits(kglob + (size_t)(c0 >> 5) * KS::BYTES, (c0 >> 4) & 1, t);
                    }
                }
            }
            // no copy may still be landing in LDS when the workgroup ends
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        } else {
            // fp32 queries: the MFMA k-slot kg of step (s, j) carries dimension 16s + 4kg + j
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
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (t < nt) {
                    const int c = min(RS::tile_chunk(t, cw) + n16, nvis - 1);   // A row = chunk
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
                        const int ch = RS::tile_chunk(t, cw) + 4 * kg + i;
                        sv[t][i] = (ch < nvis) ? acc[i] : -INFINITY;
                        smax = fmaxf(smax, sv[t][i]);
                    }
                }
            }
        }
        smax = pair32_max(pair16_max(smax));
        if constexpr (CW > 1) {
            if (kg == 0) xred[(gid * CW + cw) * 16 + n16] = smax;
            __syncthreads();
            smax = -INFINITY;
#pragma unroll
            for (int k = 0; k < CW; ++k) smax = fmaxf(smax, xred[(gid * CW + k) * 16 + n16]);
        }
        // thresholded argument shifted by the row maximum: y = (α-1)γ(z̄ - max z̄) <= 0
        // (α = 1: y = γ log2(e)(z̄ - max z̄))
#pragma unroll
        for (int t = 0; t < NT; ++t)
            if (t < nt) {                             // later tiles are never read
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[t][i] = p.cs * (sv[t][i] - smax);
            }

        if constexpr (PM == kSoftmaxRouting) {
            // per-head softmax in log2 units, log2 ŵ = y - log2 Σ 2^y, then the group
            // weight log2 w = log2((1/g) Σ_h ŵ_h) taken stably across the g lanes
            float se = 0.f;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                if (t < nt) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) se += fast_exp2(sv[t][i]);
                }
            se = pair32_sum(pair16_sum(se));
            if constexpr (CW > 1) {
                float* buf = xsum + ((size_t)gid * CW) * 32;
                if (kg == 0) buf[(cw * 16 + n16) * 2] = se;
                __syncthreads();
                se = 0.f;
#pragma unroll
                for (int k = 0; k < CW; ++k) se += buf[(k * 16 + n16) * 2];
            }
            const float lse = fast_log2(se);
            if (p.stats && kg == 0 && cw == 0 && wave_live && row_ok) {
                float* so = p.stats + 2 * (((size_t)bi * p.h_q + my_head) * p.n + my_row);
                so[0] = smax;
                so[1] = lse;
            }
            const float lg_g = (float)lg;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (t < nt) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float lw = sv[t][i] - lse;
                        const float m = row_group_max(lw, lg);
                        const float sm = row_group_sum(m == -INFINITY ? 0.f : fast_exp2(lw - m), lg);
                        sv[t][i] = m == -INFINITY ? -INFINITY : m + fast_log2(sm) - lg_g;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) sv[t][i] = -INFINITY;
                }
            }
        } else {
        float tau;
        if constexpr (CW == 1) tau = solve_tau<NT, PM>(sv, nt, p.pexp, row_ok && wave_live);
        else tau = solve_tau_split<NT, PM, CW>(sv, nt, p.pexp, row_ok && wave_live, xsum, G, gid, cw, n16, kg);
        if (p.stats && kg == 0 && cw == 0 && wave_live && row_ok) {
            float* so = p.stats + 2 * (((size_t)bi * p.h_q + my_head) * p.n + my_row);
            so[0] = smax;
            so[1] = tau;
        }
        // per-head weights, then the group average across the g lanes of each row
        group_weights<NT, PM>(sv, nt, tau, p.pexp, row_ok, lg, 1.f / (float)g);
        }
    } else {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[t][i] = 0.f;
    }
    // group weights to LDS: the first lane of each row writes its chunks
    if (wave_live && (n16 & (g - 1)) == 0) {
        float* wr = wl + (n16 >> lg) * WS;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) wr[RS::tile_chunk(t, cw) + 4 * kg + i] = sv[t][i];
    }
    if constexpr (CW > 1) {
        __syncthreads();                              // the rows' chunks come from CW wavefronts
        if (cw != 0) return;
    } else {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (!wave_live) return;                           // no barrier follows

    // compaction: ascending chunk ids of the support, with d = (ln w - μ)/σ (with
    // α = 1 the LDS holds log2 w and every visible chunk is in the support). With a
    // top-k budget the support keeps its top_k largest weights (ties to the lower
    // chunk): the k-th largest key is found by bisection on the key bits, counted
    // with ballots over the row.
    constexpr bool SOFT = PM == kSoftmaxRouting;
    route_compact<SOFT, (WS + 63) / 64>(p, wl, WS, R, row0, nb, nvis, bi, r, lane);
}

// ---------------------------------------------------------------------------------
// Candidate router for long rows (bf16 queries, α > 1): the same routing as
// entmax_route_kernel, without keeping a row's logits in registers.
//  * One wavefront per group of 16 (row, head) pairs; the W groups of a workgroup
//    share one stream of split summaries through the LDS ring, so a workgroup reads
//    the summaries once for W·16/g rows.
//  * While the logits stream by, a lane keeps in LDS only its chunks whose logit can
//    still reach the support: since τ >= -1 on y = cs(z̄ - max z̄), a chunk with
//    z̄ <= max - 1/cs never enters it, and the lane's running maximum is a lower
//    bound of the row maximum. When a lane's list fills up, Newton's iterate on the
//    kept chunks gives a lower bound θ of the threshold (the root of a sum over fewer
//    terms lies left of the full root), and chunks below θ are dropped.
//  * The kept chunks then give τ (Newton from the left, as in the register kernel),
//    the group weights w_c = mean_h ŵ_hc are summed into an LDS row by LDS atomic
//    adds issued in a fixed order by one wavefront, and the rows are compacted by
//    route_compact. A group whose lists overflow writes count -1 on its rows, and a
//    second launch of entmax_route_kernel (redo) routes those rows.
constexpr int kCandCap = 24;            // kept chunks per lane
constexpr float kCandMargin = 1.0f / 1024.0f;  // slack on every bound, in units of y

template <int PM>
__device__ __forceinline__ float cand_newton(const float (&cv)[kCandCap], int n, float m, float cs, float pexp,
                                             bool active, float tau, int max_it = 100) {
    bool done = !active;
    for (int it = 0; it < max_it; ++it) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int j = 0; j < kCandCap; ++j)
            if (j < n) accum_pow<PM>(pos_part(cs * (cv[j] - m) - tau), pexp, a0, a1);
        a0 = pair32_sum(pair16_sum(a0));
        a1 = pair32_sum(pair16_sum(a1));
        float delta;
        if (PM == 1) {
            delta = (a1 - 1.f) / a0;
        } else {
            const float nrm = (PM == 2) ? sqrtf(a1) : (PM == 4) ? sqrtf(sqrtf(a1)) : fast_exp2(fast_log2(a1) / pexp);
            delta = (nrm - 1.f) * (a1 / nrm) / a0;
        }
        if (!(a0 > 0.f)) delta = 0.f;
        if (!done) tau += delta;
        done = done || !(fabsf(delta) > 1e-6f);
        if (ballot(!done) == 0) break;
    }
    return tau;
}

template <int D> constexpr int cand_ring_stages() { return 3; }

template <int D, int PM, int TB>
__global__ __launch_bounds__(512) void entmax_route_cand_kernel(RouteParams p) {
    typedef KSplitStage<D, 32> KS;
    typedef __bf16 b8 __attribute__((ext_vector_type(8)));
    constexpr int RSTG = cand_ring_stages<D>();
    constexpr int CAP = kCandCap;
    extern __shared__ __attribute__((aligned(16))) char rsm[];
    const int W = blockDim.x >> 6;
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n16 = lane & 15, kg = lane >> 4;
    const int g = p.g, lg = p.log2g;
    const int R = 16 >> lg;
    const int r = blockIdx.y, bi = blockIdx.z;
    const int wg_row0 = blockIdx.x * W * R;
    const int row0 = wg_row0 + wid * R;
    const bool wave_live = row0 < p.n;
    const int nb = p.seq_len ? min(max(p.seq_len[bi], 0), p.n) : p.n;
    const int Tb = nb / p.B;
    const int nvis = p.causal ? min(wg_row0 / p.B, Tb) : Tb;
    const int my_row = row0 + (n16 >> lg);
    const int my_head = r * g + (n16 & (g - 1));
    const bool row_ok = wave_live && my_row < nb;
    // LDS: the summary ring, later the rows' weights; then the lanes' kept chunks
    const size_t region = max((size_t)RSTG * KS::BYTES, (size_t)W * R * TB * 4);
    char* kstage = rsm;
    float* cval = reinterpret_cast<float*>(rsm + region);               // [W][CAP][64]
    uint16_t* cidx = reinterpret_cast<uint16_t*>(cval + (size_t)W * CAP * 64);   // [W][CAP][64]
    auto slot = [&](int j) { return ((size_t)wid * CAP + j) * 64 + lane; };

    const float cs = p.cs, inv_cs = 1.f / p.cs;
    float mlane = -INFINITY;     // the lane's running maximum of z̄
    float theta = -INFINITY;     // lower bound of the threshold on z̄ (the same in a pair's lanes)
    int ncand = 0;
    bool ovf = false;

    if (nvis > 0) {                                   // workgroup-uniform
        b8 qb[D / 32];
        {
            const uint16_t* qrow = static_cast<const uint16_t*>(p.Q) +
                (((size_t)bi * p.h_q + my_head) * p.n + (row_ok ? my_row : 0)) * D + 8 * kg;
#pragma unroll
            for (int s = 0; s < D / 32; ++s) {
                qb[s] = *reinterpret_cast<const b8*>(qrow + 32 * s);
                if (!row_ok) qb[s] = b8{};
            }
        }
        const int nst = (nvis + KS::CH - 1) / KS::CH;
        constexpr int CPI = KS::BYTES / 1024;
        const int cps = (CPI + W - 1) / W;
        const uint8_t* ksrc = p.ksplit + ((size_t)bi * p.h_kv + r) * (size_t)p.T_pad * KS::ROWB;
        // the lane's A-operand offsets inside a stage, the same for every stage
        int aoff[2][3][D / 32];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int h = 0; h < 3; ++h)
#pragma unroll
                for (int s = 0; s < D / 32; ++s) aoff[tt][h][s] = KS::off(16 * tt + n16, h, 4 * s + kg);
        auto issue = [&](int st) {
            char* dst = kstage + (st % RSTG) * KS::BYTES;
            const uint8_t* src = ksrc + (size_t)min(st, nst - 1) * KS::BYTES + lane * 16;
            for (int i = 0; i < cps; ++i) {
                int j = wid + i * W;
                if (j >= CPI) j -= CPI;
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(src + j * 1024),
                                                 reinterpret_cast<uint32_t*>(dst + j * 1024), 16, 0, 0);
            }
        };
        // drop the kept chunks below the bound that Newton's iterate on them gives
        auto prune = [&]() {
            float cv[CAP];
#pragma unroll
            for (int j = 0; j < CAP; ++j) cv[j] = j < ncand ? cval[slot(j)] : -INFINITY;
            const float m = pair32_max(pair16_max(mlane));
            // θ is below the root over the kept chunks (their set only grew above θ),
            // so Newton may start there. Every iterate from the left is a lower bound of
            // that root, so two steps suffice for a bound: at 96K they take the routing
            // from 9.4 / 7.7 / 5.9 to 8.2 / 7.0 / 5.8 ms at 75 / 87.5 / 93.75% group
            // sparsity (one step: the same; three: 8.6 / 7.3 / 5.8)
            const float tau0 = fmaxf(-1.f, cs * (theta - m));
            const float tau = cand_newton<PM>(cv, ncand, m, cs, p.pexp, row_ok && m > -INFINITY, tau0, 2);
            if (row_ok && m > -INFINITY) theta = fmaxf(theta, m + (tau - kCandMargin) * inv_cs);
            int k = 0;
#pragma unroll
            for (int j = 0; j < CAP; ++j) {
                if (j < ncand && cv[j] > theta) {
                    const uint16_t c = cidx[slot(j)];
                    cval[slot(k)] = cv[j];
                    cidx[slot(k)] = c;
                    ++k;
                }
            }
            ncand = k;
        };
        for (int j = 0; j < RSTG - 1; ++j) issue(j);
        for (int st = 0; st < nst; ++st) {
            wait_vm_at_most((RSTG - 2) * cps);
            __syncthreads();
            issue(st + RSTG - 1);
            const char* stg = kstage + (st % RSTG) * KS::BYTES;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int cb = KS::CH * st + 16 * tt;
                if (cb < nvis) {                      // workgroup-uniform
                    f32x4 acc[3];
#pragma unroll
                    for (int h = 0; h < 3; ++h) {
                        acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s = 0; s < D / 32; ++s) {
                            const b8 a = *reinterpret_cast<const b8*>(stg + aoff[tt][h][s]);
                            acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[s], acc[h], 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int c = cb + 4 * kg + i;
                        const float x = acc[0][i] + (acc[1][i] + acc[2][i]);
                        const bool valid = row_ok && c < nvis;
                        if (valid) mlane = fmaxf(mlane, x);
                        const float lim = fmaxf(theta, mlane - (1.f + kCandMargin) * inv_cs);
                        if (valid && x > lim) {
                            if (ncand < CAP) {
                                cval[slot(ncand)] = x;
                                cidx[slot(ncand)] = (uint16_t)c;
                                ++ncand;
                            } else {
                                ovf = true;
                            }
                        }
                    }
                }
            }
            // the pair's lanes share their maxima: a tighter bound for the next stage
            mlane = pair32_max(pair16_max(mlane));
            if (ballot(ncand > CAP - 8) != 0) prune();
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();                                  // the ring is free: it holds the weights now
    if (!wave_live) return;                           // no barrier follows
    const size_t rowbase = ((size_t)bi * p.h_kv + r) * p.n;
    if (ballot(ovf) != 0) {
        // this group's lists overflowed: its rows are routed by the second pass
        if (lane < R && row0 + lane < nb) p.cnt[rowbase + row0 + lane] = -1;
        else if (lane < R && row0 + lane < p.n) p.cnt[rowbase + row0 + lane] = 0;
        return;
    }
    float cv[CAP];
    int cc[CAP];
#pragma unroll
    for (int j = 0; j < CAP; ++j) {
        cv[j] = j < ncand ? cval[slot(j)] : -INFINITY;
        cc[j] = j < ncand ? cidx[slot(j)] : 0;
    }
    const float m = pair32_max(pair16_max(mlane));
    const bool active = row_ok && m > -INFINITY;
    const float tau = cand_newton<PM>(cv, ncand, m, cs, p.pexp, active, fmaxf(-1.f, cs * (theta - m)));
    if (p.stats && kg == 0 && row_ok) {
        float* so = p.stats + 2 * (((size_t)bi * p.h_q + my_head) * p.n + my_row);
        so[0] = m;
        so[1] = tau;
    }
    // group weights: zero the rows' visible chunks, then every head adds its weight
    // over g (exact: g is a power of two) by LDS atomic adds issued in a fixed order
    // within this wavefront
    float* wlw = reinterpret_cast<float*>(rsm) + (size_t)wid * R * TB;
    const int nz = (nvis + 63) & ~63;
    for (int j = 0; j < R; ++j)
        for (int c = lane; c < nz; c += 64) wlw[j * TB + c] = 0.f;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float* wr = wlw + (size_t)(n16 >> lg) * TB;
    const float inv_g = 1.f / (float)g;
#pragma unroll
    for (int j = 0; j < CAP; ++j) {
        if (active && j < ncand) {
            const float v = pow_p<PM>(pos_part(cs * (cv[j] - m) - tau), p.pexp);
            if (v > 0.f) atomicAdd(wr + cc[j], v * inv_g);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    route_compact<false, TB / 64>(p, wlw, TB, R, row0, nb, nvis, bi, r, lane);
}

// Workgroup geometry: up to 8 wavefronts = G groups x CW; all rows of a workgroup
// must share one chunk, and the LDS (the summary ring for bf16 queries, the rows'
// weights, the cross-wavefront partials) must fit 96 KiB (G shrinks until it does;
// a single group that still does not fit is rejected on the host).
constexpr size_t kRouteMaxLds = 96 * 1024;
template <typename T, int D, int NT, int CW>
inline int route_groups_per_block(int R, int B, size_t* lds) {
    const size_t stage = route_uses_ring<T, CW>() ? route_ring_stages<NT, CW>() * (size_t)KSplitStage<D, 32>::BYTES : 0;
    auto bytes = [&](int G) {
        return stage + (size_t)G * R * CW * NT * 16 * 4 + (size_t)G * CW * 16 * 4 + (size_t)2 * G * CW * 32 * 4;
    };
    int G = route_max_groups<T, NT, CW>();
    while (G > 1 && (B % (G * R) != 0 || bytes(G) > kRouteMaxLds)) G >>= 1;
    *lds = bytes(G);
    return G;
}

template <typename T, int D, int NT, int PM, int CW>
static hipError_t launch_route_pm(const RouteParams& p, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
    auto kern = entmax_route_kernel<T, D, NT, PM, CW>;
    if (lds > 64 * 1024) {
        // allow dynamic LDS up to the CU's 160 KiB less the kernel's static LDS
        static hipError_t configured = [&] {
            hipFuncAttributes fa;
            hipError_t e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kern));
            if (e != hipSuccess) return e;
            return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(160 * 1024 - fa.sharedSizeBytes));
        }();
        if (configured != hipSuccess) return configured;
    }
    hipLaunchKernelGGL(kern, grid, block, lds, s, p);
    return hipGetLastError();
}

// Candidate router geometry: W wavefronts (one group of 16 pairs each) with W·R | B
// and the LDS (ring or weight rows, plus the kept chunks) within 160 KiB; 0 if none.
template <int D, int TB>
inline int cand_waves(int R, int B, size_t* lds) {
    for (int W = 8; W >= 1; W >>= 1) {
        if (B % (W * R) != 0) continue;
        const size_t region = std::max((size_t)cand_ring_stages<D>() * KSplitStage<D, 32>::BYTES,
                                       (size_t)W * R * TB * 4);
        const size_t bytes = region + (size_t)W * kCandCap * 64 * 6;
        if (bytes <= 160 * 1024) {
            *lds = bytes;
            return W;
        }
    }
    return 0;
}

template <int D, int PM, int TB>
static hipError_t launch_cand_pm(const RouteParams& p, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
    auto kern = entmax_route_cand_kernel<D, PM, TB>;
    static hipError_t configured = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (configured != hipSuccess) return configured;
    hipLaunchKernelGGL(kern, grid, block, lds, s, p);
    return hipGetLastError();
}

template <typename T, int D, int NT, int CW>
static hipError_t launch_route_nt(const RouteParams& p, int b, hipStream_t s) {
    const int R = 16 / p.g;
    size_t lds = 0;
    const int G = route_groups_per_block<T, D, NT, CW>(R, p.B, &lds);
    const int groups = (p.n + R - 1) / R;
    dim3 grid((groups + G - 1) / G, p.h_kv, b), block(64 * G * CW);
    switch (p.pmode) {
        case kSoftmaxRouting: return launch_route_pm<T, D, NT, kSoftmaxRouting, CW>(p, grid, block, lds, s);
        case 1: return launch_route_pm<T, D, NT, 1, CW>(p, grid, block, lds, s);
        case 2: return launch_route_pm<T, D, NT, 2, CW>(p, grid, block, lds, s);
        case 4: return launch_route_pm<T, D, NT, 4, CW>(p, grid, block, lds, s);
        default: return launch_route_pm<T, D, NT, 0, CW>(p, grid, block, lds, s);
    }
}

// Long rows with bf16 queries and α > 1: the candidate router, then the register
// kernel on the row groups it could not finish. Returns hipErrorNotSupported when
// the candidate router does not apply (the caller runs the register kernel alone).
template <int D, int NT, int CW, int TB>
static hipError_t launch_route_cand(const RouteParams& p, int b, hipStream_t s) {
    const int R = 16 / p.g;
    size_t lds = 0;
    const int W = cand_waves<D, TB>(R, p.B, &lds);
    if (W < 4 || p.pmode == kSoftmaxRouting) return hipErrorNotSupported;
    dim3 grid((p.n + W * R - 1) / (W * R), p.h_kv, b), block(64 * W);
    hipError_t e;
    switch (p.pmode) {
        case 1: e = launch_cand_pm<D, 1, TB>(p, grid, block, lds, s); break;
        case 2: e = launch_cand_pm<D, 2, TB>(p, grid, block, lds, s); break;
        case 4: e = launch_cand_pm<D, 4, TB>(p, grid, block, lds, s); break;
        default: e = launch_cand_pm<D, 0, TB>(p, grid, block, lds, s); break;
    }
    if (e != hipSuccess) return e;
    RouteParams q = p;
    q.redo = 1;
    return launch_route_nt<uint16_t, D, NT, CW>(q, b, s);
}

template <typename T, int D>
static hipError_t launch_route_d(const RouteParams& p, int b, hipStream_t s) {
    switch (route_tiles_bucket(p.T_c)) {
        case 2: return launch_route_nt<T, D, 2, 1>(p, b, s);
        case 8: return launch_route_nt<T, D, 8, 1>(p, b, s);
        case 32: return launch_route_nt<T, D, 32, 1>(p, b, s);
        case 64:
            if constexpr (sizeof(T) == 2) {
                const hipError_t e = launch_route_cand<D, 32, 2, 1024>(p, b, s);
                if (e != hipErrorNotSupported) return e;
            }
            return launch_route_nt<T, D, 32, 2>(p, b, s);
        default:
            if constexpr (sizeof(T) == 2) {
                const hipError_t e = launch_route_cand<D, 32, 4, 2048>(p, b, s);
                if (e != hipErrorNotSupported) return e;
            }
            return launch_route_nt<T, D, 32, 4>(p, b, s);
    }
}

hipError_t launch_route_f32_64(const RouteParams& p, int b, hipStream_t s);
hipError_t launch_route_f32_128(const RouteParams& p, int b, hipStream_t s);
hipError_t launch_route_bf16_64(const RouteParams& p, int b, hipStream_t s);
hipError_t launch_route_bf16_128(const RouteParams& p, int b, hipStream_t s);

}  // namespace dash
