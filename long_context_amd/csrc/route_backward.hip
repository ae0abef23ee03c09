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
#include "route_impl.h"

#include <math.h>

#include <algorithm>

namespace dash {

struct RouteBwdParams {
    const void* Q; const float* kbar; const int32_t* idx; const int32_t* cnt; const float* dbias;
    const float* stats;
    float* dQ; float* dkbar;
    int h_q, h_kv, n, kbar_cap, list_cap, g, soft, T;
    int pmode;          // ŵ = t^p with p = 1, 2, 4 (plain products) or 0 (exp2/log2)
    const uint8_t* ksplit;   // bf16 queries: k̄ as three bf16 terms, the router's layout
    int T_pad;               // chunks per (b, KV head) in ksplit
    float cs;           // scale of y: (α-1)γ/sqrt(d), or γ log2(e)/sqrt(d) when soft
    float pexp;         // 1/(α-1)
    float inv_sigma, dz_scale;   // 1/σ and γ/sqrt(d)
};

// ---------------------------------------------------------------------------------
// Stage-1 backward with dk̄ accumulated in LDS (the form used whenever one column
// slice of dk̄ for all chunks fits in LDS).
//
// A workgroup of 8 wavefronts owns one (b, KV head), one slice of DS columns of dq
// and dk̄, and a strided set of rows (row = wavefront index + k x wavefronts in the
// grid's x dimension, which evens out the causal growth of the lists). Per row, one
// wavefront walks the list in tiles of 16 entries with 16x16 MFMA tiles whose 16
// columns are the heads of the group (columns past g stay zero):
//  * logits z[entry][head] rebuilt with the router's own arithmetic (bf16 queries:
//    k̄ split into three bf16 terms, the same k-slot order and partial-sum order;
//    fp32 queries: fp32 MFMA with the router's k-slot order), so ŵ = [y - τ]_+^p
//    and the support agree with the forward bit for bit;
//  * first walk: Σ_c s ∂ŵ and Σ_c s per head; second walk: dz per (entry, head);
//  * dq[head][col] += Σ_entries dz k̄ (fp32 MFMA, k = entries; added to dQ once);
//  * dk̄[entry][col] += Σ_heads dz q (dz through a per-wavefront LDS transpose;
//    bf16 queries: dz in three bf16 terms against the exact bf16 q; fp32 queries:
//    fp32 MFMA), added into the workgroup's LDS accumulator [T][DS + 1].
// After the last row the accumulator goes to dkbar with one atomic add per nonzero
// element, so global atomics scale with workgroups, not with rows.
constexpr int kRbWaves = 8;
constexpr int kRbTr = 16 * 17;                       // transpose tile floats per wavefront
constexpr size_t kRbMaxLds = 160 * 1024;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float rb_row16_sum(float v) {
    v += dpp_partner<0xB1>(v);
    v += dpp_partner<0x4E>(v);
    v += dpp_partner<0x141>(v);
    v += dpp_partner<0x140>(v);
    return v;
}

// [y - τ]_+ for y <= 0 and τ >= -1 (a clamp to [0, 1]), as the router forms it.
__device__ __forceinline__ float rb_pos(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 1.f); }

// ŵ = t^p and s = ŵ^(2-α) = t^(p-1) for the exponent mode of the router.
__device__ __forceinline__ void rb_weight(float t, int pm, float pexp, float& w, float& sj) {
    switch (pm) {
        case 1: w = t; sj = t > 0.f ? 1.f : 0.f; break;
        case 2: w = t * t; sj = t; break;
        case 4: { const float t2 = t * t; w = t2 * t2; sj = t2 * t; } break;
        default:
            if (t > 0.f) {
                const float lt = fast_log2(t);
                w = fast_exp2(pexp * lt);
                sj = fast_exp2((pexp - 1.f) * lt);
            } else {
                w = 0.f; sj = 0.f;
            }
    }
}

__device__ __forceinline__ void rb_split3(float x, __bf16& h, __bf16& m, __bf16& l) {
    h = (__bf16)x;
    const float r1 = x - (float)h;
    m = (__bf16)r1;
    l = (__bf16)(r1 - (float)m);
}

__device__ __forceinline__ short rb_bits(__bf16 v) { return __builtin_bit_cast(short, v); }

// acc[ci[i] * st + n16 + 16 dt] += v[dt][i] for the entries with ci[i] >= 0, as
// compare-and-swap on the words (the LDS float add runs far below the rate of the
// integer atomics on this chip). All words are read, then swapped; a lane whose swap
// lost to another wavefront retries with the value it found. Every round at least one
// of the competing updates of a word succeeds, so the loop ends.
template <int NDT>
__device__ __forceinline__ void rb_lds_add(float* acc, int st, const int (&ci)[4], int n16,
                                           const f32x4 (&v)[NDT]) {
    uint32_t* base = reinterpret_cast<uint32_t*>(acc);
#pragma unroll
    for (int half = 0; half < 2; ++half) {            // two entries at a time (registers)
        uint32_t cur[2][NDT];
        bool pend[2][NDT];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const int i = 2 * half + u;
                pend[u][dt] = ci[i] >= 0;
                cur[u][dt] = pend[u][dt] ? base[ci[i] * st + n16 + 16 * dt] : 0u;
            }
        for (;;) {
            bool again = false;
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    if (pend[u][dt]) {
                        const int i = 2 * half + u;
                        const uint32_t nv = __float_as_uint(__uint_as_float(cur[u][dt]) + v[dt][i]);
                        pend[u][dt] = !__hip_atomic_compare_exchange_strong(
                            base + ci[i] * st + n16 + 16 * dt, &cur[u][dt], nv, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_WORKGROUP);   // on failure cur holds the word found
                        again = again || pend[u][dt];
                    }
                }
            if (ballot(again) == 0) break;
        }
    }
}

template <typename T, int D, int DS>
__global__ __launch_bounds__(512) void route_backward_lds_kernel(RouteBwdParams p, int nb) {
    extern __shared__ __attribute__((aligned(16))) float rb_lds[];
    constexpr int ST = DS + 1;                        // accumulator row stride (floats)
    constexpr int NDT = DS / 16;                      // 16-column tiles of the slice
    constexpr bool BF = sizeof(T) == 2;
    typedef __bf16 b8 __attribute__((ext_vector_type(8)));
    float* acc = rb_lds;                              // [T][ST]
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n16 = lane & 15, kg = lane >> 4;
    float* tr = rb_lds + (size_t)p.T * ST + wid * kRbTr;   // [16 entries][17]
    const size_t bh = blockIdx.y;
    const int bi = (int)(bh / p.h_kv), r = (int)(bh % p.h_kv);
    const int col0 = blockIdx.z * DS;
    const int g = p.g;
    const bool head_ok = n16 < g;
    const T* Qb = static_cast<const T*>(p.Q);
    const float* kb = p.kbar + bh * (size_t)p.kbar_cap * D;
    const uint8_t* ksb = BF ? p.ksplit + bh * (size_t)p.T_pad * KSplitStage<D, 32>::ROWB : nullptr;

    for (int e = threadIdx.x; e < p.T * ST; e += blockDim.x) acc[e] = 0.f;
    __syncthreads();

    // The walk is software pipelined: the row's list entries and dbias sit in
    // registers, a window of 256 at a time (register k of lane l: entry 256w + 64k + l),
    // loaded with one coalesced access per window; the logits operands of tile t + 1
    // are loaded while tile t computes.
    constexpr int WINK = 4;
    constexpr int NOB = BF ? D / 32 : 1;             // bf16 operands per split
    constexpr int NOF = BF ? 1 : D / 16;             // fp32 operands
    for (int row = blockIdx.x * kRbWaves + wid; row < p.n; row += nb * kRbWaves) {
        const size_t rb = bh * p.n + row;
        const int cn = min(p.cnt[rb], p.list_cap);
        if (cn <= 0) continue;                        // wavefront-uniform
        const int32_t* li = p.idx + rb * p.list_cap;
        const float* ldb = p.dbias + rb * p.list_cap;
        const size_t qrow_h = (((size_t)bi * p.h_q + r * g + (head_ok ? n16 : 0)) * p.n + row) * D;

        // statistics of head n16 (max raw logit, threshold or log2 Σ 2^y)
        float smax = 0.f, thr = 0.f;
        if (head_ok) {
            const float* st = p.stats + 2 * (((size_t)bi * p.h_q + r * g + n16) * p.n + row);
            smax = st[0];
            thr = st[1];
        }
        // logits operand: q of head n16 at the router's k-slots
        b8 qb[NOB];
        float qv[BF ? 1 : D / 4];
        if constexpr (BF) {
#pragma unroll
            for (int s = 0; s < D / 32; ++s)
                qb[s] = head_ok ? *reinterpret_cast<const b8*>(Qb + qrow_h + 32 * s + 8 * kg) : b8{};
        } else {
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                const f32x4 v = head_ok ? *reinterpret_cast<const f32x4*>(Qb + qrow_h + 16 * s + 4 * kg)
                                        : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) qv[4 * s + j] = v[j];
            }
        }
        // dk̄ operand: q of heads 4kg..4kg+3 (bf16) or kg + 4j (fp32) at column 16dt + n16
        s16x4 qk16[BF ? NDT : 1];
        float qk32[BF ? 1 : NDT][4];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int col = col0 + 16 * dt + n16;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int h = BF ? 4 * kg + j : kg + 4 * j;
                const size_t o = (((size_t)bi * p.h_q + r * g + (h < g ? h : 0)) * p.n + row) * D + col;
                if constexpr (BF) qk16[dt][j] = h < g ? static_cast<short>(reinterpret_cast<const uint16_t*>(Qb)[o]) : 0;
                else qk32[dt][j] = h < g ? reinterpret_cast<const float*>(Qb)[o] : 0.f;
            }
        }

        // lreg[k] / dreg[k] hold block cb + k of 64 entries (chunk id or -1, dbias); the
        // walk asks for blocks in increasing order, so a new block rotates the registers
        // down by one and every WINK blocks the next window is loaded
        int lreg[WINK];
        float dreg[WINK];
        int cb = 0;
        auto load_window = [&](int blk0) {
#pragma unroll
            for (int k = 0; k < WINK; ++k) {
                const int e = 64 * (blk0 + k) + lane;
                int c = -1;
                float d = 0.f;
                if (e < cn) {
                    c = li[e];
                    d = ldb[e];
                    if ((unsigned)c >= (unsigned)p.T) c = -1;
                }
                lreg[k] = c;
                dreg[k] = d;
            }
            cb = blk0;
        };
        load_window(0);
        float dsum = 0.f;
#pragma unroll
        for (int k = 0; k < WINK; ++k) dsum += dreg[k];
        for (int e = 64 * WINK + lane; e < cn; e += 64) dsum += ldb[e];
        const float dmean = wave_sum(dsum) / (float)cn;

        // chunk id and dbias of the A-operand row of lane (kg, n16) in tile t: entry 16t + n16
        auto tile_entry = [&](int t, int& ca, float& dba) {
            const int blk = t >> 2;
            if (blk != cb) {                          // wavefront-uniform
                if (blk == cb + 1 && (blk & (WINK - 1)) != 0) {
#pragma unroll
                    for (int k = 0; k + 1 < WINK; ++k) { lreg[k] = lreg[k + 1]; dreg[k] = dreg[k + 1]; }
                    cb = blk;
                } else {
                    load_window(blk);
                }
            }
            const int src = (((t & 3) << 4) | n16) << 2;
            ca = __builtin_amdgcn_ds_bpermute(src, lreg[0]);
            dba = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(dreg[0])));
        };
        // logits operands of one A row (zero for no chunk)
        auto load_ops = [&](int ca, b8 (&ob)[3][NOB], f32x4 (&of)[NOF]) {
            if constexpr (BF) {
                typedef KSplitStage<D, 32> KS;
#pragma unroll
                for (int h = 0; h < 3; ++h)
#pragma unroll
                    for (int s = 0; s < NOB; ++s)
                        ob[h][s] = ca >= 0 ? *reinterpret_cast<const b8*>(ksb + KS::off(ca, h, 4 * s + kg)) : b8{};
            } else {
                const float* krow = kb + (ca < 0 ? 0 : ca) * D + 4 * kg;
#pragma unroll
                for (int s = 0; s < NOF; ++s)
                    of[s] = ca >= 0 ? *reinterpret_cast<const f32x4*>(krow + 16 * s) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        };
        // chunk ids of the output entries 16t + 4kg + i, from the lanes holding them
        auto out_ids = [&](int ca, float dba, int (&ci)[4], float (&db)[4]) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int src = ((lane & 48) | (4 * kg + i)) << 2;
                ci[i] = __builtin_amdgcn_ds_bpermute(src, ca);
                db[i] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(dba)));
            }
        };
        // lane (kg, n16) ends with entries 16t + 4kg + i of head n16: s and ∂L/∂ŵ (the
        // same for every head)
        auto weights = [&](const b8 (&ob)[3][NOB], const f32x4 (&of)[NOF], const int (&ci)[4],
                           const float (&db)[4], float (&sj)[4], float (&dw)[4]) {
            f32x4 z;
            if constexpr (BF) {
                f32x4 a3[3];
#pragma unroll
                for (int h = 0; h < 3; ++h) {
                    a3[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < NOB; ++s)
                        a3[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ob[h][s], qb[s], a3[h], 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) z[i] = a3[0][i] + (a3[1][i] + a3[2][i]);
            } else {
                z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NOF; ++s)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        z = __builtin_amdgcn_mfma_f32_16x16x4f32(of[s][j], qv[4 * s + j], z, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float w = 0.f, sv = 0.f;
                if (ci[i] >= 0 && head_ok) {
                    const float y = p.cs * (z[i] - smax);
                    if (p.soft) { w = fast_exp2(y - thr); sv = w; }
                    else rb_weight(rb_pos(y - thr), p.pmode, p.pexp, w, sv);
                }
                const float wsum = rb_row16_sum(w);
                sj[i] = sv;
                dw[i] = (ci[i] >= 0 && wsum > 0.f) ? (db[i] - dmean) * p.inv_sigma * __builtin_amdgcn_rcpf(wsum) : 0.f;
            }
        };

        const int ntile = (cn + 15) / 16;
        float corr = 0.f;
        f32x4 dq[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // pass 0: Σ_c s ∂ŵ and Σ_c s per head; pass 1: dz, dq and dk̄
        for (int pass = 0; pass < 2; ++pass) {
            float Ah = 0.f, Bh = 0.f;
            int ca_n;
            float dba_n;
            b8 ob_n[3][NOB];
            f32x4 of_n[NOF];
            tile_entry(0, ca_n, dba_n);
            load_ops(ca_n, ob_n, of_n);
            for (int t = 0; t < ntile; ++t) {
                const int ca = ca_n;
                const float dba = dba_n;
                b8 ob[3][NOB];
                f32x4 of[NOF];
#pragma unroll
                for (int h = 0; h < 3; ++h)
#pragma unroll
                    for (int s = 0; s < NOB; ++s) ob[h][s] = ob_n[h][s];
#pragma unroll
                for (int s = 0; s < NOF; ++s) of[s] = of_n[s];
                if (t + 1 < ntile) {
                    tile_entry(t + 1, ca_n, dba_n);
                    load_ops(ca_n, ob_n, of_n);
                }
                int ci[4];
                float db[4], sj[4], dw[4];
                out_ids(ca, dba, ci, db);
                if (pass == 0) {
                    weights(ob, of, ci, db, sj, dw);
#pragma unroll
                    for (int i = 0; i < 4; ++i) { Ah = fmaf(sj[i], dw[i], Ah); Bh += sj[i]; }
                    continue;
                }
                weights(ob, of, ci, db, sj, dw);
                // dq operand k̄[entry][column]
                float kv[NDT][4];
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        kv[dt][i] = ci[i] >= 0 ? kb[ci[i] * D + col0 + 16 * dt + n16] : 0.f;
                float dz[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) dz[i] = ci[i] >= 0 ? p.dz_scale * sj[i] * (dw[i] - corr) : 0.f;
                // dq[head][col] += Σ_entries dz[entry][head] k̄[entry][col]: the k-slot kg of
                // step i is entry 4kg + i, the A row is head n16
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        dq[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(dz[i], kv[dt][i], dq[dt], 0, 0, 0);
                // dz to [entry][head] through LDS
#pragma unroll
                for (int i = 0; i < 4; ++i) tr[(4 * kg + i) * 17 + n16] = dz[i];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                f32x4 dk[NDT];
                if constexpr (BF) {
                    // A row = entry n16, k-slots = heads 4kg..4kg+3, dz in three bf16 terms
                    s16x4 zh, zm, zl;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        __bf16 hh, mm, ll;
                        rb_split3(tr[n16 * 17 + 4 * kg + j], hh, mm, ll);
                        zh[j] = rb_bits(hh); zm[j] = rb_bits(mm); zl[j] = rb_bits(ll);
                    }
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        f32x4 a = {0.f, 0.f, 0.f, 0.f};
                        a = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(zl, qk16[dt], a, 0, 0, 0);
                        a = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(zm, qk16[dt], a, 0, 0, 0);
                        dk[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(zh, qk16[dt], a, 0, 0, 0);
                    }
                } else {
                    float za[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) za[j] = tr[n16 * 17 + kg + 4 * j];
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int j = 0; j < 4; ++j) a = __builtin_amdgcn_mfma_f32_16x16x4f32(za[j], qk32[dt][j], a, 0, 0, 0);
                        dk[dt] = a;
                    }
                }
                // lane (kg, n16) holds dk̄[entry 4kg + i][column 16dt + n16]; the lanes of one
                // wavefront address distinct elements, other wavefronts may add to the same
                // chunk at the same time
                rb_lds_add<NDT>(acc, ST, ci, n16, dk);
                __builtin_amdgcn_wave_barrier();      // the transpose tile is rewritten next
            }
            if (pass == 0) {
                Ah = pair32_sum(pair16_sum(Ah));
                Bh = pair32_sum(pair16_sum(Bh));
                corr = Bh > 0.f ? Ah / Bh : 0.f;
            }
        }
        // dQ: lane (kg, n16) holds dq[head 4kg + j][column 16dt + n16]
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int h = 4 * kg + j;
            if (h < g) {
                float* out = p.dQ + (((size_t)bi * p.h_q + r * g + h) * p.n + row) * D + col0 + n16;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) out[16 * dt] += dq[dt][j];
            }
        }
    }
    __syncthreads();
    float* dk = p.dkbar + bh * (size_t)p.kbar_cap * D + col0;
    for (int e = threadIdx.x; e < p.T * DS; e += blockDim.x) {
        const int c = e / DS, cc = e % DS;
        const float v = acc[c * ST + cc];
        if (v != 0.f) unsafeAtomicAdd(dk + (size_t)c * D + cc, v);
    }
}

template <typename T>
__device__ __forceinline__ float load_f(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_f<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_f<uint16_t>(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }

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

// Widest column slice (64, 32, 16) whose LDS accumulator [T][DS + 1] fits beside the
// transpose tiles (128 columns would not fit the registers). Every chunk count the
// router accepts (≤ 2048) fits a 16-column slice.
static int route_bwd_slice(int d, int T) {
    for (int ds = d == 128 ? 64 : d; ds >= 16; ds /= 2)
        if ((size_t)T * (ds + 1) * 4 + (size_t)kRbWaves * kRbTr * 4 <= kRbMaxLds) return ds;
    return 0;
}

template <typename T, int D, int DS>
static hipError_t launch_rb_lds(const RouteBwdParams& p, int bh, hipStream_t s) {
    auto kern = route_backward_lds_kernel<T, D, DS>;
    static hipError_t configured = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kRbMaxLds);
    if (configured != hipSuccess) return configured;
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
    }
    const size_t lds = (size_t)p.T * (DS + 1) * 4 + (size_t)kRbWaves * kRbTr * 4;
    const int per_cu = (int)std::max<size_t>(1, std::min<size_t>(4, kRbMaxLds / lds));
    const int slices = D / DS;
    const int want = (cus * per_cu + bh * slices - 1) / (bh * slices);
    const int nb = std::max(1, std::min(want, (p.n + kRbWaves - 1) / kRbWaves));
    hipLaunchKernelGGL(kern, dim3(nb, bh, slices), dim3(64 * kRbWaves), lds, s, p, nb);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_rb_lds_d(const RouteBwdParams& p, int bh, int ds, hipStream_t s) {
    switch (ds) {
        case 64: return launch_rb_lds<T, D, 64>(p, bh, s);
        case 32: return launch_rb_lds<T, D, 32>(p, bh, s);
        default: return launch_rb_lds<T, D, 16>(p, bh, s);
    }
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
    p.pmode = pmode_of(a.alpha);
    p.cs = route_scale(a.alpha, a.gamma, a.d);
    p.pexp = p.soft ? 1.f : (float)(1.0 / ((double)a.alpha - 1.0));
    p.inv_sigma = 1.f / a.sigma;
    p.dz_scale = (float)(a.gamma / sqrt((double)a.d));
    p.ksplit = static_cast<const uint8_t*>(a.ws);
    p.T_pad = (p.T + 31) / 32 * 32;
    if (p.T == 0) return hipSuccess;
    const int bh = a.b * a.h_kv;
    const int ds = route_bwd_slice(a.d, p.T);
    if (ds > 0) {
        if (a.q_bf16) {
            const hipError_t e = launch_kbar_split(a.kbar, a.ws, a.b, a.h_kv, a.kbar_cap, p.T, a.d, s);
            if (e != hipSuccess) return e;
        }
        if (a.q_bf16) return a.d == 64 ? launch_rb_lds_d<uint16_t, 64>(p, bh, ds, s)
                                       : launch_rb_lds_d<uint16_t, 128>(p, bh, ds, s);
        return a.d == 64 ? launch_rb_lds_d<float, 64>(p, bh, ds, s) : launch_rb_lds_d<float, 128>(p, bh, ds, s);
    }
    return hipErrorInvalidValue;                      // rejected by the host checks first
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
