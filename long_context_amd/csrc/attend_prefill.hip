// Stage 2 prefill kernel for fp32 inputs (see prefill_common.h for the method).
//
// sparse_prior_attn_kernel: the tile is R_t rows times the g heads of a KV group
// (M = g*R_t pairs, 32 per wavefront, up to 8 wavefronts):
//   * tiles are copied global->LDS asynchronously (global_load_lds_dwordx4) into a
//     two-stage ring; the copy of tile k+1 runs while tile k is computed, and one
//     barrier per tile separates the stages;
//   * a wavefront skips a chunk none of its rows routes to;
//   * S^T = K Q^T on MFMA (lane = one (row, head) column), logits in log2 units
//     with the bias folded into the exp2 argument, online softmax per lane with
//     lazy rescaling, O^T += V^T P^T on MFMA; the division by the softmax
//     denominator happens once at the end.
// The kernel is generic in the element type; bf16 inputs take the kernel of
// attend_prefill_bf16.hip.
#include "kernels.h"
#include "prefill_common.h"

#include <math.h>

namespace dash {

constexpr int kWaves = 8;                 // wavefronts per workgroup (256 pairs)

template <typename T, int D, int TT, bool PAGED>
__global__ __launch_bounds__(64 * kWaves) void sparse_prior_attn_kernel(PrefillParams p) {
    typedef SwzTile<T, D, TT> S;
    typedef Mfma<T> MM;
    typedef typename MM::Op Op;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* ring = smem;                                             // 2 stages
    TileTables tabs;
    tabs.carve(smem + 2 * S::STAGE, p.T_c);

    constexpr int nthr = 64 * kWaves;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hl = lane >> 5;
    const int r = blockIdx.y, bi = blockIdx.z;
    const int g = p.g, lg = p.log2g, R_t = p.R_t;
    // causal tiles near the end of the sequence carry the most work: launch them first
    const int row0 = (gridDim.x - 1 - blockIdx.x) * R_t;
    // ragged batch: the sequence's own tokens and complete chunks; a tile past them
    // has nothing to do (workgroup-uniform, before any barrier)
    const int nb = seq_tokens(p, bi), Tb = nb / p.B;
    if (row0 >= nb) return;
    const int cq = row0 / p.B;
    const int nvis = p.causal ? min(cq, Tb) : Tb;
    const int last_row = min(row0 + R_t, nb) - 1;
    const size_t bhkv = (size_t)bi * p.h_kv + r;
    // K and V rows: the sequence's own rows, or (paged) the whole cache with per-chunk
    // row offsets
    const T* Kg = static_cast<const T*>(p.K) + (PAGED ? 0 : bhkv * (size_t)p.n * D);
    const T* Vg = static_cast<const T*>(p.V) + (PAGED ? 0 : bhkv * (size_t)p.n * D);
    auto krow0 = [&](int t) { return PAGED ? paged_row0(p, bi, r, t) : 0; };
    const int U = tabs.build(p, bhkv, row0, nvis, tid, nthr, nb);
    const int* ulist = tabs.ulist;

    // ---- this lane's (row, head) pair ----
    const int pair = wid * 32 + l32;
    const bool wave_active = wid * 32 < g * R_t;
    const int j = pair >> lg;
    const int hh = r * g + (pair & (g - 1));
    const int my_row = row0 + j;
    const bool pair_ok = wave_active && j < R_t && my_row < nb;
    ListCursor lc;
    lc.init(p, bhkv * p.n + (pair_ok ? my_row : 0), pair_ok);
    Op qf[D / 16];
    if (pair_ok) {
        const T* qrow = static_cast<const T*>(p.Q) + (((size_t)bi * p.h_q + hh) * p.n + my_row) * D + 8 * hl;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) qf[s] = MM::load(qrow + 16 * s);
    } else {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) qf[s] = MM::zero();
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o_acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o_acc[db][i] = 0.f;

    TileSteps st;
    st.init(p, U, cq, last_row, TT, nb, Tb);
    const int nrouted = st.nrouted, nsteps = st.nsteps, SPC = st.SPC;
    const int nmax = nb - 1;
    TileCopier<T, D, TT, kWaves> copier;
    copier.init(wid, lane);
    // the tile base and chunk of each step are read from LDS two steps ahead, so
    // that neither the cursor nor the copies wait on an LDS read
    int tb_cur, c_cur, tb_nxt, c_nxt;
    st.at(ulist, 0, tb_cur, c_cur);
    st.at(ulist, 1, tb_nxt, c_nxt);

    int ko_nxt = krow0(tb_nxt);
    if (nsteps > 0) {
        const int ko = krow0(tb_cur);
        copier.issue(ring, Kg, Vg, ko + tb_cur, ko + nmax, wid);
    }
    wait_tile_copies();
    __syncthreads();
    for (int k = 0; k < nsteps; ++k) {
        // the cursor's entry arrived during the previous tile; its next load goes
        // out ahead of the copies
        const bool routed = k < nrouted;
        float bias2 = 0.f;
        bool run = wave_active;
        if (routed && run) {
            bias2 = lc.take(c_cur, k % SPC == SPC - 1);
            run = ballot(bias2 > -INFINITY) != 0;          // some row of this wave routes c
        }
        if (k + 1 < nsteps) copier.issue(ring + ((k + 1) & 1) * S::STAGE, Kg, Vg, ko_nxt + tb_nxt, ko_nxt + nmax, wid);
        int tb_nn, c_nn;
        st.at(ulist, k + 2, tb_nn, c_nn);
        const char* ktile = ring + (k & 1) * S::STAGE;
        const char* vtile = ktile + S::BYTES;
        if (run) {
            const int tb = tb_cur;
            // S^T = K Q^T: accumulator column = this lane's pair, rows = tokens
            f32x16 sacc[TT / 32];
#pragma unroll
            for (int blk = 0; blk < TT / 32; ++blk)
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[blk][i] = 0.f;
            constexpr int NB = sizeof(T) == 2 ? 4 : 2;
#pragma unroll
            for (int s0 = 0; s0 < D / 16; s0 += NB) {
                Op ka[TT / 32][NB];
#pragma unroll
                for (int blk = 0; blk < TT / 32; ++blk)
#pragma unroll
                    for (int s = 0; s < NB; ++s)
                        ka[blk][s] = load_k_op<T, D, TT>(ktile, 32 * blk + l32, 16 * (s0 + s) + 8 * hl);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int s = 0; s < NB; ++s)
#pragma unroll
                    for (int blk = 0; blk < TT / 32; ++blk) sacc[blk] = MM::mma(ka[blk][s], qf[s0 + s], sacc[blk]);
            }
            // mask the diagonal tile on the raw scores (selects, no branches)
            if (!routed) {
                const int lim = p.causal ? my_row : nb - 1;
                const int tk0 = tb + 4 * hl;
#pragma unroll
                for (int blk = 0; blk < TT / 32; ++blk)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int tk = tk0 + 32 * blk + 8 * (i >> 2) + (i & 3);
                        sacc[blk][i] = tk > lim ? -INFINITY : sacc[blk][i];
                    }
            }
            // tile maximum; c1 = log2(e)/sqrt(d) > 0 commutes with the maximum
            float mx = -INFINITY;
#pragma unroll
            for (int blk = 0; blk < TT / 32; ++blk)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[blk][i]);
            mx = pair32_max(mx);
            const float tmax = fmaf(mx, p.scale_log2, bias2);     // -inf when nothing is visible
            // lazy rescaling: the reference maximum only moves when the tile maximum
            // exceeds it by more than 8 (probabilities stay <= 2^8 in between)
            const bool grow = tmax > m_run + 8.f;
            float alpha = 1.f;
            if (grow) {
                alpha = fast_exp2(m_run - tmax);
                m_run = tmax;
            }
            const float off = bias2 - ((m_run == -INFINITY) ? 0.f : m_run);
            float ps = 0.f;
#pragma unroll
            for (int blk = 0; blk < TT / 32; ++blk)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    sacc[blk][i] = fast_exp2(fmaf(sacc[blk][i], p.scale_log2, off));
                }
            if (ballot(grow) != 0) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o_acc[db][i] *= alpha;
            }
            // O^T += V^T P^T
#pragma unroll
            for (int s = 0; s < TT / 16; ++s) {
                float pv8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) pv8[e] = sacc[s >> 1][8 * (s & 1) + e];
                const Op pb = MM::pack(pv8);
                ps = MM::sum(pb, pv8, ps);        // the denominator sums the P fed to the MFMA
                Op va[D / 32];
#pragma unroll
                for (int db = 0; db < D / 32; ++db) va[db] = load_vt_op<T, D, TT>(vtile, s, db, lane);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) o_acc[db] = MM::mma(va[db], pb, o_acc[db]);
            }
            l_run = fmaf(l_run, alpha, ps);
        }
        wait_tile_copies();
        __syncthreads();
        tb_cur = tb_nxt; c_cur = c_nxt;
        tb_nxt = tb_nn; c_nxt = c_nn;
        ko_nxt = krow0(tb_nxt);
    }

    const float l_tot = pair32_sum(l_run);
    if (pair_ok) {
        const float inv = 1.f / l_tot;
        if (p.lse && hl == 0)
            p.lse[((size_t)bi * p.h_q + hh) * p.n + my_row] =
                (((m_run == -INFINITY) ? 0.f : m_run) + fast_log2(l_tot)) * kLn2;
        const size_t obase = (((size_t)bi * p.h_q + hh) * p.n + my_row) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int d0 = 32 * db + 8 * a + 4 * hl;
                if (p.out_bf16) {
                    u32x2 o;
                    o[0] = (uint32_t)f32_to_bf16_bits(o_acc[db][4 * a] * inv) |
                           ((uint32_t)f32_to_bf16_bits(o_acc[db][4 * a + 1] * inv) << 16);
                    o[1] = (uint32_t)f32_to_bf16_bits(o_acc[db][4 * a + 2] * inv) |
                           ((uint32_t)f32_to_bf16_bits(o_acc[db][4 * a + 3] * inv) << 16);
                    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.O) + obase + d0) = o;
                } else {
                    f32x4 o;
                    o[0] = o_acc[db][4 * a] * inv; o[1] = o_acc[db][4 * a + 1] * inv;
                    o[2] = o_acc[db][4 * a + 2] * inv; o[3] = o_acc[db][4 * a + 3] * inv;
                    *reinterpret_cast<f32x4*>(static_cast<float*>(p.O) + obase + d0) = o;
                }
            }
    }
}

static constexpr size_t kMaxLds = 160 * 1024;

static int stage_bytes(int d, bool bf16, int TT) { return 2 * TT * d * (bf16 ? 2 : 4); }

PrefillGeom prefill_geom_f32(int, int B) {
    return PrefillGeom{(B % 64 == 0) ? 64 : 32, kWaves, 32 * kWaves, 2};
}

void prefill_tiling(int g, int B, int T_c, int d, bool bf16, int* rows, size_t* lds_bytes) {
    *rows = 0;
    *lds_bytes = 0;
    if (B % 32 != 0 || g < 1 || g > 16) return;
    const PrefillGeom geo = bf16 ? prefill_geom_bf16(d, B) : prefill_geom_f32(d, B);
    const int st = stage_bytes(d, bf16, geo.TT);
    for (int m = geo.max_pairs; m >= 32; m >>= 1) {
        const int R_t = m / g;
        if (R_t < 1 || B % R_t != 0) continue;
        const int stages = bf16 ? prefill_bf16_stages(d, B, T_c) : geo.stages;
        const size_t lds = (size_t)stages * st + TileTables::bytes(T_c);
        if (lds <= kMaxLds) {
            *rows = R_t;
            *lds_bytes = lds;
            return;
        }
    }
}

// Both K/V layouts of every (d, tile) pair are instantiated explicitly: when one
// dispatcher names the two, hipcc emits the host handle of only the first.
#define DASH_PREFILL_F32_INST(D, TT)                                                   \
    template __global__ void sparse_prior_attn_kernel<float, D, TT, false>(PrefillParams); \
    template __global__ void sparse_prior_attn_kernel<float, D, TT, true>(PrefillParams);
DASH_PREFILL_F32_INST(64, 32)
DASH_PREFILL_F32_INST(64, 64)
DASH_PREFILL_F32_INST(128, 32)
DASH_PREFILL_F32_INST(128, 64)
#undef DASH_PREFILL_F32_INST

template <int D, int TT, bool PAGED>
static hipError_t launch_prefill_paged(const PrefillParams& p, int b, size_t lds, hipStream_t s) {
    static hipError_t configured = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&sparse_prior_attn_kernel<float, D, TT, PAGED>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    if (configured != hipSuccess) return configured;
    dim3 grid((p.n + p.R_t - 1) / p.R_t, p.h_kv, b), block(64 * kWaves);
    hipLaunchKernelGGL((sparse_prior_attn_kernel<float, D, TT, PAGED>), grid, block, lds, s, p);
    return hipGetLastError();
}

template <int D, int TT>
static hipError_t launch_prefill_t(const PrefillParams& p, int b, size_t lds, hipStream_t s) {
    return p.pages ? launch_prefill_paged<D, TT, true>(p, b, lds, s) : launch_prefill_paged<D, TT, false>(p, b, lds, s);
}

hipError_t launch_prefill_f32(const PrefillParams& p, int b, int d, size_t lds, hipStream_t s) {
    const bool t64 = (p.B % 64 == 0);
    if (d == 64) return t64 ? launch_prefill_t<64, 64>(p, b, lds, s) : launch_prefill_t<64, 32>(p, b, lds, s);
    return t64 ? launch_prefill_t<128, 64>(p, b, lds, s) : launch_prefill_t<128, 32>(p, b, lds, s);
}

hipError_t launch_attend_prefill(const PrefillArgs& a, hipStream_t s) {
    PrefillParams p;
    p.Q = a.Q; p.K = a.K; p.V = a.V; p.idx = a.idx; p.bias = a.bias; p.cnt = a.cnt; p.O = a.O;
    p.lse = a.lse;
    p.Vt = static_cast<const uint16_t*>(a.ws);
    p.out_bf16 = a.out_bf16; p.h_q = a.h_q; p.h_kv = a.h_kv; p.n = a.n; p.B = a.B;
    p.n_pad = prefill_n_pad(a.n);
    p.T_c = a.n / a.B; p.list_cap = a.list_cap; p.causal = a.causal;
    p.g = a.h_q / a.h_kv;
    p.log2g = 0;
    while ((1 << p.log2g) < p.g) ++p.log2g;
    p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)a.d));
    p.seq_len = a.seq_len;
    p.pages = a.pages; p.pages_per_seq = a.pages_per_seq; p.num_pages = a.num_pages;
    size_t lds = 0;
    prefill_tiling(p.g, a.B, p.T_c, a.d, a.in_bf16, &p.R_t, &lds);
    if (p.R_t == 0) return hipErrorInvalidValue;
    p.nw = (p.g * p.R_t + 31) / 32;
    if (a.n == 0) return hipSuccess;
    return a.in_bf16 ? launch_prefill_bf16(p, a.b, a.d, lds, s) : launch_prefill_f32(p, a.b, a.d, lds, s);
}

}  // namespace dash
