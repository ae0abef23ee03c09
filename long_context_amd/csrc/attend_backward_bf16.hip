// Stage 2 backward for bf16 inputs.
//
// Stage 2 is a softmax attention whose logits carry a fixed additive bias per routed
// chunk (paper review section 三, the Proposition 4.1 form). With the support and
// the bias held fixed its gradients are those of softmax attention:
//   P = exp(Z - lse),  dV = P^T dO,  dP = dO V^T,  dZ = P ∘ (dP - Δ),  Δ_i = <o_i, do_i>,
//   dQ = dZ K / sqrt(d),  dK = dZ^T Q / sqrt(d),
// and the gradient of a routed chunk's bias in row i is the sum of dZ over the
// chunk's tokens and the query heads of the row's KV group (they share one list).
//
// Kernels, in launch order:
//   bwd_prep_kernel        Δ per (row, head); dO as bf16 when it comes in fp32.
//   inv_*_kernel           the routed lists inverted into per-chunk row lists, rows
//                          ascending (a stable counting sort over 64-row blocks).
//   prior_attn_dq_kernel   query-major like the forward: a query tile walks the
//                          union of its rows' routed chunks and then the diagonal,
//                          recomputes P from the forward's lse, keeps dQ in
//                          registers and writes each routed chunk's bias gradient.
//   prior_attn_dkv_kernel  key-major: a workgroup holds K and V of 64 tokens of one
//                          chunk in registers, streams the (row, head) pairs that
//                          see them (a segment of the chunk's row list and its
//                          diagonal rows) and keeps dK and dV in registers; the
//                          pair-contiguous operands of dK and dV come from
//                          transposing LDS reads of the row-major Q and dO tiles.
// dQ and the bias gradients have one writer each. dK and dV add the partials of
// the segments of a chunk and of the two pair halves of a workgroup onto zeros
// with atomic adds.
#include "kernels.h"
#include "prefill_common.h"

#include <math.h>

#include <algorithm>

namespace dash {

// ---------------------------------------------------------------------------------
// Preparation: Δ, transposed Q and dO, bf16 dO
// ---------------------------------------------------------------------------------

struct BwdPrepParams {
    const void* O; const void* dO;
    uint16_t* dOb;                   // nullable: bf16 copy of an fp32 dO
    float* delta;                    // [b, h_q, n]
    int h_q, h_kv, n, g, log2g;
};

// One workgroup per 64 consecutive (row, head) pairs of a KV group.
template <int D, typename OT>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdPrepParams p) {
    constexpr int PR = D / 8;                    // 16-byte pieces per row
    const int tid = threadIdx.x;
    const int hk = blockIdx.y, bi = blockIdx.z;
    const size_t P0 = (size_t)blockIdx.x * 64;
    const size_t npairs = (size_t)p.n * p.g;
    for (int q = tid; q < 64 * PR; q += 256) {
        const int t = q / PR, c = q % PR;
        const size_t pair = P0 + t;
        const int row = (int)(pair >> p.log2g), head = (int)(pair & (p.g - 1));
        const bool ok = pair < npairs;
        const size_t off = (((size_t)bi * p.h_q + (size_t)hk * p.g + head) * p.n + (ok ? row : 0)) * D + 8 * c;
        u32x4 dv;
        float part = 0.f;
        if (ok) {
            float o[8], d[8];
            Elem<OT>::load8(static_cast<const OT*>(p.O) + off, o);
            Elem<OT>::load8(static_cast<const OT*>(p.dO) + off, d);
            // Δ takes dO as the MFMAs of dP see it (rounded to bf16), so that Δ and
            // the rows of dP stay consistent and dZ cancels where it should
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = f32_to_bf16_bits(d[2 * e]), hi = f32_to_bf16_bits(d[2 * e + 1]);
                dv[e] = lo | (hi << 16);
                part = fmaf(o[2 * e], bf16_bits_to_f32(lo), part);
                part = fmaf(o[2 * e + 1], bf16_bits_to_f32(hi), part);
            }
            if (p.dOb) *reinterpret_cast<u32x4*>(p.dOb + off) = dv;
        }
        // the PR pieces of one pair sit in PR consecutive lanes
#pragma unroll
        for (int m = 1; m < PR; m <<= 1) part += shfl_xor(part, m);
        if (ok && c == 0) p.delta[(((size_t)bi * p.h_q + (size_t)hk * p.g + head) * p.n + row)] = part;
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* x, size_t n) {
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) x[i] = 0.f;
}

// ---------------------------------------------------------------------------------
// Inverted lists: for each (b, KV head, chunk c) the rows whose routed list holds c
// (visible chunks only), ascending, with the bias of that entry.
// ---------------------------------------------------------------------------------

struct InvParams {
    const int32_t* idx; const float* bias; const int32_t* cnt;
    int32_t* hist;       // [b*h_kv][T][nblk]: rows of block k routing c, then their offsets
    int32_t* coff;       // [b*h_kv][T+1]: start of chunk c's rows in the inverted list
    int32_t* inv_row; float* inv_bias;   // [b*h_kv][n*T]
    int n, B, T, nblk, list_cap, causal;
};

// Bit r of word c: row block*64 + r routes chunk c. One wavefront per 64-row block;
// lane r walks row r's list.
__device__ __forceinline__ void mark_block_rows(const InvParams& p, size_t bh, int blk, int lane,
                                                unsigned long long* msk) {
    for (int c = lane; c < p.T; c += 64) msk[c] = 0ull;
    __syncthreads();
    const int row = blk * 64 + lane;
    if (row < p.n) {
        const int nvis = p.causal ? min(row / p.B, p.T) : p.T;
        const size_t rb = bh * p.n + row;
        const int cn = min(p.cnt[rb], p.list_cap);
        const int32_t* li = p.idx + rb * p.list_cap;
        for (int e = 0; e < cn; ++e) {
            const int c = li[e];
            if (c >= 0 && c < nvis) atomicOr(&msk[c], 1ull << lane);
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(64) void inv_hist_kernel(InvParams p) {
    extern __shared__ unsigned long long msk[];
    const int blk = blockIdx.x, lane = threadIdx.x;
    const size_t bh = blockIdx.y;
    mark_block_rows(p, bh, blk, lane, msk);
    for (int c = lane; c < p.T; c += 64)
        p.hist[(bh * p.T + c) * p.nblk + blk] = __builtin_popcountll(msk[c]);
}

// Exclusive prefix sum over a 256-thread workgroup (tmp: 4 ints of LDS).
__device__ __forceinline__ int block_scan256(int v, int* tmp, int& total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __builtin_amdgcn_ds_bpermute(((lane - o) & 63) << 2, x);
        if (lane >= o) x += y;
    }
    if (lane == 63) tmp[wid] = x;
    __syncthreads();
    int off = 0;
    for (int w = 0; w < wid; ++w) off += tmp[w];
    total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
    __syncthreads();
    return off + x - v;
}

// Per (chunk, b*h_kv): block counts -> exclusive offsets inside the chunk; chunk total.
__global__ __launch_bounds__(256) void inv_scan_blocks_kernel(InvParams p) {
    __shared__ int tmp[4];
    const size_t bh = blockIdx.y;
    const int c = blockIdx.x;
    int32_t* h = p.hist + (bh * p.T + c) * p.nblk;
    const int per = (p.nblk + 255) / 256;
    const int k0 = min((int)threadIdx.x * per, p.nblk), k1 = min(k0 + per, p.nblk);
    int s = 0;
    for (int k = k0; k < k1; ++k) s += h[k];
    int total;
    int run = block_scan256(s, tmp, total);
    for (int k = k0; k < k1; ++k) {
        const int v = h[k];
        h[k] = run;
        run += v;
    }
    if (threadIdx.x == 0) p.coff[bh * (p.T + 1) + c] = total;
}

// Per b*h_kv: chunk totals -> exclusive chunk starts (entry T: the total).
__global__ __launch_bounds__(256) void inv_scan_chunks_kernel(InvParams p) {
    __shared__ int tmp[4];
    const size_t bh = blockIdx.x;
    int32_t* co = p.coff + bh * (p.T + 1);
    const int per = (p.T + 255) / 256;
    const int k0 = min((int)threadIdx.x * per, p.T), k1 = min(k0 + per, p.T);
    int s = 0;
    for (int k = k0; k < k1; ++k) s += co[k];
    int total;
    int run = block_scan256(s, tmp, total);
    for (int k = k0; k < k1; ++k) {
        const int v = co[k];
        co[k] = run;
        run += v;
    }
    if (threadIdx.x == 0) co[p.T] = total;
}

__global__ __launch_bounds__(64) void inv_scatter_kernel(InvParams p) {
    extern __shared__ unsigned long long msk[];
    const int blk = blockIdx.x, lane = threadIdx.x;
    const size_t bh = blockIdx.y;
    mark_block_rows(p, bh, blk, lane, msk);
    const int row = blk * 64 + lane;
    if (row >= p.n) return;
    const int nvis = p.causal ? min(row / p.B, p.T) : p.T;
    const size_t rb = bh * p.n + row;
    const int cn = min(p.cnt[rb], p.list_cap);
    const int32_t* li = p.idx + rb * p.list_cap;
    const float* lb = p.bias + rb * p.list_cap;
    const size_t base = bh * (size_t)p.n * p.T;
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int e = 0; e < cn; ++e) {
        const int c = li[e];
        if (c < 0 || c >= nvis) continue;
        const size_t pos = base + p.coff[bh * (p.T + 1) + c] + p.hist[(bh * p.T + c) * p.nblk + blk] +
                           __builtin_popcountll(msk[c] & below);
        p.inv_row[pos] = row;
        p.inv_bias[pos] = lb[e];
    }
}

// ---------------------------------------------------------------------------------
// dQ and the bias gradients (query-major)
// ---------------------------------------------------------------------------------

struct DqExtra {
    const uint16_t* Kt;              // [b*h_kv][D][n_pad]
    const uint16_t* dO;              // bf16 [b, h_q, n, D]
    const float* lse; const float* delta;
    float* dQ; float* dbias;
    float scale;                     // 1/sqrt(d)
};

// Copies of one stage: K tile [TT][D], V tile [TT][D] (both "K" form) and the K^T
// tile [D][TT]; wavefront w issues copy instructions w, w+NW, ...
template <int D, int TT, int NW>
struct DqCopier {
    typedef BfTiles<D, TT> S;
    static constexpr int NI = 2 * S::KINSTS + S::VINSTS;
    static constexpr int CPW = NI / NW;
    static_assert(CPW * NW == NI, "copies must divide evenly over the wavefronts");
    static constexpr int STAGE = 2 * S::KBYTES + S::VBYTES;
    int row[CPW], off[CPW], dst[CPW];

    __device__ __forceinline__ void init(int wid, int lane) {
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int j = wid + i * NW;
            if (j < 2 * S::KINSTS) {
                const int jj = j % S::KINSTS;
                const int q = jj * 64 + lane, t = q / S::KPPR, cs = q % S::KPPR;
                row[i] = t;
                off[i] = S::kslot(t, cs) * 8;
                dst[i] = (j < S::KINSTS ? 0 : S::KBYTES) + jj * 1024;
            } else {
                const int jj = j - 2 * S::KINSTS;
                const int q = jj * 64 + lane, d = q / S::VPPR, cs = q % S::VPPR;
                row[i] = d;
                off[i] = S::vslot(d, cs) * 8;
                dst[i] = 2 * S::KBYTES + jj * 1024;
            }
        }
    }
    __device__ __forceinline__ void issue(char* stage, const uint16_t* Kg, const uint16_t* Vg, const uint16_t* Ktg,
                                          int tb, int nmax, int n_pad, int wid) const {
        tb = min(max(tb, 0), n_pad - TT);
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int j = wid + i * NW;               // wavefront-uniform
            const uint16_t* src = j < S::KINSTS       ? Kg + (size_t)min(tb + row[i], nmax) * D + off[i]
                                  : j < 2 * S::KINSTS ? Vg + (size_t)min(tb + row[i], nmax) * D + off[i]
                                                      : Ktg + (size_t)row[i] * n_pad + tb + off[i];
            __builtin_amdgcn_global_load_lds(src, stage + dst[i], 16, 0, 0);
        }
    }
};

// dZ of one 32-token half of a tile from its S^T and dP^T accumulators: P =
// 2^(S c1 + off) with off = bias - lse in log2 units, zero past lim on the diagonal
// (MASK; element e of k16 step u is token tk0 + 16 u + e); returns the sum of dZ.
template <bool MASK>
__device__ __forceinline__ float dz_half(const f32x16& sacc, const f32x16& dpacc, float c1, float off, float dlt,
                                         int tk0, int lim, bf16x8 (&dz)[2]) {
    float part = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float pv = fast_exp2(fmaf(sacc[8 * u + e], c1, off));
            if (MASK && tk0 + 16 * u + e > lim) pv = 0.f;
            const float z = pv * (dpacc[8 * u + e] - dlt);
            part += z;
            dz[u][e] = (__bf16)z;
        }
    return part;
}

// NW wavefronts of one 32-pair block each; the tile geometry is the forward's
// (TT = 64 tokens when B is a multiple of 64, else 32).
template <int D, int TT, int NW>
__global__ __launch_bounds__(64 * NW) void prior_attn_dq_kernel(PrefillParams p, DqExtra x) {
    typedef BfTiles<D, TT> S;
    typedef DqCopier<D, TT, NW> CP;
    constexpr int NS = D / 16;     // k16 steps over d
    constexpr int NB = TT / 32;    // 32-token blocks of S^T
    constexpr int ND = D / 32;     // 32-wide d blocks of dQ^T
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* ring = smem;
    TileTables tabs;
    tabs.carve(smem + 2 * CP::STAGE, p.T_c);

    constexpr int nthr = 64 * NW;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hl = lane >> 5;
    const int r = blockIdx.y, bi = blockIdx.z;
    const int g = p.g, lg = p.log2g, R_t = p.R_t;
    const int row0 = (gridDim.x - 1 - blockIdx.x) * R_t;
    const int cq = row0 / p.B;
    const int nvis = p.causal ? min(cq, p.T_c) : p.T_c;
    const int last_row = min(row0 + R_t, p.n) - 1;
    const size_t bhkv = (size_t)bi * p.h_kv + r;
    const uint16_t* Kg = static_cast<const uint16_t*>(p.K) + bhkv * (size_t)p.n * D;
    const uint16_t* Vg = static_cast<const uint16_t*>(p.V) + bhkv * (size_t)p.n * D;
    const uint16_t* Ktg = x.Kt + bhkv * (size_t)D * p.n_pad;
    const int U = tabs.build(p, bhkv, row0, nvis, tid, nthr);

    // ---- the lane's (row, head) pair ----
    const int P = wid * 32 + l32;
    const int jrow = P >> lg, my_row = row0 + jrow;
    const int hh = r * g + (P & (g - 1));
    const bool live = wid * 32 < g * R_t;                     // wavefront-uniform
    const bool pok = live && jrow < R_t && my_row < p.n;
    ListCursor lc;
    lc.init(p, bhkv * p.n + (pok ? my_row : 0), pok);
    const size_t prow = ((size_t)bi * p.h_q + hh) * p.n + (pok ? my_row : 0);
    bf16x8 qf[NS], df[NS];
    {
        const uint16_t* qrow = static_cast<const uint16_t*>(p.Q) + prow * D + 8 * hl;
        const uint16_t* drow = x.dO + prow * D + 8 * hl;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
            df[s] = *reinterpret_cast<const bf16x8*>(drow + 16 * s);
            if (!pok) { qf[s] = bf16x8{}; df[s] = bf16x8{}; }
        }
    }
    const float lse_raw = pok ? x.lse[prow] : 0.f;
    // a row with nothing visible has lse = -inf and no gradient: P = 0 everywhere
    const float lse2 = (lse_raw == -INFINITY) ? INFINITY : lse_raw * kLog2e;
    const float dlt = pok ? x.delta[prow] : 0.f;

    f32x16 dq[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;
    float dbsum = 0.f;

    TileSteps st;
    st.init(p, U, cq, last_row, TT);
    const int nmax = p.n - 1;
    CP cp;
    cp.init(wid, lane);
    const int krow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
    const float c1 = p.scale_log2;
    const int lim = p.causal ? my_row : p.n - 1;

    int tb_cur, c_cur, tb_nxt, c_nxt;
    st.at(tabs.ulist, 0, tb_cur, c_cur);
    st.at(tabs.ulist, 1, tb_nxt, c_nxt);
    if (st.nsteps > 0) cp.issue(ring, Kg, Vg, Ktg, tb_cur, nmax, p.n_pad, wid);
    wait_tile_copies();
    __syncthreads();
    for (int k = 0; k < st.nsteps; ++k) {
        // dQ stays in accumulation registers across steps (both sides of the
        // step's skip branch), so no step copies it in and out
#pragma unroll
        for (int db = 0; db < ND; ++db) asm volatile("" : "+a"(dq[db]));
        const bool routed = k < st.nrouted;
        const bool last = k % st.SPC == st.SPC - 1;
        const int epos = lc.pos;                   // list position of chunk c_cur if routed
        const float bias2 = routed ? lc.take(c_cur, last) : 0.f;
        const bool hit = bias2 > -INFINITY;
        const bool run = live && (!routed || ballot(hit) != 0);
        if (k + 1 < st.nsteps)
            cp.issue(ring + ((k + 1) & 1) * CP::STAGE, Kg, Vg, Ktg, tb_nxt, nmax, p.n_pad, wid);
        int tb_nn, c_nn;
        st.at(tabs.ulist, k + 2, tb_nn, c_nn);
        const char* kt = ring + (k & 1) * CP::STAGE;
        const char* vt = kt + S::KBYTES;
        const char* ktt = kt + 2 * S::KBYTES;
        const int tb = tb_cur;
        if (run) {
            // one 32-token half of the tile at a time: S^T = K Q^T and dP^T = V dO^T,
            // then P from the forward's lse and dZ = P (dP - Δ), then dQ^T += K^T dZ^T
            // over the half's two k16 steps (token of element e of k16 step s is
            // tb + 16 s + 8 hl + e)
            const float off = bias2 - lse2;
            float part = 0.f;
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) {
                f32x16 sacc, dpacc;
#pragma unroll
                for (int i = 0; i < 16; ++i) { sacc[i] = 0.f; dpacc[i] = 0.f; }
                const int t = 32 * blk + krow;
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const int o = t * S::KROWB + S::kslot(t, 2 * s + hl) * 16;
                    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kt + o);
                    const bf16x8 va = *reinterpret_cast<const bf16x8*>(vt + o);
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], sacc, 0, 0, 0);
                    dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, df[s], dpacc, 0, 0, 0);
                }
                bf16x8 dz[2];
                part += routed ? dz_half<false>(sacc, dpacc, c1, off, dlt, 0, 0, dz)
                               : dz_half<true>(sacc, dpacc, c1, off, dlt, tb + 32 * blk + 8 * hl, lim, dz);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int sk = 2 * blk + u;
                    bf16x8 kta[ND];
#pragma unroll
                    for (int db = 0; db < ND; ++db) {
                        const int d = 32 * db + l32;
                        kta[db] = *reinterpret_cast<const bf16x8*>(ktt + d * S::VROWB + S::vslot(d, 2 * sk + hl) * 16);
                    }
#pragma unroll
                    for (int db = 0; db < ND; ++db)
                        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kta[db], dz[u], dq[db], 0, 0, 0);
                }
            }
            dbsum += part;
            // the chunk's bias gradient: its tokens (both lane halves, all its steps)
            // and the g heads of the row (g consecutive lanes)
            if (routed && last) {
                float v = pair32_sum(dbsum);
                for (int m = 1; m < g; m <<= 1) v += shfl_xor(v, m);
                if (pok && hit && hl == 0 && (P & (g - 1)) == 0)
                    x.dbias[(bhkv * p.n + my_row) * p.list_cap + epos] = v;
            }
        }
        if (last || !routed) dbsum = 0.f;
        wait_tile_copies();
        __syncthreads();
        tb_cur = tb_nxt; c_cur = c_nxt;
        tb_nxt = tb_nn; c_nxt = c_nn;
    }

    if (pok) {
        const size_t obase = prow * D;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int d0 = 32 * db + 8 * a + 4 * hl;
                f32x4 o;
                o[0] = dq[db][4 * a] * x.scale; o[1] = dq[db][4 * a + 1] * x.scale;
                o[2] = dq[db][4 * a + 2] * x.scale; o[3] = dq[db][4 * a + 3] * x.scale;
                *reinterpret_cast<f32x4*>(x.dQ + obase + d0) = o;
            }
    }
}

// ---------------------------------------------------------------------------------
// dK and dV (key-major)
// ---------------------------------------------------------------------------------

struct DkvParams {
    const uint16_t* Q; const uint16_t* dO;       // bf16 [b, h_q, n, D]
    const uint16_t* K; const uint16_t* V;        // bf16 [b, h_kv, n, D]
    const float* lse; const float* delta;        // [b, h_q, n]
    const int32_t* inv_row; const float* inv_bias; const int32_t* coff;
    float* dK; float* dV;                        // [b, h_kv, n, D], zero on entry
    const int4* items;                           // work items (b*h_kv, chunk tile, segment)
    int32_t* counters;                           // [0] next item, [1] item count
    int h_q, h_kv, n, B, T_c, causal, g, log2g, seg_rows;
    float c1, scale;                             // log2(e)/sqrt(d), 1/sqrt(d)
};

// 64-token tiles per chunk: B/64, or one (half used) for B = 32
__host__ __device__ __forceinline__ int tiles_per_chunk(int B) { return B >= 64 ? B / 64 : 1; }

// Rows of the row sequence of 64-token tile cs of chunk cs / SUB of KV group bhk
// (SUB = tiles_per_chunk(B)): the routed rows of the chunk, then its diagonal rows at
// or after the tile (causal; non-causal: every row for the tail tile). The tile's
// tokens are t0 .. tend-1 (tend - t0 < 64 for a 32-token chunk or the tail).
struct TileRows { int c, t0, tend, rbase, nrouted, dlo, dhi; };
__device__ __forceinline__ TileRows tile_rows(const int32_t* coff, size_t bhk, int cs, int n, int B, int T,
                                              int causal) {
    TileRows r;
    const int SUB = tiles_per_chunk(B);
    r.c = cs / SUB;
    r.t0 = r.c * B + 64 * (cs % SUB);
    r.tend = min(min(r.t0 + 64, r.c * B + B), n);
    r.rbase = 0; r.nrouted = 0; r.dlo = 0; r.dhi = 0;
    if (r.t0 >= n) return r;
    if (r.c < T) {
        r.rbase = coff[bhk * (T + 1) + r.c];
        r.nrouted = coff[bhk * (T + 1) + r.c + 1] - r.rbase;
    }
    if (causal) { r.dlo = r.t0; r.dhi = min(r.c * B + B, n); }
    else if (r.c == T) { r.dlo = 0; r.dhi = n; }
    return r;
}

// Exclusive prefix sum over a 1024-thread workgroup (tmp: 16 ints of LDS).
__device__ __forceinline__ int block_scan1024(int v, int* tmp, int& total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __builtin_amdgcn_ds_bpermute(((lane - o) & 63) << 2, x);
        if (lane >= o) x += y;
    }
    if (lane == 63) tmp[wid] = x;
    __syncthreads();
    int off = 0;
    total = 0;
    for (int w = 0; w < 16; ++w) {
        off += w < wid ? tmp[w] : 0;
        total += tmp[w];
    }
    __syncthreads();
    return off + x - v;
}

// The work items of the dK/dV kernel: every 64-token tile of every chunk (and the
// tail) with its row sequence cut into segments of seg_rows rows, segment 0 at the
// end of the sequence; tiles in ascending chunk order (under a causal mask the early
// chunks have the longest sequences, so the largest items go first). One workgroup.
__global__ __launch_bounds__(1024) void dkv_items_kernel(const int32_t* coff, int4* items, int32_t* counters,
                                                         int bh, int n, int B, int T, int causal, int seg_rows) {
    __shared__ int tmp[16];
    const int per_bh = (T + 1) * tiles_per_chunk(B);
    const int E = bh * per_bh;
    const int per = (E + 1023) / 1024;
    const int e0 = min((int)threadIdx.x * per, E), e1 = min(e0 + per, E);
    auto nseg = [&](int e) {
        const TileRows r = tile_rows(coff, (size_t)(e / per_bh), e % per_bh, n, B, T, causal);
        if (r.t0 >= n) return 0;
        const int rows = r.nrouted + max(r.dhi - r.dlo, 0);
        return (rows + seg_rows - 1) / seg_rows;
    };
    int sum = 0;
    for (int e = e0; e < e1; ++e) sum += nseg(e);
    int total;
    int o = block_scan1024(sum, tmp, total);
    for (int e = e0; e < e1; ++e) {
        const int k = nseg(e);
        for (int s = 0; s < k; ++s) items[o + s] = make_int4(e / per_bh, e % per_bh, s, 0);
        o += k;
    }
    if (threadIdx.x == 0) { counters[0] = 0; counters[1] = total; }
}

// A stage: Q and dO of a group of 64 (row, head) pairs, both row-major [64][D] with
// the "K" swizzle; pair index = row_slot * g + head.
template <int D>
struct DkvStage {
    typedef BfTiles<D, 64> S;
    static constexpr int BYTES = 2 * S::KBYTES;
    static constexpr int NI = 2 * S::KINSTS;                     // wavefront copies
    static constexpr int NST = 3;                                // ring stages
};

// The chunk's row sequence: the routed rows (inverted list, ascending), then the
// diagonal rows dlo, dlo+1, ...; a workgroup walks its segment [j0, j1) from the
// end, so the workgroups running at one time start on the same late rows. Row m of
// the walk is entry j = j1 - 1 - m.
struct RowSeq {
    const int32_t* irow; const float* ibias;
    const int32_t* safe_i; const float* safe_f;  // readable stand-ins when nothing is routed
    int nrouted, dlo, j0, j1;
    __device__ __forceinline__ int entry(int m) const { return j1 - 1 - m; }
    // list slots read for entry j (clamped into the list: always a valid address)
    __device__ __forceinline__ const int32_t* row_src(int j) const {
        return nrouted > 0 ? irow + min(max(j, 0), nrouted - 1) : safe_i;
    }
    __device__ __forceinline__ const float* bias_src(int j) const {
        return nrouted > 0 ? ibias + min(max(j, 0), nrouted - 1) : safe_f;
    }
    __device__ __forceinline__ bool valid(int j) const { return j >= j0; }
    __device__ __forceinline__ bool routed(int j) const { return j >= j0 && j < nrouted; }
    // the row of entry j given the list value loaded for it
    __device__ __forceinline__ int row(int j, int loaded) const {
        return routed(j) ? loaded : (valid(j) ? dlo + (j - nrouted) : 0);
    }
};

typedef short i16x4 __attribute__((ext_vector_type(4)));

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives as element k the
// 16-bit element i % 4 of the 8 bytes that lane 4k + i/4 of the group addressed.
// The N reads of one call go out together and are waited for inside the same asm
// block (the compiler's own form of this read makes it wait for every copy into
// LDS in flight first, which stalls the copy pipeline).
template <int N>
__device__ __forceinline__ void lds_read_tr16(const uint32_t (&a)[N], i16x4 (&r)[N]) {
    static_assert(N == 8 || N == 16, "8 or 16 reads");
    if constexpr (N == 16) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %16\n ds_read_b64_tr_b16 %1, %17\n ds_read_b64_tr_b16 %2, %18\n"
            "ds_read_b64_tr_b16 %3, %19\n ds_read_b64_tr_b16 %4, %20\n ds_read_b64_tr_b16 %5, %21\n"
            "ds_read_b64_tr_b16 %6, %22\n ds_read_b64_tr_b16 %7, %23\n ds_read_b64_tr_b16 %8, %24\n"
            "ds_read_b64_tr_b16 %9, %25\n ds_read_b64_tr_b16 %10, %26\n ds_read_b64_tr_b16 %11, %27\n"
            "ds_read_b64_tr_b16 %12, %28\n ds_read_b64_tr_b16 %13, %29\n ds_read_b64_tr_b16 %14, %30\n"
            "ds_read_b64_tr_b16 %15, %31\n s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
              "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]),
              "=&v"(r[14]), "=&v"(r[15])
            : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
              "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]), "v"(a[14]), "v"(a[15])
            : "memory");
    } else {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8\n ds_read_b64_tr_b16 %1, %9\n ds_read_b64_tr_b16 %2, %10\n"
            "ds_read_b64_tr_b16 %3, %11\n ds_read_b64_tr_b16 %4, %12\n ds_read_b64_tr_b16 %5, %13\n"
            "ds_read_b64_tr_b16 %6, %14\n ds_read_b64_tr_b16 %7, %15\n s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
              "=&v"(r[7])
            : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
            : "memory");
    }
}



// LDS of one work item: the tile ring, the tables and the loaded-value rings.
template <int D>
constexpr size_t dkv_item_lds_bytes() {
    return (size_t)DkvStage<D>::NST * DkvStage<D>::BYTES + 3 * 128 * 4 + (8 + 8 + 4 + 4) * 64 * 4;
}

// Piece slot of the Q and dO tiles of the dK/dV kernel: 16-byte piece c of row t sits
// at slot c ^ swz(t). At d = 128 swz swaps the two 2-bit halves of t mod 16: the 16
// rows of a row read still fill 16 distinct slots, and the 4 rows x 4 pieces of a
// transposing read do too (with t mod 16 itself they fold onto 4 slots, four lanes'
// words per bank).
template <int D>
__device__ __forceinline__ int dkv_slot(int t, int c) {
    if constexpr (D == 128) return c ^ (((t & 3) << 2) | ((t >> 2) & 3));
    else return BfTiles<D, 64>::kslot(t, c);
}

// The 16 transposing reads of k16 step S at d = 128, read (db, t) from its own
// per-lane address a[2 db + t] (the Q tile; the dO tile is 16 KiB above, step S at
// +4096 S, both immediates). Reads 0..7: dO, 8..15: Q.
template <int S>
__device__ __forceinline__ void tr_reads_d128_sw(const uint32_t (&a)[8], i16x4 (&r)[16]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16 offset:%24\n ds_read_b64_tr_b16 %1, %17 offset:%24\n"
        "ds_read_b64_tr_b16 %2, %18 offset:%24\n ds_read_b64_tr_b16 %3, %19 offset:%24\n"
        "ds_read_b64_tr_b16 %4, %20 offset:%24\n ds_read_b64_tr_b16 %5, %21 offset:%24\n"
        "ds_read_b64_tr_b16 %6, %22 offset:%24\n ds_read_b64_tr_b16 %7, %23 offset:%24\n"
        "ds_read_b64_tr_b16 %8, %16 offset:%25\n ds_read_b64_tr_b16 %9, %17 offset:%25\n"
        "ds_read_b64_tr_b16 %10, %18 offset:%25\n ds_read_b64_tr_b16 %11, %19 offset:%25\n"
        "ds_read_b64_tr_b16 %12, %20 offset:%25\n ds_read_b64_tr_b16 %13, %21 offset:%25\n"
        "ds_read_b64_tr_b16 %14, %22 offset:%25\n ds_read_b64_tr_b16 %15, %23 offset:%25\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
          "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]),
          "=&v"(r[14]), "=&v"(r[15])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
          "n"(16384 + 4096 * S), "n"(4096 * S)
        : "memory");
}

// One work item: up to 64 tokens of one chunk (tile cs) of KV group bhk against
// segment seg of its row sequence. Tokens from tend on (a 32-token chunk's second
// half, the sequence end) are computed on and never written.
template <int D>
__device__ __forceinline__ void dkv_item(const DkvParams& p, size_t bhk, int cs, int seg, char* smem) {
    typedef BfTiles<D, 64> S;
    typedef DkvStage<D> ST;
    constexpr int NS = D / 16, ND = D / 32;
    constexpr int CPW = ST::NI / 4;
    char* ring = smem;                                                  // NST stages
    float* t_off = reinterpret_cast<float*>(smem + ST::NST * ST::BYTES);  // [2][64] bias2 - lse2
    int* t_lim = reinterpret_cast<int*>(t_off + 128);                  // [2][64] last visible token
    float* t_dlt = reinterpret_cast<float*>(t_lim + 128);              // [2][64] Δ
    int* r_row = reinterpret_cast<int*>(t_dlt + 128);                  // [8][64] list rows as loaded
    float* r_bias = reinterpret_cast<float*>(r_row + 512);             // [8][64] list biases as loaded
    float* r_lse = r_bias + 512;                                       // [4][64] lse as loaded
    float* r_dlt = r_lse + 256;                                        // [4][64] Δ as loaded

    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hl = lane >> 5;
    const int bi = (int)(bhk / p.h_kv), hk = (int)(bhk % p.h_kv);
    const int T = p.T_c;
    const TileRows tr = tile_rows(p.coff, bhk, cs, p.n, p.B, T, p.causal);
    const int t0 = tr.t0, tend = tr.tend, rbase = tr.rbase, nrouted = tr.nrouted, dlo = tr.dlo, dhi = tr.dhi;
    if (t0 >= p.n) return;
    const int nrows = nrouted + max(dhi - dlo, 0);
    // segment 0 holds the end of the sequence
    const int j1 = nrows - seg * p.seg_rows, j0 = max(j1 - p.seg_rows, 0);
    if (j1 <= 0) return;
    const int g = p.g, lg = p.log2g, RG = 64 >> lg;
    const int ngroups = (j1 - j0 + RG - 1) / RG;
    RowSeq rs;
    rs.irow = p.inv_row + bhk * (size_t)p.n * T + rbase;
    rs.ibias = p.inv_bias + bhk * (size_t)p.n * T + rbase;
    rs.safe_i = p.coff; rs.safe_f = p.lse;
    rs.nrouted = nrouted; rs.dlo = dlo; rs.j0 = j0; rs.j1 = j1;

    // ---- K and V of the wavefront's 32 tokens as B operands (token = lane column) ----
    const int tbk = wid & 1, half = wid >> 1;
    const int tok = t0 + 32 * tbk + l32;
    bf16x8 kreg[NS], vreg[NS];
    {
        const size_t kb = (bhk * p.n + min(tok, p.n - 1)) * D + 8 * hl;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            kreg[s] = *reinterpret_cast<const bf16x8*>(p.K + kb + 16 * s);
            vreg[s] = *reinterpret_cast<const bf16x8*>(p.V + kb + 16 * s);
            if (tok >= p.n) { kreg[s] = bf16x8{}; vreg[s] = bf16x8{}; }
        }
    }

    // ---- the table pipeline ----
    // Every value a step needs from memory besides the Q / dO tiles arrives by a copy
    // straight into LDS, so no register waits for a load across steps. In step k:
    //   wavefront 0 / 1 copies the list rows / biases of group k+5 (64 lanes = the
    //   group's 64 pairs) into ring slot (k+5) % 8;
    //   wavefront 2 / 3 copies lse / Δ of group k+3 (rows from slot (k+3) % 8) into
    //   ring slot (k+3) % 4;
    //   all wavefronts copy the Q / dO tiles of group k+2 (rows from slot (k+2) % 8);
    //   lanes 0..15 of each wavefront turn the loaded values of group k+1 into its
    //   tables (slot (k+1) % 2).
    // Each wavefront so issues one table copy plus its tile copies per step; the wait
    // at the end of step k leaves exactly those in flight, so everything older has
    // landed and every read above finds its data.
    const int pr_slot = lane >> lg, pr_head = lane & (g - 1);    // pair = lane (table copies)
    const size_t hbase_l = ((size_t)bi * p.h_q + (size_t)hk * g + pr_head) * p.n;
    auto table_copy = [&](int k) {
        if (wid < 2) {
            const int m = k + 5;
            const int j = rs.entry(m * RG + pr_slot);
            const void* src = wid == 0 ? (const void*)rs.row_src(j) : (const void*)rs.bias_src(j);
            char* dst = reinterpret_cast<char*>(wid == 0 ? r_row + (m & 7) * 64 : reinterpret_cast<int*>(r_bias) + (m & 7) * 64);
            __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
        } else {
            const int m = k + 3;
            const int j = rs.entry(m * RG + pr_slot);
            const int row = rs.row(j, r_row[(m & 7) * 64 + lane]);
            const float* src = (wid == 2 ? p.lse : p.delta) + hbase_l + row;
            char* dst = reinterpret_cast<char*>((wid == 2 ? r_lse : r_dlt) + (m & 3) * 64);
            __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
        }
    };
    const bool TL = lane < 16;
    const int tp = 16 * wid + (lane & 15);
    const int tslot = tp >> lg;
    auto make_tables = [&](int m) {
        const int j = rs.entry(m * RG + tslot);
        const int row = rs.row(j, r_row[(m & 7) * 64 + tp]);
        const float lse = r_lse[(m & 3) * 64 + tp];
        const float l2 = (lse == -INFINITY) ? INFINITY : lse * kLog2e;
        const float bias = rs.routed(j) ? r_bias[(m & 7) * 64 + tp] : 0.f;
        const int slot = m & 1;
        t_off[slot * 64 + tp] = rs.valid(j) ? bias * kLog2e - l2 : -INFINITY;
        t_lim[slot * 64 + tp] = !rs.valid(j) ? -1 : rs.routed(j) ? 0x7fffffff : (p.causal ? row : p.n - 1);
        t_dlt[slot * 64 + tp] = rs.valid(j) ? r_dlt[(m & 3) * 64 + tp] : 0.f;
    };

    // ---- copies of a group's Q / dO stage (rows from its ring slot) ----
    const uint16_t* Qg = p.Q + ((size_t)bi * p.h_q + (size_t)hk * g) * p.n * D;
    const uint16_t* dOg = p.dO + ((size_t)bi * p.h_q + (size_t)hk * g) * p.n * D;
    auto issue = [&](char* stage, int m) {
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int j = wid + 4 * i;                 // wavefront-uniform
            const int jj = j % S::KINSTS;
            const int q = jj * 64 + lane, t = q / S::KPPR, cc = q % S::KPPR;
            const int e = rs.entry(m * RG + (t >> lg));
            const int row = min(max(rs.row(e, r_row[(m & 7) * 64 + t]), 0), p.n - 1);
            const size_t o = ((size_t)(t & (g - 1)) * p.n + row) * D + dkv_slot<D>(t, cc) * 8;
            // source and destination as named pointers: a conditional expression
            // inside the builtin's argument list loses the kernel's host stub
            const uint16_t* src = (j < S::KINSTS ? Qg : dOg) + o;
            char* dst = stage + (j < S::KINSTS ? 0 : S::KBYTES) + jj * 1024;
            __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
        }
    };

    // ---- prologue (plain loads): list values of groups 0..4, lse / Δ of groups
    // 0..2, tables of group 0, tiles of groups 0 and 1 ----
    for (int x = tid; x < 5 * 64; x += 256) {
        const int m = x >> 6, pp = x & 63;
        const int j = rs.entry(m * RG + (pp >> lg));
        r_row[(m & 7) * 64 + pp] = *rs.row_src(j);
        r_bias[(m & 7) * 64 + pp] = *rs.bias_src(j);
    }
    __syncthreads();
    for (int x = tid; x < 3 * 64; x += 256) {
        const int m = x >> 6, pp = x & 63;
        const int j = rs.entry(m * RG + (pp >> lg));
        const int row = rs.row(j, r_row[(m & 7) * 64 + pp]);
        const size_t hb = ((size_t)bi * p.h_q + (size_t)hk * g + (pp & (g - 1))) * p.n;
        r_lse[(m & 3) * 64 + pp] = p.lse[hb + row];
        r_dlt[(m & 3) * 64 + pp] = p.delta[hb + row];
    }
    __syncthreads();
    if (TL) make_tables(0);
    issue(ring, 0);
    if (ngroups > 1) issue(ring + ST::BYTES, 1);
    wait_vm<0>();
    __syncthreads();

    f32x16 dk[ND], dv[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) { dk[db][i] = 0.f; dv[db][i] = 0.f; }
    // A row l32 presents pair (bits 2 and 3 swapped): accumulator element 8s + e of a
    // lane is then pair 16s + 8hl + e, the k-slot order of the pair contraction
    const int prow_a = 32 * half + ((l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1));
    // transposing reads of the B operands: lane group G = lane/16 covers columns
    // 16(G&1) .. +15 of a 32-wide d block and k-slot half hl; its lane 4k + q reads
    // pair base + k at d offset 4q
    const int tr_k = (lane & 15) >> 2, tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    // d = 128: the lane's offset of read (db, t) of k16 step 0 inside the Q tile
    // (row 32 half + 8 hl + 4 t + tr_k, piece 4 db + tr_d / 8, slot by dkv_slot)
    uint32_t tr_off[8];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int pr = 32 * half + 8 * hl + 4 * t + tr_k;
            tr_off[2 * db + t] = pr * 256 + 16 * dkv_slot<128>(pr, 4 * db + (tr_d >> 3)) + 8 * (lane & 1);
        }
    const float c1 = p.c1;
    char* st_cur = ring;
    char* st_nxt = ring + ST::BYTES;
    char* st_nn = ring + 2 * ST::BYTES;

    for (int k = 0; k < ngroups; ++k) {
        // dK and dV stay in accumulation registers across groups
#pragma unroll
        for (int db = 0; db < ND; ++db) asm volatile("" : "+a"(dk[db]), "+a"(dv[db]));
        table_copy(k);
        const bool more = k + 2 < ngroups;
        if (more) issue(st_nn, k + 2);

        const char* qt = st_cur;
        const char* dot = qt + S::KBYTES;
        // S = Q K^T and dP = dO V^T for this wavefront's 32 pairs x 32 tokens
        f32x16 sacc, dpacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) { sacc[i] = 0.f; dpacc[i] = 0.f; }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int o = prow_a * S::KROWB + dkv_slot<D>(prow_a, 2 * s + hl) * 16;
            const bf16x8 qa8 = *reinterpret_cast<const bf16x8*>(qt + o);
            const bf16x8 da8 = *reinterpret_cast<const bf16x8*>(dot + o);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa8, kreg[s], sacc, 0, 0, 0);
            dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da8, vreg[s], dpacc, 0, 0, 0);
        }
        // P and dZ per pair: element 8s + e is pair 32 half + 16 s + 8 hl + e
        const int tb = (k & 1) * 64 + 32 * half + 8 * hl;
        bf16x8 pa[2], za[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const f32x4 o0 = *reinterpret_cast<const f32x4*>(t_off + tb + 16 * s);
            const f32x4 o1 = *reinterpret_cast<const f32x4*>(t_off + tb + 16 * s + 4);
            const u32x4 m0 = *reinterpret_cast<const u32x4*>(t_lim + tb + 16 * s);
            const u32x4 m1 = *reinterpret_cast<const u32x4*>(t_lim + tb + 16 * s + 4);
            const f32x4 d0 = *reinterpret_cast<const f32x4*>(t_dlt + tb + 16 * s);
            const f32x4 d1 = *reinterpret_cast<const f32x4*>(t_dlt + tb + 16 * s + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float off = e < 4 ? o0[e & 3] : o1[e & 3];
                const int lim = (int)(e < 4 ? m0[e & 3] : m1[e & 3]);
                const float dl = e < 4 ? d0[e & 3] : d1[e & 3];
                float pv = fast_exp2(fmaf(sacc[8 * s + e], c1, off));
                if (tok > lim) pv = 0.f;
                const float z = pv * (dpacc[8 * s + e] - dl);
                pa[s][e] = (__bf16)pv;
                za[s][e] = (__bf16)z;
            }
        }
        // dV += P^T dO and dK += dZ^T Q over the 32 pairs; B operands by transposing
        // reads of the row-major tiles
        const uint32_t qt_lds = lds_addr(qt);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            // reads 0 .. 2ND-1: dO, then 2ND .. 4ND-1: Q; read 2 db + t of a tensor
            // holds pairs base + 4t .. +3 of d block db
            i16x4 x[4 * ND];
            if constexpr (D == 128) {
                uint32_t a8[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) a8[u] = qt_lds + tr_off[u];
                if (s == 0) tr_reads_d128_sw<0>(a8, x);
                else tr_reads_d128_sw<1>(a8, x);
            } else {
                uint32_t a[4 * ND];
#pragma unroll
                for (int db = 0; db < ND; ++db) {
                    const int d = 32 * db + tr_d;
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const int pr = 32 * half + 16 * s + 8 * hl + 4 * t + tr_k;
                        const uint32_t o = pr * S::KROWB + dkv_slot<D>(pr, d >> 3) * 16 + ((d >> 2) & 1) * 8;
                        a[2 * db + t] = qt_lds + S::KBYTES + o;
                        a[2 * ND + 2 * db + t] = qt_lds + o;
                    }
                }
                lds_read_tr16<4 * ND>(a, x);
            }
            bf16x8 ob[ND], qb8[ND];
#pragma unroll
            for (int db = 0; db < ND; ++db) {
                ob[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x[2 * db], x[2 * db + 1], 0, 1, 2, 3, 4, 5, 6, 7));
                qb8[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x[2 * ND + 2 * db], x[2 * ND + 2 * db + 1],
                                                                             0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int db = 0; db < ND; ++db) {
                dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[s], ob[db], dv[db], 0, 0, 0);
                dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(za[s], qb8[db], dk[db], 0, 0, 0);
            }
        }

        // tables of group k+1 (their slot was last read in step k-1)
        if (TL) make_tables(k + 1);
        // everything issued before this step has landed; this step's table copy and
        // tile copies may stay in flight
        if (more) wait_vm<CPW + 1>();
        else wait_vm<1>();
        barrier_lds();
        char* t = st_cur; st_cur = st_nxt; st_nxt = st_nn; st_nn = t;
    }

    wait_vm<0>();      // no copy into LDS outlives the loop

    // ---- add the partials: element i of lane l is token 8(i/4) + 4hl + i%4 of the
    // wavefront's 32, column d = 32 db + l32 ----
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = t0 + 32 * tbk + 8 * (i >> 2) + 4 * hl + (i & 3);
            if (t < tend) {
                const size_t o = (bhk * p.n + t) * D + 32 * db + l32;
                unsafeAtomicAdd(p.dK + o, dk[db][i] * p.scale);
                unsafeAtomicAdd(p.dV + o, dv[db][i]);
            }
        }
}

// Persistent: each workgroup takes work items from a counter until none is left.
template <int D>
__global__ __launch_bounds__(256) void prior_attn_dkv_kernel(DkvParams p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    int* s_item = reinterpret_cast<int*>(smem + dkv_item_lds_bytes<D>());
    const int nitems = p.counters[1];
    for (;;) {
        if (threadIdx.x == 0) *s_item = atomicAdd(p.counters, 1);
        __syncthreads();
        const int it = *s_item;
        __syncthreads();
        if (it >= nitems) break;
        const int4 w = p.items[it];
        dkv_item<D>(p, (size_t)w.x, w.y, w.z, smem);
    }
}

// ---------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------

static constexpr int kDqWaves = 4;
static constexpr size_t kBwdMaxLds = 160 * 1024;

static size_t dq_lds_bytes(int d, int B, int T_c) {
    const bool t64 = B % 64 == 0;
    const size_t stage = d == 64 ? (t64 ? DqCopier<64, 64, kDqWaves>::STAGE : DqCopier<64, 32, kDqWaves>::STAGE)
                                 : (t64 ? DqCopier<128, 64, kDqWaves>::STAGE : DqCopier<128, 32, kDqWaves>::STAGE);
    return 2 * stage + TileTables::bytes(T_c);
}
static size_t dkv_lds_bytes(int d) {
    return (d == 64 ? dkv_item_lds_bytes<64>() : dkv_item_lds_bytes<128>()) + 16;
}

int backward_tile_rows(int g, int B, int T_c, int d) {
    if (g < 1 || g > 16 || (g & (g - 1)) != 0 || B % 32 != 0 || (d != 64 && d != 128)) return 0;
    if (dq_lds_bytes(d, B, T_c) > kBwdMaxLds) return 0;
    return std::min(32 * kDqWaves / g, std::min(B, 64));      // a query tile stays inside one chunk
}

// Rows per dK/dV work item and an upper bound on the number of items: over the tiles
// of one KV group the sequences hold each routed entry SUB = tiles_per_chunk(B) times
// (at most n floor(n/B) entries) plus diagonal rows (at most SUB (n + B)); every tile
// adds at most one partial segment.
static int dkv_seg_rows(int g) { return 8192 / g; }
static size_t dkv_item_bound(int b, int h_q, int h_kv, int n, int B) {
    const size_t T = (size_t)(n / B), SUB = (size_t)tiles_per_chunk(B), seg = (size_t)dkv_seg_rows(h_q / h_kv);
    return (size_t)b * h_kv * ((T + 1) * SUB + (SUB * ((size_t)n * T + n + B) + seg - 1) / seg);
}

namespace {
struct BwdLayout {
    size_t kt, dob, delta, hist, coff, inv_row, inv_bias, items, counters, total;
};
size_t up256(size_t x) { return (x + 255) / 256 * 256; }
BwdLayout bwd_layout(int b, int h_q, int h_kv, int n, int d, int B) {
    BwdLayout L;
    const size_t T = (size_t)(n / B), nblk = ((size_t)n + 63) / 64;
    size_t o = 0;
    L.kt = o;       o += up256(prefill_workspace_bytes(b, h_kv, n, d));
    L.dob = o;      o += up256((size_t)b * h_q * n * d * 2);
    L.delta = o;    o += up256((size_t)b * h_q * n * 4);
    L.hist = o;     o += up256((size_t)b * h_kv * T * nblk * 4);
    L.coff = o;     o += up256((size_t)b * h_kv * (T + 1) * 4);
    L.inv_row = o;  o += up256((size_t)b * h_kv * n * T * 4);
    L.inv_bias = o; o += up256((size_t)b * h_kv * n * T * 4);
    L.items = o;    o += up256(dkv_item_bound(b, h_q, h_kv, n, B) * 16);
    L.counters = o; o += 256;
    L.total = o;
    return L;
}
}  // namespace

size_t backward_workspace_bytes(int b, int h_q, int h_kv, int n, int d, int B) {
    return bwd_layout(b, h_q, h_kv, n, d, B).total;
}

static hipError_t fill_zero(float* x, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const size_t blocks = std::min<size_t>((n + 255) / 256, 65536);
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, n);
    return hipGetLastError();
}

template <int D, int TT>
static hipError_t launch_dq(const PrefillParams& p, const DqExtra& x, const PrefillBwdArgs& a, int T, hipStream_t s) {
    auto kern = prior_attn_dq_kernel<D, TT, kDqWaves>;
    static hipError_t configured = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kBwdMaxLds);
    if (configured != hipSuccess) return configured;
    dim3 grid((a.n + p.R_t - 1) / p.R_t, a.h_kv, a.b);
    hipLaunchKernelGGL(kern, grid, dim3(64 * kDqWaves), dq_lds_bytes(D, a.B, T), s, p, x);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_t(const PrefillBwdArgs& a, const BwdLayout& L, hipStream_t s) {
    char* ws = static_cast<char*>(a.ws);
    const int g = a.h_q / a.h_kv;
    int lg = 0;
    while ((1 << lg) < g) ++lg;
    const int T = a.n / a.B, n_pad = prefill_n_pad(a.n), nblk = (a.n + 63) / 64;
    const int bh = a.b * a.h_kv;
    uint16_t* kt = reinterpret_cast<uint16_t*>(ws + L.kt);
    uint16_t* dob = a.o_bf16 ? nullptr : reinterpret_cast<uint16_t*>(ws + L.dob);
    float* delta = reinterpret_cast<float*>(ws + L.delta);
    const uint16_t* dO16 = a.o_bf16 ? static_cast<const uint16_t*>(a.dO) : dob;

    hipError_t e;
    if ((e = fill_zero(a.dK, (size_t)bh * a.n * D, s)) != hipSuccess) return e;
    if ((e = fill_zero(a.dV, (size_t)bh * a.n * D, s)) != hipSuccess) return e;
    if ((e = fill_zero(a.dbias, (size_t)bh * a.n * a.list_cap, s)) != hipSuccess) return e;
    if ((e = launch_transpose_rows(static_cast<const uint16_t*>(a.K), kt, bh, a.n, n_pad, D, s)) != hipSuccess)
        return e;

    BwdPrepParams pp{a.O, a.dO, dob, delta, a.h_q, a.h_kv, a.n, g, lg};
    const dim3 pgrid((unsigned)(((size_t)a.n * g + 63) / 64), a.h_kv, a.b);
    if (a.o_bf16) hipLaunchKernelGGL((bwd_prep_kernel<D, uint16_t>), pgrid, dim3(256), 0, s, pp);
    else hipLaunchKernelGGL((bwd_prep_kernel<D, float>), pgrid, dim3(256), 0, s, pp);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    InvParams ip{a.idx, a.bias, a.cnt,
                 reinterpret_cast<int32_t*>(ws + L.hist), reinterpret_cast<int32_t*>(ws + L.coff),
                 reinterpret_cast<int32_t*>(ws + L.inv_row), reinterpret_cast<float*>(ws + L.inv_bias),
                 a.n, a.B, T, nblk, a.list_cap, a.causal};
    if (T > 0) {
        const size_t mlds = (size_t)T * 8;
        hipLaunchKernelGGL(inv_hist_kernel, dim3(nblk, bh), dim3(64), mlds, s, ip);
        hipLaunchKernelGGL(inv_scan_blocks_kernel, dim3(T, bh), dim3(256), 0, s, ip);
        hipLaunchKernelGGL(inv_scan_chunks_kernel, dim3(bh), dim3(256), 0, s, ip);
        hipLaunchKernelGGL(inv_scatter_kernel, dim3(nblk, bh), dim3(64), mlds, s, ip);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    // dQ and the bias gradients
    PrefillParams p;
    p.Q = a.Q; p.K = a.K; p.V = a.V; p.Vt = nullptr;
    p.idx = a.idx; p.bias = a.bias; p.cnt = a.cnt; p.O = nullptr; p.lse = nullptr;
    p.out_bf16 = 0; p.h_q = a.h_q; p.h_kv = a.h_kv; p.n = a.n; p.n_pad = n_pad; p.B = a.B;
    p.T_c = T; p.list_cap = a.list_cap; p.causal = a.causal; p.g = g; p.log2g = lg;
    p.R_t = backward_tile_rows(g, a.B, T, D);
    p.nw = kDqWaves;
    p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    const float scale = (float)(1.0 / sqrt((double)D));
    DqExtra x{kt, dO16, a.lse, delta, a.dQ, a.dbias, scale};
    if ((e = a.B % 64 == 0 ? launch_dq<D, 64>(p, x, a, T, s) : launch_dq<D, 32>(p, x, a, T, s)) != hipSuccess)
        return e;

    // dK and dV
    DkvParams q;
    q.Q = static_cast<const uint16_t*>(a.Q); q.dO = dO16;
    q.K = static_cast<const uint16_t*>(a.K); q.V = static_cast<const uint16_t*>(a.V);
    q.lse = a.lse; q.delta = delta;
    q.inv_row = ip.inv_row; q.inv_bias = ip.inv_bias; q.coff = ip.coff;
    q.dK = a.dK; q.dV = a.dV;
    q.h_q = a.h_q; q.h_kv = a.h_kv; q.n = a.n; q.B = a.B; q.T_c = T; q.causal = a.causal;
    q.g = g; q.log2g = lg;
    q.seg_rows = dkv_seg_rows(g);
    q.items = reinterpret_cast<const int4*>(ws + L.items);
    q.counters = reinterpret_cast<int32_t*>(ws + L.counters);
    q.c1 = p.scale_log2; q.scale = scale;
    {
        auto kern = prior_attn_dkv_kernel<D>;
        static hipError_t configured = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kBwdMaxLds);
        if (configured != hipSuccess) return configured;
        hipLaunchKernelGGL(dkv_items_kernel, dim3(1), dim3(1024), 0, s, ip.coff,
                           reinterpret_cast<int4*>(ws + L.items), q.counters, bh, a.n, a.B, T, a.causal, q.seg_rows);
        static int cus = 0;
        if (cus == 0) {
            int dev = 0;
            if (hipGetDevice(&dev) != hipSuccess ||
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
                cus = 256;
        }
        hipLaunchKernelGGL(kern, dim3(cus), dim3(256), dkv_lds_bytes(D), s, q);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_attend_prefill_backward(const PrefillBwdArgs& a, hipStream_t s) {
    if (a.n == 0) return hipSuccess;
    const BwdLayout L = bwd_layout(a.b, a.h_q, a.h_kv, a.n, a.d, a.B);
    return a.d == 64 ? launch_bwd_t<64>(a, L, s) : launch_bwd_t<128>(a, L, s);
}

}  // namespace dash
