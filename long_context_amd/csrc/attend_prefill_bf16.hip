// Stage 2 prefill kernel for bf16 inputs (the method is stated in prefill_common.h).
//
// sparse_prior_attn_bf16_kernel: NW wavefronts, each owning PBW blocks of 32
// (row, head) pairs.
//   * On gfx950 LDS throughput is bounded by the number of read instructions, so
//     every MFMA operand read from LDS is one 16-byte read.
//   * V is transposed once per call into [d][n_pad] (transpose_v_kernel): the A
//     operand of O^T += V^T P^T (8 consecutive tokens of one d) is then a plain
//     16-byte read of the V^T tile.
//   * The A operand of S^T = K Q^T presents the K rows of a 32-token block with bits
//     2 and 3 of the row index swapped. The S^T accumulator element i of lane l
//     (rows 8(i/4) + 4(l/32) + i%4) then holds token 16(i/8) + 8(l/32) + i%8, which
//     is exactly the token order k-slot (l/32, e) of a k16 step needs in the B
//     operand P^T: P leaves the accumulator in natural token order.
//   * Tiles of K and V^T are copied global->LDS asynchronously into a two-stage
//     ring (one barrier per tile); a pair block skips a routed chunk none of its
//     rows routes to. Each lane finds its row's bias by walking the row's routed
//     list alongside the tile's union of chunks (no per-row table in LDS).
#include "kernels.h"
#include "prefill_common.h"

#include <math.h>

namespace dash {


// Copies of one stage split over NW wavefronts: wavefront w issues copy
// instructions w, w+NW, ...; instructions 0..KINSTS-1 copy K pieces, the rest V^T.
template <int D, int TT, int NW>
struct BfCopier {
    typedef BfTiles<D, TT> S;
    static constexpr int CPW = (S::KINSTS + S::VINSTS) / NW;
    static_assert(CPW * NW == S::KINSTS + S::VINSTS, "copies must divide evenly over the wavefronts");
    int row[CPW];      // K: tile token; V^T: d
    int off[CPW];      // element offset of the piece inside its row
    int dst[CPW];      // byte offset of the wavefront's 1 KiB block inside a stage

    __device__ __forceinline__ void init(int wid, int lane) {
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int j = wid + i * NW;
            if (j < S::KINSTS) {
                const int q = j * 64 + lane, t = q / S::KPPR, cs = q % S::KPPR;
                row[i] = t;
                off[i] = S::kslot(t, cs) * 8;             // the swizzle is an involution
                dst[i] = j * 1024;
            } else {
                const int jj = j - S::KINSTS;
                const int q = jj * 64 + lane, d = q / S::VPPR, cs = q % S::VPPR;
                row[i] = d;
                off[i] = S::vslot(d, cs) * 8;
                dst[i] = S::KBYTES + jj * 1024;
            }
        }
    }
    // K rows ko + min(tb + t, nmax) (ko: 0, or the paged cache's row offset of the tile's
    // chunk); V^T columns tb .. tb+TT-1 (inside n_pad). Tile bases are multiples of TT
    // below n_pad by construction; the clamp keeps every source address inside the
    // tensors even if a table were corrupted.
    __device__ __forceinline__ void issue(char* stage, const uint16_t* Kg, int ko, const uint16_t* Vtg, int tb,
                                          int nmax, int n_pad, int wid) const {
        tb = min(max(tb, 0), n_pad - TT);
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const bool isk = wid + i * NW < S::KINSTS;     // wavefront-uniform
            const uint16_t* src = isk ? Kg + (size_t)(ko + min(tb + row[i], nmax)) * D + off[i]
                                      : Vtg + (size_t)row[i] * n_pad + tb + off[i];
            __builtin_amdgcn_global_load_lds(src, stage + dst[i], 16, 0, 0);
        }
    }
};

// V [b, h_kv, n, D] -> Vt [b, h_kv, D, n_pad], tokens n .. n_pad-1 zero (in a ragged
// batch, tokens from seq_len[b] on: padding rows may hold anything).
// A paged V (pages != nullptr) is [num_pages, h_kv, B, D] with chunk c of sequence b in
// page pages[b * pages_per_seq + c].
template <int D>
__global__ __launch_bounds__(256) void transpose_v_kernel(const uint16_t* V, uint16_t* Vt, int n, int n_pad,
                                                          const int32_t* seq_len = nullptr, int h_kv = 1,
                                                          const int32_t* pages = nullptr, int pages_per_seq = 0,
                                                          int num_pages = 0, int B = 1) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[64][D + 8];
    const int t0 = blockIdx.x * 64;
    const size_t bh = blockIdx.y;
    const int nv = seq_len ? min(max(seq_len[bh / h_kv], 0), n) : n;   // tokens copied
    uint16_t* dst = Vt + bh * (size_t)D * n_pad;
    // V row of token t
    auto vrow = [&](int t) -> const uint16_t* {
        if (pages) {
            const int pg = min(max(pages[(bh / h_kv) * pages_per_seq + t / B], 0), num_pages - 1);
            return V + (((size_t)pg * h_kv + bh % h_kv) * B + t % B) * D;
        }
        return V + (bh * (size_t)n + t) * D;
    };
    constexpr int PR = D / 8;                          // 16-byte pieces per V row
    for (int q = threadIdx.x; q < 64 * PR; q += 256) {
        const int t = q / PR, c = q % PR;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (t0 + t < nv) v = *reinterpret_cast<const u32x4*>(vrow(t0 + t) + 8 * c);
        *reinterpret_cast<u32x4*>(&tile[t][8 * c]) = v;
    }
    __syncthreads();
    for (int q = threadIdx.x; q < D * 8; q += 256) {
        const int d = q / 8, c = q % 8;
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = (uint32_t)tile[8 * c + 2 * e][d] | ((uint32_t)tile[8 * c + 2 * e + 1][d] << 16);
        *reinterpret_cast<u32x4*>(dst + (size_t)d * n_pad + t0 + 8 * c) = o;
    }
}


// NW wavefronts of PBW pair blocks (32 (row, head) pairs each); PAGED: K read through
// the page table; PS tiles per barrier.
template <int D, int TT, int NW, int PBW, bool PAGED, int PS>
__global__ __launch_bounds__(64 * NW) void sparse_prior_attn_bf16_kernel(PrefillParams p) {
    typedef BfTiles<D, TT> S;
    constexpr int NS = D / 16;     // k16 steps of S^T
    constexpr int NB = TT / 32;    // 32-token blocks of S^T
    constexpr int NP = TT / 16;    // k16 steps of O^T
    constexpr int ND = D / 32;     // 32-wide d blocks of O^T
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* ring = smem;                                   // two stages of PS tiles
    TileTables tabs;
    tabs.carve(smem + 2 * PS * S::STAGE, p.T_c);

    constexpr int nthr = 64 * NW;
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
    // K rows: the sequence's own rows, or (paged) the whole cache with per-chunk offsets
    const uint16_t* Kg = static_cast<const uint16_t*>(p.K) + (PAGED ? 0 : bhkv * (size_t)p.n * D);
    auto krow0 = [&](int t) { return PAGED ? paged_row0(p, bi, r, t) : 0; };
    const uint16_t* Vtg = p.Vt + bhkv * (size_t)D * p.n_pad;
    const int U = tabs.build(p, bhkv, row0, nvis, tid, nthr, nb);

    // ---- the lane's (row, head) pair in each of its pair blocks ----
    int jrow[PBW], my_row[PBW];
    bool pok[PBW], live[PBW];
    ListCursor lc[PBW];
    bf16x8 qf[PBW][NS];
#pragma unroll
    for (int pb = 0; pb < PBW; ++pb) {
        const int P = (wid * PBW + pb) * 32 + l32;
        jrow[pb] = P >> lg;
        my_row[pb] = row0 + jrow[pb];
        const int hh = r * g + (P & (g - 1));
        live[pb] = (wid * PBW + pb) * 32 < g * R_t;              // wavefront-uniform
        pok[pb] = live[pb] && jrow[pb] < R_t && my_row[pb] < nb;
        lc[pb].init(p, bhkv * p.n + (pok[pb] ? my_row[pb] : 0), pok[pb]);
        const uint16_t* qrow = static_cast<const uint16_t*>(p.Q) +
            (((size_t)bi * p.h_q + hh) * p.n + (pok[pb] ? my_row[pb] : 0)) * D + 8 * hl;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            qf[pb][s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
            if (!pok[pb]) qf[pb][s] = bf16x8{};
        }
    }

    float m_run[PBW], l_run[PBW];
    f32x16 o_acc[PBW][ND];
#pragma unroll
    for (int pb = 0; pb < PBW; ++pb) {
        m_run[pb] = -INFINITY;
        l_run[pb] = 0.f;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o_acc[pb][db][i] = 0.f;
    }

    TileSteps st;
    st.init(p, U, cq, last_row, TT, nb, Tb);
    const int nmax = nb - 1;
    BfCopier<D, TT, NW> cp;
    cp.init(wid, lane);
    // tile row presented by A row l32 of a 32-token block: bits 2 and 3 swapped
    const int krow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
    const float c1 = p.scale_log2;

    // K operands of the tile (shared by the pair blocks)
    auto load_k = [&](const char* kt, bf16x8 (&ka)[NB][NS]) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int t = 32 * blk + krow;
                ka[blk][s] = *reinterpret_cast<const bf16x8*>(kt + t * S::KROWB + S::kslot(t, 2 * s + hl) * 16);
            }
    };
    auto load_v = [&](const char* vt, bf16x8 (&va)[NP][ND]) {
#pragma unroll
        for (int s = 0; s < NP; ++s)
#pragma unroll
            for (int db = 0; db < ND; ++db) {
                const int d = 32 * db + l32;
                va[s][db] = *reinterpret_cast<const bf16x8*>(vt + d * S::VROWB + S::vslot(d, 2 * s + hl) * 16);
            }
    };
    // S^T of pair block pb over the tile
    auto scores = [&](int pb, const bf16x8 (&ka)[NB][NS], f32x16 (&sacc)[NB]) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[blk][i] = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
                sacc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[blk][s], qf[pb][s], sacc[blk], 0, 0, 0);
    };
    // online softmax of pair block pb: P (bf16) into pp, running max and sum; returns
    // the rescale factor of the output accumulator (1 when the maximum stays)
    auto softmax = [&](int pb, bool diag, int tb, float bias2, f32x16 (&sacc)[NB], bf16x8 (&pp)[NP],
                       bool& grow) -> float {
        if (diag) {
            const int lim = p.causal ? my_row[pb] : nb - 1;
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int tk = tb + 32 * blk + 16 * (i >> 3) + 8 * hl + (i & 7);
                    sacc[blk][i] = tk > lim ? -INFINITY : sacc[blk][i];
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[blk][i]);
        mx = pair32_max(mx);
        const float tmax = fmaf(mx, c1, bias2);              // -inf when nothing is visible
        // lazy rescaling: the reference maximum only moves when the tile maximum
        // exceeds it by more than 8 (probabilities stay <= 2^8 in between)
        grow = tmax > m_run[pb] + 8.f;
        const float alpha = grow ? fast_exp2(m_run[pb] - tmax) : 1.f;
        m_run[pb] = grow ? tmax : m_run[pb];
        const float off = bias2 - ((m_run[pb] == -INFINITY) ? 0.f : m_run[pb]);
        float ps = 0.f;
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int s = 0; s < NP; ++s) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pp[s][e] = (__bf16)fast_exp2(fmaf(sacc[s >> 1][8 * (s & 1) + e], c1, off));
            // the denominator sums the rounded P fed to the MFMA
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const bf16x2 pr = {pp[s][e], pp[s][e + 1]};
                ps = __builtin_amdgcn_fdot2_f32_bf16(pr, one, ps, false);
            }
        }
        l_run[pb] = fmaf(l_run[pb], alpha, ps);
        return alpha;
    };
    auto rescale = [&](int pb, bool grow, float alpha) {
        if (ballot(grow) != 0) {
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o_acc[pb][db][i] *= alpha;
        }
    };
    auto pv = [&](int pb, const bf16x8 (&va)[NP][ND], const bf16x8 (&pp)[NP]) {
#pragma unroll
        for (int s = 0; s < NP; ++s)
#pragma unroll
            for (int db = 0; db < ND; ++db)
                o_acc[pb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[s][db], pp[s], o_acc[pb][db], 0, 0, 0);
    };

    // PS steps per barrier: ring stage j & 1 holds the PS tiles of group j, and a
    // wavefront takes the tiles of the group it has rows for one after the other (a
    // wavefront idle on a tile no longer waits at a barrier of that tile's own). The
    // tile bases and chunks are read from LDS two groups ahead, so that neither the
    // cursors nor the copies wait on an LDS read.
    const int npairs = (st.nsteps + PS - 1) / PS;
    int tb_cur[PS], c_cur[PS], tb_nxt[PS], c_nxt[PS], ko_nxt[PS];
#pragma unroll
    for (int u = 0; u < PS; ++u) {
        st.at(tabs.ulist, u, tb_cur[u], c_cur[u]);
        st.at(tabs.ulist, PS + u, tb_nxt[u], c_nxt[u]);
        ko_nxt[u] = krow0(tb_nxt[u]);
    }
#pragma unroll
    for (int u = 0; u < PS; ++u)
        if (u < st.nsteps) cp.issue(ring + u * S::STAGE, Kg, krow0(tb_cur[u]), Vtg, tb_cur[u], nmax, p.n_pad, wid);
    wait_tile_copies();
    __syncthreads();
    for (int j = 0; j < npairs; ++j) {
        const int k0 = PS * j;
#pragma unroll
        for (int u = 0; u < PS; ++u)
            if (k0 + PS + u < st.nsteps)
                cp.issue(ring + (((j + 1) & 1) * PS + u) * S::STAGE, Kg, ko_nxt[u], Vtg, tb_nxt[u], nmax, p.n_pad, wid);
        int tb_nn[PS], c_nn[PS], ko_nn[PS];
#pragma unroll
        for (int u = 0; u < PS; ++u) {
            st.at(tabs.ulist, k0 + 2 * PS + u, tb_nn[u], c_nn[u]);
            ko_nn[u] = krow0(tb_nn[u]);      // (paged) a page-table load with a group to arrive
        }
#pragma unroll
        for (int u = 0; u < PS; ++u) {
            const int k = k0 + u;
            if (k >= st.nsteps) break;
            const bool routed = k < st.nrouted;
            float bias2[PBW];
            bool run[PBW];
#pragma unroll
            for (int pb = 0; pb < PBW; ++pb) {
                bias2[pb] = routed ? lc[pb].take(c_cur[u], k % st.SPC == st.SPC - 1) : 0.f;
                run[pb] = live[pb] && (!routed || ballot(bias2[pb] > -INFINITY) != 0);
            }
            const char* kt = ring + ((j & 1) * PS + u) * S::STAGE;
            const char* vt = kt + S::KBYTES;
            const int tb = tb_cur[u];
#pragma unroll
            for (int pb = 0; pb < PBW; ++pb) {
                if (run[pb]) {
                    bf16x8 ka[NB][NS];
                    load_k(kt, ka);
                    f32x16 sacc[NB];
                    scores(pb, ka, sacc);
                    bf16x8 pp[NP];
                    bool grow;
                    const float alpha = softmax(pb, !routed, tb, bias2[pb], sacc, pp, grow);
                    rescale(pb, grow, alpha);
                    bf16x8 va[NP][ND];
                    load_v(vt, va);
                    pv(pb, va, pp);
                }
            }
        }
        wait_tile_copies();
        __syncthreads();
#pragma unroll
        for (int u = 0; u < PS; ++u) {
            tb_cur[u] = tb_nxt[u]; c_cur[u] = c_nxt[u];
            tb_nxt[u] = tb_nn[u]; c_nxt[u] = c_nn[u];
            ko_nxt[u] = ko_nn[u];
        }
    }

#pragma unroll
    for (int pb = 0; pb < PBW; ++pb) {
        const float l_tot = pair32_sum(l_run[pb]);
        if (pok[pb]) {
            const int hh = r * g + (((wid * PBW + pb) * 32 + l32) & (g - 1));
            const float inv = 1.f / l_tot;
            // log-sum-exp of the row's logits: P was taken relative to 2^m (m = 0 if
            // nothing was visible), so sum_j e^{z_j} = 2^m l
            if (p.lse && hl == 0)
                p.lse[((size_t)bi * p.h_q + hh) * p.n + my_row[pb]] =
                    (((m_run[pb] == -INFINITY) ? 0.f : m_run[pb]) + fast_log2(l_tot)) * kLn2;
            const size_t obase = (((size_t)bi * p.h_q + hh) * p.n + my_row[pb]) * D;
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int d0 = 32 * db + 8 * a + 4 * hl;
                    if (p.out_bf16) {
                        u32x2 o;
                        o[0] = (uint32_t)f32_to_bf16_bits(o_acc[pb][db][4 * a] * inv) |
                               ((uint32_t)f32_to_bf16_bits(o_acc[pb][db][4 * a + 1] * inv) << 16);
                        o[1] = (uint32_t)f32_to_bf16_bits(o_acc[pb][db][4 * a + 2] * inv) |
                               ((uint32_t)f32_to_bf16_bits(o_acc[pb][db][4 * a + 3] * inv) << 16);
                        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.O) + obase + d0) = o;
                    } else {
                        f32x4 o;
                        o[0] = o_acc[pb][db][4 * a] * inv; o[1] = o_acc[pb][db][4 * a + 1] * inv;
                        o[2] = o_acc[pb][db][4 * a + 2] * inv; o[3] = o_acc[pb][db][4 * a + 3] * inv;
                        *reinterpret_cast<f32x4*>(static_cast<float*>(p.O) + obase + d0) = o;
                    }
                }
        }
    }
}

int prefill_n_pad(int n) { return (n + 63) / 64 * 64; }

hipError_t launch_transpose_rows(const uint16_t* src, uint16_t* dst, int bh, int n, int n_pad, int d, hipStream_t s) {
    if (n_pad == 0) return hipSuccess;
    if (d == 64)
        hipLaunchKernelGGL((transpose_v_kernel<64>), dim3(n_pad / 64, bh), dim3(256), 0, s, src, dst, n, n_pad);
    else
        hipLaunchKernelGGL((transpose_v_kernel<128>), dim3(n_pad / 64, bh), dim3(256), 0, s, src, dst, n, n_pad);
    return hipGetLastError();
}

size_t prefill_workspace_bytes(int b, int h_kv, int n, int d) {
    return (size_t)b * h_kv * d * (size_t)prefill_n_pad(n) * sizeof(uint16_t);
}

constexpr int kWavesB = 8;        // wavefronts per workgroup
constexpr int kPairBlocks = 1;    // 32-pair blocks per wavefront

static int bf16_tile_tokens(int, int B) { return (B % 64 == 0) ? 64 : 32; }

PrefillGeom prefill_geom_bf16(int d, int B) {
    return PrefillGeom{bf16_tile_tokens(d, B), kWavesB, 32 * kWavesB * kPairBlocks, 2};
}

// Ring stages of tiles: two groups of two tiles (two steps per barrier) when they and
// the tile tables fit LDS, else two single tiles (contexts of more than about 4K chunks
// at d = 128 and 64-token tiles).
int prefill_bf16_stages(int d, int B, int T_c) {
    const size_t stage = (size_t)2 * bf16_tile_tokens(d, B) * d * 2;     // K and V^T tiles
    return 4 * stage + TileTables::bytes(T_c) <= (size_t)160 * 1024 ? 4 : 2;
}

// Every (d, tile, K/V layout, tiles per barrier) combination is instantiated
// explicitly: when one dispatcher names two, hipcc emits the host handle of only the
// first.
#define DASH_PREFILL_BF16_INST(D, TT, PS)                                                                   \
    template __global__ void sparse_prior_attn_bf16_kernel<D, TT, kWavesB, kPairBlocks, false, PS>(PrefillParams); \
    template __global__ void sparse_prior_attn_bf16_kernel<D, TT, kWavesB, kPairBlocks, true, PS>(PrefillParams);
DASH_PREFILL_BF16_INST(64, 32, 1)
DASH_PREFILL_BF16_INST(64, 64, 1)
DASH_PREFILL_BF16_INST(128, 32, 1)
DASH_PREFILL_BF16_INST(128, 64, 1)
DASH_PREFILL_BF16_INST(64, 32, 2)
DASH_PREFILL_BF16_INST(64, 64, 2)
DASH_PREFILL_BF16_INST(128, 32, 2)
DASH_PREFILL_BF16_INST(128, 64, 2)
#undef DASH_PREFILL_BF16_INST

template <int D, int TT, bool PAGED, int PS>
static hipError_t launch_bf16_paged(const PrefillParams& p, int b, size_t lds, hipStream_t s) {
    auto kern = sparse_prior_attn_bf16_kernel<D, TT, kWavesB, kPairBlocks, PAGED, PS>;
    static hipError_t configured = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (configured != hipSuccess) return configured;
    hipLaunchKernelGGL((transpose_v_kernel<D>), dim3(p.n_pad / 64, b * p.h_kv), dim3(256), 0, s,
                       static_cast<const uint16_t*>(p.V), const_cast<uint16_t*>(p.Vt), p.n, p.n_pad, p.seq_len,
                       p.h_kv, p.pages, p.pages_per_seq, p.num_pages, p.B);
    dim3 grid((p.n + p.R_t - 1) / p.R_t, p.h_kv, b), block(64 * kWavesB);
    hipLaunchKernelGGL(kern, grid, block, lds, s, p);
    return hipGetLastError();
}

template <int D, int TT, int PS>
static hipError_t launch_bf16_ps(const PrefillParams& p, int b, size_t lds, hipStream_t s) {
    return p.pages ? launch_bf16_paged<D, TT, true, PS>(p, b, lds, s) : launch_bf16_paged<D, TT, false, PS>(p, b, lds, s);
}

template <int D, int TT>
static hipError_t launch_bf16_t(const PrefillParams& p, int b, size_t lds, hipStream_t s) {
    return prefill_bf16_stages(D, p.B, p.T_c) == 4 ? launch_bf16_ps<D, TT, 2>(p, b, lds, s)
                                                   : launch_bf16_ps<D, TT, 1>(p, b, lds, s);
}

hipError_t launch_prefill_bf16(const PrefillParams& p, int b, int d, size_t lds, hipStream_t s) {
    const bool t64 = bf16_tile_tokens(d, p.B) == 64;
    if (d == 64) return t64 ? launch_bf16_t<64, 64>(p, b, lds, s) : launch_bf16_t<64, 32>(p, b, lds, s);
    return t64 ? launch_bf16_t<128, 64>(p, b, lds, s) : launch_bf16_t<128, 32>(p, b, lds, s);
}

}  // namespace dash
