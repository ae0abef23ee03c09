// Pieces shared by the two Stage-2 prefill kernels (fp32 and bf16 inputs).
//
// Stage 2 of DashAttention for a prefill (paper review section 三, Eq. 9-12 through
// the additive-bias form of Proposition 4.1):
//   o_i = sum_{j in R_i ∪ D_i} softmax_j(<q_i, k_j>/sqrt(d) + d_ij) v_j,
// with d_ij = bias of chunk c(j) on the routed tokens R_i and 0 on the diagonal
// branch D_i (the query's own chunk up to itself, causal).
//
// Both kernels take one workgroup per (query tile, KV group, batch). The tile is
// R_t consecutive rows inside one chunk times all g query heads of the group; the
// heads of a group share one routed list, so packing them costs no extra work. The
// workgroup first merges its rows' lists into the union of routed chunks
// (ascending) and a per-(row, chunk) bias table in LDS, then walks the union and
// finally the diagonal chunk in token tiles.
#pragma once

#include "attn_common.h"

namespace dash {

struct PrefillParams {
    const void* Q; const void* K; const void* V;
    const uint16_t* Vt;  // bf16 path: V transposed per (b, KV head): [d][n_pad]
    const int32_t* idx; const float* bias; const int32_t* cnt;
    void* O;
    float* lse;          // nullable: per (b, query head, row) log-sum-exp of the logits
    int out_bf16, h_q, h_kv, n, n_pad, B, T_c, list_cap, causal, g, log2g, R_t, nw;
    float scale_log2;    // log2(e)/sqrt(d)
    const int32_t* seq_len = nullptr;  // ragged batch (nullable): tokens of each sequence
    // paged K/V (nullable): K and V are [num_pages, h_kv, B, D] and chunk c of sequence b
    // lives in page pages[b * pages_per_seq + c]
    const int32_t* pages = nullptr;
    int pages_per_seq = 0, num_pages = 0;
};

// Paged K/V: the row of token t of sequence bi, KV head r, is paged_row0(p, bi, r, t) + t
// in the cache viewed as [num_pages * h_kv * B, D] (page ids outside the cache are
// clamped: a bad table gives wrong output, never a stray read).
__device__ __forceinline__ int paged_row0(const PrefillParams& p, int bi, int r, int t) {
    const int c = t / p.B;
    const int pg = min(max(p.pages[(size_t)bi * p.pages_per_seq + c], 0), p.num_pages - 1);
    return (pg * p.h_kv + r) * p.B - c * p.B;
}

// Tokens of sequence bi: seq_len[bi] clamped to [0, n] in a ragged batch, else n.
__device__ __forceinline__ int seq_tokens(const PrefillParams& p, int bi) {
    return p.seq_len ? min(max(p.seq_len[bi], 0), p.n) : p.n;
}

// LDS tables of one query tile: the ascending union of the chunks its rows route.
struct TileTables {
    int* uflag;    // [T_c] scratch flags
    int* ulist;    // [T_c] ascending union of routed chunks
    int* s_U;      // union size
    __host__ __device__ static size_t bytes(int T_c) { return (size_t)2 * T_c * 4 + 16; }
    __device__ __forceinline__ void carve(char* base, int T_c) {
        uflag = reinterpret_cast<int*>(base);
        ulist = uflag + T_c;
        s_U = ulist + T_c;
    }
    // Fill the union for rows row0 .. row0+R_t-1 of KV group bhkv (visible chunks
    // 0..nvis-1) and return its size. Every row has nthr/R_t threads, which read its
    // list four entries apart at a time, so all rows' loads are in flight together.
    // Ends with a workgroup barrier.
    __device__ int build(const PrefillParams& p, size_t bhkv, int row0, int nvis, int tid, int nthr, int nb = -1) {
        if (nb < 0) nb = p.n;
        for (int c = tid; c < nvis; c += nthr) uflag[c] = 0;
        __syncthreads();
        const int tpr = max(nthr / p.R_t, 1);
        const int j = tid / tpr, sub = tid % tpr, row = row0 + j;
        if (j < p.R_t && row < nb) {
            const size_t rb = bhkv * p.n + row;
            const int cn = min(p.cnt[rb], p.list_cap);
            const int32_t* li = p.idx + rb * p.list_cap;
            for (int e0 = sub; e0 < cn; e0 += 4 * tpr) {
                int c[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) c[u] = e0 + u * tpr < cn ? li[e0 + u * tpr] : -1;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (c[u] >= 0 && c[u] < nvis) uflag[c[u]] = 1;
            }
        }
        __syncthreads();
        if (tid < 64) {
            const int lane = tid;
            int base = 0;
            for (int c0 = 0; c0 < nvis; c0 += 64) {
                const int c = c0 + lane;
                const bool f = c < nvis && uflag[c] != 0;
                const uint64_t m = ballot(f);
                if (f) ulist[base + __builtin_popcountll(m & ((1ull << lane) - 1ull))] = c;
                base += __builtin_popcountll(m);
            }
            if (lane == 0) *s_U = base;
        }
        __syncthreads();
        return *s_U;
    }
};

// A lane's walk along the routed list of its query row, in step with the tile's
// ascending union: both are ascending, so the bias of union chunk c for this row
// is the list's next entry when that entry is c, and the row does not route c
// otherwise. The entry after a consumed one is loaded at once and has a whole
// tile of work to arrive.
struct ListCursor {
    const int32_t* idx; const float* bias;
    int cn, pos, next;
    float nb;
    __device__ __forceinline__ void fetch() {
        next = pos < cn ? idx[pos] : 0x7fffffff;
        nb = pos < cn ? bias[pos] : 0.f;
    }
    __device__ __forceinline__ void init(const PrefillParams& p, size_t rb, bool ok) {
        idx = p.idx + rb * p.list_cap;
        bias = p.bias + rb * p.list_cap;
        cn = ok ? min(p.cnt[rb], p.list_cap) : 0;
        pos = 0;
        fetch();
    }
    // bias of union chunk c in log2 units (-inf: not routed); `last` marks the
    // chunk's last token tile, after which the cursor moves past c
    __device__ __forceinline__ float take(int c, bool last) {
        float b = next == c ? nb * kLog2e : -INFINITY;
        // b is fixed here, before the cursor moves: the old entry is then dead when
        // the next one is loaded into its registers, and nothing waits on that load
        // until the following tile
        asm volatile("" : "+v"(b));
        if (last && next <= c) { ++pos; fetch(); }
        return b;
    }
};

// Steps of a query tile: U routed chunks of B tokens in TT-token tiles, then the
// diagonal branch.
struct TileSteps {
    int SPC, nrouted, ndiag, nsteps, diag_base, TT;
    // nb, Tb: the sequence's tokens and complete chunks (a ragged batch), else n and T_c
    __device__ __forceinline__ void init(const PrefillParams& p, int U, int cq, int last_row, int tt,
                                         int nb = -1, int Tb = -1) {
        if (nb < 0) { nb = p.n; Tb = p.T_c; }
        TT = tt;
        SPC = p.B / TT;
        if (p.causal) {
            diag_base = cq * p.B;
            ndiag = (last_row - diag_base) / TT + 1;
        } else {
            diag_base = Tb * p.B;
            ndiag = (nb - diag_base + TT - 1) / TT;
        }
        nrouted = U * SPC;
        nsteps = nrouted + ndiag;
    }
    __device__ __forceinline__ int base(const int* ulist, int k) const {
        return k < nrouted ? ulist[k / SPC] * (SPC * TT) + (k % SPC) * TT
                           : diag_base + (k - nrouted) * TT;
    }
    // first token and routed chunk (0 on the diagonal) of step k; zeros past the end
    __device__ __forceinline__ void at(const int* ulist, int k, int& tb, int& c) const {
        c = k < nrouted ? ulist[k / SPC] : 0;
        tb = k < nrouted ? c * (SPC * TT) + (k % SPC) * TT : k < nsteps ? diag_base + (k - nrouted) * TT : 0;
    }
};

// bf16 tiles in LDS: a row-major tile [TT][D] ("K" form) and a transposed tile
// [D][TT] ("V^T" form), both unpadded, split into 16-byte pieces stored at piece
// slot c ^ swz(row) so that 16 lanes reading one piece column of 16 different rows
// hit 16 distinct bank groups (RPB rows share one 256-byte bank row).
template <int D, int TT>
struct BfTiles {
    static constexpr int KROWB = D * 2;
    static constexpr int KPPR = KROWB / 16;
    static constexpr int KRPB = KROWB >= 256 ? 1 : 256 / KROWB;
    static constexpr int KBYTES = TT * KROWB;
    static constexpr int VROWB = TT * 2;
    static constexpr int VPPR = VROWB / 16;
    static constexpr int VRPB = 256 / VROWB;
    static constexpr int VBYTES = D * VROWB;
    static constexpr int STAGE = KBYTES + VBYTES;
    static constexpr int KINSTS = KBYTES / 1024;     // wavefront copy instructions per tile
    static constexpr int VINSTS = VBYTES / 1024;
    __device__ __forceinline__ static int kslot(int t, int c) { return c ^ ((t / KRPB) & (KPPR - 1)); }
    __device__ __forceinline__ static int vslot(int d, int c) { return c ^ ((d / VRPB) & (VPPR - 1)); }
};

// Launch geometry of a prefill kernel: tokens per tile, wavefronts per workgroup,
// the most (row, head) pairs a workgroup takes, and LDS ring stages.
struct PrefillGeom { int TT, waves, max_pairs, stages; };
PrefillGeom prefill_geom_f32(int d, int B);
PrefillGeom prefill_geom_bf16(int d, int B);
// LDS tile stages of the bf16 kernel (4: two tiles per barrier; 2: one), by context length
int prefill_bf16_stages(int d, int B, int T_c);

// fp32-input kernel (attend_prefill.hip) and bf16-input kernel with its V
// transposition (attend_prefill_bf16.hip).
hipError_t launch_prefill_f32(const PrefillParams& p, int b, int d, size_t lds, hipStream_t s);
hipError_t launch_prefill_bf16(const PrefillParams& p, int b, int d, size_t lds, hipStream_t s);

}  // namespace dash
