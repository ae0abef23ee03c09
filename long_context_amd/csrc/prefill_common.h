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
    int out_bf16, h_q, h_kv, n, n_pad, B, T_c, list_cap, causal, g, log2g, R_t, nw;
    float scale_log2;    // log2(e)/sqrt(d)
};

// LDS tables of one query tile: the union of routed chunks and the bias table.
struct TileTables {
    float* btab;   // [R_t][T_c] bias of chunk c for tile row j (-inf: not routed)
    int* uflag;    // [T_c] scratch flags
    int* ulist;    // [T_c] ascending union of routed chunks
    int* s_U;      // union size
    __host__ __device__ static size_t bytes(int R_t, int T_c) {
        return (size_t)R_t * T_c * 4 + (size_t)2 * T_c * 4 + 16;
    }
    __device__ __forceinline__ void carve(char* base, int R_t, int T_c) {
        btab = reinterpret_cast<float*>(base);
        uflag = reinterpret_cast<int*>(btab + R_t * T_c);
        ulist = uflag + T_c;
        s_U = ulist + T_c;
    }
    // Fill the tables for rows row0 .. row0+R_t-1 of KV group bhkv (visible chunks
    // 0..nvis-1) and return the union size. Ends with a workgroup barrier.
    __device__ int build(const PrefillParams& p, size_t bhkv, int row0, int nvis, int tid, int nthr) {
        const int R_t = p.R_t;
        for (int i = tid; i < R_t * nvis; i += nthr) btab[(i / nvis) * p.T_c + i % nvis] = -INFINITY;
        for (int c = tid; c < nvis; c += nthr) uflag[c] = 0;
        __syncthreads();
        for (int j = 0; j < R_t; ++j) {
            const int row = row0 + j;
            if (row >= p.n) break;
            const size_t rb = bhkv * p.n + row;
            const int cn = min(p.cnt[rb], p.list_cap);
            for (int e = tid; e < cn; e += nthr) {
                const int c = p.idx[rb * p.list_cap + e];
                if (c >= 0 && c < nvis) {
                    btab[j * p.T_c + c] = p.bias[rb * p.list_cap + e];
                    uflag[c] = 1;
                }
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

// Steps of a query tile: U routed chunks of B tokens in TT-token tiles, then the
// diagonal branch.
struct TileSteps {
    int SPC, nrouted, ndiag, nsteps, diag_base, TT;
    __device__ __forceinline__ void init(const PrefillParams& p, int U, int cq, int last_row, int tt) {
        TT = tt;
        SPC = p.B / TT;
        if (p.causal) {
            diag_base = cq * p.B;
            ndiag = (last_row - diag_base) / TT + 1;
        } else {
            diag_base = p.T_c * p.B;
            ndiag = (p.n - diag_base + TT - 1) / TT;
        }
        nrouted = U * SPC;
        nsteps = nrouted + ndiag;
    }
    __device__ __forceinline__ int base(const int* ulist, int k) const {
        return k < nrouted ? ulist[k / SPC] * (SPC * TT) + (k % SPC) * TT
                           : diag_base + (k - nrouted) * TT;
    }
};

// Launch geometry of a prefill kernel: tokens per tile, wavefronts per workgroup,
// the most (row, head) pairs a workgroup takes, and LDS ring stages.
struct PrefillGeom { int TT, waves, max_pairs, stages; };
PrefillGeom prefill_geom_f32(int d, int B);
PrefillGeom prefill_geom_bf16(int d, int B);

// fp32-input kernel (attend_prefill.hip) and bf16-input kernel with its V
// transposition (attend_prefill_bf16.hip).
hipError_t launch_prefill_f32(const PrefillParams& p, int b, int d, size_t lds, hipStream_t s);
hipError_t launch_prefill_bf16(const PrefillParams& p, int b, int d, size_t lds, hipStream_t s);

}  // namespace dash
