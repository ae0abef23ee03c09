// Shared pieces of the Stage-2 attention kernels (prefill and decode).
//
// Both kernels compute S^T = K Q^T and O^T = V^T P^T with 32x32 MFMAs so that a
// lane owns one (query row, head) column: its softmax statistics and its output
// rows live in the same lane, and P leaves the S^T accumulator already laid out as
// the B operand of the second product.
//   * v_mfma_f32_32x32x16_bf16 (bf16 inputs) or 8 x v_mfma_f32_32x32x2_f32 (fp32
//     inputs) consume a "k16 step": lane l supplies 8 values with k-slots
//     (h = l/32, e = 0..7); A and B use the same slot convention, so which real
//     index a slot carries is free as long as both operands agree.
//   * Accumulator layout (32x32): lane l holds column l%32 and rows
//     8*(i/4) + 4*(l/32) + i%4 for i = 0..15.
//   * K tile in LDS: row-major [token][d] with a 16-byte pad per row (conflict-free
//     128-bit reads of one column block across 32 rows).
//   * V tile in LDS: transposed [d][slot]. In each 16-token group, token
//     8q + 4h + x sits at slot 8h + 4q + x, which is exactly the token order of
//     the P values a lane holds for k-slot (h, e) of a k16 step.
#pragma once

#include "common.h"

namespace dash {

template <typename T> struct Mfma;

template <> struct Mfma<uint16_t> {       // bf16 inputs
    typedef bf16x8 Op;
    __device__ __forceinline__ static f32x16 mma(const Op& a, const Op& b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static Op load(const uint16_t* p) {
        return *reinterpret_cast<const Op*>(p);
    }
    __device__ __forceinline__ static Op pack(const float* v) {
        Op o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (__bf16)v[e];
        return o;
    }
    __device__ __forceinline__ static Op zero() {
        Op o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (__bf16)0.f;
        return o;
    }
    // acc + sum of the 8 (already rounded) values of a packed operand
    __device__ __forceinline__ static float sum(const Op& o, const float*, float acc) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const bf16x2 pr = {o[e], o[e + 1]};
            acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
        }
        return acc;
    }
};

struct F32x8 { float v[8]; };

template <typename Op>
__device__ __forceinline__ Op pack_f32x8(Op r, const f32x4& a, const f32x4& b);

template <> struct Mfma<float> {          // fp32 inputs
    typedef F32x8 Op;
    __device__ __forceinline__ static f32x16 mma(const Op& a, const Op& b, f32x16 c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[e], b.v[e], c, 0, 0, 0);
        return c;
    }
    __device__ __forceinline__ static Op load(const float* p) {
        Op o;
        const f32x4* q = reinterpret_cast<const f32x4*>(p);
        f32x4 x = q[0], y = q[1];
        o.v[0] = x[0]; o.v[1] = x[1]; o.v[2] = x[2]; o.v[3] = x[3];
        o.v[4] = y[0]; o.v[5] = y[1]; o.v[6] = y[2]; o.v[7] = y[3];
        return o;
    }
    __device__ __forceinline__ static Op pack(const float* v) {
        Op o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o.v[e] = v[e];
        return o;
    }
    __device__ __forceinline__ static Op zero() {
        Op o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o.v[e] = 0.f;
        return o;
    }
    __device__ __forceinline__ static float sum(const Op&, const float* v, float acc) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += v[e];
        return acc;
    }
};

template <>
__device__ __forceinline__ F32x8 pack_f32x8<F32x8>(F32x8 r, const f32x4& a, const f32x4& b) {
    r.v[0] = a[0]; r.v[1] = a[1]; r.v[2] = a[2]; r.v[3] = a[3];
    r.v[4] = b[0]; r.v[5] = b[1]; r.v[6] = b[2]; r.v[7] = b[3];
    return r;
}
template <>
__device__ __forceinline__ bf16x8 pack_f32x8<bf16x8>(bf16x8 r, const f32x4&, const f32x4&) { return r; }

// S^T blocks (NBLK x 32 tokens x 32 pairs) = K rows [32 tokens][D] (LDS, row
// stride KROW bytes, block stride 32 rows) times the lane's q fragments. The K
// fragments of a group of k16 steps are read from LDS before the MFMAs start, and
// the NBLK independent accumulation chains are interleaved so that consecutive
// MFMAs never depend on each other.
template <typename T, int D, int NBLK, int KROW>
__device__ __forceinline__ void score_blocks(f32x16 (&acc)[NBLK], const char* krow_lds,
                                             const typename Mfma<T>::Op* qf) {
    typedef Mfma<T> MM;
    constexpr int NB = sizeof(T) == 2 ? (NBLK == 1 ? D / 16 : 4) : 2;   // k16 steps per group
#pragma unroll
    for (int b = 0; b < NBLK; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[b][i] = 0.f;
#pragma unroll
    for (int s0 = 0; s0 < D / 16; s0 += NB) {
        typename MM::Op ka[NBLK][NB];
#pragma unroll
        for (int b = 0; b < NBLK; ++b)
#pragma unroll
            for (int s = 0; s < NB; ++s)
                ka[b][s] = MM::load(reinterpret_cast<const T*>(krow_lds + 32 * b * KROW) + 16 * (s0 + s));
        __builtin_amdgcn_sched_barrier(0);     // keep the reads ahead of the MFMAs
#pragma unroll
        for (int s = 0; s < NB; ++s)
#pragma unroll
            for (int b = 0; b < NBLK; ++b) acc[b] = MM::mma(ka[b][s], qf[s0 + s], acc[b]);
    }
}

// ---------------------------------------------------------------------------------
// Swizzled tiles filled by asynchronous global->LDS copies (global_load_lds_dwordx4:
// a wavefront instruction writes 64 x 16 bytes contiguously, lane l at +16l).
// Rows are unpadded (D*ES bytes) and split into PPR 16-byte pieces; piece c of row t
// is stored at piece slot c ^ swz(t):
//   K:  swz(t) = t mod PPR            (16 consecutive rows read one column: all banks)
//   V:  swz(t) = 4 (t mod 4) mod PPR  (bf16; the transposing reads of a k16 step
//                                      touch 4 rows x 4 pieces: all distinct)
// ---------------------------------------------------------------------------------
template <typename T, int D, int TT>
struct SwzTile {
    static constexpr int ES = sizeof(T);
    static constexpr int ROWB = D * ES;              // bytes per row
    static constexpr int PPR = ROWB / 16;            // 16-byte pieces per row
    static constexpr int BYTES = TT * ROWB;          // one K (or V) tile
    static constexpr int STAGE = 2 * BYTES;          // K tile then V tile
    static constexpr int INSTS = TT * PPR / 64;      // wavefront copies per K (or V) tile
    __device__ __forceinline__ static int kslot(int t, int c) { return c ^ (t & (PPR - 1)); }
    __device__ __forceinline__ static int vslot(int t, int c) {
        return ES == 2 ? (c ^ ((4 * (t & 3)) & (PPR - 1))) : c;
    }
};

// The copies of one K/V tile, split over NW wavefronts: wavefront `wid` issues copy
// instructions wid, wid + NW, ... (CPW of them). Each lane's tile row and source
// element offset per copy depend only on (wid, lane), so they are computed once.
template <typename T, int D, int TT, int NW>
struct TileCopier {
    typedef SwzTile<T, D, TT> S;
    static constexpr int CPW = 2 * S::INSTS / NW;   // copies per wavefront per tile
    static_assert(CPW * NW == 2 * S::INSTS, "copies must divide evenly over the wavefronts");
    int row[CPW];      // tile row (token) of this lane's piece
    int off[CPW];      // element offset of the piece inside its row
    int dst[CPW];      // byte offset of the wavefront's 1 KiB block inside a stage

    __device__ __forceinline__ void init(int wid, int lane) {
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int j = wid + i * NW;
            const bool isv = j >= S::INSTS;
            const int jj = isv ? j - S::INSTS : j;
            const int slot = jj * 64 + lane;
            const int t = slot / S::PPR, cs = slot % S::PPR;
            const int c = isv ? S::vslot(t, cs) : S::kslot(t, cs);   // the swizzle is an involution
            row[i] = t;
            off[i] = c * (16 / S::ES);
            dst[i] = (isv ? S::BYTES : 0) + jj * 1024;
        }
    }
    // Copy the tile whose token t lives in row min(tb + t, nmax) of K and V.
    __device__ __forceinline__ void issue(char* stage, const T* Kg, const T* Vg, int tb, int nmax,
                                          int wid) const {
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int j = wid + i * NW;
            const T* base = (j >= S::INSTS) ? Vg : Kg;            // wavefront-uniform
            const T* src = base + (size_t)max(min(tb + row[i], nmax), 0) * D + off[i];
            __builtin_amdgcn_global_load_lds(src, stage + dst[i], 16, 0, 0);
        }
    }
};

// Wait until at most N vector memory operations of this wavefront are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier after this wavefront's LDS writes and reads have completed. Unlike
// __syncthreads() it does not also wait for the copies into LDS still in flight
// (their landing is ordered by explicit vmcnt waits).
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n s_barrier" ::: "memory");
}

__device__ __forceinline__ void wait_tile_copies() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// 8 consecutive elements (one k16-step operand) of row t starting at element e0 of
// a K tile stored with the K swizzle.
template <typename T, int D, int TT>
__device__ __forceinline__ typename Mfma<T>::Op load_k_op(const char* ktile, int t, int e0) {
    typedef SwzTile<T, D, TT> S;
    typedef Mfma<T> MM;
    constexpr int EPP = 16 / S::ES;                  // elements per piece
    const char* row = ktile + t * S::ROWB;
    if constexpr (S::ES == 2) {
        return MM::load(reinterpret_cast<const T*>(row + S::kslot(t, e0 / EPP) * 16));
    } else {
        const f32x4 a = *reinterpret_cast<const f32x4*>(row + S::kslot(t, e0 / EPP) * 16);
        const f32x4 b = *reinterpret_cast<const f32x4*>(row + S::kslot(t, e0 / EPP + 1) * 16);
        return pack_f32x8(MM::zero(), a, b);
    }
}

// A operand of O^T += V^T P^T for k16 step s and d-block db (rows d = 32db + lane%32,
// k-slot (h = lane/32, e) = token 16s + 8(e/4) + 4h + e%4) from a V tile stored
// row-major with the V swizzle.
//  * bf16: two transposing reads. In a 16-lane group, lane 4k+c addresses the 4
//    elements of row t_k at d0 + 4c and lane i receives element d0 + i of rows
//    t_0..t_3; the two reads cover e = 0..3 and e = 4..7.
//  * fp32: no transpose is needed for one element per MFMA: 8 scalar reads.
template <typename T, int D, int TT>
__device__ __forceinline__ typename Mfma<T>::Op load_vt_op(const char* vtile, int s, int db, int lane) {
    typedef SwzTile<T, D, TT> S;
    if constexpr (S::ES == 2) {
        const int G = lane >> 4, i = lane & 15, k = i >> 2, c = i & 3;
        const int h = G >> 1, dh = G & 1;
        const int cp = 4 * db + 2 * dh + (c >> 1);
        const int boff = (c & 1) * 8;
        s16x4 r[2];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int t = 16 * s + 8 * rr + 4 * h + k;
            const char* a = vtile + t * S::ROWB + S::vslot(t, cp) * 16 + boff;
            r[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(a));
        }
        typename Mfma<T>::Op o;
        o = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r[0], r[1], 0, 1, 2, 3, 4, 5, 6, 7));
        return o;
    } else {
        const int d = 32 * db + (lane & 31), h = lane >> 5;
        typename Mfma<T>::Op o;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = 16 * s + 8 * (e >> 2) + 4 * h + (e & 3);
            o.v[e] = *reinterpret_cast<const float*>(vtile + t * S::ROWB + S::vslot(t, d >> 2) * 16 + (d & 3) * 4);
        }
        return o;
    }
}

// LDS geometry of one token tile of TT tokens.
template <typename T, int D, int TT>
struct TileGeom {
    static constexpr int ES = sizeof(T);
    static constexpr int KROW = D * ES + 16;           // bytes per K row
    static constexpr int VROW = TT * ES + 16;          // bytes per V^T row (one d)
    static constexpr int KBYTES = TT * KROW;
    static constexpr int VBYTES = D * VROW;
    static constexpr int BYTES = KBYTES + VBYTES;
    static constexpr int KPIECES = TT * D * ES / 16;   // 16-byte pieces of the K tile
};

// slot of token t (0..TT-1) in the V^T tile: swap bits 2 and 3 within each 16-group
__device__ __forceinline__ int v_slot(int t) {
    return (t & ~15) | ((t & 4) << 1) | ((t & 8) >> 1) | (t & 3);
}

// Registers holding one K/V tile in flight from global memory. K is copied as
// 16-byte pieces of its rows; V is read as blocks of 4 consecutive tokens x 16 bytes
// (8 bf16 or 4 fp32 of d) and transposed in registers, so every global load is 16
// bytes wide. Consecutive lanes take consecutive 4-token groups of one d-block: the
// transposed stores of a wavefront then fill whole V^T rows (every LDS bank once
// per pass), while each load instruction still reads 64-byte row segments.
template <typename T, int D, int TT, int NTHR>
struct TileRegs {
    typedef TileGeom<T, D, TT> G;
    static constexpr int VE = 16 / G::ES;                  // elements of d per V block
    static constexpr int VBLK = (TT / 4) * (D / VE);       // V blocks per tile
    static constexpr int KP = (G::KPIECES + NTHR - 1) / NTHR;
    static constexpr int VB = (VBLK + NTHR - 1) / NTHR;
    u32x4 k[KP];
    u32x4 v[VB][4];

    // row_of(t) gives the global row index (element offset / D) of tile token t.
    template <typename RowFn>
    __device__ __forceinline__ void load(const T* Kg, const T* Vg, RowFn row_of, int tid) {
        constexpr int PPR = D * G::ES / 16;             // pieces per K row
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            const int q = tid + i * NTHR;
            if (G::KPIECES % NTHR == 0 || q < G::KPIECES) {
                const int t = q / PPR, c = q % PPR;
                k[i] = *reinterpret_cast<const u32x4*>(
                    reinterpret_cast<const char*>(Kg + (size_t)row_of(t) * D) + 16 * c);
            }
        }
        constexpr int TQ = TT / 4;                        // 4-token groups per tile
#pragma unroll
        for (int i = 0; i < VB; ++i) {
            const int q = tid + i * NTHR;
            if (VBLK % NTHR == 0 || q < VBLK) {
                const int tq = q % TQ, dg = q / TQ;
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    v[i][x] = *reinterpret_cast<const u32x4*>(Vg + (size_t)row_of(4 * tq + x) * D + dg * VE);
            }
        }
    }

    __device__ __forceinline__ void store(char* lds, int tid) const {
        constexpr int PPR = D * G::ES / 16;
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            const int q = tid + i * NTHR;
            if (G::KPIECES % NTHR == 0 || q < G::KPIECES) {
                const int t = q / PPR, c = q % PPR;
                *reinterpret_cast<u32x4*>(lds + t * G::KROW + 16 * c) = k[i];
            }
        }
        char* vt = lds + G::KBYTES;
        constexpr int TQ = TT / 4;
#pragma unroll
        for (int i = 0; i < VB; ++i) {
            const int q = tid + i * NTHR;
            if (VBLK % NTHR == 0 || q < VBLK) {
                const int tq = q % TQ, dg = q / TQ;
                const int sl = v_slot(4 * tq);            // 4 tokens -> 4 consecutive slots
                if (G::ES == 2) {
                    // token x holds d = dg*8 + 2j (low half) and + 2j + 1 (high half) in dword j
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        u32x2 lo, hi;
                        lo[0] = __builtin_amdgcn_perm(v[i][1][j], v[i][0][j], 0x05040100u);
                        lo[1] = __builtin_amdgcn_perm(v[i][3][j], v[i][2][j], 0x05040100u);
                        hi[0] = __builtin_amdgcn_perm(v[i][1][j], v[i][0][j], 0x07060302u);
                        hi[1] = __builtin_amdgcn_perm(v[i][3][j], v[i][2][j], 0x07060302u);
                        const int d0 = dg * 8 + 2 * j;
                        *reinterpret_cast<u32x2*>(vt + d0 * G::VROW + sl * 2) = lo;
                        *reinterpret_cast<u32x2*>(vt + (d0 + 1) * G::VROW + sl * 2) = hi;
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        u32x4 o;
                        o[0] = v[i][0][j]; o[1] = v[i][1][j]; o[2] = v[i][2][j]; o[3] = v[i][3][j];
                        *reinterpret_cast<u32x4*>(vt + (dg * 4 + j) * G::VROW + sl * 4) = o;
                    }
                }
            }
        }
    }
};

}  // namespace dash
