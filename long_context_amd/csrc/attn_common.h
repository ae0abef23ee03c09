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
};

struct F32x8 { float v[8]; };

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
};

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
            if (q < G::KPIECES) {
                const int t = q / PPR, c = q % PPR;
                k[i] = *reinterpret_cast<const u32x4*>(
                    reinterpret_cast<const char*>(Kg + (size_t)row_of(t) * D) + 16 * c);
            }
        }
        constexpr int TQ = TT / 4;                        // 4-token groups per tile
#pragma unroll
        for (int i = 0; i < VB; ++i) {
            const int q = tid + i * NTHR;
            if (q < VBLK) {
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
            if (q < G::KPIECES) {
                const int t = q / PPR, c = q % PPR;
                *reinterpret_cast<u32x4*>(lds + t * G::KROW + 16 * c) = k[i];
            }
        }
        char* vt = lds + G::KBYTES;
        constexpr int TQ = TT / 4;
#pragma unroll
        for (int i = 0; i < VB; ++i) {
            const int q = tid + i * NTHR;
            if (q < VBLK) {
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
