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
    static constexpr int EPD = 4 / ES;                 // elements per dword (2 bf16, 1 f32)
    static constexpr int VBLOCKS = (TT / 8) * (D / EPD);   // (8 tokens x 1 dword) blocks of V
};

// slot of token t (0..TT-1) in the V^T tile: swap bits 2 and 3 within each 16-group
__device__ __forceinline__ int v_slot(int t) {
    return (t & ~15) | ((t & 4) << 1) | ((t & 8) >> 1) | (t & 3);
}

// Registers holding one K/V tile in flight from global memory.
template <typename T, int D, int TT, int NTHR>
struct TileRegs {
    typedef TileGeom<T, D, TT> G;
    static constexpr int KP = (G::KPIECES + NTHR - 1) / NTHR;
    static constexpr int VB = (G::VBLOCKS + NTHR - 1) / NTHR;
    u32x4 k[KP];
    uint32_t v[VB][8];

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
        constexpr int DW = D / G::EPD;                   // dwords per V row
#pragma unroll
        for (int i = 0; i < VB; ++i) {
            const int q = tid + i * NTHR;
            if (q < G::VBLOCKS) {
                const int dw = q % DW, tg = q / DW;
#pragma unroll
                for (int x = 0; x < 8; ++x)
                    v[i][x] = reinterpret_cast<const uint32_t*>(Vg + (size_t)row_of(8 * tg + x) * D)[dw];
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
        constexpr int DW = D / G::EPD;
#pragma unroll
        for (int i = 0; i < VB; ++i) {
            const int q = tid + i * NTHR;
            if (q < G::VBLOCKS) {
                const int dw = q % DW, tg = q / DW;
                const int t0 = 8 * tg;
                // tokens t0..t0+3 and t0+4..t0+7 land on two runs of 4 consecutive slots
                const int s0 = v_slot(t0), s1 = v_slot(t0 + 4);
                if (G::ES == 2) {
                    // dword x holds (d = 2dw, 2dw+1) of token t0+x
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const uint32_t* w = &v[i][4 * half];
                        const int sl = half ? s1 : s0;
                        u32x2 lo, hi;
                        lo[0] = (w[0] & 0xFFFFu) | (w[1] << 16);
                        lo[1] = (w[2] & 0xFFFFu) | (w[3] << 16);
                        hi[0] = (w[0] >> 16) | (w[1] & 0xFFFF0000u);
                        hi[1] = (w[2] >> 16) | (w[3] & 0xFFFF0000u);
                        *reinterpret_cast<u32x2*>(vt + (2 * dw) * G::VROW + sl * 2) = lo;
                        *reinterpret_cast<u32x2*>(vt + (2 * dw + 1) * G::VROW + sl * 2) = hi;
                    }
                } else {
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const uint32_t* w = &v[i][4 * half];
                        const int sl = half ? s1 : s0;
                        u32x4 o;
                        o[0] = w[0]; o[1] = w[1]; o[2] = w[2]; o[3] = w[3];
                        *reinterpret_cast<u32x4*>(vt + dw * G::VROW + sl * 4) = o;
                    }
                }
            }
        }
    }
};

}  // namespace dash
