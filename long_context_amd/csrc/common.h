// Device helpers shared by the DashAttention HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dash {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 raw bits <-> fp32. bf16 -> fp32 is exact; fp32 -> bf16 rounds to nearest even
// (gfx950 has a native conversion instruction for the __bf16 cast).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
}

// 2^x on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the hardware unit (v_log_f32).
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Cross-lane exchange within the wave (ds_bpermute based).
__device__ __forceinline__ float shfl_xor(float v, int mask) {
    int l = lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute(((l ^ mask) & 63) << 2, __float_as_int(v)));
}
__device__ __forceinline__ int shfl_xor_i(int v, int mask) {
    int l = lane_id();
    return __builtin_amdgcn_ds_bpermute(((l ^ mask) & 63) << 2, v);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Sum / max of the values of lanes l and l^16 (l^32) without LDS traffic:
// v_permlane16_swap (v_permlane32_swap) with both operands equal hands every lane
// its own and its partner's value; sum and max are symmetric in the two, so both
// lanes of a pair get the same, order-independent result.
__device__ __forceinline__ float pair16_sum(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair16_max(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Value of the partner lane within a 16-lane row: xor 1, xor 2, mirror within 8
// lanes, mirror within 16 (DPP). Applied in this order with a symmetric combine,
// they reduce a whole row and leave the result in every lane of it.
template <int CTRL>
__device__ __forceinline__ float dpp_partner(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum / max over all 64 lanes (the same value in every lane): DPP within each
// 16-lane row, then the cross-row swaps; no LDS traffic.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_partner<0xB1>(v);
    v += dpp_partner<0x4E>(v);
    v += dpp_partner<0x141>(v);
    v += dpp_partner<0x140>(v);
    return pair32_sum(pair16_sum(v));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_partner<0xB1>(v));
    v = fmaxf(v, dpp_partner<0x4E>(v));
    v = fmaxf(v, dpp_partner<0x141>(v));
    v = fmaxf(v, dpp_partner<0x140>(v));
    return pair32_max(pair16_max(v));
}

// Load 8 consecutive elements of a row as fp32 (T = float or raw bf16 bits).
template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kBytes = 4;
    __device__ __forceinline__ static void load8(const float* p, float* out) {
        const f32x4* q = reinterpret_cast<const f32x4*>(p);
        f32x4 a = q[0], b = q[1];
        out[0] = a[0]; out[1] = a[1]; out[2] = a[2]; out[3] = a[3];
        out[4] = b[0]; out[5] = b[1]; out[6] = b[2]; out[7] = b[3];
    }
};
template <> struct Elem<uint16_t> {
    static constexpr int kBytes = 2;
    __device__ __forceinline__ static void load8(const uint16_t* p, float* out) {
        u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(v[i] << 16);
            out[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
        }
    }
};

}  // namespace dash
