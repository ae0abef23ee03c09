// Routed lists -> bitpacked block mask (paper review section 三, GPU kernel table: the
// mask M_i in {0,1}^{T_c} that marks the routed chunks of a query row, 32 chunks per
// 32-bit word). One wavefront per (b, KV group, row): the row's words live in LDS,
// the listed chunks set their bits with LDS atomics, and the words go out coalesced.
#include "kernels.h"
#include "common.h"

namespace dash {

constexpr int kMaskWaves = 4;
constexpr int kMaskMaxWords = 64;     // 2048 chunks

__global__ __launch_bounds__(64 * kMaskWaves) void lists_to_mask_kernel(const int32_t* idx, const int32_t* cnt,
                                                                        size_t rows, int list_cap, int T_c,
                                                                        uint32_t* mask, int words) {
    __shared__ uint32_t s_w[kMaskWaves][kMaskMaxWords];
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const size_t row = (size_t)blockIdx.x * kMaskWaves + wid;
    if (row >= rows) return;                       // no barrier follows
    for (int k = lane; k < words; k += 64) s_w[wid][k] = 0u;
    __builtin_amdgcn_wave_barrier();
    const int cn = min(max(cnt[row], 0), list_cap);
    const int32_t* li = idx + row * (size_t)list_cap;
    for (int e = lane; e < cn; e += 64) {
        const int c = li[e];
        if (c >= 0 && c < T_c) atomicOr(&s_w[wid][c >> 5], 1u << (c & 31));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint32_t* out = mask + row * (size_t)words;
    for (int k = lane; k < words; k += 64) out[k] = s_w[wid][k];
}

hipError_t launch_lists_to_mask(const int32_t* idx, const int32_t* cnt, size_t rows, int list_cap, int T_c,
                                uint32_t* mask, int words, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const size_t blocks = (rows + kMaskWaves - 1) / kMaskWaves;
    hipLaunchKernelGGL(lists_to_mask_kernel, dim3((unsigned)blocks), dim3(64 * kMaskWaves), 0, s, idx, cnt, rows,
                       list_cap, T_c, mask, words);
    return hipGetLastError();
}

}  // namespace dash
