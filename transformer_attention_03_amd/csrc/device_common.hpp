// Device helpers shared by the attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ta03 {

constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

// 2^x on the transcendental unit (v_exp_f32).  exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 1/x on the transcendental unit (v_rcp_f32, 1 ulp).
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// tanh from the identity tanh(x) = 1 - 2 / (exp(2x) + 1), with exp(2x) = 2^(2x log2 e).
// For large |x| the exponential saturates to 0 or +inf and the result to -1 or +1.
// Absolute error is a few f32 ulps of 1 (cancellation near 0 costs relative, not
// absolute, accuracy), which is what a logit cap c * tanh(s / c) needs.
__device__ __forceinline__ float tanh_via_exp(float x) {
    const float e = fast_exp2(x * (2.0f * kLog2e));
    return 1.0f - 2.0f * fast_rcp(e + 1.0f);
}

// tanh with a small relative error for every argument: below |x| = 1/4 the odd Taylor series
// x - x^3/3 + 2x^5/15 - 17x^7/315 (remainder under 4e-7 relative there), above it the
// identity above, whose absolute error of a few f32 ulps of 1 is then under 1e-6 of |x|.
// A logit cap c tanh(s / c) needs this when c is large: the identity alone errs by about
// 1.2e-7 c in absolute terms, which for c = 1e6 is 0.1 on every score.
__device__ __forceinline__ float tanh_accurate(float x) {
    const float x2 = x * x;
    float p = __builtin_fmaf(x2, -17.f / 315.f, 2.f / 15.f);
    p = __builtin_fmaf(x2, p, -1.f / 3.f);
    const float small = __builtin_fmaf(x * x2, p, x);
    return __builtin_fabsf(x) < 0.25f ? small : tanh_via_exp(x);
}

// ---- cross-lane helpers (DPP inside a row of 16 lanes, ds_bpermute across rows) ------------

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
// quad_perm encodings: xor 1 -> [1,0,3,2], xor 2 -> [2,3,0,1]
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7 - i inside each group of 8
constexpr int kDppMirror = 0x140;       // lane i <-> 15 - i inside each row of 16

__device__ __forceinline__ float shfl_xor_f(float x, int m) {
    return __shfl_xor(x, m, 64);
}

// Sum over aligned groups of N lanes (N in 1,2,4,8,16,32,64); every lane gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (N >= 2) x += dpp_f<kDppXor1>(x);
    if constexpr (N >= 4) x += dpp_f<kDppXor2>(x);
    if constexpr (N >= 8) x += dpp_f<kDppHalfMirror>(x);
    if constexpr (N >= 16) x += dpp_f<kDppMirror>(x);
    if constexpr (N >= 32) x += shfl_xor_f(x, 16);
    if constexpr (N >= 64) x += shfl_xor_f(x, 32);
    return x;
}

// Max over aligned groups of N lanes (N in 1,2,4,8,16); every lane gets the max.
template <int N>
__device__ __forceinline__ float group_max(float x) {
    if constexpr (N >= 2) x = fmaxf(x, dpp_f<kDppXor1>(x));
    if constexpr (N >= 4) x = fmaxf(x, dpp_f<kDppXor2>(x));
    if constexpr (N >= 8) x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
    if constexpr (N >= 16) x = fmaxf(x, dpp_f<kDppMirror>(x));
    return x;
}

// Max over aligned groups of 16 lanes (one DPP row); every lane gets the max.
__device__ __forceinline__ float group_max16(float x) {
    x = fmaxf(x, dpp_f<kDppXor1>(x));
    x = fmaxf(x, dpp_f<kDppXor2>(x));
    x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
    return fmaxf(x, dpp_f<kDppMirror>(x));
}

// Lane n of each row of 16 lanes, to every lane of that row (DPP row_newbcast).  n must be a
// compile-time constant after inlining and unrolling (the switch then folds to one case).
template <int N>
__device__ __forceinline__ float row_bcast16_c(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_bcast16(float x, int n) {
    switch (n & 15) {
        case 0: return row_bcast16_c<0>(x);
        case 1: return row_bcast16_c<1>(x);
        case 2: return row_bcast16_c<2>(x);
        case 3: return row_bcast16_c<3>(x);
        case 4: return row_bcast16_c<4>(x);
        case 5: return row_bcast16_c<5>(x);
        case 6: return row_bcast16_c<6>(x);
        case 7: return row_bcast16_c<7>(x);
        case 8: return row_bcast16_c<8>(x);
        case 9: return row_bcast16_c<9>(x);
        case 10: return row_bcast16_c<10>(x);
        case 11: return row_bcast16_c<11>(x);
        case 12: return row_bcast16_c<12>(x);
        case 13: return row_bcast16_c<13>(x);
        case 14: return row_bcast16_c<14>(x);
        default: return row_bcast16_c<15>(x);
    }
}

// Integer sum over the wave (every lane gets it) and inclusive prefix sum by lane.
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}
__device__ __forceinline__ int wave_incl_scan_i(int x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

// Max over lanes that are congruent modulo N (N = 1..64, power of two): reduces across
// the 64/N groups of N lanes.  Every lane gets the max of its residue class.
template <int N>
__device__ __forceinline__ float strided_max(float x) {
#pragma unroll
    for (int m = N; m < 64; m <<= 1) x = fmaxf(x, shfl_xor_f(x, m));
    return x;
}
template <int N>
__device__ __forceinline__ float strided_sum(float x) {
#pragma unroll
    for (int m = N; m < 64; m <<= 1) x += shfl_xor_f(x, m);
    return x;
}

// Reductions across the four 16-lane rows (lanes congruent mod 16) with the gfx950 lane
// swaps: after permlane16_swap(x, x) (resp. permlane32_swap) a lane holds its own value
// and that of lane ^ 16 (resp. ^ 32), in an order that depends on the lane.
__device__ __forceinline__ float rows_max(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---- memory ---------------------------------------------------------------------------------

// Byte offset in LDS of a generic pointer into shared memory: the LDS aperture is 4 GB
// aligned, so the low 32 bits of the generic address are the offset (no null check).
__device__ __forceinline__ uint32_t lds_offset(const void* p) { return (uint32_t)(uintptr_t)p; }

// Device-scope (all XCDs) relaxed store / load: written through, resp. fetched past, the
// XCD-private L2, so another workgroup on any XCD observes them without cache-wide fences.
__device__ __forceinline__ void store_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's outstanding vector-memory operations (including stores) completed.
__device__ __forceinline__ void wait_stores_complete() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint4 ld_global_b128(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// int8 x 16 in a uint4 -> 16 floats
__device__ __forceinline__ void i8x16_to_f32(const uint4& w, float* f) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
            f[4 * i + b] = (float)(int8_t)((ws[i] >> (8 * b)) & 0xFF);
    }
}

// int8 x 8 in two words -> 8 floats
__device__ __forceinline__ void i8x8_to_f32(uint32_t lo, uint32_t hi, float* f) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        f[b] = (float)(int8_t)((lo >> (8 * b)) & 0xFF);
        f[4 + b] = (float)(int8_t)((hi >> (8 * b)) & 0xFF);
    }
}

// f16 x 8 in a uint4 -> 8 floats
__device__ __forceinline__ void f16x8_to_f32(const uint4& w, float* f) {
    half8_t h = __builtin_bit_cast(half8_t, w);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
}

}  // namespace ta03
