// Device-side types and conversions shared by the kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace stem {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// The 16 bytes of a load, widened to fp32.  ES = element size in bytes.
// FP8 uses the gfx950 hardware conversion of OCP E4M3.
template <int ES>
__device__ __forceinline__ void widen16(const uint4 &u, float *out) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    if constexpr (ES == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
    } else if constexpr (ES == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
            out[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[4 * i + 0] = __builtin_amdgcn_cvt_f32_fp8((int)w[i], 0);
            out[4 * i + 1] = __builtin_amdgcn_cvt_f32_fp8((int)w[i], 1);
            out[4 * i + 2] = __builtin_amdgcn_cvt_f32_fp8((int)w[i], 2);
            out[4 * i + 3] = __builtin_amdgcn_cvt_f32_fp8((int)w[i], 3);
        }
    }
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// max / sum of x over lanes l and l ^ 32 (v_permlane32_swap: VALU, no LDS).
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Order-preserving key of a score for top-k selection: larger score -> larger
// key; NaN below everything (key 0); -0 == +0.
__device__ __forceinline__ uint32_t order_key(float x) {
    if (x != x) return 0u;
    if (x == 0.0f) x = 0.0f;
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Starting point of a bitwise search for a k-th largest key among keys that
// all lie in [kmin, kmax]: the bits they share above the highest differing
// bit, and that bit (-1 when kmin == kmax, in which case the prefix is the key).
__device__ __forceinline__ uint32_t key_prefix(uint32_t kmin, uint32_t kmax, int &top) {
    const uint32_t diff = kmin ^ kmax;
    top = diff ? 31 - __builtin_clz(diff) : -1;
    return top < 0 ? kmax : (kmin & ~((2u << top) - 1u));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, off));
    return x;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, off));
    return x;
}

// Number of set bits of `m` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

}  // namespace stem
