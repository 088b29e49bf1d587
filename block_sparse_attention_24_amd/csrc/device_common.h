// Device-side types and conversions shared by the kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace stem {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// 16 bytes read once (a streaming pass): a non-temporal load, which keeps the
// stream from displacing reused data in the caches.
__device__ __forceinline__ uint4 load16_stream(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

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

// Reductions across lanes on the VALU (DPP within 16-lane rows,
// v_permlane16_swap / v_permlane32_swap across rows), so that no step takes
// an LDS round trip.  Every lane of a group receives the same result.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum_xor16(float x) {       // x of lanes l and l ^ 16
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Sum / max over each aligned group of N consecutive lanes (N a power of two
// up to 64).  Pairs: lanes l ^ 1, l ^ 2 (quad permutes), then the halves of
// 8 and of 16 lanes (mirrors, which pair the same partial sums as l ^ 4 and
// l ^ 8), then l ^ 16 and l ^ 32.
template <int N>
__device__ __forceinline__ float sum_lanes(float x) {
    if constexpr (N >= 2) x += dpp_f32<0xB1>(x);             // quad_perm [1, 0, 3, 2]
    if constexpr (N >= 4) x += dpp_f32<0x4E>(x);             // quad_perm [2, 3, 0, 1]
    if constexpr (N >= 8) x += dpp_f32<0x141>(x);            // row_half_mirror
    if constexpr (N >= 16) x += dpp_f32<0x140>(x);           // row_mirror
    if constexpr (N >= 32) x = sum_xor16(x);
    if constexpr (N >= 64) x = sum_xor32(x);
    return x;
}
template <int N>
__device__ __forceinline__ float max_lanes(float x) {
    if constexpr (N >= 2) x = fmaxf(x, dpp_f32<0xB1>(x));
    if constexpr (N >= 4) x = fmaxf(x, dpp_f32<0x4E>(x));
    if constexpr (N >= 8) x = fmaxf(x, dpp_f32<0x141>(x));
    if constexpr (N >= 16) x = fmaxf(x, dpp_f32<0x140>(x));
    if constexpr (N >= 32) x = max_xor16(x);
    if constexpr (N >= 64) x = max_xor32(x);
    return x;
}
// Sum over the lanes that share lane % S (S a power of two, 4 to 64): every
// lane receives the sum over lanes l, l + S, l + 2S, ... of the wave.
template <int S>
__device__ __forceinline__ float sum_stride(float x) {
    if constexpr (S <= 4) x += dpp_f32<0x124>(x);            // row_ror 4
    if constexpr (S <= 8) x += dpp_f32<0x128>(x);            // row_ror 8
    if constexpr (S <= 16) x = sum_xor16(x);
    if constexpr (S <= 32) x = sum_xor32(x);
    return x;
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

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}
// Minimum / maximum of x over the wave, on the VALU (the pairing of max_lanes).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
    x = min(x, dpp_u32<0xB1>(x));
    x = min(x, dpp_u32<0x4E>(x));
    x = min(x, dpp_u32<0x141>(x));
    x = min(x, dpp_u32<0x140>(x));
    auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = min(r[0], r[1]);
    r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return min(r[0], r[1]);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    x = max(x, dpp_u32<0xB1>(x));
    x = max(x, dpp_u32<0x4E>(x));
    x = max(x, dpp_u32<0x141>(x));
    x = max(x, dpp_u32<0x140>(x));
    auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = max(r[0], r[1]);
    r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max(r[0], r[1]);
}

// Sum of x over the wave, in every lane (the pairing of wave_min_u32).
__device__ __forceinline__ int wave_sum_i32(int x) {
    x += (int)dpp_u32<0xB1>((uint32_t)x);
    x += (int)dpp_u32<0x4E>((uint32_t)x);
    x += (int)dpp_u32<0x141>((uint32_t)x);
    x += (int)dpp_u32<0x140>((uint32_t)x);
    auto r = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
    x = (int)(r[0] + r[1]);
    r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    return (int)(r[0] + r[1]);
}

// Number of set bits of `m` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Threshold of a top-k among keys held as key[c] for J = 64 c + lane (c < NCH),
// the candidates being J in [1, I-1] (every other J holds key 0, which no
// trial value counts): t is the want-th largest key, or a value with exactly
// `want` keys at or above it; the kept set is every key > t plus the first
// need_eq keys == t in J order.  Needs 0 < want < ncand = I - 1.
// A bitwise search from the highest bit on which the candidates differ (the
// bits above it are common to all of them, so to t as well).  While the
// bucket of keys sharing t's decided bits holds more than 64 keys, each bit is
// counted per lane on the VALU and summed across the wave once; then the
// bucket is gathered into one key per lane through buf (64 u32 of LDS, this
// wave's) and each further bit costs one ballot.  all_eq: every key == t is
// kept (need_eq covers them all), so the kept set is simply the keys >= t.
template <int NCH>
__device__ __forceinline__ void topk_threshold(const uint32_t (&key)[NCH], int I, int want, int ncand,
                                               uint32_t *buf, int lane, uint32_t &t, int &need_eq,
                                               bool &all_eq) {
    all_eq = true;
    uint32_t kmin = ~0u, kmax = 0u;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int j = c * 64 + lane;
        kmin = min(kmin, (j >= 1 && j < I) ? key[c] : ~0u);
        kmax = max(kmax, key[c]);              // invalid J: 0, and some J is valid here
    }
    int bit;
    t = key_prefix(wave_min_u32(kmin), wave_max_u32(kmax), bit);
    // The bucket: the keys whose bits above `bit` equal t's; `above` keys lie
    // above it.  A trial value t | 2^bit is reached by the keys above the
    // bucket and the bucket's keys with that bit set.
    int above = 0, size = ncand;
    for (; bit >= 0 && size > 64; --bit) {
        const uint32_t cand = t | (1u << bit);
        int cl = 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) cl += key[c] >= cand ? 1 : 0;
        const int cnt = __builtin_amdgcn_readfirstlane(wave_sum_i32(cl));
        if (cnt >= want) {
            t = cand;
            size = cnt - above;
        } else {
            size -= cnt - above;
            above = cnt;
        }
        // Exactly `want` keys are >= cand: they are the kept set whatever the
        // lower bits hold, and the rule keeps every key > t and every key == t.
        if (cnt == want) {
            need_eq = want;                    // every key == t (there are want - #{> t} of them)
            return;
        }
    }
    if (bit >= 0) {
        // gather the bucket (at most 64 keys) into one key per lane
        const uint32_t hi = bit >= 31 ? 0u : ~0u << (bit + 1);
        int run = 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int j = c * 64 + lane;
            const bool in = j >= 1 && j < I && ((key[c] ^ t) & hi) == 0u;
            const uint64_t m = ballot64(in);
            if (in) buf[run + lanes_below(m)] = key[c];
            run += __popcll(m);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        const uint32_t kb = lane < run ? buf[lane] : 0u;
        for (; bit >= 0; --bit) {
            const uint32_t cand = t | (1u << bit);
            const int cnt = above + __popcll(ballot64(kb >= cand));
            if (cnt >= want) t = cand;
            if (cnt == want) {
                need_eq = want;
                return;
            }
        }
        // t is the want-th largest key: the keys above it lie above the bucket
        // or in it, and the keys equal to it all lie in it
        need_eq = want - (above + __popcll(ballot64(kb > t)));
        all_eq = need_eq >= __popcll(ballot64(kb == t));
        return;
    }
    int gt = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) gt += __popcll(ballot64(key[c] > t));
    need_eq = want - gt;
    all_eq = need_eq >= size;                      // every bit decided: the bucket is the keys == t
}

}  // namespace stem
