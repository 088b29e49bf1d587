// OAM block scoring (Stem article on cn486.com, §一.3.2 "Output-Aware Metric";
// §二.2.1: compact block-level Q/K representations, then one GEMM gives every
// block score, with no softmax, no gather and no token-level intermediate).
//
// Two kernels:
//   pool_kernel   one HBM pass over Q, K, V: per block the mean of the Q rows
//                 and of the K rows, and ln of the Frobenius norm of the V rows.
//   score_kernel  per head, fp32 tiles of tau * qbar kbar^T + lvn on and below
//                 the diagonal, -inf above it.
// Both use a fixed summation order, so results are bit-reproducible.
#include "device_common.h"
#include "stem_internal.h"

namespace stem {
namespace {

constexpr int kPoolThreads = 256;

struct PoolArgs {
    const char *base;          // Q, K or V
    float *out;                // qbar/kbar [b, H, Nb, d] or lvn [b, H, Nb]
    const int32_t *table;      // paged K/V, else nullptr
    int page_log2, pages_per_seq;
    int heads, d, blk, seq, nb;
    int chunks_per_row;        // 16-byte chunks in one token row (H * d * ES / 16)
    float scale;               // dequantisation scale
};

// Thread = one 16-byte column chunk of a token row; a workgroup covers 256
// chunks of one block and walks its blk rows in order.  MODE 0: mean of the
// rows; MODE 1: sum of squares, reduced over each head's chunks -> lvn.
template <int ES, int MODE>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(PoolArgs a) {
    constexpr int EPC = 16 / ES;              // elements per chunk
    const int chunk = blockIdx.x * kPoolThreads + threadIdx.x;
    const int blk_j = blockIdx.y;
    const int b = blockIdx.z;
    const bool active = chunk < a.chunks_per_row;
    const size_t row_bytes = (size_t)a.chunks_per_row * 16;

    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.0f;

    if (active) {
        const int tok0 = blk_j * a.blk;
#pragma unroll 8
        for (int t = 0; t < a.blk; ++t) {
            const int tok = tok0 + t;
            size_t row;
            if (a.table) {
                const int page = a.table[(size_t)b * a.pages_per_seq + (tok >> a.page_log2)];
                row = ((size_t)page << a.page_log2) + (tok & ((1 << a.page_log2) - 1));
            } else {
                row = (size_t)b * a.seq + tok;
            }
            const uint4 u = *reinterpret_cast<const uint4 *>(a.base + row * row_bytes + (size_t)chunk * 16);
            float x[EPC];
            widen16<ES>(u, x);
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                if constexpr (MODE == 0) acc[e] += x[e];
                else acc[e] = fmaf(x[e], x[e], acc[e]);
            }
        }
    }

    const int col = chunk * EPC;              // first element (head-major, then d)
    const int h = col / a.d;
    const int dd = col % a.d;
    if constexpr (MODE == 0) {
        if (!active) return;
        const float f = 1.0f / (float)a.blk;
        float *dst = a.out + (((size_t)b * a.heads + h) * a.nb + blk_j) * a.d + dd;
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
            f32x4 v;
            v[0] = acc[e] * f * a.scale;
            v[1] = acc[e + 1] * f * a.scale;
            v[2] = acc[e + 2] * f * a.scale;
            v[3] = acc[e + 3] * f * a.scale;
            *reinterpret_cast<f32x4 *>(dst + e) = v;
        }
    } else {
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) s += acc[e];
        // butterfly over the chunks of one head (a power of two <= 32, aligned)
        const int cph = a.d / EPC;
        for (int off = 1; off < cph; off <<= 1) s += __shfl_xor(s, off);
        if (active && (chunk % cph) == 0)
            a.out[((size_t)b * a.heads + h) * a.nb + blk_j] = 0.5f * logf(s) + logf(a.scale);
    }
}

template <int ES>
hipError_t pool_all(const Shape &s, const void *q, const KvView &kv, float *qbar, float *kbar,
                    float *lvn, hipStream_t st) {
    PoolArgs a{};
    a.d = s.d;
    a.blk = s.blk;
    a.seq = s.seq;
    a.nb = s.nb;
    // Q: always contiguous
    a.base = static_cast<const char *>(q);
    a.out = qbar;
    a.table = nullptr;
    a.heads = s.hq;
    a.chunks_per_row = s.hq * s.d * ES / 16;
    a.scale = s.q_scale;
    dim3 grid((a.chunks_per_row + kPoolThreads - 1) / kPoolThreads, s.nb, s.batch);
    hipLaunchKernelGGL((pool_kernel<ES, 0>), grid, dim3(kPoolThreads), 0, st, a);
    // K and V: contiguous or paged
    a.table = kv.table;
    a.page_log2 = kv.page_log2;
    a.pages_per_seq = kv.pages_per_seq;
    a.heads = s.hkv;
    a.chunks_per_row = s.hkv * s.d * ES / 16;
    grid.x = (a.chunks_per_row + kPoolThreads - 1) / kPoolThreads;
    a.base = static_cast<const char *>(kv.k);
    a.out = kbar;
    a.scale = s.k_scale;
    hipLaunchKernelGGL((pool_kernel<ES, 0>), grid, dim3(kPoolThreads), 0, st, a);
    a.base = static_cast<const char *>(kv.v);
    a.out = lvn;
    a.scale = s.v_scale;
    hipLaunchKernelGGL((pool_kernel<ES, 1>), grid, dim3(kPoolThreads), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Score GEMM: a 64 x 64 tile of (I, J) per workgroup, 4 x 4 outputs per
// thread, d streamed through LDS in slices of 32 (stored d-major so a thread
// reads its four rows as one 16-byte word).
// ---------------------------------------------------------------------------
constexpr int kTile = 64;
constexpr int kSlice = 32;

struct ScoreArgs {
    const float *qbar, *kbar, *lvn;
    float *scores;
    int hq, hkv, nb, d;
    float tau;
};

__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
    __shared__ float qs[kSlice][kTile + 4];
    __shared__ float ks[kSlice][kTile + 4];
    const int tiles = (a.nb + kTile - 1) / kTile;
    const int ti = blockIdx.x / tiles;          // I tile
    const int tj = blockIdx.x % tiles;          // J tile
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int g = h / (a.hq / a.hkv);
    const int tid = threadIdx.x;
    const int r0 = (tid / 16) * 4;              // 4 rows (I) of this thread
    const int c0 = (tid % 16) * 4;              // 4 cols (J)
    float *out = a.scores + (((size_t)b * a.hq + h) * a.nb) * a.nb;
    const float ninf = -__builtin_huge_valf();

    if (tj > ti) {                              // wholly above the diagonal
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int I = ti * kTile + r0 + r;
            if (I >= a.nb) continue;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int J = tj * kTile + c0 + c;
                if (J < a.nb) out[(size_t)I * a.nb + J] = ninf;
            }
        }
        return;
    }

    const float *qb = a.qbar + (((size_t)b * a.hq + h) * a.nb) * a.d;
    const float *kb = a.kbar + (((size_t)b * a.hkv + g) * a.nb) * a.d;
    float acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = 0.0f;

    for (int d0 = 0; d0 < a.d; d0 += kSlice) {
        // 64 rows x 32 d of each operand: 2048 floats, 8 per thread
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = tid + 256 * i;
            const int row = e / kSlice, dd = e % kSlice;
            const int I = ti * kTile + row, J = tj * kTile + row;
            qs[dd][row] = I < a.nb ? qb[(size_t)I * a.d + d0 + dd] : 0.0f;
            ks[dd][row] = J < a.nb ? kb[(size_t)J * a.d + d0 + dd] : 0.0f;
        }
        __syncthreads();
#pragma unroll 8
        for (int dd = 0; dd < kSlice; ++dd) {
            const f32x4 qv = *reinterpret_cast<const f32x4 *>(&qs[dd][r0]);
            const f32x4 kv = *reinterpret_cast<const f32x4 *>(&ks[dd][c0]);
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(qv[r], kv[c], acc[r][c]);
        }
        __syncthreads();
    }

    const float *lv = a.lvn + ((size_t)b * a.hkv + g) * a.nb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int I = ti * kTile + r0 + r;
        if (I >= a.nb) continue;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int J = tj * kTile + c0 + c;
            if (J >= a.nb) continue;
            out[(size_t)I * a.nb + J] = J <= I ? fmaf(acc[r][c], a.tau, lv[J]) : ninf;
        }
    }
}

}  // namespace

hipError_t launch_pool(const Shape &s, const void *q, const KvView &kv, float *qbar, float *kbar,
                       float *lvn, hipStream_t st) {
    switch (s.dtype) {
        case STEM_F32: return pool_all<4>(s, q, kv, qbar, kbar, lvn, st);
        case STEM_BF16: return pool_all<2>(s, q, kv, qbar, kbar, lvn, st);
        default: return pool_all<1>(s, q, kv, qbar, kbar, lvn, st);
    }
}

hipError_t launch_score(const Shape &s, const float *qbar, const float *kbar, const float *lvn,
                        float *scores, hipStream_t st) {
    ScoreArgs a{qbar, kbar, lvn, scores, s.hq, s.hkv, s.nb, s.d, s.tau};
    const int tiles = (s.nb + kTile - 1) / kTile;
    hipLaunchKernelGGL(score_kernel, dim3(tiles * tiles, s.hq, s.batch), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace stem
