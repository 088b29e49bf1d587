// OAM block scoring (Stem article on cn486.com, §一.3.2 "Output-Aware Metric";
// §二.2.1: compact block-level Q/K representations, then one GEMM gives every
// block score, with no softmax, no gather and no token-level intermediate).
//
// Kernels:
//   pool_kernel         one HBM pass over Q, K and V (one launch): per block
//                       the mean of the rows, or ln of the Frobenius norm of
//                       the V rows.
//   cache_write_kernel  the same block reductions fused into writing a
//                       prefill's K and V into the (FP8, paged) cache: one pass
//                       over the new tokens stores them and pools them.
//   score_kernel        per head, tau * qbar kbar^T (+ lvn) on the matrix
//                       cores, on and below the diagonal only (selection
//                       never reads J > I, so nothing is written there).
// All use a fixed summation order, so results are bit-reproducible; the cache
// write accumulates exactly as pool_kernel does over the stored values, so
// its representations equal, bit for bit, those pooled later from the cache.
#include "device_common.h"
#include "stem_internal.h"

namespace stem {
namespace {

// Pooling workgroups: 64 column chunks x 4 row groups (one wave each).
constexpr int kPoolThreads = 256;
constexpr int kPoolChunks = 64;
constexpr int kRowGroups = kPoolThreads / kPoolChunks;

struct PoolArgs {
    const char *base;          // Q, K or V
    float *out;                // qbar/kbar [b, H, Nb, d] or lvn [b, H, Nb]
    const int32_t *table;      // paged K/V, else nullptr
    int page_log2, pages_per_seq;
    int heads, d, blk, seq, nb;
    int chunks_per_row;        // 16-byte chunks in one token row (H * d * ES / 16)
    float scale;               // dequantisation scale
};

// Row of token tok of sequence b in a contiguous or paged [rows, H, d] tensor.
__device__ __forceinline__ size_t token_row(const int32_t *table, int page_log2, int pages_per_seq,
                                            int seq, int b, int tok) {
    if (table) {
        const int page = table[(size_t)b * pages_per_seq + (tok >> page_log2)];
        return ((size_t)page << page_log2) + (tok & ((1 << page_log2) - 1));
    }
    return (size_t)b * seq + tok;
}

// Block reductions, shared by pool_kernel and cache_write_kernel so that both
// produce the same bits.  A thread owns EPC consecutive elements (one 16-byte
// chunk of the stored row) and sees its row group's rows in order.
//   MODE 0: acc = sum of the rows; out = acc / blk * scale (the mean).
//   MODE 1: acc = sum of squares; the chunks of one head are reduced by a
//           butterfly and out = ln(sqrt(sum)) + ln(scale).
template <int EPC, int MODE>
__device__ __forceinline__ void pool_add(float *acc, const float *x) {
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
        if constexpr (MODE == 0) acc[e] += x[e];
        else acc[e] = fmaf(x[e], x[e], acc[e]);
    }
}

template <int EPC, int MODE>
__device__ __forceinline__ void pool_store(const float *acc, bool active, int chunk, float *out,
                                           int b, int heads, int nb, int d, int blk_j, int blk,
                                           float scale) {
    const int col = chunk * EPC;              // first element (head-major, then d)
    const int h = col / d;
    const int dd = col % d;
    if constexpr (MODE == 0) {
        if (!active) return;
        const float f = 1.0f / (float)blk;
        float *dst = out + (((size_t)b * heads + h) * nb + blk_j) * d + dd;
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
            f32x4 v;
            v[0] = acc[e] * f * scale;
            v[1] = acc[e + 1] * f * scale;
            v[2] = acc[e + 2] * f * scale;
            v[3] = acc[e + 3] * f * scale;
            *reinterpret_cast<f32x4 *>(dst + e) = v;
        }
    } else {
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) s += acc[e];
        // butterfly over the chunks of one head (a power of two <= 32, aligned)
        const int cph = d / EPC;
        for (int off = 1; off < cph; off <<= 1) s += __shfl_xor(s, off);
        if (active && (chunk % cph) == 0)
            out[((size_t)b * heads + h) * nb + blk_j] = 0.5f * logf(s) + logf(scale);
    }
}

// Row groups: wave w accumulates rows [w blk/4, (w+1) blk/4) of the block in
// order; the other waves' partial sums are then added to wave 0's in wave
// order through LDS (part: (kRowGroups - 1) * EPC * 64 floats).  Returns true
// in wave 0, which holds the block's sums.
template <int EPC>
__device__ __forceinline__ bool combine_row_groups(float *acc, float *part) {
    const int lane = threadIdx.x % kPoolChunks, wave = threadIdx.x / kPoolChunks;
    if (wave) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) part[((wave - 1) * EPC + e) * kPoolChunks + lane] = acc[e];
    }
    __syncthreads();
    if (wave) return false;
#pragma unroll
    for (int g = 0; g < kRowGroups - 1; ++g)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] += part[(g * EPC + e) * kPoolChunks + lane];
    return true;
}

// Thread = one 16-byte column chunk of a token row in one row group; bx is
// the workgroup's column group within its tensor.
template <int ES, int MODE>
__device__ __forceinline__ void pool_body(const PoolArgs &a, int bx, float *part) {
    constexpr int EPC = 16 / ES;              // elements per chunk
    const int chunk = bx * kPoolChunks + threadIdx.x % kPoolChunks;
    const int group = threadIdx.x / kPoolChunks;
    const int blk_j = blockIdx.y;
    const int b = blockIdx.z;
    const bool active = chunk < a.chunks_per_row;
    const size_t row_bytes = (size_t)a.chunks_per_row * 16;

    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.0f;

    if (active) {
        const int rows = a.blk / kRowGroups;
        const int tok0 = blk_j * a.blk + group * rows;
#pragma unroll 16
        for (int t = 0; t < rows; ++t) {
            const size_t row = token_row(a.table, a.page_log2, a.pages_per_seq, a.seq, b, tok0 + t);
            const uint4 u = load16_stream(a.base + row * row_bytes + (size_t)chunk * 16);
            float x[EPC];
            widen16<ES>(u, x);
            pool_add<EPC, MODE>(acc, x);
        }
    }
    if (combine_row_groups<EPC>(acc, part))
        pool_store<EPC, MODE>(acc, active, chunk, a.out, b, a.heads, a.nb, a.d, blk_j, a.blk, a.scale);
}

// Q, K and V pooled in one launch: column groups [0, g0) are Q's (means),
// [g0, g1) K's (means), [g1, gridDim.x) V's (log-norms); n tensors are set
// (Q alone when the keys' representations come from elsewhere, no V for SAM).
struct PoolSet {
    PoolArgs t[3];
    int g0, g1;
};

template <int ES>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(PoolSet p) {
    __shared__ float part[(kRowGroups - 1) * (16 / ES) * kPoolChunks];
    const int x = blockIdx.x;
    if (x < p.g0) pool_body<ES, 0>(p.t[0], x, part);
    else if (x < p.g1) pool_body<ES, 0>(p.t[1], x - p.g0, part);
    else pool_body<ES, 1>(p.t[2], x - p.g1, part);
}

// ---------------------------------------------------------------------------
// Cache write with the K/V block reductions fused in.
// ---------------------------------------------------------------------------
struct CacheArgs {
    const char *src[2];        // new K, V: [b, S, Hkv, d] in the input type
    char *dst[2];              // cache K, V: contiguous or paged, in the cache type
    float *kbar, *lvn;
    const int32_t *table;
    int page_log2, pages_per_seq;
    int heads, d, blk, seq, nb;
    int chunks_per_row;        // 16-byte chunks of one cached token row
    float scale[2];            // K and V quantisation scales (1 unless FP8)
};

// Nearest OCP E4M3 codes of x / scale for 16 values, ties to even, saturating
// at +-448 (the conversion instruction rounds to nearest even; the clamp makes
// out-of-range values saturate instead of overflowing).
__device__ __forceinline__ uint4 quantize16_e4m3(const float *x, float scale) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float q[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = fminf(fmaxf(x[4 * i + e] / scale, -448.0f), 448.0f);
        int p = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], p, true);
        w[i] = (uint32_t)p;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Thread = one 16-byte chunk of the cached row (EPC = 16 / ES_OUT elements,
// read from EPC * ES_IN input bytes); blockIdx.z = 2 * b + (0: K, 1: V).
template <int ES_IN, int ES_OUT, int MODE>
__device__ __forceinline__ void cache_write_body(const CacheArgs &a, int b, float *part) {
    constexpr int EPC = 16 / ES_OUT;
    constexpr int IN_VEC = EPC * ES_IN / 16;  // 16-byte input loads per chunk
    const int chunk = blockIdx.x * kPoolChunks + threadIdx.x % kPoolChunks;
    const int group = threadIdx.x / kPoolChunks;
    const int blk_j = blockIdx.y;
    const bool active = chunk < a.chunks_per_row;
    const size_t out_row_bytes = (size_t)a.chunks_per_row * 16;
    const size_t in_row_bytes = out_row_bytes * ES_IN / ES_OUT;
    const char *src = a.src[MODE];
    char *dst = a.dst[MODE];
    const float scale = a.scale[MODE];

    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.0f;

    if (active) {
        const int rows = a.blk / kRowGroups;
        const int tok0 = blk_j * a.blk + group * rows;
#pragma unroll 4
        for (int t = 0; t < rows; ++t) {
            const int tok = tok0 + t;
            const char *in = src + ((size_t)b * a.seq + tok) * in_row_bytes + (size_t)chunk * 16 * IN_VEC;
            uint4 stored;
            if constexpr (ES_OUT == 1) {
                float x[EPC];
#pragma unroll
                for (int i = 0; i < IN_VEC; ++i)
                    widen16<ES_IN>(load16_stream(in + 16 * i), x + i * (16 / ES_IN));
                stored = quantize16_e4m3(x, scale);
            } else {
                stored = load16_stream(in);                       // same type: a copy
            }
            const size_t row = token_row(a.table, a.page_log2, a.pages_per_seq, a.seq, b, tok);
            *reinterpret_cast<uint4 *>(dst + row * out_row_bytes + (size_t)chunk * 16) = stored;
            float x[EPC];
            widen16<ES_OUT>(stored, x);       // exactly what pool_kernel reads back
            pool_add<EPC, MODE>(acc, x);
        }
    }
    if (combine_row_groups<EPC>(acc, part))
        pool_store<EPC, MODE>(acc, active, chunk, MODE == 0 ? a.kbar : a.lvn, b, a.heads, a.nb, a.d,
                              blk_j, a.blk, scale);
}

template <int ES_IN, int ES_OUT>
__global__ __launch_bounds__(kPoolThreads) void cache_write_kernel(CacheArgs a) {
    __shared__ float part[(kRowGroups - 1) * (16 / ES_OUT) * kPoolChunks];
    const int b = blockIdx.z >> 1;
    if (blockIdx.z & 1) cache_write_body<ES_IN, ES_OUT, 1>(a, b, part);
    else cache_write_body<ES_IN, ES_OUT, 0>(a, b, part);
}

template <int ES>
PoolArgs pool_args(const Shape &s, const void *base, const int32_t *table, int page_log2, int pages_per_seq,
                   int heads, float scale, float *out) {
    PoolArgs a{};
    a.base = static_cast<const char *>(base);
    a.out = out;
    a.table = table;
    a.page_log2 = page_log2;
    a.pages_per_seq = pages_per_seq;
    a.heads = heads;
    a.d = s.d;
    a.blk = s.blk;
    a.seq = s.seq;
    a.nb = s.nb;
    a.chunks_per_row = heads * s.d * ES / 16;
    a.scale = scale;
    return a;
}

template <int ES>
hipError_t pool_all(const Shape &s, const void *q, const KvView *kv, float *qbar, float *kbar,
                    float *lvn, hipStream_t st) {
    PoolSet p{};
    auto groups = [](const PoolArgs &a) { return (a.chunks_per_row + kPoolChunks - 1) / kPoolChunks; };
    p.t[0] = pool_args<ES>(s, q, nullptr, 0, 0, s.hq, s.q_scale, qbar);
    p.g0 = p.g1 = groups(p.t[0]);
    int gx = p.g0;
    if (kv) {
        p.t[1] = pool_args<ES>(s, kv->k, kv->table, kv->page_log2, kv->pages_per_seq, s.hkv, s.k_scale, kbar);
        p.g1 = gx = p.g0 + groups(p.t[1]);
        if (lvn) {
            p.t[2] = pool_args<ES>(s, kv->v, kv->table, kv->page_log2, kv->pages_per_seq, s.hkv, s.v_scale, lvn);
            gx += groups(p.t[2]);
        }
    }
    hipLaunchKernelGGL((pool_kernel<ES>), dim3(gx, s.nb, s.batch), dim3(kPoolThreads), 0, st, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Score GEMM on the matrix cores, bf16 MFMA (v_mfma_f32_32x32x16_bf16) on a
// two-term split of each fp32 operand: x = hi + lo with hi = bf16(x) and
// lo = bf16(x - hi), and q.k summed as hi.hi + hi.lo + lo.hi in fp32.  The
// dropped lo.lo term and the rounding of lo leave each product within about
// 3 * 2^-18 of |q_i k_i|, a 16-bit-significand product at a tenth of the
// fp32 MFMA time.  A workgroup owns a 128 x 128 tile of (I, J) on or below
// the diagonal, each of its four waves a 64 x 64 quarter held as 2 x 2 MFMA
// tiles; a quarter wholly above the diagonal is not computed, and elements
// with J > I are not stored.  The tile's qbar and kbar rows pass through LDS
// in chunks of 32 dimensions, split once as they are written (two stages:
// the next chunk is written while this one is multiplied).  The order of the
// sum is fixed, so the scores are bit-reproducible.  Workgroups are
// renumbered so that each XCD (workgroup id mod 8) takes a contiguous eighth
// of the heads and reads their representations into its own L2.
// ---------------------------------------------------------------------------
constexpr int kTile = 128;

struct ScoreArgs {
    const float *qbar, *kbar, *lvn;   // lvn == nullptr: no value term (SAM)
    float *scores;
    int hq, hkv, nb, tiles;
    float tau;
};

template <int D>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
    // XCD-contiguous renumbering of (tile, head, batch); the tiles of a head
    // are the tiles.(tiles+1)/2 on or below the diagonal, numbered row by row
    const unsigned n = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const unsigned total = gridDim.x * gridDim.y * gridDim.z;
    const unsigned m = (total & 7u) ? n : (n & 7u) * (total >> 3) + (n >> 3);
    const int tile = (int)(m % gridDim.x);
    const int h = (int)((m / gridDim.x) % gridDim.y);
    const int b = (int)(m / (gridDim.x * gridDim.y));
    int ti = (int)((__builtin_sqrtf(8.0f * (float)tile + 1.0f) - 1.0f) * 0.5f);
    while (ti * (ti + 1) / 2 > tile) --ti;              // exact triangular root
    while ((ti + 1) * (ti + 2) / 2 <= tile) ++ti;
    const int tj = tile - ti * (ti + 1) / 2;            // 0 <= tj <= ti
    const int g = h / (a.hq / a.hkv);
    const int tid = threadIdx.x;
    float *out = a.scores + ((size_t)b * a.hq + h) * a.nb * a.nb;

    const int w = tid >> 6, lane = tid & 63;
    const int r = lane & 31, kh = lane >> 5;
    const int TI = ti * kTile, TJ = tj * kTile;         // the workgroup's tile
    if (TI >= a.nb || TJ >= a.nb) return;               // (whole workgroup: uniform)
    const int I0 = TI + (w >> 1) * 64;
    const int J0 = TJ + (w & 1) * 64;
    // a quarter wholly above the diagonal, or past the end, is not computed;
    // its wave still stages operands for the others
    const bool live = I0 < a.nb && J0 < a.nb && J0 <= I0 + 63;

    // value term of this lane's two columns, loaded ahead of the operands so
    // that the waits of the loop cover it: read between the conditional
    // stores below, it would make every store wait for the one before
    const float *lv = a.lvn ? a.lvn + ((size_t)b * a.hkv + g) * a.nb : nullptr;
    float lj[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) lj[j] = lv ? lv[min(J0 + 32 * j + r, a.nb - 1)] : 0.0f;

    // Staging: per chunk of 32 dimensions the workgroup loads the tile's 128
    // qbar rows and 128 kbar rows (rows past the end read the last row; their
    // results are never stored), splits each float once into bf16 hi and lo
    // and writes the four planes [Q hi, Q lo, K hi, K lo] of 128 rows x 64
    // bytes into one of two LDS stages.  Thread t moves 4-dim groups
    // t + 256 u (u = 0..3) of each operand: row (t + 256 u) / 8, group t % 8.
    // The 16-byte chunk c of row x sits at position c ^ ((x >> 2) & 3), so
    // an MFMA read (16 consecutive rows, one chunk each) covers 16 different
    // 16-byte bank slots of a 256-byte line instead of 4.
    constexpr int CH = 32, NC = D / CH, PLANE = 128 * CH * 2, STAGE = 4 * PLANE;
    __shared__ __attribute__((aligned(16))) char st[2 * STAGE];
    const float *qsrc[4], *ksrc[4];
    int woff[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int x = (tid + 256 * u) >> 3, c4 = tid & 7;
        qsrc[u] = a.qbar + (((size_t)b * a.hq + h) * a.nb + min(TI + x, a.nb - 1)) * D + 4 * c4;
        ksrc[u] = a.kbar + (((size_t)b * a.hkv + g) * a.nb + min(TJ + x, a.nb - 1)) * D + 4 * c4;
        woff[u] = x * 64 + (((c4 >> 1) ^ ((x >> 2) & 3)) << 4) + 8 * (c4 & 1);
    }
    f32x4 gq[4], gk[4];
    auto fetch = [&](int c) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            gq[u] = *reinterpret_cast<const f32x4 *>(qsrc[u] + CH * c);
            gk[u] = *reinterpret_cast<const f32x4 *>(ksrc[u] + CH * c);
        }
    };
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    auto put = [&](int stage) {
        char *base = st + stage * STAGE;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int op = 0; op < 2; ++op) {
                const f32x4 &x = op ? gk[u] : gq[u];
                bf16x4 hi, lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const __bf16 t = (__bf16)x[e];
                    hi[e] = t;
                    lo[e] = (__bf16)(x[e] - (float)t);
                }
                *reinterpret_cast<bf16x4 *>(base + (2 * op) * PLANE + woff[u]) = hi;
                *reinterpret_cast<bf16x4 *>(base + (2 * op + 1) * PLANE + woff[u]) = lo;
            }
    };
    // MFMA operand of k step s (16 dimensions) for tile rows x0 + r: this
    // lane's 8 dimensions 16 s + 8 kh, chunk 2 s + kh of the row
    auto opnd = [&](int stage, int plane, int x0, int s) {
        const int x = x0 + r;
        return *reinterpret_cast<const bf16x8 *>(st + stage * STAGE + plane * PLANE + x * 64 +
                                                 (((2 * s + kh) ^ ((x >> 2) & 3)) << 4));
    };
    auto mfma = [](const bf16x8 &x, const bf16x8 &y, const f32x16 &c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    const int xi = (w >> 1) * 64, xj = (w & 1) * 64;   // the quarter's rows within the tile
    fetch(0);
    put(0);
    if (NC > 1) fetch(1);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        __syncthreads();                                // stage c & 1 written; the other one free
        if (c + 1 < NC) {
            put((c + 1) & 1);
            if (c + 2 < NC) fetch(c + 2);
        }
        if (live) {
#pragma unroll
            for (int s = 0; s < CH / 16; ++s) {
                bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    ah[i] = opnd(c & 1, 0, xi + 32 * i, s);
                    al[i] = opnd(c & 1, 1, xi + 32 * i, s);
                    bh[i] = opnd(c & 1, 2, xj + 32 * i, s);
                    bl[i] = opnd(c & 1, 3, xj + 32 * i, s);
                }
                // small terms first, then hi.hi; four independent accumulators apart
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) acc[i][j] = mfma(al[i], bh[j], acc[i][j]);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) acc[i][j] = mfma(ah[i], bl[j], acc[i][j]);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) acc[i][j] = mfma(ah[i], bh[j], acc[i][j]);
            }
        }
    }
    if (!live) return;

    // lane holds column J0 + 32 j + r and rows I0 + 32 i + 8 (v / 4) + 4 kh + v % 4
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int J = J0 + 32 * j + r;
        if (J >= a.nb) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int I = I0 + 32 * i + 8 * (v >> 2) + 4 * kh + (v & 3);
                if (I < a.nb && J <= I) out[(size_t)I * a.nb + J] = fmaf(acc[i][j][v], a.tau, lj[j]);
            }
    }
}

}  // namespace

hipError_t launch_pool(const Shape &s, const void *q, const KvView *kv, float *qbar, float *kbar,
                       float *lvn, hipStream_t st) {
    switch (s.dtype) {
        case STEM_F32: return pool_all<4>(s, q, kv, qbar, kbar, lvn, st);
        case STEM_BF16: return pool_all<2>(s, q, kv, qbar, kbar, lvn, st);
        default: return pool_all<1>(s, q, kv, qbar, kbar, lvn, st);
    }
}

hipError_t launch_score(const Shape &s, const float *qbar, const float *kbar, const float *lvn,
                        float *scores, hipStream_t st) {
    const int tiles = (s.nb + kTile - 1) / kTile;
    ScoreArgs a{qbar, kbar, lvn, scores, s.hq, s.hkv, s.nb, tiles, s.tau};
    const dim3 grid(tiles * (tiles + 1) / 2, s.hq, s.batch);
    if (s.d == 64) hipLaunchKernelGGL(score_kernel<64>, grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(score_kernel<128>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_cache_write(const Shape &s, const void *k_in, const void *v_in, const KvView &cache,
                              float *kbar, float *lvn, hipStream_t st) {
    CacheArgs a{};
    a.src[0] = static_cast<const char *>(k_in);
    a.src[1] = static_cast<const char *>(v_in);
    a.dst[0] = static_cast<char *>(const_cast<void *>(cache.k));
    a.dst[1] = static_cast<char *>(const_cast<void *>(cache.v));
    a.kbar = kbar;
    a.lvn = lvn;
    a.table = cache.table;
    a.page_log2 = cache.page_log2;
    a.pages_per_seq = cache.pages_per_seq;
    a.heads = s.hkv;
    a.d = s.d;
    a.blk = s.blk;
    a.seq = s.seq;
    a.nb = s.nb;
    a.scale[0] = s.k_scale;
    a.scale[1] = s.v_scale;
    const int es = s.dtype == STEM_F32 ? 4 : s.dtype == STEM_BF16 ? 2 : 1;
    a.chunks_per_row = s.hkv * s.d * es / 16;
    const dim3 grid((a.chunks_per_row + kPoolChunks - 1) / kPoolChunks, s.nb, 2 * s.batch);
    switch (s.dtype) {
        case STEM_F32: hipLaunchKernelGGL((cache_write_kernel<4, 4>), grid, dim3(kPoolThreads), 0, st, a); break;
        case STEM_BF16: hipLaunchKernelGGL((cache_write_kernel<2, 2>), grid, dim3(kPoolThreads), 0, st, a); break;
        default: hipLaunchKernelGGL((cache_write_kernel<2, 1>), grid, dim3(kPoolThreads), 0, st, a); break;
    }
    return hipGetLastError();
}

}  // namespace stem
