#pragma once
// Kernels of the causal block-sparse flash attention for prefill (Stem article on cn486.com,
// §二.2.2 "BSA operator optimisation": per Q tile the block mask is staged in
// on-chip memory and the list of KV blocks to compute is built before the
// loop; the inner loop visits only those blocks and is the dense loop; a
// skipped block is equivalent to -inf scores).  The dense causal kernel used
// as the baseline (§二.3) is the same template without any mask logic.
//
// Design for gfx950 (wave64, 32x32 MFMA, 160 KiB LDS):
//   * One workgroup per (batch, head, query block I) with 2 * BLK/32 waves:
//     each 32-row query group has two waves, each taking half of every key
//     block, so every SIMD runs two waves; their partial softmax states are
//     merged through LDS at the end.  Workgroups run heaviest-first (I
//     descending), and the heads that share a KV head are spread so that they
//     land on one XCD (workgroup ids go round-robin over the 8 XCDs), to reuse
//     K/V in its L2.
//   * S^T = K Q^T on MFMA (keys are the M dimension), so after the MFMA every
//     lane holds one query's scores: the row max needs one cross-lane swap
//     (lane ^ 32) and the running sum none until the end.
//   * O^T += V^T P^T: the probabilities stay in registers as the B operand.
//     The K rows are fed to the first MFMA in a permuted order chosen so that
//     the keys a lane holds afterwards are contiguous in V; V is read with the
//     transposing LDS loads (ds_read_b64_tr_b8 / tr_b16).  K and V sit in LDS
//     as [key][d] with 16-byte chunks swizzled by row.
//   * bf16: v_mfma_f32_32x32x16_bf16; fp32: v_mfma_f32_32x32x2f32; fp8 (OCP
//     E4M3): v_mfma_f32_32x32x64_f8f6f4 with P cast per query and block as
//     P * 2^e and the E8M0 operand scale undoing 2^e.
//   * Three kernels.  bsa_fp8_kernel (fp8, d = 128, 128-token blocks) and
//     bsa_bf16_kernel (bf16, same shape) are software pipelines that load K/V
//     straight into LDS; bsa_kernel (all other shapes) alternates MFMA and
//     softmax phases between the two waves of a SIMD, with register-staged
//     loads.  Each is described where it is defined.
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "stem_internal.h"

namespace stem {
namespace {

enum { kF32 = 0, kBF16 = 1, kFP8 = 2 };

struct BsaArgs {
    const char *q, *k, *v;
    const int32_t *table;
    int page_log2, pages_per_seq;
    const uint32_t *mask;
    void *o;
    float *lse;
    int batch, seq, hq, hkv, nb, words;
    float c_exp2;     // tau * q_scale * k_scale * log2(e): logits -> exp2 argument
    float tau_eff;    // tau * q_scale * k_scale
    float o_scale;    // v_scale, divided by the P scale for fp8
    float skip_log2;  // online skip: log2(lambda) (-inf: never)
    int32_t *skipped; // online skip: blocks dropped per query row, or null
};

template <int DT, int D, int BLK>
struct Geo {
    static constexpr int DTYPE = DT;
    static constexpr int ES = DT == kF32 ? 4 : DT == kBF16 ? 2 : 1;
    static constexpr int KROWB = D * ES;
    static constexpr int KCH = KROWB / 16;
    static constexpr int TILEB = BLK * D * ES;
    static constexpr int STAGES = (2 * 2 * TILEB <= 128 * 1024) ? 2 : 1;
    // Waves: NWQ groups of 32 query rows; each block's keys are split over
    // KSPLIT waves per group (partial softmax states merged after the loop),
    // which puts two waves on every SIMD.
    static constexpr int KGRAN = DT == kFP8 ? 64 : 32;  // keys of one PV MFMA step group
    static constexpr int KSPLIT = BLK / 2 >= KGRAN ? 2 : 1;
    static constexpr int NWQ = BLK / 32;
    static constexpr int NW = NWQ * KSPLIT;
    static constexpr int NT = NW * 64;
    static constexpr int KPW = BLK / KSPLIT;          // keys of a block per wave
    static constexpr int NTW = KPW / 32;              // 32-key tiles per wave
    static constexpr int NTILE = BLK / 32;
    static constexpr int NDT = D / 32;                // 32-wide d tiles of O
    static constexpr int NKC = BLK * KCH / NT;        // K 16-byte chunks per thread
    static constexpr int LIST = 4096;                 // max blocks per row
    static constexpr int COMB = KSPLIT == 2 ? NWQ * 64 * (D / 2) * 4 : 0;   // partial O bytes
    static constexpr int SMEM = STAGES * 2 * TILEB > COMB ? STAGES * 2 * TILEB : COMB;
    // Lazy rescaling: the running max only moves when a block's max exceeds it
    // by more than THRESH (log2 units), so P stays below 2^THRESH.
    static constexpr float THRESH = 8.0f;
    // FP8: normalise O by the MFMA-accumulated sum of the quantised P (an
    // all-ones row of V^T) instead of the exact fp32 sum.
    static constexpr bool QSUM = DT == kFP8;
    static_assert(BLK * KCH % NT == 0, "K chunks must divide over the threads");
};

// Key (within the block) that MFMA row r of 32-key tile t stands for.
template <int DT>
__device__ __forceinline__ int keymap(int t, int r) {
    const int i = r >> 3, gg = (r >> 2) & 1, j = r & 3;
    if constexpr (DT == kBF16) return 32 * t + 16 * (i >> 1) + 8 * gg + 4 * (i & 1) + j;
    else if constexpr (DT == kFP8) return 64 * (t >> 1) + 32 * gg + 16 * (t & 1) + 4 * i + j;
    else return 32 * t + r;
}

// Chunk swizzle of row `key`: chosen so that the 8 rows a group of 8 lanes
// feeds to the first MFMA (whose row order keymap() permutes) and the 4 or 8
// consecutive rows of a transposing read all land on distinct bank groups.
template <int DT, int KCH>
__device__ __forceinline__ int swz(int key) {
    if constexpr (DT == kFP8) return ((key ^ (key >> 3) ^ (key >> 5)) & 7) & (KCH - 1);
    else if constexpr (DT == kBF16) return ((key ^ ((key >> 3) << 2)) & 7) * (KCH / 8);
    else return (key & 7) * (KCH / 8);
}

template <class G>
__device__ __forceinline__ int k_off(int key, int chunk) {
    return key * G::KROWB + ((chunk ^ swz<G::DTYPE, G::KCH>(key)) << 4);
}

// One K or V block: BLK rows of D elements in LDS, row-major, 16-byte chunks
// XOR-swizzled by row.  Thread `tid` moves chunks tid, tid + NT, ...: a wave
// covers RPW consecutive rows per step, which never straddle a page (pages are
// at least 16 tokens), so the page lookup is wave-uniform (a scalar load).
template <class G>
using TileRegs = u32x4[G::NKC];

// Loop-invariant part of a thread's tile traffic: for each of its chunks the
// first row its wave covers (wave-uniform), the byte offset of the thread's
// chunk from that row, and the swizzled LDS offset of the chunk.
template <class G>
struct TileMap {
    int key0[G::NKC];
    int voff[G::NKC];
    int loff[G::NKC];
};

template <int DT, int D, int BLK>
__device__ __forceinline__ void tile_map(TileMap<Geo<DT, D, BLK>> &tm, const BsaArgs &a, int tid) {
    using G = Geo<DT, D, BLK>;
    const int row_bytes = a.hkv * (D * G::ES);
#pragma unroll
    for (int i = 0; i < G::NKC; ++i) {
        const int qid = tid + G::NT * i;
        const int key = qid / G::KCH, c = qid % G::KCH;
        tm.key0[i] = __builtin_amdgcn_readfirstlane(key);
        tm.voff[i] = (key - tm.key0[i]) * row_bytes + c * 16;
        tm.loff[i] = k_off<G>(key, c);
    }
}

// Scalar byte offsets (from the start of the K or V tensor; both have the same
// layout) of the rows each wave step of block J starts at.  Paged: one
// wave-uniform page lookup per step.
template <class G>
struct BlockOffs {
    int s[G::NKC];
};

template <int DT, int D, int BLK, bool PAGED>
__device__ __forceinline__ BlockOffs<Geo<DT, D, BLK>> block_offs(const BsaArgs &a, const TileMap<Geo<DT, D, BLK>> &tm,
                                                                 int b, int g, int J) {
    using G = Geo<DT, D, BLK>;
    BlockOffs<G> bo;
    const unsigned row_bytes = (unsigned)a.hkv * (D * G::ES);
    const unsigned head = (unsigned)g * (D * G::ES);
#pragma unroll
    for (int i = 0; i < G::NKC; ++i) {
        const int tok = J * BLK + tm.key0[i];
        unsigned row;
        if constexpr (PAGED) {
            const int page = a.table[b * a.pages_per_seq + (tok >> a.page_log2)];
            row = ((unsigned)page << a.page_log2) | (unsigned)(tok & ((1 << a.page_log2) - 1));
        } else {
            row = (unsigned)(b * a.seq + tok);
        }
        bo.s[i] = (int)(row * row_bytes + head);
    }
    return bo;
}

// Global -> registers: buffer loads with a constant descriptor for the whole
// tensor (smaller than 4 GiB, checked on the host), the scalar row offset of
// the wave step and the loop-invariant per-thread offset.
template <int DT, int D, int BLK>
__device__ __forceinline__ void load_tile(TileRegs<Geo<DT, D, BLK>> &st, __amdgpu_buffer_rsrc_t rsrc,
                                          const BlockOffs<Geo<DT, D, BLK>> &bo, const TileMap<Geo<DT, D, BLK>> &tm) {
    using G = Geo<DT, D, BLK>;
#pragma unroll
    for (int i = 0; i < G::NKC; ++i)
        st[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, tm.voff[i], bo.s[i], 0));
}

template <int DT, int D, int BLK>
__device__ __forceinline__ void store_tile(const TileRegs<Geo<DT, D, BLK>> &st, char *tl,
                                           const TileMap<Geo<DT, D, BLK>> &tm) {
    using G = Geo<DT, D, BLK>;
#pragma unroll
    for (int i = 0; i < G::NKC; ++i) *reinterpret_cast<u32x4 *>(tl + tm.loff[i]) = st[i];
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

// Transposing LDS reads (gfx950).  Within each 16-lane group, source lane s
// points at a row; ds_read_b64_tr_b8 returns to lane i byte (i % 8) of the
// rows of source lanes i/8, i/8 + 2, ..., i/8 + 14, and ds_read_b64_tr_b16
// returns halfword (i % 4) of the rows of source lanes i/4, i/4 + 4, ..., i/4 + 12.
__device__ __forceinline__ i32x2 lds_tr8(const char *p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2 *)(lds_char *)p);
}
__device__ __forceinline__ i16x4 lds_tr16(const char *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(lds_char *)p);
}

// Q operand of S^T = K Q^T for this lane's query row.
template <int DT, int D>
struct QFrag {
    static constexpr int N = DT == kF32 ? D / 2 : DT == kBF16 ? D / 16 : D / 32;
    u32x4 u[DT == kF32 ? 1 : N];
    float f[DT == kF32 ? N : 1];
};

template <int DT, int D>
__device__ __forceinline__ void load_q(QFrag<DT, D> &qf, const char *qrow, int g) {
    if constexpr (DT == kF32) {
        const float *p = reinterpret_cast<const float *>(qrow);
#pragma unroll
        for (int s = 0; s < D / 2; ++s) qf.f[s] = p[2 * s + g];
    } else if constexpr (DT == kBF16) {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) qf.u[s] = *reinterpret_cast<const u32x4 *>(qrow + (16 * s + 8 * g) * 2);
    } else {
#pragma unroll
        for (int s = 0; s < D / 64; ++s) {
            qf.u[2 * s] = *reinterpret_cast<const u32x4 *>(qrow + 64 * s + 32 * g);
            qf.u[2 * s + 1] = *reinterpret_cast<const u32x4 *>(qrow + 64 * s + 32 * g + 16);
        }
    }
}

// S^T tile (32 keys of global tile tg x this lane's query) = K Q^T.
template <int DT, int D, int BLK>
__device__ __forceinline__ f32x16 qk_tile(const QFrag<DT, D> &qf, const char *kl, int tg, int lane) {
    using G = Geo<DT, D, BLK>;
    const int r = lane & 31, g = lane >> 5;
    const int key = keymap<DT>(tg, r);
    f32x16 acc = {};
    if constexpr (DT == kBF16) {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(kl + k_off<G>(key, 2 * s + g));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, qf.u[s]), acc, 0, 0, 0);
        }
    } else if constexpr (DT == kFP8) {
#pragma unroll
        for (int s = 0; s < D / 64; ++s) {
            const u32x4 a0 = *reinterpret_cast<const u32x4 *>(kl + k_off<G>(key, 4 * s + 2 * g));
            const u32x4 a1 = *reinterpret_cast<const u32x4 *>(kl + k_off<G>(key, 4 * s + 2 * g + 1));
            i32x8 av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            const u32x4 b0 = qf.u[2 * s], b1 = qf.u[2 * s + 1];
            i32x8 bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int s = 0; s < D / 2; ++s) {
            const int dd = 2 * s + g;
            const float a = *reinterpret_cast<const float *>(kl + k_off<G>(key, dd >> 2) + (dd & 3) * 4);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf.f[s], acc, 0, 0, 0);
        }
    }
    return acc;
}

// O^T[dt] += V^T P^T over this wave's keys of the block (tiles t0 .. t0+NTW-1).
// P of this wave's keys of one block, packed as the B operand of the PV MFMAs.
template <int DT, int D, int BLK>
struct PPack {
    static constexpr int NTW = Geo<DT, D, BLK>::NTW;
    i32x8 f8[DT == kFP8 ? NTW / 2 : 1];       // 64 keys per FP8 MFMA step
    bf16x8 b16[DT == kBF16 ? 2 * NTW : 1];    // 16 keys per BF16 MFMA step
    f32x16 f32[DT == kF32 ? NTW : 1];         // one key pair per FP32 MFMA step
};

template <int DT, int D, int BLK>
__device__ __forceinline__ void pack_p(PPack<DT, D, BLK> &pk, const f32x16 (&p)[Geo<DT, D, BLK>::NTW]) {
    using G = Geo<DT, D, BLK>;
    if constexpr (DT == kBF16) {
#pragma unroll
        for (int t = 0; t < G::NTW; ++t)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 8; ++e) pk.b16[2 * t + hh][e] = (__bf16)p[t][8 * hh + e];
    } else if constexpr (DT == kFP8) {
#pragma unroll
        for (int t = 0; t < G::NTW; t += 2)
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const int e = 4 * w;
                const f32x16 &src = p[t + (e >> 4)];
                const int ee = e & 15;
                // the high half is written next: its old contents do not matter
                int x = __builtin_amdgcn_cvt_pk_fp8_f32(src[ee], src[ee + 1], __builtin_nondeterministic_value(0), false);
                pk.f8[t >> 1][w] = __builtin_amdgcn_cvt_pk_fp8_f32(src[ee + 2], src[ee + 3], x, true);
            }
    } else {
#pragma unroll
        for (int t = 0; t < G::NTW; ++t) pk.f32[t] = p[t];
    }
}

// FP8: the residual P - E4M3(P) of every packed P, itself rounded to E4M3 (the
// difference is exact in fp32: P and its E4M3 value lie within a factor of
// two).  PV with both terms carries about seven significant bits of P.
template <int DT, int D, int BLK>
__device__ __forceinline__ void pack_residual(PPack<DT, D, BLK> &lo, const PPack<DT, D, BLK> &hi,
                                              const f32x16 (&p)[Geo<DT, D, BLK>::NTW]) {
    using G = Geo<DT, D, BLK>;
    static_assert(DT == kFP8, "FP8 only");
#pragma unroll
    for (int t = 0; t < G::NTW; t += 2)
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int e = 4 * w;
            const f32x16 &src = p[t + (e >> 4)];
            const int ee = e & 15;
            const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi.f8[t >> 1][w], false);
            const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi.f8[t >> 1][w], true);
            const int x = __builtin_amdgcn_cvt_pk_fp8_f32(src[ee] - h01[0], src[ee + 1] - h01[1], 0, false);
            lo.f8[t >> 1][w] = __builtin_amdgcn_cvt_pk_fp8_f32(src[ee + 2] - h23[0], src[ee + 3] - h23[1], x, true);
        }
}

// O^T[dt] += V^T P^T over this wave's keys of the block (tiles t0 .. t0+NTW-1).
// For FP8 the softmax denominator is accumulated by the MFMA as well (an
// all-ones row of V^T), so that it sums exactly the quantised P that
// multiplied V: every lane's lacc[] then holds its query's sum.
template <int DT, int D, int BLK>
__device__ __forceinline__ void pv_block(f32x16 (&o)[D / 32], f32x16 &lacc, const PPack<DT, D, BLK> &pk,
                                         const char *vl, int t0, int lane, int pscale) {
    using G = Geo<DT, D, BLK>;
    const int r = lane & 31, g = lane >> 5;
    const int i16 = lane & 15;                            // lane within its 16-lane group
    const int dhalf = 16 * ((lane >> 4) & 1);             // d offset of the group within a 32-d tile
    if constexpr (DT == kBF16) {
#pragma unroll
        for (int t = 0; t < G::NTW; ++t) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int kb = 32 * (t0 + t) + 16 * hh + 8 * g;
#pragma unroll
                for (int dt = 0; dt < G::NDT; ++dt) {
                    // V^T operand: 8 consecutive keys at d = 32 dt + (lane & 31), two transposing reads
                    const int d0 = 32 * dt + dhalf;
                    const int r0 = kb + (i16 >> 2), r1 = kb + 4 + (i16 >> 2);
                    const int ch = d0 / 8 + ((i16 & 3) >> 1), off = 8 * (i16 & 1);
                    const i16x4 v0 = lds_tr16(vl + k_off<G>(r0, ch) + off);
                    const i16x4 v1 = lds_tr16(vl + k_off<G>(r1, ch) + off);
                    typedef short i16x8 __attribute__((ext_vector_type(8)));
                    const i16x8 av = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pk.b16[2 * t + hh],
                                                                    o[dt], 0, 0, 0);
                }
            }
        }
    } else if constexpr (DT == kFP8) {
#pragma unroll
        for (int t = 0; t < G::NTW; t += 2) {
            const int pp = (t0 + t) >> 1;
            const int kb = 64 * pp + 32 * g;
#pragma unroll
            for (int dt = 0; dt < G::NDT; ++dt) {
                // V^T operand: 32 consecutive keys at d = 32 dt + (lane & 31), four transposing reads
                const int d0 = 32 * dt + dhalf;
                const int ch = d0 / 16, off = 8 * (i16 & 1);
                i32x8 av;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const i32x2 x = lds_tr8(vl + k_off<G>(kb + 8 * q + (i16 >> 1), ch) + off);
                    av[2 * q] = x[0];
                    av[2 * q + 1] = x[1];
                }
                o[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pk.f8[t >> 1], o[dt], 0, 0, 0, 127, 0, pscale);
            }
            if constexpr (G::QSUM) {
                const int one = 0x38383838;               // four E4M3 1.0
                const i32x8 ones = {one, one, one, one, one, one, one, one};
                lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pk.f8[t >> 1], lacc, 0, 0, 0, 127, 0, pscale);
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < G::NTW; ++t) {
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) {
                const int key = keymap<DT>(t0 + t, 8 * (vv >> 2) + 4 * g + (vv & 3));
#pragma unroll
                for (int dt = 0; dt < G::NDT; ++dt) {
                    const int d = 32 * dt + r;
                    const float a = *reinterpret_cast<const float *>(vl + k_off<G>(key, d >> 2) + (d & 3) * 4);
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, pk.f32[t][vv], o[dt], 0, 0, 0);
                }
            }
        }
    }
}

// FP8 MFMA phase in one piece: S = K(j) Q^T for this wave's two 32-key tiles
// and O += V(j-1)^T P(j-1).  It runs unconditionally (at the edges of the loop
// the extra products are discarded or add zeros), so it is one scheduling
// region, and its order is pinned: LDS operands are fetched ahead of the MFMAs
// that consume them, so the matrix core does not wait on LDS round trips.
template <int D, int BLK>
__device__ __forceinline__ void mfma_phase_fp8(f32x16 (&s)[2], f32x16 (&o)[D / 32], f32x16 &lacc,
                                               const QFrag<kFP8, D> &qf,
                                               const PPack<kFP8, D, BLK> &pk, int pscale, const char *kl,
                                               const char *vl, int t0, int lane) {
    using G = Geo<kFP8, D, BLK>;
    static_assert(G::NTW == 2 && D == 128, "one 64-key PV step per wave, four 32-d tiles");
    const int r = lane & 31, g = lane >> 5;
    const int i16 = lane & 15, dhalf = 16 * ((lane >> 4) & 1);
    auto kop = [&](int t, int st) {
        const int key = keymap<kFP8>(t0 + t, r);
        const u32x4 a0 = *reinterpret_cast<const u32x4 *>(kl + k_off<G>(key, 4 * st + 2 * g));
        const u32x4 a1 = *reinterpret_cast<const u32x4 *>(kl + k_off<G>(key, 4 * st + 2 * g + 1));
        return i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    };
    auto qop = [&](int st) {
        const u32x4 b0 = qf.u[2 * st], b1 = qf.u[2 * st + 1];
        return i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    };
    const int kb = 64 * (t0 >> 1) + 32 * g;
    auto vop = [&](int dt) {
        const int ch = (32 * dt + dhalf) / 16, off = 8 * (i16 & 1);
        i32x8 av;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const i32x2 x = lds_tr8(vl + k_off<G>(kb + 8 * q + (i16 >> 1), ch) + off);
            av[2 * q] = x[0];
            av[2 * q + 1] = x[1];
        }
        return av;
    };
    const i32x8 k00 = kop(0, 0), k01 = kop(0, 1), k10 = kop(1, 0), k11 = kop(1, 1);
    const i32x8 v0 = vop(0);
    f32x16 a0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k00, qop(0), f32x16{}, 0, 0, 0, 0, 0, 0);
    s[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k01, qop(1), a0, 0, 0, 0, 0, 0, 0);
    const i32x8 v1 = vop(1);
    f32x16 a1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k10, qop(0), f32x16{}, 0, 0, 0, 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k11, qop(1), a1, 0, 0, 0, 0, 0, 0);
    const i32x8 v2 = vop(2);
    o[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v0, pk.f8[0], o[0], 0, 0, 0, 127, 0, pscale);
    const i32x8 v3 = vop(3);
    o[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v1, pk.f8[0], o[1], 0, 0, 0, 127, 0, pscale);
    o[2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v2, pk.f8[0], o[2], 0, 0, 0, 127, 0, pscale);
    o[3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v3, pk.f8[0], o[3], 0, 0, 0, 127, 0, pscale);
    const int one = 0x38383838;                            // four E4M3 1.0: the sum of the quantised P
    const i32x8 ones = {one, one, one, one, one, one, one, one};
    lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pk.f8[0], lacc, 0, 0, 0, 127, 0, pscale);
    // issue order: 8 K reads + 4 V reads, 2 MFMA, 4 V reads, 2 MFMA, 4 V reads, 1 MFMA, 4 V reads, 4 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// Kept blocks J <= I of row (b, h, I), in ascending order, into list[];
// returns their count.  Every thread of the workgroup calls it (two barriers).
template <int NW, bool SPARSE>
__device__ __forceinline__ int build_block_list(const BsaArgs &a, int b, int h, int I, uint16_t *list,
                                                int *wave_sum, int tid, int lane, int wave) {
    if constexpr (!SPARSE) {
        return I + 1;
    } else {
        const int nw = (I >> 5) + 1;                          // words holding J <= I
        uint32_t w = 0;
        if (tid < nw) {
            w = a.mask[(((size_t)b * a.hq + h) * a.nb + I) * a.words + tid];
            if (tid == nw - 1 && (I & 31) != 31) w &= (2u << (I & 31)) - 1u;
        }
        const int cnt = __popc(w);
        int incl = cnt;                                       // inclusive scan in the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
        if (lane == 63) wave_sum[wave] = incl;
        __syncthreads();
        int base = 0, n = 0;
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            base += k < wave ? wave_sum[k] : 0;
            n += wave_sum[k];
        }
        int pos = base + incl - cnt;
        while (w) {
            const int bit = __builtin_ctz(w);
            list[pos++] = (uint16_t)(32 * tid + bit);
            w &= w - 1;
        }
        __syncthreads();
        return n;
    }
}

// Output of a query row that sees no key: O = 0, LSE = -inf.  Lanes l and
// l ^ 32 of the calling wave share the row and write alternate elements.
template <int DT, int D>
__device__ __forceinline__ void write_empty_row(const BsaArgs &a, int b, int h, int token, int g32) {
    if constexpr (DT == kF32) {
        float *op = reinterpret_cast<float *>(a.o) + (((size_t)b * a.seq + token) * a.hq + h) * D;
        for (int d = g32; d < D; d += 2) op[d] = 0.0f;
    } else {
        uint16_t *op = reinterpret_cast<uint16_t *>(a.o) + (((size_t)b * a.seq + token) * a.hq + h) * D;
        for (int d = g32; d < D; d += 2) op[d] = 0;
    }
    if (a.lse && g32 == 0) a.lse[((size_t)b * a.hq + h) * a.seq + token] = -__builtin_huge_valf();
}

template <int DT, int D, int BLK, bool SPARSE, bool PAGED>
__global__ __launch_bounds__((Geo<DT, D, BLK>::NT), 1) void bsa_kernel(BsaArgs a) {
    using G = Geo<DT, D, BLK>;
    __shared__ __attribute__((aligned(16))) char smem[G::SMEM];
    __shared__ uint16_t list[SPARSE ? G::LIST : 1];
    __shared__ int wave_sum[G::NW];
    __shared__ float part_ml[G::KSPLIT == 2 ? 3 * G::NWQ * 64 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g32 = lane >> 5;
    const int wq = wave % G::NWQ;                          // query group of this wave
    const int ks = wave / G::NWQ;                          // key part of this wave
    const int t0 = ks * G::NTW;                            // its first 32-key tile

    // heaviest query blocks first; the heads of one KV group on one XCD
    const int wg = blockIdx.x;
    const int qidx = wg / a.hq, j = wg % a.hq;
    const int I = a.nb - 1 - qidx / a.batch;
    const int b = qidx % a.batch;
    const int h = (a.hq % 8 == 0) ? (j % 8) * (a.hq / 8) + j / 8 : j;
    const int g = h / (a.hq / a.hkv);

    const int n = build_block_list<G::NW, SPARSE>(a, b, h, I, list, wave_sum, tid, lane, wave);

    const int qrow = 32 * wq + (lane & 31);               // query row in the block
    const int token = I * BLK + qrow;
    if (n == 0) {                                         // nothing visible: O = 0, LSE = -inf
        if (ks == 0) write_empty_row<DT, D>(a, b, h, token, g32);
        return;
    }

    QFrag<DT, D> qf;
    load_q<DT, D>(qf, a.q + (((size_t)b * a.seq + token) * a.hq + h) * (size_t)(D * G::ES), g32);

    f32x16 o[G::NDT];
#pragma unroll
    for (int dt = 0; dt < G::NDT; ++dt) o[dt] = f32x16{};
    const float ninf = -__builtin_huge_valf();
    float m = ninf;                                       // running max (raw logit units)
    float l = 0.0f;                                       // this lane's partial sum of P
    f32x16 lacc = {};                                     // FP8: the sum of P from the MFMA
    const float c = a.c_exp2;

    // Ping-pong schedule.  Every block takes two barrier-separated phases per
    // wave: an MFMA phase (S = K(j) Q^T and O += V(j-1)^T P(j-1)) and a VALU
    // phase (softmax of block j).  The two waves of a query group share a SIMD
    // and run one phase apart, so one wave's MFMAs overlap the other's
    // softmax.  K stages hold K(j), K(j+1); V stages V(j-1), V(j).  Global
    // loads are two phases ahead of their LDS store.
    TileMap<G> tm;
    tile_map<DT, D, BLK>(tm, a, tid);
    u32x4 kst[G::NKC];
    u32x4 vst[G::NKC];
    auto list_at = [&](int i) { return SPARSE ? __builtin_amdgcn_readfirstlane((int)list[i]) : i; };
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)a.k, 0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)a.v, 0, -1, 0x00020000);
    constexpr int KBASE = 0, VBASE = G::STAGES * G::TILEB;
    const int lag = G::STAGES == 2 ? ks : 0;
    const bool diag_last = list_at(n - 1) == I;            // the diagonal block, if kept, is the last
    BlockOffs<G> off_v;                                    // offsets of the next V block to fetch
    {
        const BlockOffs<G> off0 = block_offs<DT, D, BLK, PAGED>(a, tm, b, g, list_at(0));
        load_tile<DT, D, BLK>(kst, krs, off0, tm);
        store_tile<DT, D, BLK>(kst, smem + KBASE, tm);
        const BlockOffs<G> off1 = n > 1 ? block_offs<DT, D, BLK, PAGED>(a, tm, b, g, list_at(1)) : off0;
        load_tile<DT, D, BLK>(kst, krs, off1, tm);
        load_tile<DT, D, BLK>(vst, vrs, off0, tm);
        off_v = off1;
    }
    if constexpr (DT == kFP8) {
        // the first MFMA phase multiplies this V stage by P = 0: it must hold no NaN
        u32x4 *vz = reinterpret_cast<u32x4 *>(smem + VBASE + (G::STAGES == 2 ? 1 : 0) * G::TILEB);
        for (int i = tid; i < G::TILEB / 16; i += G::NT) vz[i] = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();

    f32x16 s[G::NTW];                                     // scores of the block awaiting softmax
    PPack<DT, D, BLK> pk = {};                            // P of the block awaiting PV (zero before the first)
    int pscale = 127;                                     // its E8M0 scale (FP8)
    // FP8: the row's first kept block (the forced sink block of a Stem mask,
    // where attention mass concentrates) also multiplies V by the residual of
    // its P, so that its P carries about seven significant bits.
    PPack<DT, D, BLK> plo = {};
    const int nph = 2 * n + 2;

    auto phase = [&](auto R, int p) {
        constexpr int r = decltype(R)::value;
        constexpr int ST = G::STAGES == 2 ? (r >> 1) : 0;     // K stage of this phase's MFMA work
        // odd phases fetch K(jj+2): look its rows up first, so the list read and
        // the page-table loads overlap this phase's work
        const int jj = (p - 1) >> 1;
        BlockOffs<G> off_k;
        if constexpr ((r & 1) != 0) {
            const int last = n - 1;
            off_k = block_offs<DT, D, BLK, PAGED>(a, tm, b, g, list_at(jj + 2 < last ? jj + 2 : last));
        }
        const int q = p - lag;
        if (q >= 0) {
            const int j = q >> 1;
            if ((q & 1) == 0) {
                // ---- MFMA phase: S = K(j) Q^T, O += V(j-1)^T P(j-1)
                const char *kl = smem + KBASE + ST * G::TILEB;
                const char *vl = smem + VBASE + (G::STAGES == 2 ? 1 - ST : 0) * G::TILEB;
                if constexpr (DT == kFP8 && G::NTW == 2 && D == 128) {
                    // unconditional: at j == n the scores are never used; at j == 0 P and
                    // the V stage read are zero (cleared before the loop)
                    mfma_phase_fp8<D, BLK>(s, o, lacc, qf, pk, pscale, kl, vl, t0, lane);
                } else {
                    if (j < n) {
#pragma unroll
                        for (int t = 0; t < G::NTW; ++t) s[t] = qk_tile<DT, D, BLK>(qf, kl, t0 + t, lane);
                    }
                    if (j >= 1) pv_block<DT, D, BLK>(o, lacc, pk, vl, t0, lane, pscale);
                }
                if constexpr (DT == kFP8) {
                    if (j == 1) pv_block<DT, D, BLK>(o, lacc, plo, vl, t0, lane, pscale);   // residual of P(0)
                }
            } else if (j < n) {
                // ---- VALU phase: online softmax of block j
                if (diag_last && j == n - 1) {            // causal mask inside the diagonal block
#pragma unroll
                    for (int t = 0; t < G::NTW; ++t)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int key = keymap<DT>(t0 + t, 8 * (e >> 2) + 4 * g32 + (e & 3));
                            if (key > qrow) s[t][e] = ninf;
                        }
                }
                // (NaN never arises: -inf - -inf is kept out of every expression below)
                // block max of this lane's scores as a balanced tree, then across lane ^ 32
                float mt[G::NTW * 4];
#pragma unroll
                for (int t = 0; t < G::NTW; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        mt[4 * t + e] = fmaxf(fmaxf(s[t][4 * e], s[t][4 * e + 1]), fmaxf(s[t][4 * e + 2], s[t][4 * e + 3]));
#pragma unroll
                for (int w = G::NTW * 4; w > 1; w >>= 1)
#pragma unroll
                    for (int e = 0; e < w / 2; ++e) mt[e] = fmaxf(mt[e], mt[e + w / 2]);
                const float mx = max_xor32(mt[0]);
                // lazy rescale: only when some row's max grew by more than THRESH
                const bool grow = m == ninf ? mx != ninf : (mx - m) * c > G::THRESH;
                if (__ballot(grow)) {
                    const float m_new = fmaxf(m, mx);
                    const float alpha =
                        m == ninf ? (m_new == ninf ? 1.0f : 0.0f) : __builtin_amdgcn_exp2f((m - m_new) * c);
                    m = m_new;
                    l *= alpha;
                    if constexpr (DT == kFP8 && G::QSUM) {
#pragma unroll
                        for (int e = 0; e < 16; ++e) lacc[e] *= alpha;
                    }
#pragma unroll
                    for (int dt = 0; dt < G::NDT; ++dt)
#pragma unroll
                        for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
                }
                // FP8: P of this block is cast as P * 2^e with e chosen per query so
                // that the block's largest P lands in (128, 256]; the MFMA multiplies
                // by the E8M0 scale 2^-e, so every block uses the full E4M3 range.
                int e = 0;
                if constexpr (DT == kFP8) {
                    const float x = (mx == ninf || m == ninf) ? -1000.0f : (mx - m) * c;   // log2 of the largest P
                    e = 8 - (int)ceilf(fmaxf(x, -92.0f));   // e in [0, 100]
                }
                const float mc = m == ninf ? 0.0f : m * c - (float)e;
                float ls4[4] = {0.0f, 0.0f, 0.0f, 0.0f};    // four partial sums: short add chains
#pragma unroll
                for (int t = 0; t < G::NTW; ++t)
#pragma unroll
                    for (int e2 = 0; e2 < 16; ++e2) {
                        const float pe = __builtin_amdgcn_exp2f(fmaf(s[t][e2], c, -mc));
                        s[t][e2] = pe;
                        ls4[e2 & 3] += pe;
                    }
                const float ls = (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);
                l += DT == kFP8 ? ldexpf(ls, -e) : ls;
                pack_p<DT, D, BLK>(pk, s);
                if constexpr (DT == kFP8) {
                    if (j == 0) pack_residual<DT, D, BLK>(plo, pk, s);
                }
                pscale = 127 - e;
            }
        }
        if constexpr ((r & 1) != 0) {
            // ---- store K(jj+1) and V(jj), then fetch K(jj+2) and V(jj+1)
            constexpr int KS = G::STAGES == 2 ? ((r >> 1) ^ 1) : 0;
            constexpr int VS = G::STAGES == 2 ? (r >> 1) : 0;
            if (jj + 1 < n) store_tile<DT, D, BLK>(kst, smem + KBASE + KS * G::TILEB, tm);
            if (jj < n) store_tile<DT, D, BLK>(vst, smem + VBASE + VS * G::TILEB, tm);
            load_tile<DT, D, BLK>(kst, krs, off_k, tm);
            load_tile<DT, D, BLK>(vst, vrs, off_v, tm);
            off_v = off_k;                                    // V(jj+2) is K(jj+2)'s block
        }
        __syncthreads();
    };
    for (int p0 = 0; p0 < nph; p0 += 4) {
        phase(std::integral_constant<int, 0>{}, p0);
        if (p0 + 1 < nph) phase(std::integral_constant<int, 1>{}, p0 + 1);
        if (p0 + 2 < nph) phase(std::integral_constant<int, 2>{}, p0 + 2);
        if (p0 + 3 < nph) phase(std::integral_constant<int, 3>{}, p0 + 3);
    }

    // ---- merge the key parts, normalise, store --------------------------------
    l = sum_xor32(l);                                      // exact sum of P: the LSE
    float lq = DT == kFP8 && G::QSUM ? lacc[0] : l;        // the sum O is normalised by
    if constexpr (G::KSPLIT == 2) {
        __syncthreads();                                  // stages are free: reuse for partial O
        float *po = reinterpret_cast<float *>(smem) + wq * 64 * (D / 2);
        if (ks == 1) {
#pragma unroll
            for (int dt = 0; dt < G::NDT; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) po[(dt * 16 + e) * 64 + lane] = o[dt][e];
            part_ml[(3 * wq) * 64 + lane] = m;
            part_ml[(3 * wq + 1) * 64 + lane] = l;
            part_ml[(3 * wq + 2) * 64 + lane] = lq;
        }
        __syncthreads();
        if (ks == 1) return;
        const float m1 = part_ml[(3 * wq) * 64 + lane];
        const float l1 = part_ml[(3 * wq + 1) * 64 + lane];
        const float lq1 = part_ml[(3 * wq + 2) * 64 + lane];
        const float mm = fmaxf(m, m1);
        const float a0 = m == ninf ? 0.0f : __builtin_amdgcn_exp2f((m - mm) * c);
        const float a1 = m1 == ninf ? 0.0f : __builtin_amdgcn_exp2f((m1 - mm) * c);
#pragma unroll
        for (int dt = 0; dt < G::NDT; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[dt][e] = o[dt][e] * a0 + po[(dt * 16 + e) * 64 + lane] * a1;
        l = l * a0 + l1 * a1;
        lq = lq * a0 + lq1 * a1;
        m = mm;
    }
    const float inv = lq > 0.0f ? a.o_scale / lq : 0.0f;
    const size_t obase = (((size_t)b * a.seq + token) * a.hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < G::NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 32 * dt + 8 * i + 4 * g32;
            const float x0 = o[dt][4 * i] * inv, x1 = o[dt][4 * i + 1] * inv;
            const float x2 = o[dt][4 * i + 2] * inv, x3 = o[dt][4 * i + 3] * inv;
            if constexpr (DT == kF32) {
                *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.o) + obase + d0) = f32x4{x0, x1, x2, x3};
            } else {
                u32x2 u;
                u.x = f32_to_bf16_bits(x0) | (f32_to_bf16_bits(x1) << 16);
                u.y = f32_to_bf16_bits(x2) | (f32_to_bf16_bits(x3) << 16);
                *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(a.o) + obase + d0) = u;
            }
        }
    if (a.lse && g32 == 0)
        a.lse[((size_t)b * a.hq + h) * a.seq + token] =
            l > 0.0f ? fmaf(m, a.tau_eff, logf(l)) : ninf;
}

// ---------------------------------------------------------------------------
// FP8, d = 128, 128-token blocks: a software-pipelined kernel.
//
// One wave issues a VALU instruction only every few cycles, while the two
// waves of a SIMD together reach about twice that rate, and a wave keeps
// issuing independent VALU work while its own MFMAs run.  So all eight waves
// run one pipeline: while a wave computes the softmax of block j it also
// issues the MFMAs of S = K(j+1) Q^T (under the row max) and of
// O += V(j-1)^T P(j-1) (under the exponentials).  K and V move from global
// memory straight into LDS (buffer loads that write LDS, no staging
// registers), three blocks ahead of use, through four LDS stages each, with
// one barrier per block.  Both waves of a SIMD are in the softmax at the same
// time, so its VALU issues at the two-wave rate while the MFMAs of both fill
// the matrix core.
//
// When the running max moves, O and the MFMA row sums are rescaled at the
// start of the next block, after the PV MFMA of the old scale has been added,
// so that the rescale needs no branch inside the scheduling region.
namespace fp8p {
constexpr int D = 128, BLK = 128, NT = 512, NW = 8;
constexpr int NST = 4;                           // LDS stages of K and of V
constexpr int TILE = BLK * D;                    // bytes of one K or V block
constexpr int KST = 0, VST = NST * TILE;         // K stages, then V stages
constexpr int LIST_OFF = 2 * NST * TILE;         // kept-block list (u16) after the stages
constexpr int LIST = 4096 + 8;                   // up to 4096 kept blocks, plus 8 pad entries
constexpr int WSUM_OFF = LIST_OFF + 2 * LIST;    // per-wave counts of the list scan
constexpr int ML_OFF = WSUM_OFF + 4 * NW;        // (M, l, lq) of every wave, for the key-half merge
constexpr int HM_OFF = ML_OFF + 3 * NW * 64 * 4; // online skip: half-block maxima, [parity][wave][lane]
constexpr int SMEM = HM_OFF;
constexpr int SMEM_SKIP = HM_OFF + 2 * NW * 64 * 4;
static_assert(SMEM_SKIP <= 160 * 1024, "LDS of one CU");
constexpr int VM_ITER = 4;                       // loads into LDS per wave and iteration
constexpr float THRESH = 8.0f;                   // lazy rescale: P stays below 2^THRESH
constexpr float M_NONE = -3.0e38f;               // running max before any finite score

// 16-byte chunk swizzles of a K and a V row (key = row within the block).
// K: the 8 rows of equal parity that a 16-lane group reads for S = K Q^T
// ({0..7, 32..39} plus a multiple of 16) get 8 distinct chunks, and key + 16
// keeps the pattern, so the second key tile is an immediate offset.  V: the 4
// rows of equal parity under one transposing read get distinct chunk pairs,
// and key + 8 keeps the pattern.
__device__ __forceinline__ int swz_k(int key) { return ((key >> 1) & 3) | (((key >> 5) & 1) << 2); }
__device__ __forceinline__ int swz_v(int key) { return ((key >> 1) & 3) << 1; }

// s_waitcnt vmcnt(VM) (and lgkmcnt(0) if LGKM), then the workgroup barrier.
// The barrier itself waits for nothing, so the last VM loads into LDS stay in
// flight across it.
template <int VM, bool LGKM = false>
__device__ __forceinline__ void sync_vm() {
    static_assert(VM < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | ((LGKM ? 0 : 15) << 8) | ((VM >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
typedef __attribute__((address_space(4))) const int32_t const_i32;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor of a whole tensor (smaller than 4 GiB: checked on the host).
__device__ __forceinline__ i32x4 buffer_rsrc(const void *p) {
    const unsigned long long a = (unsigned long long)p;
    return i32x4{(int)(unsigned)a, (int)((unsigned)(a >> 32) & 0xffffu), -1, 0x00020000};
}

// 16 bytes per lane from global memory (descriptor + soff + voff) straight
// into LDS at byte lds + OFF + 16 * lane.  Written as asm so that the compiler,
// which would otherwise make every later transposing LDS read wait for all such
// loads, leaves the pacing to the explicit vmcnt waits.  The asm has no
// outputs; m0 is used by nothing else in these kernels.  s_add_u32 writes
// the scalar condition code (its carry), so SCC is declared clobbered: a
// comparison the compiler placed before the asm must not be branched on after it.
template <int OFF>
__device__ __forceinline__ void load_lds16(i32x4 rsrc, unsigned lds, unsigned voff, unsigned soff) {
    asm volatile("s_add_u32 m0, %0, %4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc),
                    "s"(__builtin_amdgcn_readfirstlane(soff)), "i"(OFF) : "memory", "m0", "scc");
}
}  // namespace fp8p

// Thread tid's 32-bit word of the mask row of attention row wg (rows numbered
// as in the pipelined kernels): words 0 .. I/32 hold the blocks J <= I; the
// other threads get 0.  Issued a row ahead by the persistent kernels.
__device__ __forceinline__ uint32_t mask_word(const BsaArgs &a, int wg, int tid) {
    const int qidx = wg / a.hq, jh = wg % a.hq;
    const int I = a.nb - 1 - qidx / a.batch, b = qidx % a.batch;
    const int h = (a.hq % 8 == 0) ? (jh % 8) * (a.hq / 8) + jh / 8 : jh;
    return tid <= (I >> 5) ? a.mask[(((size_t)b * a.hq + h) * a.nb + I) * a.words + tid] : 0u;
}

// The kept-block list of row I from its mask words (thread tid holds word
// tid, as mask_word gives it), in increasing J, into LDS; returns its length.
// The words and their list offsets pass through wbuf (2 x 128 u32 of LDS);
// then every thread places the kept blocks among 32 J at a time, so a dense
// word costs one pass, not 32.  Up to 4096 blocks (128 words, two waves).
template <int NW>
__device__ __forceinline__ int build_list_words(int I, uint32_t w, uint16_t *list, uint32_t *wbuf, int *wave_sum,
                                                int tid, int lane, int wave) {
    const int nw = (I >> 5) + 1;                          // words holding J <= I
    if (tid == nw - 1 && (I & 31) != 31) w &= (2u << (I & 31)) - 1u;
    const int cnt = __popc(w);
    int incl = cnt;                                       // inclusive scan in the wave
    if (wave < 2) {                                       // words live in waves 0 and 1 only
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
    }
    if (lane == 63) wave_sum[wave] = incl;
    if (tid < nw) {
        wbuf[tid] = w;
        wbuf[128 + tid] = (uint32_t)(incl - cnt);         // offset within its wave
    }
    __syncthreads();
    const int off1 = wave_sum[0];                         // kept blocks of words 0..63
    const int n = off1 + wave_sum[1];
    for (int k = tid; k < 32 * nw; k += NW * 64) {
        const int x = k >> 5, bit = k & 31;
        const uint32_t ww = wbuf[x];
        if ((ww >> bit) & 1u)
            list[(x >= 64 ? off1 : 0) + (int)wbuf[128 + x] + __popc(ww & ((1u << bit) - 1u))] = (uint16_t)k;
    }
    __syncthreads();
    return n;
}

// Row taken by a persistent workgroup at step t, where r = blockIdx.x +
// t gridDim.x.  Rows are numbered query block major (qidx = r / hq, heaviest
// first) and head minor, so a grid that is a multiple of hq keeps each
// workgroup on one head (and one KV group per XCD).  Odd steps take their
// query blocks in reverse order, so that each workgroup's sum of row lengths
// (causal: longest first) comes out about equal.
__device__ __forceinline__ int persistent_row(const BsaArgs &a, int r, int t) {
    const int per = (int)gridDim.x / a.hq;                 // query blocks per step
    if ((t & 1) && per > 0 && (int)gridDim.x == per * a.hq && (t + 1) * per <= a.batch * a.nb)
        return (t * per + (per - 1 - (int)blockIdx.x / a.hq)) * a.hq + r % a.hq;
    return r;
}

template <bool SPARSE, bool PAGED, bool SKIP>
__global__ __launch_bounds__(512, 1) void bsa_fp8_kernel(BsaArgs a) {
    using namespace fp8p;
    // One LDS object: the compiler then leaves LDS reads that follow a load
    // into LDS unordered with it, and the explicit waits and barriers below
    // order them.
    __shared__ __attribute__((aligned(1024))) char smem[SKIP ? SMEM_SKIP : SMEM];
    uint16_t *list = reinterpret_cast<uint16_t *>(smem + LIST_OFF);
    int *wave_sum = reinterpret_cast<int *>(smem + WSUM_OFF);
    float *part_ml = reinterpret_cast<float *>(smem + ML_OFF);
    float *half_max = reinterpret_cast<float *>(smem + HM_OFF);   // SKIP only

    // Persistent workgroups: one per CU, each walking rows wg = blockIdx.x,
    // blockIdx.x + gridDim.x, ... (row_body below), with a barrier between
    // rows so that a row's loads into LDS never overwrite what the previous
    // row still reads.
    uint32_t wcur = 0, wnext = 0;                          // this row's and the next row's mask word
    auto row_body = [&](const int wg, const int next) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));                          // derived per row, not held across rows
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g32 = lane >> 5, r32 = lane & 31;
    const int wq = wave & 3;                               // query group: rows 32 wq .. 32 wq + 31
    const int ks = wave >> 2;                              // key half: keys 64 ks .. 64 ks + 63 of each block
    // heaviest query blocks first; the heads of one KV group on one XCD
    // (workgroup ids, and so the rows a persistent workgroup takes, go round-
    // robin over the 8 XCDs)
    const int qidx = wg / a.hq, jh = wg % a.hq;
    const int I = a.nb - 1 - qidx / a.batch;
    const int b = qidx % a.batch;
    const int h = (a.hq % 8 == 0) ? (jh % 8) * (a.hq / 8) + jh / 8 : jh;
    const int g = h / (a.hq / a.hkv);

    const int qrow = 32 * wq + r32;
    const int token = I * BLK + qrow;
    QFrag<kFP8, D> qf;                                     // in flight while the list is built
    load_q<kFP8, D>(qf, a.q + (((size_t)b * a.seq + token) * a.hq + h) * (size_t)D, g32);
    int n = I + 1;
    if constexpr (SPARSE) {
        // the stages are free here: the previous row ended with every load done
        n = build_list_words<NW>(I, wcur, list, reinterpret_cast<uint32_t *>(smem), wave_sum, tid, lane, wave);
        // the next row's word, in flight through this row (issued after Q, so
        // that the wait for Q below leaves it outstanding)
        wnext = next >= 0 ? mask_word(a, next, tid) : 0u;
    }
    if (n == 0) {
        if (ks == 0) write_empty_row<kFP8, D>(a, b, h, token, g32);
        if (SKIP && a.skipped && ks == 0 && g32 == 0) a.skipped[((size_t)b * a.hq + h) * a.seq + token] = 0;
        return;
    }
    // Q has landed before the first load into LDS: the compiler does not count
    // those loads, so a wait for Q after them would drain them too.
    asm volatile("" :: "v"(qf.u[0]), "v"(qf.u[1]), "v"(qf.u[2]), "v"(qf.u[3]));

    // Loop-invariant LDS offsets.  K operand of S = K Q^T: row kkey of a K
    // stage (+16 rows for the second tile), d chunk 4 st + 2 g32 + hh.  V^T
    // operand: rows vrow + 8 q of a V stage, d chunk 2 dt + ((lane >> 4) & 1),
    // byte half lane & 1.
    const int kkey = 64 * ks + 32 * ((r32 >> 2) & 1) + 4 * (r32 >> 3) + (r32 & 3);
    int koff[4];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            koff[2 * st + hh] = KST + kkey * D + (((4 * st + 2 * g32 + hh) ^ swz_k(kkey)) << 4);
    const int vrow = 64 * ks + 32 * g32 + ((lane & 15) >> 1);
    int voff[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
        voff[dt] = VST + vrow * D + (((2 * dt + ((lane >> 4) & 1)) ^ swz_v(vrow)) << 4) + 8 * (lane & 1);

    // Global -> LDS: wave w moves rows 16 w + 8 i + (lane >> 3) of a block into
    // LDS chunk lane & 7 of the row (i = 0, 1); its 16 rows lie in one page.
    const unsigned row_bytes = (unsigned)a.hkv * D;
    int dk[2], dv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 16 * wave + 8 * i + (lane >> 3), cl = lane & 7;
        dk[i] = (8 * i + (lane >> 3)) * (int)row_bytes + ((cl ^ swz_k(row)) << 4);
        dv[i] = (8 * i + (lane >> 3)) * (int)row_bytes + ((cl ^ swz_v(row)) << 4);
    }
    auto list_at = [&](int i) { return SPARSE ? __builtin_amdgcn_readfirstlane((int)list[i]) : i; };
    const int last = n - 1;
    if constexpr (SPARSE) {
        // pad the list with copies of its last entry, so that reads up to 8 entries
        // ahead need no clamp (visible after the prologue's barrier)
        if (tid < 8) list[n + tid] = list[last];
    }
    // The block table is read-only here: reading it through the constant
    // address space makes the lookups scalar loads, off the vector memory
    // counter that paces the loads into LDS.
    const_i32 *table = PAGED ? (const_i32 *)a.table + b * a.pages_per_seq : nullptr;   // this row's pages
    // byte offset of this wave's first row of a block: its token, and its page when paged
    auto page_of = [&](int tok) -> int { return PAGED ? table[(unsigned)tok >> a.page_log2] : 0; };
    auto row_off = [&](int tok, int page) -> unsigned {
        unsigned row;
        if constexpr (PAGED) row = ((unsigned)page << a.page_log2) | (unsigned)(tok & ((1 << a.page_log2) - 1));
        else row = (unsigned)(b * a.seq + tok);
        return row * row_bytes + (unsigned)g * D;
    };
    auto tok_of = [&](int J) { return J * BLK + 16 * wave; };
    auto src_off = [&](int J) -> unsigned { return row_off(tok_of(J), page_of(tok_of(J))); };
    auto list_raw = [&](int i) -> int { return SPARSE ? (int)list[i] : min(i, last); };   // i <= n + 7
    const i32x4 krs = buffer_rsrc(a.k), vrs = buffer_rsrc(a.v);
    const unsigned lds_wave = (unsigned)(size_t)(lds_char *)smem + 16 * wave * D;   // this wave's rows in a stage
    auto dma = [&](i32x4 rs, auto STAGE_OFF, unsigned so, const int (&vo)[2]) {
        constexpr int OFF = decltype(STAGE_OFF)::value;
        load_lds16<OFF>(rs, lds_wave, (unsigned)vo[0], so);
        load_lds16<OFF + 8 * D>(rs, lds_wave, (unsigned)vo[1], so);
    };
    using std::integral_constant;

    auto qop = [&](int st) {
        const u32x4 b0 = qf.u[2 * st], b1 = qf.u[2 * st + 1];
        return i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    };
    // K operand of tile t, d step st, from the K stage at byte offset ko
    auto kop = [&](int ko, int t, int st) {
        const u32x4 a0 = *reinterpret_cast<const u32x4 *>(smem + ko + koff[2 * st] + t * 16 * D);
        const u32x4 a1 = *reinterpret_cast<const u32x4 *>(smem + ko + koff[2 * st + 1] + t * 16 * D);
        return i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    };
    // V^T operand of d tile dt from the V stage at byte offset vo (from VST)
    auto vop = [&](int vo, int dt) {
        i32x8 av;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const i32x2 x = lds_tr8(smem + vo + voff[dt] + q * 8 * D);
            av[2 * q] = x[0];
            av[2 * q + 1] = x[1];
        }
        return av;
    };
    auto mfma8 = [](const i32x8 &x, const i32x8 &y, const f32x16 &acc, int sy) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, acc, 0, 0, 0, 127, 0, sy);
    };
    const int one = 0x38383838;                            // four E4M3 1.0
    i32x8 ones = {one, one, one, one, one, one, one, one};

    const float c = a.c_exp2;
    const float ninf = -__builtin_huge_valf();
    f32x16 o[4] = {};
    f32x16 lacc = {};                                      // sum of the quantised P, by MFMA (all-ones row)
    float M = M_NONE, Mthr = M_NONE;                       // running max (log2 units) and M + THRESH
    float l = 0.0f;                                        // this lane's exact sum of P (relative to 2^M)
    f32x16 s[2];                                           // scores of the block awaiting softmax
    i32x8 pk = {};                                         // P of the block awaiting PV, E4M3
    int psc = 127;                                         // its E8M0 scale
    const int jdiag = list_at(last) == I ? last : -1;     // the diagonal block, if kept, is the last

    // ---- prologue --------------------------------------------------------------
    // As if iterations -3 .. -1 had run: K(0..3) and V(0..1) loading, and V
    // stage 3 loaded with a copy of V(0) that no iteration reads (iteration 0
    // has no PV of a previous block); it keeps the count of loads in flight
    // the same at every iteration's wait.
    {
        const unsigned s0 = src_off(list_at(0));
        const unsigned s1 = src_off(list_at(min(1, last)));
        dma(krs, integral_constant<int, KST>{}, s0, dk);
        dma(krs, integral_constant<int, KST + TILE>{}, s1, dk);
        dma(vrs, integral_constant<int, VST + 3 * TILE>{}, s0, dv);
        dma(krs, integral_constant<int, KST + 2 * TILE>{}, src_off(list_at(min(2, last))), dk);
        dma(vrs, integral_constant<int, VST>{}, s0, dv);
        dma(krs, integral_constant<int, KST + 3 * TILE>{}, src_off(list_at(min(3, last))), dk);
        dma(vrs, integral_constant<int, VST + TILE>{}, s1, dv);
    }
    // Row lookups run ahead of the loads that use them, so that no wave waits
    // on them: the list entry is read at the end of iteration i-3, the page
    // table at the end of iteration i-2, the offset computed at the end of
    // iteration i-1 for the loads of iteration i (K(i+4), V(i+2)).
    unsigned so_k = src_off(list_at(min(4, last))), so_v = src_off(list_at(min(2, last)));   // iteration 0
    int tk = tok_of(list_at(min(5, last))), tv = tok_of(list_at(min(3, last)));             // iteration 1
    int pgk = page_of(tk), pgv = page_of(tv);
    int lk = list_raw(min(6, last)), lv = list_raw(min(4, last));                          // iteration 2
    sync_vm<10, true>();                                   // K(0) and K(1) have landed
#pragma unroll
    for (int t = 0; t < 2; ++t) s[t] = mfma8(kop(KST, t, 1), qop(1), mfma8(kop(KST, t, 0), qop(0), f32x16{}, 127), 127);
    i32x8 kfirst = kop(KST + TILE, 0, 0);                  // first K operand of S(1)

    // causal mask inside the diagonal block: keys past this lane's query
    auto mask_diag = [&](f32x16(&x)[2]) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (keymap<kFP8>(2 * ks + t, 8 * (e >> 2) + 4 * g32 + (e & 3)) > qrow) x[t][e] = ninf;
    };
    // Online skip (BLASST summary §2.1), on top of the mask: a row drops block
    // j when the block's largest logit lies more than log2(1/lambda) below the
    // row's running maximum (log2 units).  The two waves of a query group each
    // hold half of the block's keys, so each passes the maximum of its half,
    // taken at the end of the previous iteration, through LDS (one slot per
    // block parity), and both decide on the same whole-block maximum.  A
    // dropped row's P is exactly zero (its exp2 offset is +inf); when every
    // row of the wave drops the block, the iteration issues its MFMAs and
    // loads without the softmax.
    auto half_block_max = [&](const f32x16(&x)[2]) {
        auto max3 = [](float p, float q, float r) { return fmaxf(p, fmaxf(q, r)); };
        float u[4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            u[2 * t] = max3(max3(x[t][0], x[t][1], x[t][2]), max3(x[t][3], x[t][4], x[t][5]), max3(x[t][6], x[t][7], x[t][8]));
            u[2 * t + 1] = max3(max3(x[t][9], x[t][10], x[t][11]), max3(x[t][12], x[t][13], x[t][14]), x[t][15]);
        }
        return max_xor32(fmaxf(max3(u[0], u[1], u[2]), u[3]));
    };
    float hmine = 0.0f;                                    // this half's max of the next block (raw)
    float pmax = ninf;                                     // the row's running max (log2 units)
    int nskip = 0;                                         // blocks the row dropped
    if constexpr (SKIP) {
        if (jdiag == 0) mask_diag(s);
        hmine = half_block_max(s);
        half_max[64 * wave + lane] = hmine;                // parity 0 (block 0)
    }

    // ---- main loop: iteration j = softmax(j) with QK(j+1) and PV(j-1) ---------
    // Stages (R = j mod 4): K(j+1) is read from K stage R+1 while K(j+4) loads
    // into K stage R; V(j-1) is read from V stage R+3 while V(j+2) loads into V
    // stage R+2.  Every iteration issues VM_ITER loads per wave, so "all but the
    // last VM_ITER" are the loads of iterations up to j-2: K(j+2) is then in LDS
    // too, and the first K operand of the next block is read at the end of this one.
    float alpha = 1.0f;                                    // rescale of O and lacc still to apply
    auto rescale_o = [&]() {
        // O holds the PV MFMAs up to block j-2 at the scale of M before block
        // j-1 moved it; bring it (and lacc) to the current scale before PV(j-1).
        if (__ballot(alpha != 1.0f)) {
            asm volatile("");                              // (a real branch: taken a few times per row)
#pragma unroll
            for (int e = 0; e < 16; ++e) lacc[e] *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
        }
    };
    // Scores and P alternate between two register sets from one block to the
    // next (the loop is unrolled by an even count), so nothing is copied.
    f32x16 sB[2];
    i32x8 pkB = {};
    int pscB = 127;
    // The row's first kept block carries a second E4M3 term: the residual
    // P - E4M3(P) at the same scale, so that its P reaches O with about seven
    // significant bits instead of four.  The first block is the forced sink
    // block of a Stem mask, where attention mass concentrates.  Iteration 0
    // has no previous block to multiply, so its PV slots are free: at its
    // barrier V(0) has already landed, O and the MFMA row sums are still zero
    // (so block 0 needs no rescale), and the residual's PV is added at the end
    // of the iteration at block 0's scale.  The MFMA count per row is unchanged.
    // PH: 0 any iteration; 1 iteration 0.
    auto iter = [&](auto RR, auto PHC, int j) {
        constexpr int R = decltype(RR)::value;
        constexpr int PH = decltype(PHC)::value;
        constexpr int KRD = KST + ((R + 1) % NST) * TILE, VRD = ((R + 3) % NST) * TILE;
        f32x16(&sc)[2] = (R & 1) ? sB : s;                 // scores of block j
        f32x16(&sn)[2] = (R & 1) ? s : sB;                 // scores of block j+1
        i32x8 &pv_in = (R & 1) ? pkB : pk;                 // P(j-1) and its scale
        int &psc_in = (R & 1) ? pscB : psc;
        i32x8 &pv_out = (R & 1) ? pk : pkB;                // P(j)
        int &psc_out = (R & 1) ? psc : pscB;

        // K(j+1), K(j+2), V(j-1) have landed; stages R, R+2 are free.  (The lookups
        // issued at the end of the last iteration are waited for here, inside the
        // barrier's own skew, rather than at the first LDS wait of the region.)
        sync_vm<VM_ITER, true>();
        float hother = 0.0f;                               // the other key half's max of block j
        if constexpr (SKIP) hother = half_max[64 * (NW * (R & 1) + (wave ^ 4)) + lane];
        if constexpr (!SKIP) asm volatile("" : "+v"(ones));   // kept in registers, not rebuilt per block
        rescale_o();
        if constexpr (!SKIP) {
            if (j == jdiag) {                              // causal mask inside the diagonal block
                asm volatile("");                          // (a real branch: taken once per row)
                mask_diag(sc);
            }
        }
        // ---- the region, in a fixed order: every MFMA is followed by a slice of
        // the softmax of block j, and every LDS operand is read one MFMA ahead.
        // The loads of K(j+4) and V(j+2) into LDS are spread over it, so that
        // the waves of the workgroup do not all queue them behind the barrier.
        constexpr int KDM = KST + R * TILE, VDM = VST + ((R + 2) % NST) * TILE;   // stages being loaded
        auto dma_k = [&](auto I) { load_lds16<KDM + 8 * decltype(I)::value * D>(krs, lds_wave, (unsigned)dk[I], so_k); };
        auto dma_v = [&](auto I) { load_lds16<VDM + 8 * decltype(I)::value * D>(vrs, lds_wave, (unsigned)dv[I], so_v); };
#define SB() __builtin_amdgcn_sched_barrier(0)
        i32x8 ka = kfirst, kb = kop(KRD, 1, 0);
        i32x8 va = PH == 1 ? i32x8{} : vop(VRD, 0);
        i32x8 plo = {};                                    // PH == 1: residual of P(0)
        // the decision, after the first operand reads so that their latency and
        // the other half's maximum overlap.  A row that drops block j runs its
        // softmax like the others with an exp2 offset of +inf: its P are 0 and
        // its M, l and O stay as they are.  (Branching the softmax over when
        // the whole wave drops the block costs registers and spills in every
        // block, for a saving only in the rare blocks all 32 rows drop.)
        bool skip = false;
        if constexpr (SKIP) {
            const float xb = fmaxf(hmine, hother) * c;     // block j's max for this row, log2 units
            skip = xb < pmax + a.skip_log2;
            pmax = fmaxf(pmax, xb);
            nskip += skip ? 1 : 0;
        }
        // row max: a tree of three-input maxima (v_max3), 16 for the 32 scores
        auto max3 = [](float x, float y, float z) { return fmaxf(x, fmaxf(y, z)); };
        auto tile_max = [&](const f32x16 &x, float &u, float &v) {
            u = max3(max3(x[0], x[1], x[2]), max3(x[3], x[4], x[5]), max3(x[6], x[7], x[8]));
            v = max3(max3(x[9], x[10], x[11]), max3(x[12], x[13], x[14]), x[15]);
        };
        float m0, m1, m2, m3;
        if constexpr (!SKIP) tile_max(sc[0], m0, m1);
        SB();
        sn[0] = mfma8(ka, qop(0), f32x16{}, 127);
        SB();
        dma_k(integral_constant<int, 0>{});
        ka = kop(KRD, 0, 1);
        float ce = 0.0f, mc = 0.0f;
        {
            float mx;                                      // this half's max of block j (raw)
            if constexpr (SKIP) {
                mx = hmine;
            } else {
                tile_max(sc[1], m2, m3);
                mx = max_xor32(fmaxf(max3(m0, m1, m2), m3));
            }
            const float xm = mx * c;                       // the block's row max in log2 units
            const float Mn = xm > Mthr ? xm : M;           // lazy: move only past M + THRESH
            alpha = __builtin_amdgcn_exp2f(M - Mn);        // 1 unless the max moved
            M = Mn;
            Mthr = Mn + THRESH;
            // P is cast as P * 2^e, e = 8 - ce, so that the block's largest P lands in
            // (128, 256]; the PV MFMA multiplies by 2^-e through the E8M0 scale 127 - e.
            ce = ceilf(fmaxf(xm - M, -92.0f));             // xm - M <= THRESH, so e >= 0
            mc = (M - 8.0f) + ce;
            if constexpr (SKIP) mc = skip ? __builtin_huge_valf() : mc;   // dropped: P = 0
        }
        // The softmax of block j runs on quads of scores (quad q: tile q >> 2,
        // scores 4 (q & 3) .. 4 (q & 3) + 3) in three steps, the exp2 argument,
        // the exp2, then the sums and the E4M3 pack, each one MFMA slot after
        // the one before, so that no step waits on its predecessor's latency.
        float ls[4];
        auto fq = [&](int q) {
#pragma unroll
            for (int e = 4 * (q & 3); e < 4 * (q & 3) + 4; ++e) sc[q >> 2][e] = fmaf(sc[q >> 2][e], c, -mc);
        };
        auto eq = [&](int q) {
#pragma unroll
            for (int e = 4 * (q & 3); e < 4 * (q & 3) + 4; ++e) sc[q >> 2][e] = __builtin_amdgcn_exp2f(sc[q >> 2][e]);
        };
        auto packq = [&](int w) {                          // 4 P of P word w as E4M3
            const f32x16 &src = sc[w >> 2];
            const int ee = 4 * (w & 3);
            // the word's old contents (P of block j-2, consumed) are the tied operand
            const int x = __builtin_amdgcn_cvt_pk_fp8_f32(src[ee], src[ee + 1], pv_out[w], false);
            pv_out[w] = __builtin_amdgcn_cvt_pk_fp8_f32(src[ee + 2], src[ee + 3], x, true);
            if constexpr (PH == 1) {
                // residual of P(0): exact in fp32 (P and its E4M3 value lie within
                // a factor of two), then rounded to E4M3 itself
                const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(pv_out[w], false);
                const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(pv_out[w], true);
                const int y = __builtin_amdgcn_cvt_pk_fp8_f32(src[ee] - h01[0], src[ee + 1] - h01[1], plo[w], false);
                plo[w] = __builtin_amdgcn_cvt_pk_fp8_f32(src[ee + 2] - h23[0], src[ee + 3] - h23[1], y, true);
            }
        };
        auto aq = [&](int q) {                            // P into the partial sums, then packed
#pragma unroll
            for (int e = 4 * (q & 3); e < 4 * (q & 3) + 4; ++e) ls[e & 3] = q == 0 ? sc[0][e] : ls[e & 3] + sc[q >> 2][e];
            packq(q);
        };
        // one softmax slice per MFMA slot
        auto slice = [&](auto f) { f(); };
        slice([&] { fq(0); });
        SB();
        sn[1] = mfma8(kb, qop(0), f32x16{}, 127);
        SB();
        dma_k(integral_constant<int, 1>{});
        kb = kop(KRD, 1, 1);
        slice([&] { fq(1); eq(0); });
        SB();
        sn[0] = mfma8(ka, qop(1), sn[0], 127);
        SB();
        dma_v(integral_constant<int, 0>{});
        i32x8 vb = PH == 1 ? i32x8{} : vop(VRD, 1);
        slice([&] { fq(2); eq(1); aq(0); });
        SB();
        sn[1] = mfma8(kb, qop(1), sn[1], 127);
        SB();
        kfirst = kop(KST + ((R + 2) % NST) * TILE, 0, 0);  // K(j+2): the first operand of S(j+2)
        dma_v(integral_constant<int, 1>{});
        slice([&] { fq(3); eq(2); aq(1); });
        // PV(j-1) (none in iteration 0)
        auto pv = [&](int dt, const i32x8 &vx) {
            if constexpr (PH != 1) o[dt] = mfma8(vx, pv_in, o[dt], psc_in);
        };
        SB();
        pv(0, va);
        SB();
        if constexpr (PH != 1) va = vop(VRD, 2);
        slice([&] { fq(4); eq(3); aq(2); });
        SB();
        pv(1, vb);
        SB();
        if constexpr (PH != 1) vb = vop(VRD, 3);
        slice([&] { fq(5); eq(4); aq(3); });
        SB();
        pv(2, va);
        SB();
        slice([&] { fq(6); fq(7); eq(5); aq(4); });
        SB();
        pv(3, vb);
        SB();
        slice([&] { eq(6); eq(7); aq(5); });
        if constexpr (SKIP) {
            // made here, each block, so that it holds no registers through the region
#pragma unroll
            for (int w = 0; w < 8; ++w) asm volatile("v_mov_b32 %0, 0x38383838" : "=v"(ones[w]));
        }
        SB();
        if constexpr (PH != 1) lacc = mfma8(ones, pv_in, lacc, psc_in);
        SB();
        slice([&] { aq(6); aq(7); });
        {
            const int ice = (int)ce;
            l = fmaf(l, alpha, ldexpf((ls[0] + ls[1]) + (ls[2] + ls[3]), ice - 8));
            psc_out = 119 + ice;
        }
        SB();
        if constexpr (PH == 1) {
            // O and lacc are zero: no rescale is due, and the residual of P(0)
            // multiplies V(0) (V stage 0) at block 0's scale
            alpha = 1.0f;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) o[dt] = mfma8(vop(0, dt), plo, o[dt], psc_out);
            lacc = mfma8(ones, plo, lacc, psc_out);
        }
        if constexpr (SKIP) {
            // the next block's half max, for the decision at the next barrier
            if (j + 1 == jdiag) {
                asm volatile("");
                mask_diag(sn);
            }
            hmine = half_block_max(sn);
            half_max[64 * (NW * ((R + 1) & 1) + wave) + lane] = hmine;
        }
#undef SB
        // ---- lookups, after the region: they complete across the barrier
        so_k = row_off(tk, pgk);                           // iteration j+1
        so_v = row_off(tv, pgv);
        tk = tok_of(__builtin_amdgcn_readfirstlane(lk));   // iteration j+2
        tv = tok_of(__builtin_amdgcn_readfirstlane(lv));
        pgk = page_of(tk);
        pgv = page_of(tv);
        lk = list_raw(j + 7);                              // iteration j+3
        lv = list_raw(j + 5);
    };
    using PH0 = integral_constant<int, 0>;
    iter(integral_constant<int, 0>{}, integral_constant<int, 1>{}, 0);
    for (int j = 1; j < n; j += NST) {
        iter(integral_constant<int, 1>{}, PH0{}, j);
        if (j + 1 < n) iter(integral_constant<int, 2>{}, PH0{}, j + 1);
        if (j + 2 < n) iter(integral_constant<int, 3>{}, PH0{}, j + 2);
        if (j + 3 < n) iter(integral_constant<int, 0>{}, PH0{}, j + 3);
    }
    sync_vm<2 * VM_ITER>();                                // V(n-1) has landed
    rescale_o();
    {
        // block n-1 ran as an iteration with R = (n-1) mod 4: its P is in pkB for even R
        const bool odd = ((n - 1) & 1) != 0;
        const i32x8 pl = odd ? pk : pkB;
        const int sl = odd ? psc : pscB;
        const int vo = ((n - 1) % NST) * TILE;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] = mfma8(vop(vo, dt), pl, o[dt], sl);
        lacc = mfma8(ones, pl, lacc, sl);
    }

    // ---- merge the key halves, normalise, store -------------------------------
    // Sparse: the two waves of a query group each finalise two of the four d
    // tiles (key half ks: tiles 2 ks, 2 ks + 1).  Each hands the other two tiles
    // and its (M, l, lq) to its partner (wave ^ 4) through LDS.
    l = sum_xor32(l);                                      // exact sum of P: the LSE
    float lq = lacc[0];                                    // sum of the quantised P: O's denominator
    sync_vm<0, true>();                                    // every load into LDS is done: stages are free
    if constexpr (!SPARSE) {
    // Dense: the key-half-1 wave hands all four d tiles to its partner, which
    // finalises them alone (measured faster for the dense kernel than the
    // split below).
    float *po = reinterpret_cast<float *>(smem) + wq * 64 * (D / 2);
    if (ks == 1) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) po[(dt * 16 + e) * 64 + lane] = o[dt][e];
        part_ml[(3 * wq) * 64 + lane] = M;
        part_ml[(3 * wq + 1) * 64 + lane] = l;
        part_ml[(3 * wq + 2) * 64 + lane] = lq;
    }
    __syncthreads();
    if (ks == 1) return;
    const float M1 = part_ml[(3 * wq) * 64 + lane];
    const float l1 = part_ml[(3 * wq + 1) * 64 + lane];
    const float lq1 = part_ml[(3 * wq + 2) * 64 + lane];
    const float mm = fmaxf(M, M1);
    const float a0 = __builtin_amdgcn_exp2f(M - mm), a1 = __builtin_amdgcn_exp2f(M1 - mm);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] = fmaf(o[dt][e], a0, po[(dt * 16 + e) * 64 + lane] * a1);
    l = fmaf(l, a0, l1 * a1);                            // key half 0 fused onto half 1: as the sparse merge
    lq = fmaf(lq, a0, lq1 * a1);
    const float inv = lq > 0.0f ? a.o_scale / lq : 0.0f;
    const size_t obase = (((size_t)b * a.seq + token) * a.hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 32 * dt + 8 * i + 4 * g32;
            u32x2 u;
            u.x = f32_to_bf16_bits(o[dt][4 * i] * inv) | (f32_to_bf16_bits(o[dt][4 * i + 1] * inv) << 16);
            u.y = f32_to_bf16_bits(o[dt][4 * i + 2] * inv) | (f32_to_bf16_bits(o[dt][4 * i + 3] * inv) << 16);
            *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(a.o) + obase + d0) = u;
        }
    if (a.lse && g32 == 0)
        a.lse[((size_t)b * a.hq + h) * a.seq + token] = l > 0.0f ? fmaf(mm, 0.6931471805599453f, logf(l)) : ninf;
    if (SKIP && a.skipped && g32 == 0) a.skipped[((size_t)b * a.hq + h) * a.seq + token] = nskip;
    } else {
    auto hand_over = [&](auto KSC) {
        constexpr int K = decltype(KSC)::value;
        float *pout = reinterpret_cast<float *>(smem) + wave * (32 * 64);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 16; ++e) pout[(u * 16 + e) * 64 + lane] = o[2 * (1 - K) + u][e];
    };
    if (ks == 0) hand_over(integral_constant<int, 0>{});
    else hand_over(integral_constant<int, 1>{});
    part_ml[(3 * wave) * 64 + lane] = M;
    part_ml[(3 * wave + 1) * 64 + lane] = l;
    part_ml[(3 * wave + 2) * 64 + lane] = lq;
    __syncthreads();
    auto finish = [&](auto KSC) {
        constexpr int K = decltype(KSC)::value;
        const int pw = wave ^ 4;                           // the partner: the other key half
        const float Mp = part_ml[(3 * pw) * 64 + lane];
        const float lp = part_ml[(3 * pw + 1) * 64 + lane];
        const float lqp = part_ml[(3 * pw + 2) * 64 + lane];
        // key half 0 first, so that both waves form identical sums
        const float M0 = K ? Mp : M, M1 = K ? M : Mp;
        const float mm = fmaxf(M0, M1);
        const float a0 = __builtin_amdgcn_exp2f(M0 - mm), a1 = __builtin_amdgcn_exp2f(M1 - mm);
        const float lt = fmaf(K ? lp : l, a0, (K ? l : lp) * a1);
        const float lqt = fmaf(K ? lqp : lq, a0, (K ? lq : lqp) * a1);
        const float inv = lqt > 0.0f ? a.o_scale / lqt : 0.0f;
        const float *pin = reinterpret_cast<const float *>(smem) + pw * (32 * 64);
        const size_t obase = (((size_t)b * a.seq + token) * a.hq + h) * D;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int dt = 2 * K + u;
            f32x16 x;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                // key half 0's value fused onto half 1's product, on either wave
                const float own = o[2 * K + u][e], other = pin[(u * 16 + e) * 64 + lane];
                x[e] = fmaf(K ? other : own, a0, (K ? own : other) * a1) * inv;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * dt + 8 * i + 4 * g32;
                u32x2 v2;
                v2.x = f32_to_bf16_bits(x[4 * i]) | (f32_to_bf16_bits(x[4 * i + 1]) << 16);
                v2.y = f32_to_bf16_bits(x[4 * i + 2]) | (f32_to_bf16_bits(x[4 * i + 3]) << 16);
                *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(a.o) + obase + d0) = v2;
            }
        }
        if (K == 0 && a.lse && g32 == 0)
            a.lse[((size_t)b * a.hq + h) * a.seq + token] = lt > 0.0f ? fmaf(mm, 0.6931471805599453f, logf(lt)) : ninf;
        if (SKIP && K == 0 && a.skipped && g32 == 0) a.skipped[((size_t)b * a.hq + h) * a.seq + token] = nskip;
    };
    if (ks == 0) finish(integral_constant<int, 0>{});
    else finish(integral_constant<int, 1>{});
    }
    };
    const int rows = a.batch * a.hq * a.nb;
    if (SPARSE && (int)blockIdx.x < rows) wcur = mask_word(a, persistent_row(a, blockIdx.x, 0), threadIdx.x);
    for (int r = blockIdx.x, t = 0; r < rows; r += gridDim.x, ++t) {
        const int rn = r + (int)gridDim.x;
        row_body(persistent_row(a, r, t), rn < rows ? persistent_row(a, rn, t + 1) : -1);
        wcur = wnext;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// BF16, d = 128, 128-token blocks: the pipeline of bsa_fp8_kernel with bf16
// operands (v_mfma_f32_32x32x16_bf16: per block and wave 16 MFMAs of
// S = K(j+1) Q^T and 16 of O += V(j-1)^T P(j-1), interleaved with the softmax
// of block j).  A K or V block is 32 KB in LDS, so there are two stages of
// each and the loads run one block ahead: K(j+2) and V(j) are loaded during
// block j and waited for at the next block's barrier.  P is rounded to bf16
// with no scale, and O is normalised by the exact fp32 sum of P.
//
// LDS swizzles of the 16-byte chunks of a 256-byte row.  K: chunk c of row r
// sits at c ^ (r & 15), so the 16 rows a 16-lane group reads for one MFMA
// step land on 16 distinct chunk positions, and a lane's address for step s
// is its base XOR 32 s.  V: chunk c of row r sits at c ^ ((r & 3) << 2), so
// the 4 rows x 2 chunks of one transposing read land on 8 distinct positions,
// and every V operand address is one of four per-lane registers (one per d
// tile) plus an immediate.
namespace bf16p {
constexpr int D = 128, BLK = 128, NT = 512, NW = 8;
constexpr int ROWB = D * 2;                      // bytes of a K or V row
constexpr int TILE = BLK * ROWB;                 // bytes of a K or V block
constexpr int KST = 0, VST = 2 * TILE;           // two K stages, then two V stages
constexpr int LIST_OFF = 4 * TILE;               // kept-block list (u16) after the stages
constexpr int LIST = 4096 + 8;                   // up to 4096 kept blocks, plus 8 pad entries
constexpr int WSUM_OFF = LIST_OFF + 2 * LIST;    // per-wave counts of the list scan
constexpr int ML_OFF = WSUM_OFF + 4 * NW;        // (M, l) of every wave, for the key-half merge
constexpr int HM_OFF = ML_OFF + 2 * NW * 64 * 4; // online skip: half-block maxima, [parity][wave][lane]
constexpr int SMEM = HM_OFF;
constexpr int SMEM_SKIP = HM_OFF + 2 * NW * 64 * 4;
constexpr float THRESH = 8.0f;                   // lazy rescale: P stays below 2^THRESH
constexpr float M_NONE = -3.0e38f;               // running max before any finite score
__device__ __forceinline__ int swz_k(int row) { return row & 15; }
__device__ __forceinline__ int swz_v(int row) { return (row & 3) << 2; }
}  // namespace bf16p

template <bool SPARSE, bool PAGED, bool SKIP>
__global__ __launch_bounds__(512, 1) void bsa_bf16_kernel(BsaArgs a) {
    using namespace bf16p;
    using fp8p::buffer_rsrc;
    using fp8p::const_i32;
    using fp8p::i32x4;
    using fp8p::load_lds16;
    using fp8p::sync_vm;
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    __shared__ __attribute__((aligned(1024))) char smem[SKIP ? SMEM_SKIP : SMEM];
    uint16_t *list = reinterpret_cast<uint16_t *>(smem + LIST_OFF);
    int *wave_sum = reinterpret_cast<int *>(smem + WSUM_OFF);
    float *part_ml = reinterpret_cast<float *>(smem + ML_OFF);
    float *half_max = reinterpret_cast<float *>(smem + HM_OFF);   // SKIP only

    // Persistent workgroups, as in bsa_fp8_kernel: rows wg = blockIdx.x,
    // blockIdx.x + gridDim.x, ..., with a barrier between rows.
    uint32_t wcur = 0, wnext = 0;                          // this row's and the next row's mask word
    auto row_body = [&](const int wg, const int next) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));                          // derived per row, not held across rows
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g32 = lane >> 5, r32 = lane & 31;
    const int wq = wave & 3;                               // query group: rows 32 wq .. 32 wq + 31
    const int ks = wave >> 2;                              // key half: keys 64 ks .. 64 ks + 63 of each block

    // heaviest query blocks first; the heads of one KV group on one XCD
    const int qidx = wg / a.hq, jh = wg % a.hq;
    const int I = a.nb - 1 - qidx / a.batch;
    const int b = qidx % a.batch;
    const int h = (a.hq % 8 == 0) ? (jh % 8) * (a.hq / 8) + jh / 8 : jh;
    const int g = h / (a.hq / a.hkv);

    const int qrow = 32 * wq + r32;
    const int token = I * BLK + qrow;
    QFrag<kBF16, D> qf;                                    // in flight while the list is built
    load_q<kBF16, D>(qf, a.q + (((size_t)b * a.seq + token) * a.hq + h) * (size_t)ROWB, g32);
    int n = I + 1;
    if constexpr (SPARSE) {
        // as in bsa_fp8_kernel: the stages are free here, and the next row's
        // word is issued after Q
        n = build_list_words<NW>(I, wcur, list, reinterpret_cast<uint32_t *>(smem), wave_sum, tid, lane, wave);
        wnext = next >= 0 ? mask_word(a, next, tid) : 0u;
    }
    if (n == 0) {
        if (ks == 0) write_empty_row<kBF16, D>(a, b, h, token, g32);
        if (SKIP && a.skipped && ks == 0 && g32 == 0) a.skipped[((size_t)b * a.hq + h) * a.seq + token] = 0;
        return;
    }
    // Q has landed before the first load into LDS (those loads are not counted
    // by the compiler, so a later wait for Q would drain them too).
    asm volatile("" :: "v"(qf.u[0]), "v"(qf.u[1]), "v"(qf.u[2]), "v"(qf.u[3]));
    asm volatile("" :: "v"(qf.u[4]), "v"(qf.u[5]), "v"(qf.u[6]), "v"(qf.u[7]));

    // K operand of S = K Q^T: row kkey (+32 for the second tile), d chunk
    // 2 s + g32 at position (2 s + g32) ^ (kkey & 15): base XOR 32 s.
    const int kkey = 64 * ks + keymap<kBF16>(0, r32);
    const int kbase = kkey * ROWB + 16 * (g32 ^ swz_k(kkey));
    // V^T operand of d tile dt: rows vrow + (32 t + 16 hh + 4 q) of a V stage,
    // chunk 4 dt + 2 ((lane >> 4) & 1) + ((lane & 3) >> 1), byte half lane & 1.
    const int i16 = lane & 15;
    const int vrow = 64 * ks + 8 * g32 + (i16 >> 2);
    int vbase[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
        vbase[dt] = VST + vrow * ROWB + (((4 * dt + 2 * ((lane >> 4) & 1) + ((i16 & 3) >> 1)) ^ swz_v(vrow)) << 4) +
                    8 * (i16 & 1);

    // Global -> LDS: wave w moves rows 16 w + 4 i + (lane >> 4) of a block
    // (i = 0..3) into LDS chunk position lane & 15 of the row; its 16 rows lie
    // in one page.
    const unsigned row_bytes = (unsigned)a.hkv * ROWB;
    int dk[4], dv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * wave + 4 * i + (lane >> 4), cl = lane & 15;
        dk[i] = (4 * i + (lane >> 4)) * (int)row_bytes + ((cl ^ swz_k(row)) << 4);
        dv[i] = (4 * i + (lane >> 4)) * (int)row_bytes + ((cl ^ swz_v(row)) << 4);
    }
    auto list_at = [&](int i) { return SPARSE ? __builtin_amdgcn_readfirstlane((int)list[i]) : i; };
    const int last = n - 1;
    if constexpr (SPARSE) {
        // pad the list with copies of its last entry, so that reads ahead need no clamp
        if (tid < 8) list[n + tid] = list[last];
    }
    const_i32 *table = PAGED ? (const_i32 *)a.table + b * a.pages_per_seq : nullptr;
    auto page_of = [&](int tok) -> int { return PAGED ? table[(unsigned)tok >> a.page_log2] : 0; };
    auto row_off = [&](int tok, int page) -> unsigned {
        unsigned row;
        if constexpr (PAGED) row = ((unsigned)page << a.page_log2) | (unsigned)(tok & ((1 << a.page_log2) - 1));
        else row = (unsigned)(b * a.seq + tok);
        return row * row_bytes + (unsigned)g * ROWB;
    };
    auto tok_of = [&](int J) { return J * BLK + 16 * wave; };
    auto src_off = [&](int J) -> unsigned { return row_off(tok_of(J), page_of(tok_of(J))); };
    auto list_raw = [&](int i) -> int { return SPARSE ? (int)list[i] : min(i, last); };   // i <= n + 7
    const i32x4 krs = buffer_rsrc(a.k), vrs = buffer_rsrc(a.v);
    const unsigned lds_wave = (unsigned)(size_t)(lds_char *)smem + 16 * wave * ROWB;
    auto dma = [&](i32x4 rs, auto STAGE_OFF, unsigned so, const int (&vo)[4]) {
        constexpr int OFF = decltype(STAGE_OFF)::value;
        load_lds16<OFF>(rs, lds_wave, (unsigned)vo[0], so);
        load_lds16<OFF + 4 * ROWB>(rs, lds_wave, (unsigned)vo[1], so);
        load_lds16<OFF + 8 * ROWB>(rs, lds_wave, (unsigned)vo[2], so);
        load_lds16<OFF + 12 * ROWB>(rs, lds_wave, (unsigned)vo[3], so);
    };
    using std::integral_constant;

    auto qop = [&](int st) { return __builtin_bit_cast(bf16x8, qf.u[st]); };
    // K operand of tile t, d step st, from the K stage at byte offset ko
    auto kop = [&](int ko, int t, int st) {
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(smem + ko + (kbase ^ (32 * st)) + t * 32 * ROWB));
    };
    // V^T operand of d tile dt, keys 32 t + 16 hh of this wave's half, V stage vo (from VST)
    auto vop = [&](int vo, int t, int hh, int dt) {
        const char *p = smem + vo + vbase[dt] + (32 * t + 16 * hh) * ROWB;
        const i16x4 v0 = lds_tr16(p), v1 = lds_tr16(p + 4 * ROWB);
        return __builtin_bit_cast(bf16x8, i16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
    };
    auto mfma16 = [](const bf16x8 &x, const bf16x8 &y, const f32x16 &acc) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc, 0, 0, 0);
    };

    const float c = a.c_exp2;
    const float ninf = -__builtin_huge_valf();
    f32x16 o[4] = {};
    float M = M_NONE, Mthr = M_NONE;                       // running max (log2 units) and M + THRESH
    float l = 0.0f;                                        // this lane's exact sum of P (relative to 2^M)
    f32x16 s[2] = {};                                      // scores of the block awaiting softmax
    bf16x8 pk[4] = {};                                     // P of the block awaiting PV (zero before the first)
    const int jdiag = list_at(last) == I ? last : -1;      // the diagonal block, if kept, is the last

    // ---- prologue: K(0), K(1) and, standing in for V(-1) (multiplied by P = 0,
    // so it only has to be finite), a copy of V(0) in V stage 1
    {
        const unsigned s0 = src_off(list_at(0));
        dma(krs, integral_constant<int, KST>{}, s0, dk);
        dma(krs, integral_constant<int, KST + TILE>{}, src_off(list_at(min(1, last))), dk);
        dma(vrs, integral_constant<int, VST + TILE>{}, s0, dv);
    }
    // Row lookups run ahead of the loads that use them: the list entry is read
    // at the end of iteration i-3, the page-table entry at the end of i-2, the
    // offset formed at the end of i-1, for the loads of iteration i (K(i+2), V(i)).
    unsigned so_k = src_off(list_at(min(2, last))), so_v = src_off(list_at(0));        // iteration 0
    int tk = tok_of(list_at(min(3, last))), tv = tok_of(list_at(min(1, last)));       // iteration 1
    int pgk = page_of(tk), pgv = page_of(tv);
    int lk = list_raw(min(4, last)), lv = list_raw(min(2, last));                     // iteration 2
    sync_vm<0, true>();                                    // K(0), K(1) have landed
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
        for (int t = 0; t < 2; ++t) s[t] = mfma16(kop(KST, t, st), qop(st), s[t]);

    // causal mask inside the diagonal block: keys past this lane's query
    auto mask_diag = [&](f32x16(&x)[2]) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (keymap<kBF16>(2 * ks + t, 8 * (e >> 2) + 4 * g32 + (e & 3)) > qrow) x[t][e] = ninf;
    };
    // Online skip (BLASST summary §2.1): as in bsa_fp8_kernel, the two waves of
    // a query group exchange their half-block maxima through LDS one block
    // ahead and drop block j for a row when its maximum lies more than
    // log2(1/lambda) below the row's running maximum.
    auto half_block_max = [&](const f32x16(&x)[2]) {
        auto max3 = [](float p, float q, float r) { return fmaxf(p, fmaxf(q, r)); };
        float u[4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            u[2 * t] = max3(max3(x[t][0], x[t][1], x[t][2]), max3(x[t][3], x[t][4], x[t][5]), max3(x[t][6], x[t][7], x[t][8]));
            u[2 * t + 1] = max3(max3(x[t][9], x[t][10], x[t][11]), max3(x[t][12], x[t][13], x[t][14]), x[t][15]);
        }
        return max_xor32(fmaxf(max3(u[0], u[1], u[2]), u[3]));
    };
    float hmine = 0.0f;                                    // this half's max of the next block (raw)
    float pmax = ninf;                                     // the row's running max (log2 units)
    int nskip = 0;                                         // blocks the row dropped
    if constexpr (SKIP) {
        if (jdiag == 0) mask_diag(s);
        hmine = half_block_max(s);
        half_max[64 * wave + lane] = hmine;                // parity 0 (block 0)
    }

    float alpha = 1.0f;                                    // rescale of O still to apply
    auto rescale_o = [&]() {
        if (__ballot(alpha != 1.0f)) {
            asm volatile("");                              // (a real branch: taken a few times per row)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
        }
    };
    f32x16 sB[2];
    bf16x8 pkB[4] = {};
    auto iter = [&](auto RR, int j) {
        constexpr int R = decltype(RR)::value;              // j & 1
        constexpr int KRD = KST + (1 - R) * TILE;           // K(j+1)
        constexpr int VRD = (1 - R) * TILE;                 // V(j-1), from VST
        constexpr int KDM = KST + R * TILE, VDM = VST + R * TILE;   // stages being loaded
        f32x16(&sc)[2] = R ? sB : s;                        // scores of block j
        f32x16(&sn)[2] = R ? s : sB;                        // scores of block j+1
        bf16x8(&pv_in)[4] = R ? pkB : pk;                   // P(j-1)
        bf16x8(&pv_out)[4] = R ? pk : pkB;                  // P(j)

        // K(j+1) and V(j-1) have landed; K stage R and V stage R are free
        sync_vm<0, true>();
        float hother = 0.0f;                               // the other key half's max of block j
        if constexpr (SKIP) hother = half_max[64 * (NW * R + (wave ^ 4)) + lane];
        rescale_o();
        if constexpr (!SKIP) {
            if (j == jdiag) {                              // causal mask inside the diagonal block
                asm volatile("");                          // (a real branch: taken once per row)
                mask_diag(sc);
            }
        }
#define SB() __builtin_amdgcn_sched_barrier(0)
        auto dma_k = [&](auto I) {
            load_lds16<KDM + 4 * decltype(I)::value * ROWB>(krs, lds_wave, (unsigned)dk[I], so_k);
        };
        auto dma_v = [&](auto I) {
            load_lds16<VDM + 4 * decltype(I)::value * ROWB>(vrs, lds_wave, (unsigned)dv[I], so_v);
        };
        auto max3 = [](float x, float y, float z) { return fmaxf(x, fmaxf(y, z)); };
        auto tile_max = [&](const f32x16 &x, float &u, float &v) {
            u = max3(max3(x[0], x[1], x[2]), max3(x[3], x[4], x[5]), max3(x[6], x[7], x[8]));
            v = max3(max3(x[9], x[10], x[11]), max3(x[12], x[13], x[14]), x[15]);
        };
        float ls[4];
        float Me = M;                                      // exp2 offset: +inf for a dropped row
        auto expq = [&](int t, int e0) {                   // P of 4 scores, into the partial sums
#pragma unroll
            for (int e = e0; e < e0 + 4; ++e) {
                const float pe = __builtin_amdgcn_exp2f(fmaf(sc[t][e], c, -Me));
                sc[t][e] = pe;
                ls[e & 3] = (t == 0 && e0 == 0) ? pe : ls[e & 3] + pe;
            }
        };
        auto packq = [&](int w) {                          // 8 P of word w as bf16
            const f32x16 &src = sc[w >> 1];
            const int e0 = 8 * (w & 1);
#pragma unroll
            for (int e = 0; e < 8; ++e) pv_out[w][e] = (__bf16)src[e0 + e];
        };
        // ---- the region: 32 MFMA slots.  Slots 0-15: S(j+1) tile (k & 1), d
        // step k / 2; slots 16-31: O tile (k & 3) += keys (k - 16) / 4 of V(j-1).
        // Each LDS operand is read one slot ahead; the loads into LDS go out in
        // the first eight slots; the softmax of block j is spread over the rest.
        // MFMA m < 16: S(j+1) tile m & 1, d step m / 2; m >= 16: O tile m & 3
        // += keys 16 ((m - 16) / 4) of V(j-1).  Slot k issues MFMA order(k).
        auto order = [](int k) { return k; };
        auto operand = [&](int m) {
            if (m < 16) return kop(KRD, m & 1, m >> 1);
            return vop(VRD, (m - 16) >> 3, ((m - 16) >> 2) & 1, m & 3);
        };
        bf16x8 opk = operand(order(0));
        // the decision, after the first operand read so that its latency and
        // the other half's maximum overlap; soft: some row of the wave keeps
        // block j (always, without the skip); the softmax work is branched
        // over, wave-uniformly, when none does
        bool skip = false;
        if constexpr (SKIP) {
            const float xb = fmaxf(hmine, hother) * c;     // block j's max for this row, log2 units
            skip = xb < pmax + a.skip_log2;
            pmax = fmaxf(pmax, xb);
            nskip += skip ? 1 : 0;
        }
        const bool soft = SKIP ? !__all(skip) : true;
        float m0, m1, m2, m3, mx = 0.0f;
        auto slot = [&](auto KK) {
            constexpr int k = decltype(KK)::value;
            constexpr int m = order(k);
            bf16x8 nxt;
            if constexpr (k + 1 < 32) nxt = operand(order(k + 1));   // operand of the next slot
            SB();
            if constexpr (m < 16) sn[m & 1] = mfma16(opk, qop(m >> 1), m < 2 ? f32x16{} : sn[m & 1]);
            else o[m & 3] = mfma16(opk, pv_in[((m - 16) >> 2)], o[m & 3]);
            SB();
            if constexpr (k < 4) dma_k(integral_constant<int, k>{});
            else if constexpr (k < 8) dma_v(integral_constant<int, k - 4>{});
            // softmax work of this slot
            if (soft) {
                if constexpr (k == 0 && !SKIP) tile_max(sc[0], m0, m1);
                if constexpr (k == 1 && !SKIP) tile_max(sc[1], m2, m3);
                if constexpr (k == 2) {
                    if constexpr (SKIP) mx = hmine;
                    else mx = max_xor32(fmaxf(max3(m0, m1, m2), m3));
                    const float xm = mx * c;                   // the block's row max in log2 units
                    const float Mn = xm > Mthr ? xm : M;       // lazy: move only past M + THRESH
                    alpha = __builtin_amdgcn_exp2f(M - Mn);    // 1 unless the max moved
                    M = Mn;
                    Mthr = Mn + THRESH;
                    Me = SKIP && skip ? __builtin_huge_valf() : M;
                }
                if constexpr (k >= 3 && k < 27 && (k - 3) % 3 == 0) expq(((k - 3) / 3) >> 2, 4 * (((k - 3) / 3) & 3));
                if constexpr (k >= 5 && k < 29 && (k - 5) % 3 == 0 && ((k - 5) / 3) & 1) packq(((k - 5) / 3) >> 1);
            }
            if constexpr (k + 1 < 32) opk = nxt;
        };
        slot(integral_constant<int, 0>{});
        slot(integral_constant<int, 1>{});
        slot(integral_constant<int, 2>{});
        slot(integral_constant<int, 3>{});
        slot(integral_constant<int, 4>{});
        slot(integral_constant<int, 5>{});
        slot(integral_constant<int, 6>{});
        slot(integral_constant<int, 7>{});
        slot(integral_constant<int, 8>{});
        slot(integral_constant<int, 9>{});
        slot(integral_constant<int, 10>{});
        slot(integral_constant<int, 11>{});
        slot(integral_constant<int, 12>{});
        slot(integral_constant<int, 13>{});
        slot(integral_constant<int, 14>{});
        slot(integral_constant<int, 15>{});
        slot(integral_constant<int, 16>{});
        slot(integral_constant<int, 17>{});
        slot(integral_constant<int, 18>{});
        slot(integral_constant<int, 19>{});
        slot(integral_constant<int, 20>{});
        slot(integral_constant<int, 21>{});
        slot(integral_constant<int, 22>{});
        slot(integral_constant<int, 23>{});
        slot(integral_constant<int, 24>{});
        slot(integral_constant<int, 25>{});
        slot(integral_constant<int, 26>{});
        slot(integral_constant<int, 27>{});
        slot(integral_constant<int, 28>{});
        slot(integral_constant<int, 29>{});
        slot(integral_constant<int, 30>{});
        slot(integral_constant<int, 31>{});
        if (soft) {
            l = fmaf(l, alpha, (ls[0] + ls[1]) + (ls[2] + ls[3]));
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) pv_out[w] = bf16x8{};   // P(j) = 0: PV(j) adds nothing
            alpha = 1.0f;                                  // M, l unchanged
        }
        SB();
        if constexpr (SKIP) {
            // the next block's half max, for the decision at the next barrier
            if (j + 1 == jdiag) {
                asm volatile("");
                mask_diag(sn);
            }
            hmine = half_block_max(sn);
            half_max[64 * (NW * (1 - R) + wave) + lane] = hmine;
        }
#undef SB
        // ---- lookups, after the region: they complete across the barrier
        so_k = row_off(tk, pgk);                           // iteration j+1
        so_v = row_off(tv, pgv);
        tk = tok_of(__builtin_amdgcn_readfirstlane(lk));   // iteration j+2
        tv = tok_of(__builtin_amdgcn_readfirstlane(lv));
        pgk = page_of(tk);
        pgv = page_of(tv);
        lk = list_raw(j + 5);                              // iteration j+3
        lv = list_raw(j + 3);
    };
    for (int j = 0; j < n; j += 2) {
        iter(std::integral_constant<int, 0>{}, j);
        if (j + 1 < n) iter(std::integral_constant<int, 1>{}, j + 1);
    }
    sync_vm<0>();                                          // V(n-1) has landed
    rescale_o();
    {
        // block n-1 ran as an iteration with R = (n-1) & 1: its P is in pk for odd R
        const bool odd = ((n - 1) & 1) != 0;
        const int vo = ((n - 1) & 1) * TILE;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const bf16x8 pl = odd ? pk[w] : pkB[w];
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) o[dt] = mfma16(vop(vo, w >> 1, w & 1, dt), pl, o[dt]);
        }
    }

    // ---- merge the key halves, normalise, store -------------------------------
    // As in bsa_fp8_kernel: each wave of a query group finalises two of the
    // four d tiles and hands the other two, with its (M, l), to wave ^ 4.
    l = sum_xor32(l);
    sync_vm<0, true>();                                    // every load into LDS is done: stages are free
    auto hand_over = [&](auto KSC) {
        constexpr int K = decltype(KSC)::value;
        float *pout = reinterpret_cast<float *>(smem) + wave * (32 * 64);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 16; ++e) pout[(u * 16 + e) * 64 + lane] = o[2 * (1 - K) + u][e];
    };
    if (ks == 0) hand_over(integral_constant<int, 0>{});
    else hand_over(integral_constant<int, 1>{});
    part_ml[(2 * wave) * 64 + lane] = M;
    part_ml[(2 * wave + 1) * 64 + lane] = l;
    __syncthreads();
    auto finish = [&](auto KSC) {
        constexpr int K = decltype(KSC)::value;
        const int pw = wave ^ 4;                           // the partner: the other key half
        const float Mp = part_ml[(2 * pw) * 64 + lane];
        const float lp = part_ml[(2 * pw + 1) * 64 + lane];
        const float M0 = K ? Mp : M, M1 = K ? M : Mp;     // key half 0 first: identical sums
        const float mm = fmaxf(M0, M1);
        const float a0 = __builtin_amdgcn_exp2f(M0 - mm), a1 = __builtin_amdgcn_exp2f(M1 - mm);
        const float lt = fmaf(K ? lp : l, a0, (K ? l : lp) * a1);
        const float as = K ? a1 : a0, ap = K ? a0 : a1;   // own and partner's factor
        const float inv = lt > 0.0f ? a.o_scale / lt : 0.0f;
        const float *pin = reinterpret_cast<const float *>(smem) + pw * (32 * 64);
        const size_t obase = (((size_t)b * a.seq + token) * a.hq + h) * D;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x16 x;
#pragma unroll
            for (int e = 0; e < 16; ++e) x[e] = fmaf(o[2 * K + u][e], as, pin[(u * 16 + e) * 64 + lane] * ap) * inv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * (2 * K + u) + 8 * i + 4 * g32;
                u32x2 v2;
                v2.x = f32_to_bf16_bits(x[4 * i]) | (f32_to_bf16_bits(x[4 * i + 1]) << 16);
                v2.y = f32_to_bf16_bits(x[4 * i + 2]) | (f32_to_bf16_bits(x[4 * i + 3]) << 16);
                *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(a.o) + obase + d0) = v2;
            }
        }
        if (K == 0 && a.lse && g32 == 0)
            a.lse[((size_t)b * a.hq + h) * a.seq + token] = lt > 0.0f ? fmaf(mm, 0.6931471805599453f, logf(lt)) : ninf;
        if (SKIP && K == 0 && a.skipped && g32 == 0) a.skipped[((size_t)b * a.hq + h) * a.seq + token] = nskip;
    };
    if (ks == 0) finish(integral_constant<int, 0>{});
    else finish(integral_constant<int, 1>{});
    };
    const int rows = a.batch * a.hq * a.nb;
    if (SPARSE && (int)blockIdx.x < rows) wcur = mask_word(a, persistent_row(a, blockIdx.x, 0), threadIdx.x);
    for (int r = blockIdx.x, t = 0; r < rows; r += gridDim.x, ++t) {
        const int rn = r + (int)gridDim.x;
        row_body(persistent_row(a, r, t), rn < rows ? persistent_row(a, rn, t + 1) : -1);
        wcur = wnext;
        __syncthreads();
    }
}

// Grid of the persistent attention kernels: one workgroup per compute unit
// of the current device (they use all of a CU's LDS), at most `rows`.  The
// CU count is asked once per device.
__host__ inline unsigned persistent_grid(int rows) {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return (unsigned)(rows < n ? rows : n);
}

// Kernel arguments of one attention call (no online skip).
__host__ inline BsaArgs make_args(const Shape &s, const void *q, const KvView &kv, const uint32_t *mask, void *o, float *lse) {
    BsaArgs a{};
    a.q = static_cast<const char *>(q);
    a.k = static_cast<const char *>(kv.k);
    a.v = static_cast<const char *>(kv.v);
    a.table = kv.table;
    a.page_log2 = kv.page_log2;
    a.pages_per_seq = kv.pages_per_seq;
    a.mask = mask;
    a.o = o;
    a.lse = lse;
    a.batch = s.batch;
    a.seq = s.seq;
    a.hq = s.hq;
    a.hkv = s.hkv;
    a.nb = s.nb;
    a.words = s.words;
    const float qk = s.q_scale * s.k_scale;
    a.tau_eff = s.tau * qk;
    a.c_exp2 = a.tau_eff * 1.4426950408889634f;
    a.o_scale = s.v_scale;
    a.skip_log2 = -__builtin_huge_valf();
    a.skipped = nullptr;
    return a;
}

}  // namespace
}  // namespace stem
