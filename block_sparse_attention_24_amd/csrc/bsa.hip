// Causal block-sparse flash attention for prefill (Stem article on cn486.com,
// §二.2.2 "BSA operator optimisation": per Q tile the block mask is staged in
// on-chip memory and the list of KV blocks to compute is built before the
// loop; the inner loop visits only those blocks and is the dense loop; a
// skipped block is equivalent to -inf scores).  The dense causal kernel used
// as the baseline (§二.3) is the same template without any mask logic.
//
// Design for gfx950 (wave64, 32x32 MFMA, 160 KiB LDS):
//   * One workgroup per (batch, head, query block I); BLK/32 waves, each wave
//     owns 32 query rows.  Workgroups run heaviest-first (I descending), and
//     the heads that share a KV head are spread so that they land on one XCD
//     (workgroup ids go round-robin over the 8 XCDs), to reuse K/V in its L2.
//   * S^T = K Q^T on MFMA (keys are the M dimension), so after the MFMA every
//     lane holds one query's scores: the row max needs one cross-lane swap
//     (lane ^ 32) and the running sum none until the end.
//   * O^T += V^T P^T: the probabilities stay in registers as the B operand.
//     The K rows are fed to the first MFMA in a permuted order chosen so that
//     the keys a lane holds afterwards are contiguous in V^T, making every
//     LDS read a 16-byte vector read.
//   * K is staged in LDS as [key][d], V transposed as [d][key] (a register
//     transpose on the way in); 16-byte chunks are XOR-swizzled by row to
//     keep the vector reads bank-conflict free.  Two LDS stages: the next
//     block's global loads are in flight while the current one is computed.
//   * bf16: v_mfma_f32_32x32x16_bf16; fp8 (OCP E4M3): v_mfma_f32_32x32x64_f8f6f4
//     with P scaled by 256 before its fp8 cast; fp32: v_mfma_f32_32x32x2f32.
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
};

template <int DT, int D, int BLK>
struct Geo {
    static constexpr int ES = DT == kF32 ? 4 : DT == kBF16 ? 2 : 1;
    static constexpr int NW = BLK / 32;
    static constexpr int NT = NW * 64;
    static constexpr int KROWB = D * ES;
    static constexpr int KCH = KROWB / 16;
    static constexpr int KSWZ = (KCH < 16 ? KCH : 16) - 1;
    static constexpr int TILEB = BLK * D * ES;
    static constexpr bool VT = DT != kF32;            // V stored transposed
    static constexpr int VROWB = VT ? BLK * ES : D * ES;
    static constexpr int VCH = VROWB / 16;
    static constexpr int VSWZ = (VCH < 16 ? VCH : 16) - 1;
    static constexpr int STAGES = (2 * 2 * TILEB <= 128 * 1024) ? 2 : 1;
    static constexpr int NTILE = BLK / 32;            // 32-key tiles per block
    static constexpr int NDT = D / 32;                // 32-wide d tiles of O
    static constexpr int NKC = BLK * KCH / NT;        // K 16-byte chunks per thread
    static constexpr int NSUB = BLK * D / 64;         // 8x8 V sub-tiles per block
    static constexpr int NVI = (NSUB + NT - 1) / NT;  // V sub-tiles per thread
    static constexpr int LIST = 4096;                 // max blocks per row
};

// Key (within the block) that MFMA row r of 32-key tile t stands for.
template <int DT>
__device__ __forceinline__ int keymap(int t, int r) {
    const int i = r >> 3, gg = (r >> 2) & 1, j = r & 3;
    if constexpr (DT == kBF16) return 32 * t + 16 * (i >> 1) + 8 * gg + 4 * (i & 1) + j;
    else if constexpr (DT == kFP8) return 64 * (t >> 1) + 32 * gg + 16 * (t & 1) + 4 * i + j;
    else return 32 * t + r;
}

template <class G>
__device__ __forceinline__ int k_off(int key, int chunk) {
    return key * G::KROWB + ((chunk ^ (key & G::KSWZ)) << 4);
}
template <class G>
__device__ __forceinline__ int v_off(int row, int chunk) {
    return row * G::VROWB + ((chunk ^ (row & G::VSWZ)) << 4);
}

template <int D, int ES, bool PAGED>
__device__ __forceinline__ const char *kv_row(const char *base, const BsaArgs &a, int b, int tok, int g) {
    size_t row;
    if constexpr (PAGED) {
        const int page = a.table[(size_t)b * a.pages_per_seq + (tok >> a.page_log2)];
        row = ((size_t)page << a.page_log2) + (tok & ((1 << a.page_log2) - 1));
    } else {
        row = (size_t)b * a.seq + tok;
    }
    return base + (row * a.hkv + g) * (size_t)(D * ES);
}

// Registers holding one K (or V) block on its way from HBM to LDS.  K and V
// are staged at different points of the loop so that only one is live.
template <class G>
struct KStage {
    uint4 k[G::NKC];
};
template <int DT, class G>
struct VStage {
    uint4 v[DT == kF32 ? G::NKC : G::NVI * 8];        // fp8 uses the low 8 bytes
};

template <int DT, int D, int BLK, bool PAGED>
__device__ __forceinline__ void load_k(KStage<Geo<DT, D, BLK>> &st, const BsaArgs &a, int b, int g, int J,
                                       int tid) {
    using G = Geo<DT, D, BLK>;
    const int tok0 = J * BLK;
#pragma unroll
    for (int i = 0; i < G::NKC; ++i) {
        const int qid = tid + G::NT * i;
        const int key = qid / G::KCH, c = qid % G::KCH;
        st.k[i] = *reinterpret_cast<const uint4 *>(kv_row<D, G::ES, PAGED>(a.k, a, b, tok0 + key, g) + c * 16);
    }
}

template <int DT, int D, int BLK, bool PAGED>
__device__ __forceinline__ void load_v(VStage<DT, Geo<DT, D, BLK>> &st, const BsaArgs &a, int b, int g, int J,
                                       int tid) {
    using G = Geo<DT, D, BLK>;
    const int tok0 = J * BLK;
    if constexpr (DT == kF32) {
#pragma unroll
        for (int i = 0; i < G::NKC; ++i) {
            const int qid = tid + G::NT * i;
            const int key = qid / G::KCH, c = qid % G::KCH;
            st.v[i] = *reinterpret_cast<const uint4 *>(kv_row<D, G::ES, PAGED>(a.v, a, b, tok0 + key, g) + c * 16);
        }
    } else {
#pragma unroll
        for (int s = 0; s < G::NVI; ++s) {
            const int sub = tid + G::NT * s;
            if (sub < G::NSUB) {
                const int kg = sub % (BLK / 8), dc = sub / (BLK / 8);
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const char *p = kv_row<D, G::ES, PAGED>(a.v, a, b, tok0 + 8 * kg + r, g) + dc * 8 * G::ES;
                    if constexpr (DT == kBF16) {
                        st.v[8 * s + r] = *reinterpret_cast<const uint4 *>(p);
                    } else {
                        const uint2 u = *reinterpret_cast<const uint2 *>(p);
                        st.v[8 * s + r] = make_uint4(u.x, u.y, 0u, 0u);
                    }
                }
            }
        }
    }
}

__device__ __forceinline__ uint32_t word_of(const uint4 &u, int w) {
    return w == 0 ? u.x : w == 1 ? u.y : w == 2 ? u.z : u.w;
}

template <int DT, int D, int BLK>
__device__ __forceinline__ void store_k(const KStage<Geo<DT, D, BLK>> &st, char *kl, int tid) {
    using G = Geo<DT, D, BLK>;
#pragma unroll
    for (int i = 0; i < G::NKC; ++i) {
        const int qid = tid + G::NT * i;
        const int key = qid / G::KCH, c = qid % G::KCH;
        *reinterpret_cast<uint4 *>(kl + k_off<G>(key, c)) = st.k[i];
    }
}

template <int DT, int D, int BLK>
__device__ __forceinline__ void store_v(const VStage<DT, Geo<DT, D, BLK>> &st, char *vl, int tid) {
    using G = Geo<DT, D, BLK>;
    if constexpr (DT == kF32) {
#pragma unroll
        for (int i = 0; i < G::NKC; ++i) {
            const int qid = tid + G::NT * i;
            const int key = qid / G::KCH, c = qid % G::KCH;
            *reinterpret_cast<uint4 *>(vl + v_off<G>(key, c)) = st.v[i];
        }
    } else {
#pragma unroll
        for (int s = 0; s < G::NVI; ++s) {
            const int sub = tid + G::NT * s;
            if (sub < G::NSUB) {
                const int kg = sub % (BLK / 8), dc = sub / (BLK / 8);
                const uint4 *in = &st.v[8 * s];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int d = 8 * dc + i;
                    if constexpr (DT == kBF16) {
                        // keys 8kg..8kg+7 of column d: pairs of bf16 halves
                        const int w = i >> 1;
                        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
                        uint4 o;
                        o.x = __builtin_amdgcn_perm(word_of(in[1], w), word_of(in[0], w), sel);
                        o.y = __builtin_amdgcn_perm(word_of(in[3], w), word_of(in[2], w), sel);
                        o.z = __builtin_amdgcn_perm(word_of(in[5], w), word_of(in[4], w), sel);
                        o.w = __builtin_amdgcn_perm(word_of(in[7], w), word_of(in[6], w), sel);
                        *reinterpret_cast<uint4 *>(vl + v_off<G>(d, kg)) = o;
                    } else {
                        // byte i of each of the 8 key rows
                        const int w = i >> 2, bsel = i & 3;
                        const uint32_t sel = (uint32_t)bsel | ((uint32_t)(4 + bsel) << 8) | 0x0c0c0000u;
                        const uint32_t x01 = __builtin_amdgcn_perm(word_of(in[1], w), word_of(in[0], w), sel);
                        const uint32_t x23 = __builtin_amdgcn_perm(word_of(in[3], w), word_of(in[2], w), sel);
                        const uint32_t x45 = __builtin_amdgcn_perm(word_of(in[5], w), word_of(in[4], w), sel);
                        const uint32_t x67 = __builtin_amdgcn_perm(word_of(in[7], w), word_of(in[6], w), sel);
                        uint2 o;
                        o.x = __builtin_amdgcn_perm(x23, x01, 0x05040100u);
                        o.y = __builtin_amdgcn_perm(x67, x45, 0x05040100u);
                        *reinterpret_cast<uint2 *>(vl + v_off<G>(d, kg >> 1) + ((kg & 1) << 3)) = o;
                    }
                }
            }
        }
    }
}

// Q operand of S^T = K Q^T for this lane's query row.
template <int DT, int D>
struct QFrag {
    static constexpr int N = DT == kF32 ? D / 2 : DT == kBF16 ? D / 16 : D / 32;
    uint4 u[DT == kF32 ? 1 : N];
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
        for (int s = 0; s < D / 16; ++s) qf.u[s] = *reinterpret_cast<const uint4 *>(qrow + (16 * s + 8 * g) * 2);
    } else {
#pragma unroll
        for (int s = 0; s < D / 64; ++s) {
            qf.u[2 * s] = *reinterpret_cast<const uint4 *>(qrow + 64 * s + 32 * g);
            qf.u[2 * s + 1] = *reinterpret_cast<const uint4 *>(qrow + 64 * s + 32 * g + 16);
        }
    }
}

template <int DT, int D, int BLK>
__device__ __forceinline__ void qk_tile(f32x16 &acc, const QFrag<DT, D> &qf, const char *kl, int t, int lane) {
    using G = Geo<DT, D, BLK>;
    const int r = lane & 31, g = lane >> 5;
    const int key = keymap<DT>(t, r);
    if constexpr (DT == kBF16) {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const uint4 a = *reinterpret_cast<const uint4 *>(kl + k_off<G>(key, 2 * s + g));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, qf.u[s]), acc, 0, 0, 0);
        }
    } else if constexpr (DT == kFP8) {
#pragma unroll
        for (int s = 0; s < D / 64; ++s) {
            const uint4 a0 = *reinterpret_cast<const uint4 *>(kl + k_off<G>(key, 4 * s + 2 * g));
            const uint4 a1 = *reinterpret_cast<const uint4 *>(kl + k_off<G>(key, 4 * s + 2 * g + 1));
            i32x8 av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            const uint4 b0 = qf.u[2 * s], b1 = qf.u[2 * s + 1];
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
}

// O^T[dt] += V^T P^T over the whole block.
template <int DT, int D, int BLK>
__device__ __forceinline__ void pv_block(f32x16 (&o)[D / 32], const f32x16 (&p)[BLK / 32], const char *vl,
                                         int lane) {
    using G = Geo<DT, D, BLK>;
    const int r = lane & 31, g = lane >> 5;
    if constexpr (DT == kBF16) {
#pragma unroll
        for (int t = 0; t < G::NTILE; ++t) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                bf16x8 bv;
#pragma unroll
                for (int e = 0; e < 8; ++e) bv[e] = (__bf16)p[t][8 * hh + e];
#pragma unroll
                for (int dt = 0; dt < G::NDT; ++dt) {
                    const uint4 a = *reinterpret_cast<const uint4 *>(vl + v_off<G>(32 * dt + r, 4 * t + 2 * hh + g));
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), bv, o[dt], 0, 0, 0);
                }
            }
        }
    } else if constexpr (DT == kFP8) {
#pragma unroll
        for (int pp = 0; pp < G::NTILE / 2; ++pp) {
            i32x8 bv;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const int e = 4 * w;
                const f32x16 &src = p[2 * pp + (e >> 4)];
                const int ee = e & 15;
                int x = __builtin_amdgcn_cvt_pk_fp8_f32(src[ee] * 256.0f, src[ee + 1] * 256.0f, 0, false);
                x = __builtin_amdgcn_cvt_pk_fp8_f32(src[ee + 2] * 256.0f, src[ee + 3] * 256.0f, x, true);
                bv[w] = x;
            }
#pragma unroll
            for (int dt = 0; dt < G::NDT; ++dt) {
                const int row = 32 * dt + r;
                const uint4 a0 = *reinterpret_cast<const uint4 *>(vl + v_off<G>(row, 4 * pp + 2 * g));
                const uint4 a1 = *reinterpret_cast<const uint4 *>(vl + v_off<G>(row, 4 * pp + 2 * g + 1));
                i32x8 av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                o[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, o[dt], 0, 0, 0, 0, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < G::NTILE; ++t) {
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) {
                const int key = keymap<DT>(t, 8 * (vv >> 2) + 4 * g + (vv & 3));
#pragma unroll
                for (int dt = 0; dt < G::NDT; ++dt) {
                    const int d = 32 * dt + r;
                    const float a = *reinterpret_cast<const float *>(vl + v_off<G>(key, d >> 2) + (d & 3) * 4);
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[t][vv], o[dt], 0, 0, 0);
                }
            }
        }
    }
}

template <int DT, int D, int BLK, bool SPARSE, bool PAGED>
__global__ __launch_bounds__(2 * BLK, 1) void bsa_kernel(BsaArgs a) {
    using G = Geo<DT, D, BLK>;
    __shared__ __attribute__((aligned(16))) char smem[G::STAGES * 2 * G::TILEB];
    __shared__ uint16_t list[SPARSE ? G::LIST : 1];
    __shared__ int wave_sum[G::NW];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g32 = lane >> 5;

    // heaviest query blocks first; the heads of one KV group on one XCD
    const int wg = blockIdx.x;
    const int qidx = wg / a.hq, j = wg % a.hq;
    const int I = a.nb - 1 - qidx / a.batch;
    const int b = qidx % a.batch;
    const int h = (a.hq % 8 == 0) ? (j % 8) * (a.hq / 8) + j / 8 : j;
    const int g = h / (a.hq / a.hkv);

    // ---- kept-block list, built once before the loop -------------------------
    int n;
    if constexpr (SPARSE) {
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
        int base = 0;
#pragma unroll
        for (int k = 0; k < G::NW; ++k) base += k < wave ? wave_sum[k] : 0;
        n = 0;
#pragma unroll
        for (int k = 0; k < G::NW; ++k) n += wave_sum[k];
        int pos = base + incl - cnt;
        while (w) {
            const int bit = __builtin_ctz(w);
            list[pos++] = (uint16_t)(32 * tid + bit);
            w &= w - 1;
        }
        __syncthreads();
    } else {
        n = I + 1;
    }

    const int qrow = 32 * wave + (lane & 31);               // query row in the block
    const int token = I * BLK + qrow;
    if (n == 0) {                                         // nothing visible: O = 0, LSE = -inf
        if constexpr (DT == kF32) {
            float *op = reinterpret_cast<float *>(a.o) + (((size_t)b * a.seq + token) * a.hq + h) * D;
            for (int d = g32; d < D; d += 2) op[d] = 0.0f;
        } else {
            uint16_t *op = reinterpret_cast<uint16_t *>(a.o) + (((size_t)b * a.seq + token) * a.hq + h) * D;
            for (int d = g32; d < D; d += 2) op[d] = 0;
        }
        if (a.lse && g32 == 0) a.lse[((size_t)b * a.hq + h) * a.seq + token] = -__builtin_huge_valf();
        return;
    }

    QFrag<DT, D> qf;
    load_q<DT, D>(qf, a.q + (((size_t)b * a.seq + token) * a.hq + h) * (size_t)(D * G::ES), g32);

    f32x16 o[G::NDT];
#pragma unroll
    for (int dt = 0; dt < G::NDT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] = 0.0f;
    float m = -__builtin_huge_valf();
    float l = 0.0f;
    const float c = a.c_exp2;

    KStage<G> kst;
    VStage<DT, G> vst;
    {
        const int J0 = SPARSE ? (int)list[0] : 0;
        load_k<DT, D, BLK, PAGED>(kst, a, b, g, J0, tid);
        load_v<DT, D, BLK, PAGED>(vst, a, b, g, J0, tid);
        store_k<DT, D, BLK>(kst, smem, tid);
        store_v<DT, D, BLK>(vst, smem + G::TILEB, tid);
    }
    __syncthreads();

    for (int it = 0; it < n; ++it) {
        const int J = SPARSE ? (int)list[it] : it;
        const bool more = it + 1 < n;
        // the last iteration re-fetches its own block so that loads stay unconditional
        const int Jn = more ? (SPARSE ? (int)list[it + 1] : it + 1) : J;
        const int cur = G::STAGES == 2 ? (it & 1) : 0;
        const char *kl = smem + cur * 2 * G::TILEB;
        const char *vl = kl + G::TILEB;
        char *kn = smem + (G::STAGES == 2 ? ((it + 1) & 1) : 0) * 2 * G::TILEB;
        load_k<DT, D, BLK, PAGED>(kst, a, b, g, Jn, tid);   // in flight during S = K Q^T

        f32x16 s[G::NTILE];
#pragma unroll
        for (int t = 0; t < G::NTILE; ++t) {
#pragma unroll
            for (int e = 0; e < 16; ++e) s[t][e] = 0.0f;
            qk_tile<DT, D, BLK>(s[t], qf, kl, t, lane);
        }
        if (J == I) {                                     // causal mask inside the diagonal block
#pragma unroll
            for (int t = 0; t < G::NTILE; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = keymap<DT>(t, 8 * (e >> 2) + 4 * g32 + (e & 3));
                    if (key > qrow) s[t][e] = -__builtin_huge_valf();
                }
        }
        if constexpr (G::STAGES == 2) {                   // next stage is free: store K, fetch V
            if (more) store_k<DT, D, BLK>(kst, kn, tid);
            load_v<DT, D, BLK, PAGED>(vst, a, b, g, Jn, tid);
        }
        float mx = -__builtin_huge_valf();
#pragma unroll
        for (int t = 0; t < G::NTILE; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[t][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
        const float mc = m_new * c;
        float ls = 0.0f;
#pragma unroll
        for (int t = 0; t < G::NTILE; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float pe = __builtin_amdgcn_exp2f(fmaf(s[t][e], c, -mc));
                s[t][e] = pe;
                ls += pe;
            }
        l = fmaf(l, alpha, ls);
        m = m_new;
#pragma unroll
        for (int dt = 0; dt < G::NDT; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
        pv_block<DT, D, BLK>(o, s, vl, lane);

        if (more) {
            if constexpr (G::STAGES == 1) {
                __syncthreads();                          // everyone is done with the only stage
                store_k<DT, D, BLK>(kst, kn, tid);
                load_v<DT, D, BLK, PAGED>(vst, a, b, g, Jn, tid);
            }
            store_v<DT, D, BLK>(vst, kn + G::TILEB, tid);
            __syncthreads();
        }
    }

    // ---- epilogue --------------------------------------------------------------
    const float lt = l + __shfl_xor(l, 32);
    const float inv = lt > 0.0f ? a.o_scale / lt : 0.0f;
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
                uint2 u;
                u.x = f32_to_bf16_bits(x0) | (f32_to_bf16_bits(x1) << 16);
                u.y = f32_to_bf16_bits(x2) | (f32_to_bf16_bits(x3) << 16);
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.o) + obase + d0) = u;
            }
        }
    if (a.lse && g32 == 0)
        a.lse[((size_t)b * a.hq + h) * a.seq + token] =
            lt > 0.0f ? fmaf(m, a.tau_eff, logf(lt)) : -__builtin_huge_valf();
}

template <int DT, int D, int BLK>
hipError_t launch_cfg(const BsaArgs &a, bool sparse, hipStream_t st) {
    using G = Geo<DT, D, BLK>;
    const dim3 grid((unsigned)(a.batch * a.hq * a.nb));
    const bool paged = a.table != nullptr;
    if (sparse && paged) hipLaunchKernelGGL((bsa_kernel<DT, D, BLK, true, true>), grid, dim3(G::NT), 0, st, a);
    else if (sparse) hipLaunchKernelGGL((bsa_kernel<DT, D, BLK, true, false>), grid, dim3(G::NT), 0, st, a);
    else if (paged) hipLaunchKernelGGL((bsa_kernel<DT, D, BLK, false, true>), grid, dim3(G::NT), 0, st, a);
    else hipLaunchKernelGGL((bsa_kernel<DT, D, BLK, false, false>), grid, dim3(G::NT), 0, st, a);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const Shape &s, const BsaArgs &a, bool sparse, hipStream_t st) {
    if (s.d == 64 && s.blk == 64) return launch_cfg<DT, 64, 64>(a, sparse, st);
    if (s.d == 64 && s.blk == 128) return launch_cfg<DT, 64, 128>(a, sparse, st);
    if (s.d == 128 && s.blk == 64) return launch_cfg<DT, 128, 64>(a, sparse, st);
    return launch_cfg<DT, 128, 128>(a, sparse, st);
}

}  // namespace

hipError_t launch_bsa(const Shape &s, const void *q, const KvView &kv, const uint32_t *mask, void *o,
                      float *lse, hipStream_t st) {
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
    a.o_scale = s.dtype == STEM_FP8_E4M3 ? s.v_scale / 256.0f : s.v_scale;
    const bool sparse = mask != nullptr;
    switch (s.dtype) {
        case STEM_F32: return launch_dt<kF32>(s, a, sparse, st);
        case STEM_BF16: return launch_dt<kBF16>(s, a, sparse, st);
        default: return launch_dt<kFP8>(s, a, sparse, st);
    }
}

}  // namespace stem
