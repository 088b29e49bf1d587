// One decode step of Stem block-sparse attention over the KV cache: the new
// token of every sequence scores the cache's complete blocks with the OAM
// metric (Stem article on cn486.com, §一.3.2; the token is its own query
// representation), keeps the sink block, its own (current) block and the best
// of the rest under the row's TPD budget (§一.3.1, §二.2.1), and attends to the
// keys of the kept blocks only, reading nothing else of the cache (the
// memory-bound decode case of the BLASST summary, §2.3: skipped blocks cost
// no HBM traffic).
//
// Kernels:
//   dec_score_kernel    the candidates' scores, as order-preserving keys:
//                       64 rows of one KV head per workgroup, scored for
//                       every query head of its group.
//   dec_select_kernel   one wave per (b, h) finds the top-k by a bitwise
//                       search for the k-th largest key (equal scores to the
//                       smaller J) and writes the kept list in ascending J.
//   dec_attn_kernel     split-K: a workgroup takes four consecutive kept
//                       blocks, one per wave; each wave streams its block's K
//                       and V rows once (16-byte chunks, one row per
//                       d*ES/16 lanes), and the four partial softmaxes are
//                       merged in wave order.
//   dec_combine_kernel  one workgroup per (b, h) merges the splits (four
//                       contiguous quarters, then the quarters in order).
// With BLASST's online skip (gist.science summary, §2.1 running-maximum
// pruning; §2.3: in decode the skip saves the V loads) the attention runs in
// two passes around a scan, so that the V rows of a dropped block are never
// read:
//   dec_attn_kernel<QK> each wave reads its block's K rows and writes the
//                       block's scores and their maximum (log2 units);
//   dec_prefix_kernel   one wave per (b, h): in ascending J, a block is
//                       dropped when its maximum lies more than
//                       log2(1/lambda) below the largest maximum of the
//                       earlier kept blocks; the entries not dropped are
//                       listed in order;
//   dec_attn_kernel<PV> split-K over that list: each wave forms P from its
//                       block's stored scores and reads the block's V rows
//                       (workgroups past the list exit at once), and
//                       dec_combine_kernel merges those splits.
// lambda = 0 drops nothing and runs the plain step.
// Every sum has a fixed order, so results are bit-reproducible.
#include "device_common.h"
#include "stem_internal.h"

namespace stem {
namespace {

constexpr int kSplit = 4;             // kept blocks per attention workgroup (one per wave)
enum { kFull = 0, kQK = 1, kPV = 2 };    // attention passes (kQK, kPV: with the online skip)
constexpr float kLog2e = 1.4426950408889634f;

// Orders LDS traffic between the lanes of one wave (no workgroup barrier).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct DecArgs {
    const char *q;                    // [b, hq, d]
    const char *k, *v;                // cache
    const int32_t *table;
    int page_log2, pages_per_seq;
    const int32_t *seq_lens, *keep;   // [b]; keep may be null (dense)
    const float *kbar, *lvn;          // [b, hkv, nb, d], [b, hkv, nb] (lvn null: no value term)
    int32_t *lists;                   // [b, hq, nb]
    int32_t *counts;                  // [b, hq]
    float *part;                      // [b, hq, nsplit, d + 2]
    uint32_t *keys;                   // [b, hq, nb] order keys of the candidate scores
    void *o;                          // [b, hq, d]
    float *lse;                       // [b, hq] or null
    // online skip only
    float *bmax;                      // [b, hq, nb] maximum score of each kept entry (log2 units)
    float *scores;                    // [b, hq, nb, blk] its scores (log2 units)
    int32_t *live;                    // [b, hq, nb] the entries not dropped, ascending
    int32_t *nlive;                   // [b, hq] their number
    int32_t *skipped;                 // [b, hq] dropped entries, or null
    float skip_log2;                  // log2(lambda)
    int hq, hkv, d, blk, nb, seq, nsplit;
    int off32;                        // K/V byte offsets fit in 32 bits
    float q_scale, k_scale, v_scale, tau;
};

__device__ __forceinline__ int seq_len_of(const DecArgs &a, int b) {
    return min(max(a.seq_lens[b], 1), a.seq);      // clamped into [1, capacity]
}

// Element e of the new token's query (dequantised).
template <int ES>
__device__ __forceinline__ float q_elem(const DecArgs &a, size_t idx) {
    if constexpr (ES == 4) return reinterpret_cast<const float *>(a.q)[idx];
    else if constexpr (ES == 2) return bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(a.q)[idx]);
    else return __builtin_amdgcn_cvt_f32_fp8((int)(uint8_t)a.q[idx], 0) * a.q_scale;
}

// ---------------------------------------------------------------------------
// Scores and selection
// ---------------------------------------------------------------------------
// Budget of the new token's row: k = keep clamped to [|{0, I}|, I + 1].
struct RowPlan {
    int t, I, kk, want, ncand;
};
__device__ __forceinline__ RowPlan row_plan(const DecArgs &a, int b) {
    RowPlan p;
    p.t = seq_len_of(a, b) - 1;                     // position of the new token
    p.I = p.t / a.blk;                              // its block
    const int forced = p.I == 0 ? 1 : 2;
    p.kk = a.keep ? min(max(a.keep[b], forced), p.I + 1) : p.I + 1;
    p.want = p.kk - forced;                         // candidates J in [1, I-1] to keep
    p.ncand = p.I > 1 ? p.I - 1 : 0;
    return p;
}

// Scores of the candidates J in [1, I-1]: a row of kbar is read by D/4 lanes
// (one 16-byte piece each), so a wave covers 256/D rows per load, U loads in
// flight per lane.  A workgroup scores kScoreRows rows of one KV head for
// every query head of its group: each kbar row is read once, and for each
// head the dot product is finished by a butterfly over the row's lanes.
constexpr int kScoreRows = 64;
constexpr int kScoreHeads = 64;                      // query heads staged in LDS at a time
template <int ES, int D>
__global__ __launch_bounds__(256) void dec_score_kernel(DecArgs a) {
    constexpr int LPR = D / 4;                      // lanes per kbar row
    constexpr int RPW = kWave / LPR;                // rows per wave and load
    constexpr int STEP = 4 * RPW;                   // rows per workgroup and load
    constexpr int U = kScoreRows / STEP;            // loads per lane
    const int g = blockIdx.y, b = blockIdx.z;
    const RowPlan rp = row_plan(a, b);
    const int j0 = 1 + blockIdx.x * kScoreRows;
    if (rp.want >= rp.ncand || j0 >= rp.I) return;  // no selection, or no rows here
    const int I = rp.I;
    const int G = a.hq / a.hkv;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int sub = lane / LPR, piece = lane % LPR;
    const float *kb = a.kbar + ((size_t)b * a.hkv + g) * a.nb * D + 4 * piece;
    const float *lv = a.lvn ? a.lvn + ((size_t)b * a.hkv + g) * a.nb : nullptr;
    __shared__ f32x4 qs[kScoreHeads * (D / 4)];    // the group's queries, dequantised
    f32x4 x[U];
    float lj[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int jc = min(j0 + u * STEP + wave * RPW + sub, I - 1);   // past the end: a valid row
        x[u] = *reinterpret_cast<const f32x4 *>(kb + (size_t)jc * D);
        lj[u] = lv ? lv[jc] : 0.0f;
    }
    for (int h0 = 0; h0 < G; h0 += kScoreHeads) {
        const int nh = min(kScoreHeads, G - h0);
        if (h0 > 0) __syncthreads();                // the previous heads' queries are read
        for (int i = tid; i < nh * (D / 4); i += 256) {
            const size_t base = ((size_t)b * a.hq + g * G + h0 + i / (D / 4)) * D + 4 * (i % (D / 4));
            qs[i] = f32x4{q_elem<ES>(a, base), q_elem<ES>(a, base + 1), q_elem<ES>(a, base + 2),
                          q_elem<ES>(a, base + 3)};
        }
        __syncthreads();
        for (int hh = 0; hh < nh; ++hh) {
            const int h = g * G + h0 + hh;
            const f32x4 qv = qs[hh * (D / 4) + piece];
            uint32_t *keys = a.keys + ((size_t)b * a.hq + h) * a.nb;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = j0 + u * STEP + wave * RPW + sub;
                const float acc =
                    sum_lanes<LPR>(fmaf(qv[3], x[u][3], fmaf(qv[2], x[u][2], fmaf(qv[1], x[u][1], qv[0] * x[u][0]))));
                if (piece == 0 && j < I) keys[j] = order_key(fmaf(acc, a.tau, lj[u]));
            }
        }
    }
}

// Selection, one wave per (b, h): the keys of J = 64 c + lane in registers
// (MAXC chunks; J outside [1, I-1] hold key 0), the threshold of the top-k by
// topk_threshold (equal keys to the smaller J); the kept list is written in
// ascending J.
template <int MAXC>
__global__ __launch_bounds__(64) void dec_select_kernel(DecArgs a) {
    __shared__ uint32_t buf[64];
    const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const RowPlan rp = row_plan(a, b);
    const int I = rp.I, want = rp.want;
    int32_t *lrow = a.lists + ((size_t)b * a.hq + h) * a.nb;
    if (lane == 0) {
        a.counts[(size_t)b * a.hq + h] = rp.kk;
        if (a.skipped && !a.bmax) a.skipped[(size_t)b * a.hq + h] = 0;   // lambda = 0: nothing dropped
    }
    if (want >= rp.ncand) {                         // every block up to I
        for (int j = lane; j <= I; j += kWave) lrow[j] = j;
        return;
    }
    const uint32_t *keys = a.keys + ((size_t)b * a.hq + h) * a.nb;
    uint32_t key[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int j = c * 64 + lane;
        key[c] = (j >= 1 && j < I) ? keys[j] : 0u;
    }
    uint32_t th = 0u;
    int need_eq = 0;
    bool all_eq = true;
    if (want > 0) topk_threshold<MAXC>(key, I, want, rp.ncand, buf, lane, th, need_eq, all_eq);
    int run_eq = 0, run_keep = 0;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        if (c <= (I >> 6)) {                        // uniform; keeps the loop fully unrolled
            const int j = c * 64 + lane;
            const bool valid = j >= 1 && j < I;
            bool keep = false;
            if (want > 0) {
                const bool eq = valid && key[c] == th;
                const uint64_t eqm = ballot64(eq);
                keep = valid && (key[c] > th || (eq && run_eq + lanes_below(eqm) < need_eq));
                run_eq += __popcll(eqm);
            }
            keep = keep || j == 0 || j == I;
            const uint64_t km = ballot64(keep);
            if (keep) lrow[run_keep + lanes_below(km)] = j;
            run_keep += __popcll(km);
        }
    }
}

// ---------------------------------------------------------------------------
// Split-K attention over the kept blocks
// ---------------------------------------------------------------------------
// fp8 with 32-bit offsets fits in 80 registers: six workgroups per CU (more
// workgroups in flight beat a deeper ring of loads per lane: 8 in flight at
// five per CU and 16 at four were slower)
template <int ES, int D, int BLK, int MODE, typename OFF>
__global__ __launch_bounds__(256, (ES == 1 && sizeof(OFF) == 4) ? 6 : 1) void dec_attn_kernel(DecArgs a) {
    constexpr int CPR = D * ES / 16;                // 16-byte chunks per K/V row
    constexpr int RPP = kWave / CPR;                // rows per pass
    constexpr int EPC = 16 / ES;                    // elements per chunk
    constexpr int NP = BLK / RPP;                   // passes over the block's rows
    constexpr int TOT = MODE == kFull ? 2 * NP : NP;   // K passes, then V passes (or one of them)
    constexpr int RING = ES == 1 ? 4 : 8;           // loads in flight per lane (fp8: see above)
    constexpr int DIST = TOT < RING ? TOT : RING;
    __shared__ float ps[kSplit][BLK];               // scores, then P, of each wave's block
    __shared__ float ml[kSplit][2];
    __shared__ float os[kSplit][D];
    // Renumbering: in the order (b, g, split, head of the group) each XCD
    // (workgroup id mod 8) takes a contiguous eighth, so the heads of a KV
    // group run side by side on one XCD and share the blocks they all keep
    // through its L2.
    const unsigned n = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const unsigned total = gridDim.x * gridDim.y * gridDim.z;
    const unsigned m = (total & 7u) ? n : (n & 7u) * (total >> 3) + (n >> 3);
    const int G = a.hq / a.hkv;
    const int hh = (int)(m % G);
    const int s = (int)((m / G) % gridDim.x);
    const int bg = (int)(m / (G * gridDim.x));     // b * hkv + g
    const int g = bg % a.hkv, b = bg / a.hkv;
    const int h = g * G + hh;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int slot = s * kSplit + wave;             // this wave's place in the list it walks
    const size_t row_list = ((size_t)b * a.hq + h) * a.nb;
    // The entry of the list this wave walks is read before the count is known,
    // at an index clamped into the row (a value past the count is never
    // used), so that the two loads overlap instead of following each other.
    const int first = MODE == kPV ? a.live[row_list + min(slot, a.nb - 1)] : a.lists[row_list + min(slot, a.nb - 1)];
    // the PV pass walks the entries that were not dropped
    const int count = MODE == kPV ? a.nlive[(size_t)b * a.hq + h] : a.counts[(size_t)b * a.hq + h];
    if (s * kSplit >= count) return;                // the whole workgroup exits together
    const int t = seq_len_of(a, b) - 1;
    const int e = MODE == kPV ? (slot < count ? first : 0) : slot;
    const int r = lane / CPR, c = lane % CPR;       // row within a pass, chunk within the row
    const size_t row_bytes = (size_t)a.hkv * D * ES;
    const size_t col = (size_t)g * D * ES + (size_t)c * 16;
    const float ninf = -__builtin_huge_valf();

    float m_w = ninf, l_w = 0.0f;
    float acc[EPC];
#pragma unroll
    for (int i = 0; i < EPC; ++i) acc[i] = 0.0f;
    const size_t ent = ((size_t)b * a.hq + h) * a.nb + e;   // this wave's entry in the skip arrays
    const bool live = slot < count;

    if (live) {
        const int J = MODE == kPV ? a.lists[row_list + e] : first;
        const int tok0 = J * BLK;
        const int nkeys = min(BLK, t - tok0 + 1);
        // this lane's slice of q, scaled so that q.k is in log2 units
        const float qsc = a.tau * a.k_scale * kLog2e;
        float qv[EPC];
#pragma unroll
        for (int i = 0; i < EPC; ++i) qv[i] = q_elem<ES>(a, ((size_t)b * a.hq + h) * D + c * EPC + i) * qsc;
        // byte offset of each pass's row (rows past nkeys read row nkeys-1, then
        // masked).  Paged: the block's page entries (at most BLK/16) are read
        // once, one per lane, and handed to the rows by lane shuffles.
        OFF roff[NP];                                   // 32-bit when the K/V tensors are below 4 GiB
        if (a.table) {
            const int lg = a.page_log2;
            const int pg0 = tok0 >> lg;
            const int npg = ((tok0 + BLK - 1) >> lg) - pg0 + 1;
            const int pg_lane = lane < npg ? a.table[(size_t)b * a.pages_per_seq + pg0 + lane] : 0;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int tok = tok0 + min(p * RPP + r, nkeys - 1);
                const int page = __shfl(pg_lane, (tok >> lg) - pg0);
                roff[p] = (OFF)((((size_t)page << lg) + (tok & ((1 << lg) - 1))) * row_bytes + col);
            }
        } else {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int tok = tok0 + min(p * RPP + r, nkeys - 1);
                roff[p] = (OFF)(((size_t)b * a.seq + tok) * row_bytes + col);
            }
        }
        if constexpr (MODE == kPV) {
            // the scores the QK pass stored, and the block softmax in log2 units
            const float *sc = a.scores + ent * BLK;
#pragma unroll
            for (int k = lane; k < BLK; k += kWave) ps[wave][k] = sc[k];
            wave_sync();
            const float mx = a.bmax[ent];
            float lsum = 0.0f;
#pragma unroll
            for (int k = lane; k < BLK; k += kWave) {
                const float p = __builtin_amdgcn_exp2f(ps[wave][k] - mx);   // 0 for -inf
                ps[wave][k] = p;
                lsum += p;
            }
            lsum = sum_lanes<kWave>(lsum);
            m_w = mx;
            l_w = lsum;
            wave_sync();
        }
        // pass i reads K rows for i < NP (V rows after them); the PV pass reads V only
        auto src_of = [&](int i) { return MODE == kPV ? a.v : (i < NP ? a.k : a.v); };
        uint4 ring[DIST];
        auto issue = [&](int i) {
            ring[i % DIST] = *reinterpret_cast<const uint4 *>(src_of(i) + (size_t)roff[i % NP]);
        };
#pragma unroll
        for (int i = 0; i < DIST; ++i) issue(i);
#pragma unroll
        for (int i = 0; i < TOT; ++i) {
            const uint4 u = ring[i % DIST];
            if (i + DIST < TOT) issue(i + DIST);
            const int row = (i % NP) * RPP + r;
            if (MODE != kPV && i < NP) {
                // scores: one chunk per lane, reduced over the row's CPR lanes
                float kx[EPC];
                widen16<ES>(u, kx);
                float x = 0.0f;
#pragma unroll
                for (int k = 0; k < EPC; ++k) x = fmaf(qv[k], kx[k], x);
                x = sum_lanes<CPR>(x);
                if (c == 0) ps[wave][row] = row < nkeys ? x : ninf;
            } else {
                if (MODE == kFull && i == NP) {
                    // block softmax in log2 units
                    wave_sync();
                    float mx = ninf;
#pragma unroll
                    for (int k = lane; k < BLK; k += kWave) mx = fmaxf(mx, ps[wave][k]);
                    mx = max_lanes<kWave>(mx);
                    float lsum = 0.0f;
#pragma unroll
                    for (int k = lane; k < BLK; k += kWave) {
                        const float p = __builtin_amdgcn_exp2f(ps[wave][k] - mx);   // 0 for -inf
                        ps[wave][k] = p;
                        lsum += p;
                    }
                    lsum = sum_lanes<kWave>(lsum);
                    m_w = mx;
                    l_w = lsum;
                    wave_sync();
                }
                // P V: a lane accumulates its chunk over the rows r, r + RPP, ...
                float vx[EPC];
                widen16<ES>(u, vx);
                const float p = ps[wave][row];
#pragma unroll
                for (int k = 0; k < EPC; ++k) acc[k] = fmaf(p, vx[k], acc[k]);
            }
        }
        if constexpr (MODE == kQK) {
            // the block's scores and their maximum, for the scan and the PV pass
            wave_sync();
            float mx = ninf;
#pragma unroll
            for (int k = lane; k < BLK; k += kWave) mx = fmaxf(mx, ps[wave][k]);
            mx = max_lanes<kWave>(mx);
            float *sc = a.scores + ent * BLK;
#pragma unroll
            for (int k = lane; k < BLK; k += kWave) sc[k] = ps[wave][k];
            if (lane == 0) a.bmax[ent] = mx;
        }
#pragma unroll
        for (int k = 0; k < EPC; ++k) acc[k] = sum_stride<CPR>(acc[k]);
    }
    if constexpr (MODE == kQK) return;
    if (lane < CPR) {
#pragma unroll
        for (int i = 0; i < EPC; ++i) os[wave][lane * EPC + i] = acc[i];
    }
    if (lane == 0) {
        ml[wave][0] = m_w;
        ml[wave][1] = l_w;
    }
    __syncthreads();
    if (wave != 0) return;
    // merge the four blocks in wave order
    float M = ninf;
#pragma unroll
    for (int w = 0; w < kSplit; ++w) M = fmaxf(M, ml[w][0]);
    float L = 0.0f, f[kSplit];
#pragma unroll
    for (int w = 0; w < kSplit; ++w) {
        f[w] = ml[w][0] == ninf ? 0.0f : __builtin_amdgcn_exp2f(ml[w][0] - M);
        L += ml[w][1] * f[w];
    }
    float *dst = a.part + (((size_t)b * a.hq + h) * a.nsplit + s) * (D + 2);
    for (int i = lane; i < D; i += kWave) {
        float x = 0.0f;
#pragma unroll
        for (int w = 0; w < kSplit; ++w) x += os[w][i] * f[w];
        dst[2 + i] = x;
    }
    if (lane == 0) {
        dst[0] = M;
        dst[1] = L;
    }
}

// Online skip, one wave per (b, h): entry e of the kept list (ascending J)
// is dropped when its maximum lies more than log2(1/lambda) below the largest
// maximum of entries 0 .. e-1 (a dropped entry lies below it, so it never
// raises that maximum); entry 0 is never dropped.  A wave takes 64 entries
// at a time: an inclusive max-scan over the lanes, shifted by one lane, plus
// the maximum carried from the entries before.
__global__ __launch_bounds__(64) void dec_prefix_kernel(DecArgs a) {
    const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const size_t bh = (size_t)b * a.hq + h;
    const int n = a.counts[bh];
    const float ninf = -__builtin_huge_valf();
    const float *mx = a.bmax + bh * a.nb;
    int32_t *live = a.live + bh * a.nb;
    float carry = ninf;
    int dropped = 0, kept = 0;
    for (int e0 = 0; e0 < n; e0 += kWave) {
        const int e = e0 + lane;
        const float x = e < n ? mx[e] : ninf;
        float inc = x;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float y = __shfl_up(inc, off);
            if (lane >= off) inc = fmaxf(inc, y);
        }
        float before = __shfl_up(inc, 1);
        before = lane == 0 ? carry : fmaxf(carry, before);   // maximum of entries 0 .. e-1
        const bool d = e < n && x < before + a.skip_log2;
        const uint64_t keepm = ballot64(e < n && !d);
        if (e < n && !d) live[kept + lanes_below(keepm)] = e;   // in ascending order
        kept += __popcll(keepm);
        dropped += __popcll(ballot64(d));
        carry = fmaxf(carry, __shfl(inc, kWave - 1));
    }
    if (lane == 0) {
        a.nlive[bh] = kept;
        if (a.skipped) a.skipped[bh] = dropped;
    }
}

// One workgroup per (b, h): merge the splits.  Each of the four waves sums
// a contiguous quarter of the splits in order; the quarters are then added
// in wave order.  Split weights 2^(m_s - M) go through LDS.
template <int D>
__global__ __launch_bounds__(256) void dec_combine_kernel(DecArgs a, int out_f32) {
    __shared__ float fw[1024];                      // weight of each split (nsplit <= 1024)
    __shared__ float red[4][D + 1];
    __shared__ float mred[4];
    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const size_t bh = (size_t)b * a.hq + h;
    const int ns = ((a.nlive ? a.nlive[bh] : a.counts[bh]) + kSplit - 1) / kSplit;
    const float *src = a.part + bh * a.nsplit * (D + 2);
    const float ninf = -__builtin_huge_valf();
    float m = ninf;
    for (int s = tid; s < ns; s += 256) m = fmaxf(m, src[(size_t)s * (D + 2)]);
    m = max_lanes<kWave>(m);
    if (lane == 0) mred[wave] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(mred[0], mred[1]), fmaxf(mred[2], mred[3]));
    for (int s = tid; s < ns; s += 256) {
        const float ms = src[(size_t)s * (D + 2)];
        fw[s] = ms == ninf ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
    }
    __syncthreads();
    const int q0 = (ns * wave) / 4, q1 = (ns * (wave + 1)) / 4;
    float lsum = 0.0f;
    float acc[D / kWave] = {};
#pragma unroll 4
    for (int s = q0; s < q1; ++s) {
        const float *ps = src + (size_t)s * (D + 2);
        const float f = fw[s];
        lsum += ps[1] * f;
#pragma unroll
        for (int i = 0; i < D / kWave; ++i) acc[i] += ps[2 + lane + kWave * i] * f;
    }
#pragma unroll
    for (int i = 0; i < D / kWave; ++i) red[wave][lane + kWave * i] = acc[i];
    if (lane == 0) red[wave][D] = lsum;
    __syncthreads();
    if (wave) return;
    const float L = ((red[0][D] + red[1][D]) + red[2][D]) + red[3][D];
    const float inv = a.v_scale / L;
#pragma unroll
    for (int i = 0; i < D / kWave; ++i) {
        const int dd = lane + kWave * i;
        const float x = (((red[0][dd] + red[1][dd]) + red[2][dd]) + red[3][dd]) * inv;
        const size_t idx = bh * D + dd;
        if (out_f32) reinterpret_cast<float *>(a.o)[idx] = x;
        else reinterpret_cast<uint16_t *>(a.o)[idx] = (uint16_t)f32_to_bf16_bits(x);
    }
    if (a.lse && lane == 0) a.lse[bh] = (M + log2f(L)) / kLog2e;
}

template <int ES, int D, int BLK>
hipError_t launch_all(const Shape &s, DecArgs &a, bool skip, hipStream_t st) {
    const dim3 heads(s.hq, s.batch);
    const int chunks = (s.nb + 63) / 64;
    hipLaunchKernelGGL((dec_score_kernel<ES, D>), dim3((s.nb + kScoreRows - 1) / kScoreRows, s.hkv, s.batch),
                       dim3(256), 0, st, a);
    if (chunks <= 2) hipLaunchKernelGGL((dec_select_kernel<2>), heads, dim3(64), 0, st, a);
    else if (chunks <= 8) hipLaunchKernelGGL((dec_select_kernel<8>), heads, dim3(64), 0, st, a);
    else if (chunks <= 16) hipLaunchKernelGGL((dec_select_kernel<16>), heads, dim3(64), 0, st, a);
    else if (chunks <= 32) hipLaunchKernelGGL((dec_select_kernel<32>), heads, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((dec_select_kernel<64>), heads, dim3(64), 0, st, a);
    const dim3 splits(a.nsplit, s.hq, s.batch);
    if (skip) {
        if (a.off32) hipLaunchKernelGGL((dec_attn_kernel<ES, D, BLK, kQK, uint32_t>), splits, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((dec_attn_kernel<ES, D, BLK, kQK, size_t>), splits, dim3(256), 0, st, a);
        hipLaunchKernelGGL(dec_prefix_kernel, heads, dim3(64), 0, st, a);
        if (a.off32) hipLaunchKernelGGL((dec_attn_kernel<ES, D, BLK, kPV, uint32_t>), splits, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((dec_attn_kernel<ES, D, BLK, kPV, size_t>), splits, dim3(256), 0, st, a);
    } else {
        if (a.off32) hipLaunchKernelGGL((dec_attn_kernel<ES, D, BLK, kFull, uint32_t>), splits, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((dec_attn_kernel<ES, D, BLK, kFull, size_t>), splits, dim3(256), 0, st, a);
    }
    hipLaunchKernelGGL((dec_combine_kernel<D>), heads, dim3(256), 0, st, a, ES == 4 ? 1 : 0);
    return hipGetLastError();
}

template <int ES, int D>
hipError_t launch_blk(const Shape &s, DecArgs &a, bool skip, hipStream_t st) {
    return s.blk == 64 ? launch_all<ES, D, 64>(s, a, skip, st) : launch_all<ES, D, 128>(s, a, skip, st);
}

}  // namespace

void decode_workspace_layout(const Shape &s, size_t *lists, size_t *counts, size_t *part,
                             size_t *total) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    const size_t bh = (size_t)s.batch * s.hq;
    const size_t nsplit = (size_t)(s.nb + kSplit - 1) / kSplit;
    *lists = 0;
    *counts = al(bh * s.nb * sizeof(int32_t));
    *part = *counts + al(bh * sizeof(int32_t));
    *total = *part + al(bh * nsplit * (s.d + 2) * sizeof(float)) + al(bh * s.nb * sizeof(uint32_t));
}

void decode_skip_layout(const Shape &s, size_t *bmax, size_t *live, size_t *nlive, size_t *scores,
                        size_t *total) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    const size_t bh = (size_t)s.batch * s.hq;
    size_t l, c, p, base;
    decode_workspace_layout(s, &l, &c, &p, &base);
    *bmax = base;
    *live = *bmax + al(bh * s.nb * sizeof(float));
    *nlive = *live + al(bh * s.nb * sizeof(int32_t));
    *scores = *nlive + al(bh * sizeof(int32_t));
    *total = *scores + al(bh * s.nb * s.blk * sizeof(float));
}

hipError_t launch_decode(const Shape &s, const void *q, const KvView &kv, const int32_t *seq_lens,
                         const int32_t *keep, const float *kbar, const float *lvn, void *o,
                         float *lse, void *workspace, hipStream_t st, const DecodeSkip *skip) {
    size_t ol, oc, op, total;
    decode_workspace_layout(s, &ol, &oc, &op, &total);
    char *ws = static_cast<char *>(workspace);
    DecArgs a{};
    a.q = static_cast<const char *>(q);
    a.k = static_cast<const char *>(kv.k);
    a.v = static_cast<const char *>(kv.v);
    a.table = kv.table;
    a.page_log2 = kv.page_log2;
    a.pages_per_seq = kv.pages_per_seq;
    a.seq_lens = seq_lens;
    a.keep = keep;
    a.kbar = kbar;
    a.lvn = lvn;
    a.lists = reinterpret_cast<int32_t *>(ws + ol);
    a.counts = reinterpret_cast<int32_t *>(ws + oc);
    a.part = reinterpret_cast<float *>(ws + op);
    a.keys = reinterpret_cast<uint32_t *>(ws + total - (((size_t)s.batch * s.hq * s.nb * 4 + 255) & ~size_t(255)));
    a.o = o;
    a.lse = lse;
    a.hq = s.hq;
    a.hkv = s.hkv;
    a.d = s.d;
    a.blk = s.blk;
    a.nb = s.nb;
    a.seq = s.seq;
    a.nsplit = (s.nb + kSplit - 1) / kSplit;
    const size_t es = s.dtype == STEM_F32 ? 4 : s.dtype == STEM_BF16 ? 2 : 1;
    a.off32 = kv.rows * s.hkv * s.d * es < (size_t(1) << 32) ? 1 : 0;
    a.q_scale = s.q_scale;
    a.k_scale = s.k_scale;
    a.v_scale = s.v_scale;
    a.tau = s.tau;
    // lambda = 0 drops nothing: the plain step, whose result it then is bit
    // for bit (the selection reports zero dropped blocks)
    const bool sk = skip != nullptr && skip->log2_lambda != -__builtin_huge_valf();
    if (sk) {
        size_t obm, olv, onl, osc, tot2;
        decode_skip_layout(s, &obm, &olv, &onl, &osc, &tot2);
        a.bmax = reinterpret_cast<float *>(ws + obm);
        a.live = reinterpret_cast<int32_t *>(ws + olv);
        a.nlive = reinterpret_cast<int32_t *>(ws + onl);
        a.scores = reinterpret_cast<float *>(ws + osc);
        a.skipped = skip->skipped;
        a.skip_log2 = skip->log2_lambda;
    } else if (skip) {
        a.skipped = skip->skipped;
    }
    if (s.d == 64) {
        switch (s.dtype) {
            case STEM_F32: return launch_blk<4, 64>(s, a, sk, st);
            case STEM_BF16: return launch_blk<2, 64>(s, a, sk, st);
            default: return launch_blk<1, 64>(s, a, sk, st);
        }
    }
    switch (s.dtype) {
        case STEM_F32: return launch_blk<4, 128>(s, a, sk, st);
        case STEM_BF16: return launch_blk<2, 128>(s, a, sk, st);
        default: return launch_blk<1, 128>(s, a, sk, st);
    }
}

}  // namespace stem
