// Fused TPD budget + top-k block selection (Stem article on cn486.com, §二.2.1:
// budget generation and block sorting/selection in one operator; §一.3.1 for
// the position-dependent budget).
//
// One wavefront per row (b, h, I).  The row's budget k_I is generated in the
// kernel from the plan's threshold grant (an O(1) integer computation).  The
// sink J=0 and the diagonal J=I are kept; the best k_I - |{0,I}| candidates
// J in [1, I-1] are found by a bitwise search for the k-th largest
// order-preserving 32-bit key (scores held in registers), then ties at the
// threshold go to the smallest J by a prefix count over the lanes in J order
// (when every key equal to the threshold is kept, which is the usual case,
// the kept candidates are simply the keys at or above it).
// The search counts on the VALU (per-lane counts, one wave sum per bit) while
// the bucket of keys that share the threshold's decided bits holds more than
// 64 keys; then that bucket is gathered into one key per lane and each
// further bit costs one ballot.  Output: the packed mask row (two 32-bit words
// per 64-lane chunk straight from a ballot) and, optionally, the kept list.
#include "device_common.h"
#include "stem_internal.h"

namespace stem {
namespace {

struct SelectArgs {
    const float *scores;
    uint32_t *mask;
    int32_t *list;
    int32_t *count;
    int list_stride;
    int nb, words;
    long long rows;
    TpdPlan plan;
};

// One row, its candidates in the first NCH chunks of 64 J (chunks from
// ceil(I/64) on hold only invalid J).  Every chunk loop has a compile-time
// trip count and no branch: invalid J read a clamped, in-row address and get
// key 0, which no trial value (it has a bit set) counts.
template <int NCH>
__device__ __forceinline__ void select_row(const SelectArgs &a, long long row, int I, int k_row, int want,
                                           int ncand, uint32_t *buf, int lane) {
    const float *srow = a.scores + row * a.nb;
    uint32_t key[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int j = c * 64 + lane;
        const float x = srow[min(j, I)];
        key[c] = (j >= 1 && j < I) ? order_key(x) : 0u;
    }

    // the threshold of the kept set (need_eq: keys equal to it still kept, smallest J first)
    uint32_t t = 0u;
    int need_eq = 0;
    bool all_eq = false;
    const bool all = want >= ncand;
    if (want > 0 && !all) topk_threshold<NCH>(key, I, want, ncand, buf, lane, t, need_eq, all_eq);
    // no tie to break at the threshold: the kept candidates are the keys >= t
    // (invalid J hold key 0, below any t > 0)
    const bool simple = want > 0 && !all && all_eq && t > 0u;

    // The kept set, chunk by chunk in J order; lane w collects mask words w,
    // w + 64, ... (two words per chunk).
    int32_t *lrow = a.list ? a.list + row * a.list_stride : nullptr;
    constexpr int MW = (2 * NCH + 63) / 64;
    uint32_t mword[MW];
#pragma unroll
    for (int q = 0; q < MW; ++q) mword[q] = 0u;
    int run_keep = 0;
    auto emit = [&](int c, bool keep) {         // chunk c's kept J: its two mask words and list entries
        const int j = c * 64 + lane;
        keep = keep || j == 0 || j == I;
        const uint64_t km = ballot64(keep);
        if ((lane >> 1) == (c & 31)) mword[c >> 5] = (lane & 1) ? (uint32_t)(km >> 32) : (uint32_t)km;
        if (lrow) {
            const int pos = run_keep + lanes_below(km);
            if (keep && pos < a.list_stride) lrow[pos] = j;
            run_keep += __popcll(km);
        }
    };
    if (simple) {                               // uniform branches: ballots stay wave-wide
#pragma unroll
        for (int c = 0; c < NCH; ++c) emit(c, key[c] >= t);
    } else {
        int run_eq = 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int j = c * 64 + lane;
            const bool valid = j >= 1 && j < I;
            bool keep = false;
            if (all) {
                keep = valid && want > 0;
            } else if (want > 0) {
                const bool eq = valid && key[c] == t;
                const uint64_t eqm = ballot64(eq);
                keep = valid && (key[c] > t || (eq && run_eq + lanes_below(eqm) < need_eq));
                run_eq += __popcll(eqm);
            }
            emit(c, keep);
        }
    }
    uint32_t *mrow = a.mask + row * a.words;
#pragma unroll
    for (int q = 0; q < MW; ++q) {
        const int wd = 64 * q + lane;
        if (wd < 2 * NCH && wd < a.words) mrow[wd] = mword[q];
    }
    for (int wd = 2 * NCH + lane; wd < a.words; wd += 64) mrow[wd] = 0u;   // J > I
    if (a.count && lane == 0) a.count[row] = k_row;
}

template <int MAXC>
__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
    __shared__ uint32_t gather[4][64];          // per wave: the bucket gathered for the last bits
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.rows) return;                  // whole wave exits together
    const int I = (int)(row % a.nb);
    const int k_row = tpd_row_budget(a.plan, I);
    const int forced = I == 0 ? 1 : 2;
    const int want = k_row - forced;            // candidates to keep
    const int ncand = I > 1 ? I - 1 : 0;        // J in [1, I-1]
    const int nch = (I >> 6) + 1;               // chunks holding J <= I
    uint32_t *buf = gather[threadIdx.x >> 6];
    // the smallest compiled chunk count that covers the row (uniform branches)
#define SEL(N) select_row<(MAXC < N ? MAXC : N)>(a, row, I, k_row, want, ncand, buf, lane)
    if (nch <= 1) SEL(1);
    else if (nch <= 2) SEL(2);
    else if (nch <= 4) SEL(4);
    else if (nch <= 8) SEL(8);
    else if (nch <= 12) SEL(12);
    else if (nch <= 16) SEL(16);
    else if (nch <= 24) SEL(24);
    else if (nch <= 32) SEL(32);
    else if (nch <= 48) SEL(48);
    else SEL(64);
#undef SEL
}

template <int MAXC>
hipError_t launch(const SelectArgs &a, hipStream_t st) {
    const long long blocks = (a.rows + 3) / 4;
    hipLaunchKernelGGL((select_kernel<MAXC>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const Shape &s, const TpdPlan &plan, const float *scores, uint32_t *mask,
                         int32_t *list, int list_stride, int32_t *count, hipStream_t st) {
    SelectArgs a{};
    a.scores = scores;
    a.mask = mask;
    a.list = list;
    a.count = count;
    a.list_stride = list_stride;
    a.nb = s.nb;
    a.words = s.words;
    a.rows = (long long)s.batch * s.hq * s.nb;
    a.plan = plan;
    const int chunks = (s.nb + 63) / 64;
    if (chunks <= 1) return launch<1>(a, st);
    if (chunks <= 2) return launch<2>(a, st);
    if (chunks <= 4) return launch<4>(a, st);
    if (chunks <= 8) return launch<8>(a, st);
    if (chunks <= 16) return launch<16>(a, st);
    if (chunks <= 32) return launch<32>(a, st);
    return launch<64>(a, st);
}

}  // namespace stem
