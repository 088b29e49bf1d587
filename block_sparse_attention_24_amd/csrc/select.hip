// Fused TPD budget + top-k block selection (Stem article on cn486.com, §二.2.1:
// budget generation and block sorting/selection in one operator; §一.3.1 for
// the position-dependent budget).
//
// One wavefront per row (b, h, I).  The row's budget k_I is generated in the
// kernel from the plan's threshold grant (an O(1) integer computation).  The
// sink J=0 and the diagonal J=I are kept; the best k_I - |{0,I}| candidates
// J in [1, I-1] are found by a bitwise search for the k-th largest
// order-preserving 32-bit key (scores held in registers, counted with wave
// ballots), then ties at the threshold go to the smallest J by a prefix count
// over the lanes in J order.  Output: the packed mask row (two 32-bit words
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

template <int MAXC>
__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.rows) return;                  // whole wave exits together
    const int I = (int)(row % a.nb);
    const int k_row = tpd_row_budget(a.plan, I);
    const int forced = I == 0 ? 1 : 2;
    const int want = k_row - forced;            // candidates to keep
    const int ncand = I > 1 ? I - 1 : 0;        // J in [1, I-1]
    const int nch = (I + 63) >> 6;              // chunks holding J < I
    const float *srow = a.scores + row * a.nb;

    uint32_t key[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        key[c] = 0u;
        if (c < nch) {
            const int j = c * 64 + lane;
            if (j >= 1 && j < I) key[c] = order_key(srow[j]);
        }
    }

    // Threshold key t: the want-th largest key, by a bitwise search from the
    // highest bit on which the row's candidate keys differ (the bits above it
    // are common to all of them, so to t as well).
    uint32_t t = 0u;
    int need_eq = 0;                           // keys == t still to keep, smallest J first
    const bool all = want >= ncand;
    if (want > 0 && !all) {
        uint32_t kmin = ~0u, kmax = 0u;
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int j = c * 64 + lane;
            if (c < nch && j >= 1 && j < I) {
                kmin = min(kmin, key[c]);
                kmax = max(kmax, key[c]);
            }
        }
        int top;
        t = key_prefix(wave_min_u32(kmin), wave_max_u32(kmax), top);
        for (int bit = top; bit >= 0; --bit) {
            const uint32_t cand = t | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int c = 0; c < MAXC; ++c)
                if (c < nch) cnt += __popcll(ballot64(key[c] >= cand));
            if (cnt >= want) t = cand;
            // Exactly `want` keys are >= cand: they are the kept set whatever
            // the lower bits hold, and with t = cand the rule below keeps
            // every key > t and every key == t, i.e. exactly them.
            if (cnt == want) break;
        }
        int gt = 0;
#pragma unroll
        for (int c = 0; c < MAXC; ++c)
            if (c < nch) gt += __popcll(ballot64(key[c] > t));
        need_eq = want - gt;
    }

    const int chunks_row = (a.nb + 63) >> 6;
    uint32_t *mrow = a.mask + row * a.words;
    int32_t *lrow = a.list ? a.list + row * a.list_stride : nullptr;
    int run_eq = 0, run_keep = 0;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        if (c < chunks_row) {                   // uniform; keeps the loop fully unrolled
            const int j = c * 64 + lane;
            const bool valid = j >= 1 && j < I;
            bool keep = false;
            if (all) {                          // uniform branches: ballots stay wave-wide
                keep = valid && want > 0;
            } else if (want > 0) {
                const bool eq = valid && key[c] == t;
                const uint64_t eqm = ballot64(eq);
                keep = valid && (key[c] > t || (eq && run_eq + lanes_below(eqm) < need_eq));
                run_eq += __popcll(eqm);
            }
            keep = keep || j == 0 || j == I;
            const uint64_t km = ballot64(keep);
            if (lane < 2 && 2 * c + lane < a.words)
                mrow[2 * c + lane] = lane == 0 ? (uint32_t)km : (uint32_t)(km >> 32);
            const int pos = run_keep + lanes_below(km);
            if (lrow && keep && pos < a.list_stride) lrow[pos] = j;
            run_keep += __popcll(km);
        }
    }
    if (a.count && lane == 0) a.count[row] = k_row;
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
