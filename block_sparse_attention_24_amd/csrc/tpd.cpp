// TPD budget (Stem article on cn486.com, §一.3.1 "Token Position Decay";
// setupai.cc summary, "Technical Deep Dive"): a fixed total of kept blocks per
// head, redistributed towards early query blocks.  Reading implemented: start
// at the forced minimum (1 block in row 0, 2 elsewhere: sink + diagonal) and
// grant the remaining blocks one at a time to the row with the smallest key
// (k+1)/(I+1)^(1-alpha) that still has room, equal keys to the smaller row.
//
// Instead of simulating the grants, the host finds the last grant made (the
// R-th smallest of all possible grants in (key, row) order) by a selection
// over the per-row ranges of candidate grants, each comparison exact in
// integers.  Every row's budget then follows in O(1) (tpd_nmax), which lets
// the selection kernel generate its own row budget.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "stem_internal.h"

namespace stem {
namespace {

// Is grant (r1, n1) strictly before grant (r2, n2)?
bool grant_before(int power, int r1, long long n1, int r2, long long n2) {
    unsigned long long lhs, rhs;
    if (power == 0) {
        lhs = (unsigned long long)n1;
        rhs = (unsigned long long)n2;
    } else if (power == 1) {
        lhs = (unsigned long long)n1 * (unsigned long long)(r2 + 1);
        rhs = (unsigned long long)n2 * (unsigned long long)(r1 + 1);
    } else {
        lhs = (unsigned long long)(n1 * n1) * (unsigned long long)(r2 + 1);
        rhs = (unsigned long long)(n2 * n2) * (unsigned long long)(r1 + 1);
    }
    if (lhs != rhs) return lhs < rhs;
    return r1 < r2;
}

// The plan depends only on (nb, density, alpha); callers repeat the same few,
// so the last kPlanCache plans are kept (round-robin), shared by all threads.
constexpr int kPlanCache = 8;
struct CachedPlan {
    int nb;
    double density, alpha;
    TpdPlan plan;
};
std::mutex g_plan_mutex;
CachedPlan g_plans[kPlanCache];
int g_plans_used = 0, g_plans_next = 0;

bool same_bits(double x, double y) { return std::memcmp(&x, &y, sizeof(double)) == 0; }

int make_plan_uncached(int nb, double density, double alpha, TpdPlan *out, const char **why);

}  // namespace

int tpd_make_plan(int nb, double density, double alpha, TpdPlan *out, const char **why) {
    {
        std::lock_guard<std::mutex> g(g_plan_mutex);
        for (int i = 0; i < g_plans_used; ++i)
            if (g_plans[i].nb == nb && same_bits(g_plans[i].density, density) && same_bits(g_plans[i].alpha, alpha)) {
                *out = g_plans[i].plan;
                return STEM_OK;
            }
    }
    TpdPlan p;
    const int rc = make_plan_uncached(nb, density, alpha, &p, why);
    if (rc != STEM_OK) return rc;
    std::lock_guard<std::mutex> g(g_plan_mutex);
    g_plans[g_plans_next] = CachedPlan{nb, density, alpha, p};
    g_plans_next = (g_plans_next + 1) % kPlanCache;
    g_plans_used = std::min(g_plans_used + 1, kPlanCache);
    *out = p;
    return STEM_OK;
}

namespace {

int make_plan_uncached(int nb, double density, double alpha, TpdPlan *out, const char **why) {
    if (nb < 1 || nb > 65536) { *why = "num_blocks must lie in [1, 65536]"; return STEM_EINVAL; }
    if (!(density > 0.0 && density <= 1.0)) { *why = "density must lie in (0, 1]"; return STEM_EINVAL; }
    int power;
    if (alpha == 0.0) power = 1;
    else if (alpha == 0.5) power = 2;
    else if (alpha == 1.0) power = 0;
    else { *why = "alpha must be 0, 0.5 or 1"; return STEM_EUNSUPPORTED; }

    const long long c = (long long)nb * (nb + 1) / 2;
    long long t = (long long)std::floor(density * (double)c + 0.5);
    const long long forced = 2LL * nb - 1;
    t = std::max(forced, std::min(c, t));

    TpdPlan p{};
    p.nb = nb;
    p.power = power;
    p.total = t;
    long long need = t - forced;              // grants to hand out
    if (need == 0) { p.has_threshold = 0; *out = p; return STEM_OK; }

    // Candidate grants of row I: n in (lo[I], hi[I]]; initially (min, I+1].
    std::vector<long long> lo(nb), hi(nb);
    for (int i = 0; i < nb; ++i) { lo[i] = i == 0 ? 1 : 2; hi[i] = i + 1; if (hi[i] < lo[i]) hi[i] = lo[i]; }
    struct Mid { int row; long long n; };
    std::vector<Mid> mids;
    mids.reserve(nb);
    std::vector<long long> cnt(nb, 0);
    for (;;) {
        // Pivot: the lower median, in grant order, of the rows' middle grants
        // (linear time).  Either every grant after the pivot is dropped, and
        // the rows whose middle grant lies after it lose at least half their
        // range, or every grant up to the pivot is taken, and the rows whose
        // middle grant lies at or before it do.  The lower median is never the
        // last of several middle grants, so something is dropped or taken in
        // every round.
        mids.clear();
        for (int i = 0; i < nb; ++i) {
            const long long w = hi[i] - lo[i];
            if (w > 0) mids.push_back({i, lo[i] + (w + 1) / 2});
        }
        auto med = mids.begin() + (mids.size() - 1) / 2;
        std::nth_element(mids.begin(), med, mids.end(), [&](const Mid &a, const Mid &b) {
            return grant_before(power, a.row, a.n, b.row, b.n);
        });
        const Mid piv = *med;
        // Count candidates at or before the pivot.
        long long s = 0;
        for (int i = 0; i < nb; ++i) {
            cnt[i] = 0;
            if (hi[i] <= lo[i]) continue;
            long long n = tpd_nmax(power, i, piv.row, (int)piv.n);
            long long k = std::min(hi[i], std::max(lo[i], n)) - lo[i];
            cnt[i] = k;
            s += k;
        }
        if (s == need) { p.has_threshold = 1; p.th_row = piv.row; p.th_n = (int)piv.n; break; }
        if (s > need) {
            for (int i = 0; i < nb; ++i) hi[i] = lo[i] + cnt[i];
        } else {
            for (int i = 0; i < nb; ++i) lo[i] += cnt[i];
            need -= s;
        }
    }
    *out = p;
    return STEM_OK;
}

}  // namespace
}  // namespace stem
