// Offline choice of the map-reuse interval K* (EvoCG paper, Sec. 3.4
// "Interval Reuse Scheduling"): from a per-iteration record of every column
// block's precision, the fraction of upward transitions (toward more bits)
// that reusing the window-start decision over windows of K iterations would
// delay, for K = 1, 2, 4, ...; K* is the largest K whose fraction is below a
// threshold. Host code only.
#include <algorithm>
#include <atomic>
#include <cstdint>
#include <string>
#include <vector>

#include "mpcg.h"
#include "mpcg_internal.hpp"

using mpcg::fail;

extern "C" int cg_select_reuse_interval(const uint8_t* codes, int32_t nrec, int64_t ncb, double max_fraction,
                                        int32_t* kstar, int32_t cap, int32_t* intervals, double* fractions) {
    mpcg::clear_error();
    if (!codes || !kstar) return fail(CG_EINVAL, "cg_select_reuse_interval: NULL argument");
    if (nrec < 0 || ncb < 0) return fail(CG_EINVAL, "cg_select_reuse_interval: negative size");
    for (int64_t i = 0; i < (int64_t)nrec * ncb; ++i)
        if (codes[i] > 2)
            return fail(CG_EINVAL, "cg_select_reuse_interval: code " + std::to_string(codes[i]) + " at " +
                                       std::to_string(i) + " is not 0, 1 or 2");
    // Candidate intervals below the record length (at least interval 1).
    std::vector<int32_t> cand;
    for (int64_t k = 1; k < std::max<int32_t>(nrec, 2); k *= 2) cand.push_back((int32_t)k);
    std::vector<std::atomic<int64_t>> delayed(cand.size());
    for (auto& d : delayed) d = 0;
    std::atomic<int64_t> up{0};
    // Column blocks are independent: split them over threads.
    mpcg::parallel_for(ncb, [&](int64_t lo, int64_t hi) {
        std::vector<int64_t> my_delayed(cand.size(), 0);
        int64_t my_up = 0;
        for (int64_t J = lo; J < hi; ++J)
            for (int64_t k = 1; k < nrec; ++k) {
                const uint8_t now = codes[k * ncb + J];
                if (now >= codes[(k - 1) * ncb + J]) continue;  // not an upward transition
                ++my_up;
                for (size_t c = 0; c < cand.size(); ++c) {
                    const int64_t start = k / cand[c] * cand[c];
                    if (codes[start * ncb + J] > now) ++my_delayed[c];
                }
            }
        up += my_up;
        for (size_t c = 0; c < cand.size(); ++c) delayed[c] += my_delayed[c];
    });
    int32_t best = 1;
    for (size_t c = 0; c < cand.size(); ++c) {
        const double f = up.load() ? (double)delayed[c].load() / (double)up.load() : 0.0;
        if (f < max_fraction) best = cand[c];
        if ((int32_t)c < cap) {
            if (intervals) intervals[c] = cand[c];
            if (fractions) fractions[c] = f;
        }
    }
    *kstar = best;
    return (int32_t)cand.size();
}
