// Row-block height tuning (EvoCG paper, Sec. 3.3.3 "Cross-Level Balance
// Tuning"): for every candidate height R = 32, 64, ..., 16384 the number of
// non-empty R x C tiles of each row block, how evenly they spread (coefficient
// of variation), and the tuned R: the admissible candidate (R <= max_R, at
// least min_row_blocks row blocks) with the smallest coefficient of variation,
// ties to the smaller R. Candidates are compared exactly (integer arithmetic
// on the squared coefficient), not through the rounded values. Host code
// only.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <string>
#include <vector>

#include "mpcg.h"
#include "mpcg_internal.hpp"

using mpcg::fail;

namespace {

constexpr int kCandidates = 10;  // 32 << 0 .. 32 << 9

typedef unsigned __int128 u128;

struct Balance {
    int64_t nrb = 0, tiles = 0;
    double cv = 0.0, max_ratio = 0.0;
    u128 var = 0, s1sq = 1;  // cv^2 = var / s1sq exactly (var = m S2 - S1^2, s1sq = S1^2; 0 / 1 when empty)
};

// p / q < r / s for p, r >= 0 and q, s > 0, exactly: compare the integer
// parts; when they agree, compare the reciprocals of the remainders (a
// continued-fraction step), which never overflows.
bool frac_less(u128 p, u128 q, u128 r, u128 s) {
    for (;;) {
        const u128 a = p / q, b = r / s;
        if (a != b) return a < b;
        p -= a * q;
        r -= b * s;
        if (p == 0) return r != 0;
        if (r == 0) return false;
        // p / q < r / s  <=>  s / r < q / p
        const u128 np = s, nq = r, nr = q, ns = p;
        p = np;
        q = nq;
        r = nr;
        s = ns;
    }
}

// Tile counts of every row block of height R (one stamp array of column
// blocks per worker), then the balance measures from exact integer sums: with
// m row blocks, S1 = sum c, S2 = sum c^2, cv = sqrt(m S2 - S1^2) / S1 and
// max / mean = m max(c) / S1, each operand rounded once to double.
Balance row_block_balance(int64_t n, const int64_t* rowptr, const int32_t* colind, int64_t R, int64_t C) {
    const int64_t nrb = (n + R - 1) / R, ncb = (n + C - 1) / C;
    std::vector<int64_t> counts(nrb, 0);
    mpcg::parallel_for(nrb, [&](int64_t lo, int64_t hi) {
        std::vector<int32_t> stamp(ncb, -1);  // row block that last counted column block J
        for (int64_t I = lo; I < hi; ++I) {
            int64_t c = 0;
            const int64_t r1 = std::min(n, (I + 1) * R);
            for (int64_t r = I * R; r < r1; ++r)
                for (int64_t k = rowptr[r]; k < rowptr[r + 1]; ++k) {
                    const int64_t J = colind[k] / C;
                    if (stamp[J] != (int32_t)I) {
                        stamp[J] = (int32_t)I;
                        ++c;
                    }
                }
            counts[I] = c;
        }
    });
    Balance b;
    b.nrb = nrb;
    unsigned __int128 s2 = 0;
    int64_t s1 = 0, mx = 0;
    for (int64_t c : counts) {
        s1 += c;
        s2 += (unsigned __int128)c * (unsigned __int128)c;
        mx = std::max(mx, c);
    }
    b.tiles = s1;
    if (s1 > 0) {
        const unsigned __int128 var = (unsigned __int128)nrb * s2 - (unsigned __int128)s1 * (unsigned __int128)s1;
        b.var = var;
        b.s1sq = (u128)s1 * (u128)s1;
        b.cv = std::sqrt((double)var) / (double)s1;
        b.max_ratio = (double)((unsigned __int128)nrb * (unsigned __int128)mx) / (double)s1;
    }
    return b;
}

}  // namespace

extern "C" int cg_tune_row_height(int64_t n, const int64_t* rowptr, const int32_t* colind, int32_t C,
                                  int32_t max_R, int64_t min_row_blocks, int32_t* R_out, int32_t cap,
                                  int32_t* cand_R, int64_t* cand_nrb, int64_t* cand_T, double* cand_cv,
                                  double* cand_max_ratio, uint8_t* cand_ok) {
    mpcg::clear_error();
    if (!rowptr || !R_out) return fail(CG_EINVAL, "cg_tune_row_height: NULL argument");
    if (n < 1) return fail(CG_EINVAL, "cg_tune_row_height: n must be >= 1");
    if (C < 1 || C > 256) return fail(CG_EINVAL, "cg_tune_row_height: C must lie in [1, 256]");
    if (min_row_blocks < 1) return fail(CG_EINVAL, "cg_tune_row_height: min_row_blocks must be >= 1");
    if (cap < 0) return fail(CG_EINVAL, "cg_tune_row_height: cap must be >= 0");
    if (rowptr[0] != 0) return fail(CG_EINVAL, "cg_tune_row_height: rowptr[0] must be 0");
    for (int64_t i = 0; i < n; ++i)
        if (rowptr[i + 1] < rowptr[i])
            return fail(CG_EINVAL, "cg_tune_row_height: rowptr decreases at row " + std::to_string(i));
    if (rowptr[n] > 0 && !colind) return fail(CG_EINVAL, "cg_tune_row_height: colind is NULL");
    for (int64_t k = 0; k < rowptr[n]; ++k)
        if (colind[k] < 0 || colind[k] >= n)
            return fail(CG_EINVAL, "cg_tune_row_height: colind[" + std::to_string(k) + "] is outside [0, n)");
    int32_t best = -1;
    Balance best_b;
    for (int i = 0; i < kCandidates; ++i) {
        const int32_t R = 32 << i;
        const Balance b = row_block_balance(n, rowptr, colind, R, C);
        const bool ok = R <= max_R && b.nrb >= min_row_blocks;
        if (ok && (best < 0 || frac_less(b.var, b.s1sq, best_b.var, best_b.s1sq))) {
            best = R;
            best_b = b;
        }
        if (i < cap) {
            if (cand_R) cand_R[i] = R;
            if (cand_nrb) cand_nrb[i] = b.nrb;
            if (cand_T) cand_T[i] = b.tiles;
            if (cand_cv) cand_cv[i] = b.cv;
            if (cand_max_ratio) cand_max_ratio[i] = b.max_ratio;
            if (cand_ok) cand_ok[i] = ok ? 1 : 0;
        }
    }
    *R_out = best < 0 ? 32 : best;
    return kCandidates;
}
