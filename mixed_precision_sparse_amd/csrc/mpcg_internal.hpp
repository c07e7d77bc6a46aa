// Internal declarations shared by the host layout builder and the HIP runtime.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/mpcg.h"

// Canonical Tile-CSC matrix held on the host (EvoCG, Sec. 3.3, Fig. 4).
struct cg_tilecsc {
    int64_t n = 0;
    int32_t R = 0, C = 0;
    int64_t nrb = 0;                    // ceil(n / R)
    std::vector<int64_t> tile_row_ptr;  // [nrb + 1]
    std::vector<int32_t> tile_col_idx;  // [T]
    std::vector<int64_t> tile_nnz_ptr;  // [T + 1]
    std::vector<uint16_t> row_idx;      // [nnz] row offset inside the row block (R <= 16384)
    std::vector<uint8_t> col_local;     // [nnz]
    std::vector<int64_t> perm;          // [nnz] canonical position -> CSR position
    std::vector<double> val;            // [nnz]
    int64_t T() const { return (int64_t)tile_col_idx.size(); }
    int64_t nnz() const { return (int64_t)val.size(); }
};

namespace mpcg {

// Records a message for cg_last_error() and returns code.
int fail(int code, const std::string& msg);
void clear_error();

// Runs body(lo, hi) over [0, count) split across hardware threads.
template <class F>
void parallel_for(int64_t count, F&& body);

}  // namespace mpcg

#include <algorithm>
#include <thread>

template <class F>
void mpcg::parallel_for(int64_t count, F&& body) {
    unsigned hw = std::thread::hardware_concurrency();
    int64_t nt = std::max<int64_t>(1, std::min<int64_t>(hw ? hw : 1, 16));
    if (count < 4096 || nt == 1) {
        body((int64_t)0, count);
        return;
    }
    std::vector<std::thread> th;
    int64_t chunk = (count + nt - 1) / nt;
    for (int64_t t = 0; t < nt; ++t) {
        int64_t lo = t * chunk, hi = std::min(count, lo + chunk);
        if (lo >= hi) break;
        th.emplace_back([&body, lo, hi] { body(lo, hi); });
    }
    for (auto& x : th) x.join();
}
