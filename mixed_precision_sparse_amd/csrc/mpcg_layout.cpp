// Host-side construction of the canonical Tile-CSC layout and the error channel.
//
// Layout definition: EvoCG paper, Sec. 3.3 ("Inter-Tile Row-Block
// Scheduling" and "Intra-Tile CSC Execution") and Fig. 4(a)/(b): non-empty
// R x C tiles in row-block-major order with ascending column blocks, and
// column-major (CSC) storage inside each tile with row offsets relative to
// the row block. The paper's sentinel padding of odd-length columns is a
// storage choice of its kernel and is not part of this canonical form.

#include <atomic>
#include <cmath>
#include <cstring>
#include <new>

#include "mpcg_internal.hpp"

namespace {
thread_local std::string g_last_error;
}

int mpcg::fail(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

void mpcg::clear_error() { g_last_error.clear(); }

extern "C" const char* cg_last_error(void) { return g_last_error.c_str(); }

extern "C" int cg_version(void) { return 10400; }  // 1.4.0

namespace {

// Validates the CSR input; returns CG_OK or a CG_EINVAL with a message.
int validate_csr(int64_t n, const int64_t* rowptr, const int32_t* colind, const double* val) {
    if (n < 1) return mpcg::fail(CG_EINVAL, "cg_tilecsc_from_csr: n must be >= 1");
    if (!rowptr) return mpcg::fail(CG_EINVAL, "cg_tilecsc_from_csr: rowptr is NULL");
    if (rowptr[0] != 0) return mpcg::fail(CG_EINVAL, "cg_tilecsc_from_csr: rowptr[0] must be 0");
    int64_t nnz = rowptr[n];
    if (nnz < 0 || nnz > INT32_MAX)
        return mpcg::fail(CG_EINVAL, "cg_tilecsc_from_csr: nnz must lie in [0, 2^31-1]");
    if (nnz > 0 && (!colind || !val))
        return mpcg::fail(CG_EINVAL, "cg_tilecsc_from_csr: colind or val is NULL");
    for (int64_t i = 0; i < n; ++i) {
        if (rowptr[i + 1] < rowptr[i])
            return mpcg::fail(CG_EINVAL, "cg_tilecsc_from_csr: rowptr decreases at row " +
                                             std::to_string(i));
    }
    std::atomic<int64_t> bad_row{-1};
    mpcg::parallel_for(n, [&](int64_t lo, int64_t hi) {
        for (int64_t i = lo; i < hi && bad_row.load(std::memory_order_relaxed) < 0; ++i) {
            int64_t prev = -1;
            for (int64_t k = rowptr[i]; k < rowptr[i + 1]; ++k) {
                int64_t c = colind[k];
                if (c < 0 || c >= n || c <= prev || !std::isfinite(val[k])) {
                    int64_t expect = -1;
                    bad_row.compare_exchange_strong(expect, i);
                    break;
                }
                prev = c;
            }
        }
    });
    if (bad_row.load() >= 0)
        return mpcg::fail(CG_EINVAL,
                          "cg_tilecsc_from_csr: row " + std::to_string(bad_row.load()) +
                              " has a column out of range, unsorted or duplicate columns, or a "
                              "non-finite value");
    return CG_OK;
}

}  // namespace

extern "C" int cg_tilecsc_from_csr(int64_t n, const int64_t* rowptr, const int32_t* colind,
                                   const double* val, int32_t R, int32_t C, cg_tilecsc** out) {
    mpcg::clear_error();
    if (!out) return mpcg::fail(CG_EINVAL, "cg_tilecsc_from_csr: out is NULL");
    *out = nullptr;
    if (R < 1 || R > 16384 || C < 1 || C > 256)
        return mpcg::fail(CG_EINVAL, "cg_tilecsc_from_csr: R must lie in [1, 16384] and C in [1, 256]");
    int rc = validate_csr(n, rowptr, colind, val);
    if (rc != CG_OK) return rc;

    cg_tilecsc* A = new (std::nothrow) cg_tilecsc();
    if (!A) return mpcg::fail(CG_ENOMEM, "cg_tilecsc_from_csr: out of host memory");
    try {
        const int64_t nnz = rowptr[n];
        const int64_t nrb = (n + R - 1) / R;
        const int64_t ncb = (n + C - 1) / C;
        A->n = n;
        A->R = R;
        A->C = C;
        A->nrb = nrb;

        // Pass 1: count the non-empty tiles of every row block (distinct column blocks).
        std::vector<int64_t> tiles_in_rb(nrb, 0);
        mpcg::parallel_for(nrb, [&](int64_t lo, int64_t hi) {
            std::vector<int64_t> stamp(ncb, -1);
            for (int64_t I = lo; I < hi; ++I) {
                int64_t r0 = I * R, r1 = std::min<int64_t>(n, r0 + R), cnt = 0;
                for (int64_t k = rowptr[r0]; k < rowptr[r1]; ++k) {
                    int64_t J = colind[k] / C;
                    if (stamp[J] != I) {
                        stamp[J] = I;
                        ++cnt;
                    }
                }
                tiles_in_rb[I] = cnt;
            }
        });
        A->tile_row_ptr.assign(nrb + 1, 0);
        for (int64_t I = 0; I < nrb; ++I) A->tile_row_ptr[I + 1] = A->tile_row_ptr[I] + tiles_in_rb[I];
        const int64_t T = A->tile_row_ptr[nrb];
        if (T > INT32_MAX) {
            delete A;
            return mpcg::fail(CG_EINVAL, "cg_tilecsc_from_csr: more than 2^31-1 non-empty tiles");
        }
        A->tile_col_idx.resize(T);
        A->tile_nnz_ptr.resize(T + 1);
        A->row_idx.resize(nnz);
        A->col_local.resize(nnz);
        A->perm.resize(nnz);
        A->val.resize(nnz);
        A->tile_nnz_ptr[T] = nnz;

        // Pass 2: inside each row block, order the entries by (global column, row):
        // that is column block, then local column, then local row.
        mpcg::parallel_for(nrb, [&](int64_t lo, int64_t hi) {
            struct Ent {
                int32_t col;
                int32_t row;
                int64_t k;
            };
            std::vector<Ent> ents;
            for (int64_t I = lo; I < hi; ++I) {
                int64_t r0 = I * R, r1 = std::min<int64_t>(n, r0 + R);
                int64_t base = rowptr[r0];
                ents.clear();
                for (int64_t i = r0; i < r1; ++i)
                    for (int64_t k = rowptr[i]; k < rowptr[i + 1]; ++k)
                        ents.push_back(Ent{colind[k], (int32_t)(i - r0), k});
                std::sort(ents.begin(), ents.end(), [](const Ent& a, const Ent& b) {
                    return a.col != b.col ? a.col < b.col : a.row < b.row;
                });
                int64_t t = A->tile_row_ptr[I] - 1;
                int64_t curJ = -1;
                for (size_t e = 0; e < ents.size(); ++e) {
                    int64_t pos = base + (int64_t)e;
                    int64_t J = ents[e].col / C;
                    if (J != curJ) {
                        ++t;
                        curJ = J;
                        A->tile_col_idx[t] = (int32_t)J;
                        A->tile_nnz_ptr[t] = pos;
                    }
                    A->row_idx[pos] = (uint16_t)ents[e].row;
                    A->col_local[pos] = (uint8_t)(ents[e].col - J * C);
                    A->perm[pos] = ents[e].k;
                    A->val[pos] = val[ents[e].k];
                }
            }
        });
    } catch (const std::bad_alloc&) {
        delete A;
        return mpcg::fail(CG_ENOMEM, "cg_tilecsc_from_csr: out of host memory");
    }
    *out = A;
    return CG_OK;
}

extern "C" int cg_tilecsc_get_view(const cg_tilecsc* A, cg_tilecsc_view* v) {
    mpcg::clear_error();
    if (!A || !v) return mpcg::fail(CG_EINVAL, "cg_tilecsc_get_view: NULL argument");
    v->n = A->n;
    v->T = A->T();
    v->nnz = A->nnz();
    v->R = A->R;
    v->C = A->C;
    v->tile_row_ptr = A->tile_row_ptr.data();
    v->tile_col_idx = A->tile_col_idx.data();
    v->tile_nnz_ptr = A->tile_nnz_ptr.data();
    v->row_idx = A->row_idx.data();
    v->col_local = A->col_local.data();
    v->val = A->val.data();
    return CG_OK;
}

extern "C" int cg_tilecsc_col_ptr(const cg_tilecsc* A, int32_t* out) {
    mpcg::clear_error();
    if (!A || !out) return mpcg::fail(CG_EINVAL, "cg_tilecsc_col_ptr: NULL argument");
    const int64_t T = A->T();
    const int C = A->C;
    mpcg::parallel_for(T, [&](int64_t lo, int64_t hi) {
        for (int64_t t = lo; t < hi; ++t) {
            int32_t* cp = out + t * (C + 1);
            std::memset(cp, 0, sizeof(int32_t) * (C + 1));
            int64_t s = A->tile_nnz_ptr[t], e = A->tile_nnz_ptr[t + 1];
            for (int64_t k = s; k < e; ++k) cp[A->col_local[k] + 1]++;
            for (int c = 0; c < C; ++c) cp[c + 1] += cp[c];
        }
    });
    return CG_OK;
}

extern "C" int cg_tilecsc_perm(const cg_tilecsc* A, int64_t* out) {
    mpcg::clear_error();
    if (!A || !out) return mpcg::fail(CG_EINVAL, "cg_tilecsc_perm: NULL argument");
    std::memcpy(out, A->perm.data(), sizeof(int64_t) * A->perm.size());
    return CG_OK;
}

extern "C" void cg_tilecsc_free(cg_tilecsc* A) { delete A; }
