/* Host-side driver for sanitizer builds (AddressSanitizer + UndefinedBehaviorSanitizer, or
 * ThreadSanitizer) of the library's host C++ code: the Tile-CSC layout builder, the row-block
 * height tuning and the reuse-interval selection. It builds seeded random matrices of several
 * shapes (empty rows, ragged last blocks, tall row blocks, wide tiles, one large enough for the
 * builder's worker threads), checks every invariant of the canonical layout against the CSR
 * input, and walks the error paths. Exit status 0 when every check holds; it links without
 * the HIP runtime (no device call is made). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mpcg.h"

static uint64_t rng_state;
static uint32_t rnd(void) { /* 64-bit LCG, high bits */
    rng_state = rng_state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (uint32_t)(rng_state >> 33);
}

static int failures = 0;
#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            ++failures;                                   \
            printf("FAIL %s:%d: ", __FILE__, __LINE__);   \
            printf(__VA_ARGS__);                          \
            printf("\n");                                 \
            return;                                       \
        }                                                 \
    } while (0)

/* Random square CSR with sorted unique columns: the diagonal (unless the row is left empty)
 * plus up to `extra` random columns per row. */
static void make_csr(int64_t n, int extra, int empty_every, int64_t** rowptr, int32_t** colind, double** val) {
    int64_t cap = n * (int64_t)(extra + 1) + 1;
    *rowptr = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n + 1));
    *colind = (int32_t*)malloc(sizeof(int32_t) * (size_t)cap);
    *val = (double*)malloc(sizeof(double) * (size_t)cap);
    int32_t* row = (int32_t*)malloc(sizeof(int32_t) * (size_t)(extra + 1));
    int64_t k = 0;
    (*rowptr)[0] = 0;
    for (int64_t i = 0; i < n; ++i) {
        int m = 0;
        if (!(empty_every > 0 && i % empty_every == 0)) {
            row[m++] = (int32_t)i;
            const int e = extra ? (int)(rnd() % (uint32_t)(extra + 1)) : 0;
            for (int j = 0; j < e; ++j) row[m++] = (int32_t)(rnd() % (uint32_t)n);
        }
        for (int a = 1; a < m; ++a) /* insertion sort */
            for (int b = a; b > 0 && row[b - 1] > row[b]; --b) {
                int32_t t = row[b];
                row[b] = row[b - 1];
                row[b - 1] = t;
            }
        for (int a = 0; a < m; ++a) {
            if (a > 0 && row[a] == row[a - 1]) continue;
            (*colind)[k] = row[a];
            (*val)[k] = (double)(int32_t)(rnd() % 2001u) - 1000.0;
            ++k;
        }
        (*rowptr)[i + 1] = k;
    }
    free(row);
}

static void check_layout(int64_t n, int extra, int empty_every, int32_t R, int32_t C) {
    int64_t* rowptr;
    int32_t* colind;
    double* val;
    make_csr(n, extra, empty_every, &rowptr, &colind, &val);
    const int64_t nnz = rowptr[n];
    cg_tilecsc* A = NULL;
    const int rc = cg_tilecsc_from_csr(n, rowptr, colind, val, R, C, &A);
    CHECK(rc == CG_OK && A, "build n=%lld R=%d C=%d: rc %d %s", (long long)n, R, C, rc, cg_last_error());
    cg_tilecsc_view v;
    CHECK(cg_tilecsc_get_view(A, &v) == CG_OK, "view");
    CHECK(v.n == n && v.nnz == nnz && v.R == R && v.C == C, "sizes");
    const int64_t nrb = (n + R - 1) / R, ncb = (n + C - 1) / C;
    CHECK(v.tile_row_ptr[0] == 0 && v.tile_row_ptr[nrb] == v.T, "tile_row_ptr ends");
    CHECK(v.tile_nnz_ptr[0] == 0 && v.tile_nnz_ptr[v.T] == nnz, "tile_nnz_ptr ends");
    int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nnz > 0 ? nnz : 1));
    int32_t* colptr = (int32_t*)malloc(sizeof(int32_t) * (size_t)((v.T > 0 ? v.T : 1) * (C + 1)));
    CHECK(cg_tilecsc_perm(A, perm) == CG_OK && cg_tilecsc_col_ptr(A, colptr) == CG_OK, "perm/col_ptr");
    uint8_t* seen = (uint8_t*)calloc((size_t)(nnz > 0 ? nnz : 1), 1);
    for (int64_t I = 0; I < nrb; ++I) {
        CHECK(v.tile_row_ptr[I] <= v.tile_row_ptr[I + 1], "tile_row_ptr order at %lld", (long long)I);
        for (int64_t t = v.tile_row_ptr[I]; t < v.tile_row_ptr[I + 1]; ++t) {
            const int32_t J = v.tile_col_idx[t];
            CHECK(J >= 0 && J < ncb, "column block range");
            CHECK(t == v.tile_row_ptr[I] || v.tile_col_idx[t - 1] < J, "column blocks ascending");
            CHECK(v.tile_nnz_ptr[t] < v.tile_nnz_ptr[t + 1], "empty tile listed");
            const int32_t* cp = colptr + t * (C + 1);
            CHECK(cp[0] == 0 && cp[C] == v.tile_nnz_ptr[t + 1] - v.tile_nnz_ptr[t], "col_ptr ends");
            for (int c = 0; c < C; ++c) CHECK(cp[c] <= cp[c + 1], "col_ptr order");
            for (int64_t k = v.tile_nnz_ptr[t]; k < v.tile_nnz_ptr[t + 1]; ++k) {
                const int64_t row = I * R + v.row_idx[k], col = (int64_t)J * C + v.col_local[k];
                CHECK(v.row_idx[k] < R && v.col_local[k] < C && row < n && col < n, "local indices");
                const int32_t lc = v.col_local[k];
                const int64_t pos = k - v.tile_nnz_ptr[t];
                CHECK(pos >= cp[lc] && pos < cp[lc + 1], "entry outside its column's range");
                if (k > v.tile_nnz_ptr[t]) { /* CSC order inside the tile */
                    CHECK(v.col_local[k - 1] < lc || (v.col_local[k - 1] == lc && v.row_idx[k - 1] < v.row_idx[k]),
                          "tile order");
                }
                const int64_t p = perm[k];
                CHECK(p >= 0 && p < nnz && !seen[p], "perm is a permutation");
                seen[p] = 1;
                CHECK(p >= rowptr[row] && p < rowptr[row + 1], "perm row");
                CHECK(colind[p] == col && val[p] == v.val[k], "perm column and value");
            }
        }
    }
    /* Row-block height tuning on the same structure. */
    int32_t Rt = 0, cR[10], ok_count = 0;
    int64_t cnrb[10], cT[10];
    double ccv[10], cmx[10];
    uint8_t cok[10];
    const int nc = cg_tune_row_height(n, rowptr, colind, C, 16384, 4, &Rt, 10, cR, cnrb, cT, ccv, cmx, cok);
    CHECK(nc == 10, "tune returns 10 candidates: %d %s", nc, cg_last_error());
    for (int i = 0; i < 10; ++i) {
        CHECK(cR[i] == (32 << i) && cnrb[i] == (n + cR[i] - 1) / cR[i] && cT[i] >= 1 && ccv[i] >= 0.0, "table");
        ok_count += cok[i];
    }
    CHECK(Rt >= 32 && Rt <= 16384 && (ok_count == 0 ? Rt == 32 : 1), "tuned height %d", Rt);
    free(seen);
    free(colptr);
    free(perm);
    cg_tilecsc_free(A);
    free(rowptr);
    free(colind);
    free(val);
}

static void check_errors(void) {
    const int64_t rp[4] = {0, 2, 3, 5};
    const int32_t ci[5] = {0, 1, 1, 0, 2};
    const int32_t unsorted[5] = {1, 0, 1, 0, 2};
    const int32_t dup[5] = {0, 0, 1, 0, 2};
    const int32_t outside[5] = {0, 1, 1, 0, 3};
    double v[5] = {1, 2, 3, 4, 5};
    cg_tilecsc* A = NULL;
    CHECK(cg_tilecsc_from_csr(3, rp, unsorted, v, 2, 2, &A) == CG_EINVAL && !A, "unsorted");
    CHECK(cg_tilecsc_from_csr(3, rp, dup, v, 2, 2, &A) == CG_EINVAL && !A, "duplicate");
    CHECK(cg_tilecsc_from_csr(3, rp, outside, v, 2, 2, &A) == CG_EINVAL && !A, "column outside");
    CHECK(cg_tilecsc_from_csr(0, rp, ci, v, 2, 2, &A) == CG_EINVAL && !A, "n = 0");
    CHECK(cg_tilecsc_from_csr(3, rp, ci, v, 0, 2, &A) == CG_EINVAL && !A, "R = 0");
    CHECK(cg_tilecsc_from_csr(3, rp, ci, v, 16385, 2, &A) == CG_EINVAL && !A, "R too tall");
    CHECK(cg_tilecsc_from_csr(3, rp, ci, v, 2, 257, &A) == CG_EINVAL && !A, "C too wide");
    CHECK(cg_tilecsc_from_csr(3, NULL, ci, v, 2, 2, &A) == CG_EINVAL && !A, "NULL rowptr");
    CHECK(cg_tilecsc_from_csr(3, rp, ci, v, 2, 2, NULL) == CG_EINVAL, "NULL out");
    v[3] = NAN;
    CHECK(cg_tilecsc_from_csr(3, rp, ci, v, 2, 2, &A) == CG_EINVAL && !A, "NaN value");
    v[3] = INFINITY;
    CHECK(cg_tilecsc_from_csr(3, rp, ci, v, 2, 2, &A) == CG_EINVAL && !A, "infinite value");
    const int64_t bad_rp[4] = {0, 3, 2, 5};
    v[3] = 4.0;
    CHECK(cg_tilecsc_from_csr(3, bad_rp, ci, v, 2, 2, &A) == CG_EINVAL && !A, "decreasing rowptr");
    CHECK(strlen(cg_last_error()) > 0, "message");
    int32_t R = 0;
    CHECK(cg_tune_row_height(3, rp, outside, 2, 256, 1, &R, 0, NULL, NULL, NULL, NULL, NULL, NULL) < 0, "tune");
    CHECK(cg_tune_row_height(3, rp, ci, 0, 256, 1, &R, 0, NULL, NULL, NULL, NULL, NULL, NULL) < 0, "tune C");
    int32_t k = -1;
    const uint8_t codes[4] = {2, 1, 3, 0};
    CHECK(cg_select_reuse_interval(codes, 2, 2, 0.1, &k, 0, NULL, NULL) < 0, "code 3");
    CHECK(cg_select_reuse_interval(NULL, 2, 2, 0.1, &k, 0, NULL, NULL) < 0, "NULL codes");
}

static void check_reuse(int32_t nrec, int64_t ncb) {
    uint8_t* codes = (uint8_t*)malloc((size_t)(nrec * ncb));
    for (int64_t i = 0; i < nrec * ncb; ++i) codes[i] = (uint8_t)(rnd() % 3u);
    int32_t kstar = -1, intervals[40];
    double fractions[40];
    const int nk = cg_select_reuse_interval(codes, nrec, ncb, 0.1, &kstar, 40, intervals, fractions);
    CHECK(nk >= 1 && kstar >= 1, "reuse %d: %s", nk, cg_last_error());
    for (int i = 0; i < nk && i < 40; ++i)
        CHECK(intervals[i] == (1 << i) && fractions[i] >= 0.0 && fractions[i] <= 1.0, "reuse table");
    free(codes);
}

int main(void) {
    rng_state = 12345;
    check_layout(1, 0, 0, 1, 1);
    check_layout(5, 2, 0, 2, 2);
    check_layout(37, 4, 5, 4, 8);           /* empty rows, ragged blocks */
    check_layout(300, 6, 7, 16, 16);
    check_layout(1000, 8, 0, 300, 32);      /* a height that is not a power of two */
    check_layout(3000, 5, 11, 512, 256);    /* wide tiles, tall blocks */
    check_layout(2500, 3, 0, 16384, 64);    /* one row block taller than the matrix */
    check_layout(20000, 8, 13, 32, 32);     /* large enough for the builder's worker threads */
    check_errors();
    check_reuse(1, 1);
    check_reuse(37, 5);
    check_reuse(300, 64);
    printf(failures ? "host_sanitize: %d failure(s)\n" : "host_sanitize: ok\n", failures);
    return failures ? 1 : 0;
}
