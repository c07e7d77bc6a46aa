/*
 * A plain C99 consumer of libmpcg's C ABI (include/mpcg.h), using only the
 * calls that need no GPU: the Tile-CSC builder and its views, argument
 * validation with cg_last_error, row-block height tuning and the reuse
 * interval selection. Prints one "key v0 v1 ..." line per quantity; the test
 * that compiles and runs it compares them with values derived by hand and
 * with the CPU oracle.
 */
#include <stdio.h>
#include <stdlib.h>

#include "mpcg.h"

static void print_i64(const char* key, const int64_t* v, int64_t n) {
    printf("%s", key);
    for (int64_t i = 0; i < n; ++i) printf(" %lld", (long long)v[i]);
    printf("\n");
}

static void print_i32(const char* key, const int32_t* v, int64_t n) {
    printf("%s", key);
    for (int64_t i = 0; i < n; ++i) printf(" %d", (int)v[i]);
    printf("\n");
}

static void print_u16(const char* key, const uint16_t* v, int64_t n) {
    printf("%s", key);
    for (int64_t i = 0; i < n; ++i) printf(" %u", (unsigned)v[i]);
    printf("\n");
}

static void print_u8(const char* key, const uint8_t* v, int64_t n) {
    printf("%s", key);
    for (int64_t i = 0; i < n; ++i) printf(" %u", (unsigned)v[i]);
    printf("\n");
}

int main(void) {
    /* 5 x 5 tridiagonal (2, -1) in CSR, 2 x 2 tiles. */
    const int64_t rowptr[6] = {0, 2, 5, 8, 11, 13};
    const int32_t colind[13] = {0, 1, 0, 1, 2, 1, 2, 3, 2, 3, 4, 3, 4};
    const double val[13] = {2, -1, -1, 2, -1, -1, 2, -1, -1, 2, -1, -1, 2};
    cg_tilecsc* A = NULL;
    if (cg_tilecsc_from_csr(5, rowptr, colind, val, 2, 2, &A) != CG_OK) {
        printf("error build %s\n", cg_last_error());
        return 1;
    }
    cg_tilecsc_view v;
    if (cg_tilecsc_get_view(A, &v) != CG_OK) return 1;
    printf("sizes %lld %lld %lld %d %d\n", (long long)v.n, (long long)v.T, (long long)v.nnz, (int)v.R, (int)v.C);
    print_i64("tile_row_ptr", v.tile_row_ptr, (v.n + v.R - 1) / v.R + 1);
    print_i32("tile_col_idx", v.tile_col_idx, v.T);
    print_i64("tile_nnz_ptr", v.tile_nnz_ptr, v.T + 1);
    print_u16("row_idx", v.row_idx, v.nnz);
    print_u8("col_local", v.col_local, v.nnz);
    printf("val");
    for (int64_t i = 0; i < v.nnz; ++i) printf(" %.17g", v.val[i]);
    printf("\n");
    int32_t* colptr = (int32_t*)malloc(sizeof(int32_t) * (size_t)(v.T * (v.C + 1)));
    int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (size_t)v.nnz);
    if (!colptr || !perm || cg_tilecsc_col_ptr(A, colptr) != CG_OK || cg_tilecsc_perm(A, perm) != CG_OK) return 1;
    print_i32("col_ptr", colptr, v.T * (v.C + 1));
    print_i64("perm", perm, v.nnz);
    free(colptr);
    free(perm);
    cg_tilecsc_free(A);

    /* Invalid input: columns out of order in row 1. */
    const int32_t bad[13] = {0, 1, 1, 0, 2, 1, 2, 3, 2, 3, 4, 3, 4};
    cg_tilecsc* B = NULL;
    const int rc = cg_tilecsc_from_csr(5, rowptr, bad, val, 2, 2, &B);
    printf("unsorted_rc %d %d\n", rc, B == NULL ? 1 : 0);
    printf("unsorted_msg %s\n", cg_last_error());

    /* Row-block height tuning: ten candidates, none admissible here (too few
     * row blocks), so the fallback height 32. */
    int32_t R = 0;
    const int ncand = cg_tune_row_height(5, rowptr, colind, 2, 256, 1024, &R, 0, NULL, NULL, NULL, NULL, NULL, NULL);
    printf("tune %d %d\n", ncand, (int)R);

    /* Reuse interval: two column blocks, four records; block 0 moves up
     * (code 2 -> 0) at record 1, block 1 never changes. */
    const uint8_t codes[8] = {2, 1, 0, 1, 0, 1, 0, 1};
    int32_t kstar = -1, intervals[4];
    double fractions[4];
    const int nk = cg_select_reuse_interval(codes, 4, 2, 0.1, &kstar, 4, intervals, fractions);
    printf("reuse %d %d", nk, (int)kstar);
    for (int i = 0; i < nk && i < 4; ++i) printf(" %d:%.17g", (int)intervals[i], fractions[i]);
    printf("\n");
    printf("version %d\n", cg_version());

    /* Bandwidth references: argument errors come back before any device call. */
    double sink[1];
    printf("stream_rc %d %d %d %d %d\n", cg_stream_read(NULL, 16, sink, 1, NULL),
           cg_stream_copy(val, NULL, 16, 1, NULL), cg_stream_mix(val, 15, NULL, 0, sink, 1, NULL),
           cg_stream_mix(val, 16, NULL, 16, sink, 1, NULL), cg_stream_mix(NULL, 16, NULL, 0, sink, 0, NULL));
    return 0;
}
