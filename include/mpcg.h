/*
 * mpcg.h -- C ABI of the mixed-precision Tile-CSC Conjugate Gradient library
 * for AMD Instinct MI355X (gfx950).
 *
 * The operations follow "EvoCG: Self-Evolving Precision Control for Faster
 * Conjugate Gradient" (Zhai et al.):
 *   - Tile-CSC storage: Sec. 3.3 and Fig. 4(a)/(b);
 *   - three resident value streams (FP64, FP32, BF16) selected per tile:
 *     Sec. 3.3.2 and Sec. 4.8 "Memory cost";
 *   - the precision action encoding {0, 1, 2} = {FP64, FP32, BF16}: Eq. (9);
 *   - the mixed-precision product y = (A + E(a)) p: Eq. (2) and Eq. (5);
 *   - the CG recurrence: Sec. 2.1, Eq. (1), Fig. 1 and Algorithm 1's solver
 *     lines; Jacobi-preconditioned CG: Sec. 4.6;
 *   - the stopping rule ||r_k||/||r_0|| <= tol or k = max_iter: Sec. 4.1.
 *
 * Conventions for every entry point:
 *   - Return value: CG_OK (0) on success, a positive status from cg_solve,
 *     or a negative error code. No entry point aborts; on error,
 *     cg_last_error() returns a message naming the bad argument (the message
 *     is per calling thread and valid until that thread's next call).
 *   - "host" pointers are ordinary CPU memory; "device" pointers are HIP
 *     device memory of the GPU the handle was created on (for example the
 *     data pointer of a torch tensor on that GPU).
 *   - A stream argument is a hipStream_t passed as void*; NULL means the
 *     default stream.
 *   - All device-side indices are 32-bit: a handle accepts at most
 *     2^31 - 1 nonzeros and 2^31 - 1 non-empty tiles.
 *   - Handles are not thread-safe: calls on one handle must not overlap.
 */
#ifndef MPCG_H
#define MPCG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    CG_OK = 0,
    CG_NOT_CONVERGED = 1, /* cg_solve stopped at maxit */
    CG_BREAKDOWN = 2,     /* cg_solve met p.q <= 0 or a non-finite scalar */
    CG_EINVAL = -1,       /* invalid argument or input data */
    CG_ENOMEM = -2,       /* host or device allocation failed */
    CG_EDEVICE = -3,      /* a HIP runtime call failed */
    CG_EINTERNAL = -4
};

/* Precision codes of a tile (Eq. (9)). */
enum { CG_FP64 = 0, CG_FP32 = 1, CG_BF16 = 2 };

/* Opaque host-side canonical Tile-CSC matrix. */
typedef struct cg_tilecsc cg_tilecsc;
/* Opaque solver handle: device-resident matrix, value planes, map, CG state. */
typedef struct cg_handle cg_handle;

/*
 * Read-only view of a canonical Tile-CSC matrix (Sec. 3.3, Fig. 4):
 *   tile (I, J) covers rows [I*R, (I+1)*R) and columns [J*C, (J+1)*C);
 *   non-empty tiles are listed row block by row block, column blocks
 *   ascending; tile t owns nonzeros tile_nnz_ptr[t] .. tile_nnz_ptr[t+1]-1,
 *   stored column by column (CSC) with row offsets ascending in a column.
 * Pointers are owned by the library object the view came from.
 */
typedef struct {
    int64_t n;                    /* rows (= columns) */
    int64_t T;                    /* non-empty tiles */
    int64_t nnz;
    int32_t R, C;                 /* tile height in [1, 16384], width in [1, 256] */
    const int64_t* tile_row_ptr;  /* [ceil(n/R) + 1] */
    const int32_t* tile_col_idx;  /* [T] column-block index */
    const int64_t* tile_nnz_ptr;  /* [T + 1] */
    const uint16_t* row_idx;      /* [nnz] row offset inside the row block */
    const uint8_t* col_local;     /* [nnz] column offset inside the tile */
    const double* val;            /* [nnz] FP64 values in canonical order */
} cg_tilecsc_view;

/*
 * Build the canonical Tile-CSC form of a square CSR matrix (Sec. 3.3).
 *   n       : rows and columns, n >= 1.
 *   rowptr  : host int64[n+1], rowptr[0] = 0, non-decreasing.
 *   colind  : host int32[nnz], strictly increasing inside each row, in [0, n).
 *   val     : host double[nnz], finite (explicit zeros are kept as entries).
 *   R, C    : tile shape: height R in [1, 16384] (the paper's candidates of
 *             Sec. 3.3.3 reach 16384), width C in [1, 256].
 *   out     : receives a library-owned object; free with cg_tilecsc_free.
 * Inputs are read only and may be freed after the call.
 * Errors: CG_EINVAL (bad sizes, unsorted or duplicate columns, non-finite
 * values, more than 2^31 - 1 nonzeros), CG_ENOMEM.
 */
int cg_tilecsc_from_csr(int64_t n, const int64_t* rowptr, const int32_t* colind,
                        const double* val, int32_t R, int32_t C, cg_tilecsc** out);

/* Fill *view with pointers into A (valid until cg_tilecsc_free(A)). */
int cg_tilecsc_get_view(const cg_tilecsc* A, cg_tilecsc_view* view);

/* Intra-tile column pointers (Fig. 4(b) colPtr, unpadded): host int32[T*(C+1)],
 * entry t*(C+1)+c is the start of local column c relative to the tile's first
 * nonzero. */
int cg_tilecsc_col_ptr(const cg_tilecsc* A, int32_t* out);

/* CSR position of every canonical nonzero: host int64[nnz]. */
int cg_tilecsc_perm(const cg_tilecsc* A, int64_t* out);

void cg_tilecsc_free(cg_tilecsc* A);

/*
 * Row-block height tuning (Sec. 3.3.3 "Cross-Level Balance Tuning"): the
 * tile width C stays fixed and the height R is searched over the paper's
 * candidates 32, 64, ..., 16384 so that row blocks hold similar numbers of
 * non-empty tiles. The paper names no measure; here it is the coefficient of
 * variation (population standard deviation over mean) of the non-empty tile
 * counts of the ceil(n/R) row blocks, computed as sqrt(m S2 - S1^2) / S1 from
 * the exact integer sums S1 = sum c, S2 = sum c^2 over m row blocks. A
 * candidate is admissible when R <= max_R (every candidate is a height that
 * cg_tilecsc_from_csr and cg_create accept) and it leaves at least
 * min_row_blocks row blocks; the tuned R is
 * the admissible candidate with the smallest coefficient of variation (ties
 * to the smaller R), or 32 when none is admissible.
 *   n, rowptr, colind : square CSR structure as for cg_tilecsc_from_csr
 *                       (host; values are not needed).
 *   C                 : tile width in [1, 256].
 *   max_R, min_row_blocks : admissibility bounds (min_row_blocks >= 1).
 *   R_out             : receives the tuned height.
 *   cap               : entries available in each table array (0 allowed).
 *   cand_R, cand_nrb, cand_T, cand_cv, cand_max_ratio, cand_ok : one entry per
 *                       candidate, in candidate order: height, row blocks,
 *                       non-empty tiles, coefficient of variation, largest
 *                       count over the mean, admissible (0/1). Any may be NULL.
 * Returns the number of candidates (10) or a negative error (CG_EINVAL for
 * bad sizes or a column outside [0, n)).
 */
int cg_tune_row_height(int64_t n, const int64_t* rowptr, const int32_t* colind, int32_t C, int32_t max_R,
                       int64_t min_row_blocks, int32_t* R_out, int32_t cap, int32_t* cand_R,
                       int64_t* cand_nrb, int64_t* cand_T, double* cand_cv, double* cand_max_ratio,
                       uint8_t* cand_ok);

/*
 * The paper's own SpMV numerics, as options of cg_create (bits of
 * cg_options.p1; 0 = the default product, which rounds only the matrix):
 *   CG_P1_ROUND_VECTOR : the vector entry p_j is rounded to its tile's
 *       precision before the product, as the action sets the precision of the
 *       vector tile together with its column block (Eq. (9), Eq. (10)).
 *       FP32 and BF16 are each one round-to-nearest-even step from FP64.
 *       Products and sums stay FP64. The true-residual product of cg_solve
 *       (r0 = b - A x0) never rounds.
 *   CG_P1_COLUMN_SCALE : the FP32 and BF16 values of column j are stored as
 *       fl(a_ij / s_j) and multiplied back by s_j in FP64, one factor per
 *       column (Sec. 3.3.2, "Intra-Tile CSC Execution"). The factor is not
 *       given by the paper; here s_j = 2^e_j with e_j the binary exponent of
 *       the column's largest |a_ij| (max = m 2^e_j, 0.5 <= m < 1; e_j = 0 for
 *       a column without a nonzero value), so the stored values stay inside
 *       the reduced formats' range and scaling is exact. The FP64 values are
 *       not scaled. Costs 2 bytes per row of extra SpMV traffic.
 *   CG_P1_PAD_COLUMNS  : every local column with an odd number of nonzeros
 *       gets one sentinel entry (row offset R, value +0.0) after its last
 *       nonzero, as in Fig. 4(b); the SpMV skips sentinels. Requires R <= 255.
 *       cg_get_sizes and cg_export_layout then report the padded layout.
 */
enum { CG_P1_ROUND_VECTOR = 1, CG_P1_COLUMN_SCALE = 2, CG_P1_PAD_COLUMNS = 4 };

/* Options for cg_create. Zero-initialise and set what you need. */
typedef struct {
    int32_t jacobi;      /* 1: Jacobi-preconditioned CG (Sec. 4.6), M = diag(A) */
    int32_t window;      /* iterations enqueued between stop-flag polls; 0 = default (16) */
    int32_t use_graph;   /* 1: replay each window as a captured HIP graph; 0 = plain launches;
                            -1 = default (graph) */
    int32_t p1;          /* CG_P1_* bits: the paper's own SpMV numerics (above); 0 = off */
    int32_t col_slices;  /* column slices S in [0, 64]: 0 = automatic, 1 = none (below) */
    int32_t single_block; /* cg_solve on one workgroup: 0 = automatic for small
                             systems, 1 = whenever supported, -1 = never (below) */
    int32_t stage_x;     /* 1: stage each SpMV batch's vector segments in LDS (below); 0 = off */
    int32_t reserved[1];
} cg_options;

/*
 * Vector segments staged in LDS (cg_options.stage_x = 1): before the SpMV
 * sweeps a batch of up to 64 tiles, it copies the x segments of the batch's
 * distinct column blocks (C entries each) into LDS, and the sweep reads every
 * x_j from there instead of gathering it from memory (Sec. 3.3.2 "Intra-Tile
 * CSC Execution" amortises the x_j loads of a column in the same way). Only
 * batches whose distinct column blocks hold no more entries than the batch has
 * nonzeros and fit 8 KiB are staged; the others gather as usual. Requires C a
 * power of two and none of the CG_P1_* options (otherwise ignored). Results are
 * the same products in the same order. On MI355X the gathers mostly hit the
 * L2 and the stage costs occupancy, so it is off by default.
 */

/*
 * Column slices (cg_options.col_slices = S > 1): the SpMV takes the tiles in S
 * groups of consecutive column blocks, one after the other, so that the part
 * of x a group gathers can stay in the L2 of the XCDs that sweep it. This is
 * for matrices whose columns scatter over an x much larger than one XCD's
 * L2, such as random sparsity. Each slice writes its own partial product
 * (S * 8n more bytes written, and read once more, per product). The sums are
 * formed in a fixed order: the SpMV result equals the unsliced one within
 * rounding. Every schedule, Jacobi and the CG_P1_* options are supported. The
 * device keeps the tiles in slice order and its map kernels work in that
 * order; maps, scores, window maps, the map trace and cg_export_layout use the
 * canonical tile order as everywhere else (the library translates at the call).
 * Automatic (0): S = ceil(8n / L2) (at most 64), with L2 the L2 cache of one
 * XCD (4 MiB on MI355X), when x does not fit that L2 and at least half of the
 * nonzeros lie more than L2 / 16 entries (a quarter of the L2 each side) from
 * the diagonal; otherwise no slices. On a random power-law matrix with
 * n = 4e6 that picks S = 8, the fastest of S = 1, 2, ..., 64 measured there;
 * banded and stencil matrices, which gather near the diagonal, get none.
 * cg_get_options reports the choice.
 */

/*
 * Row blocks taller than 256 rows (R in [257, 16384], Sec. 3.3.3): the device
 * runs the matrix as slabs of R' rows, R' the largest divisor of R not above
 * 256, so that a slab's rows fit one wavefront's accumulators. Each canonical
 * R x C tile is stored as the non-empty R' x C pieces of its slabs; all pieces
 * of a tile share the tile's precision, so the per-tile map, the rules and
 * the product are those of the R x C tiles. Maps, scores, traces, window maps
 * and cg_export_layout are in canonical tiles; the magnitude rule takes the
 * largest |a_ij| over the whole tile. CG_P1_PAD_COLUMNS needs R <= 255.
 */

/*
 * Single-workgroup solve (cg_options.single_block): cg_solve runs all its
 * iterations in one kernel launch of one 1024-thread workgroup, with
 * workgroup barriers between the SpMV, update and direction phases instead of
 * three launches per iteration. For systems so small that launch latency, not
 * bandwidth, bounds an iteration. Same arithmetic, stop tests, history,
 * breakdown rule and map trace as the multi-launch solve. Supported with
 * static maps (including the magnitude rule's), the residual schedule and
 * Jacobi, without column slices or CG_P1_* options, for at most 12288 rows
 * (the workgroup keeps p in LDS); elsewhere cg_solve uses the multi-launch
 * path whatever the option says. The option also sizes the handle's row
 * groups for one workgroup (about 16 groups of up to 256 rows). Automatic
 * (0) picks it for at most 24576 stored entries and 8192 rows, where it is
 * no slower than three launches per iteration; its time grows with the
 * entries, so larger systems run faster on the multi-launch path.
 */

/*
 * Threads: handles share no state, so different handles may be used at the
 * same time from different host threads; calls on one handle must not
 * overlap. cg_last_error reports the calling thread's last error.
 */

/*
 * Create a solver handle on the current HIP device.
 *   A             : canonical matrix; copied to library-owned device memory
 *                   (index arrays, the FP64 values, and the FP32 and BF16 value
 *                   planes rounded on the device by round-to-nearest-even from
 *                   FP64). A may be freed right after the call.
 *   precision_map : host uint8[T] with codes 0/1/2, or NULL for all FP64.
 *   opt           : NULL for defaults.
 *   stream        : stream for the set-up copies and kernels.
 * Errors: CG_EINVAL (map code > 2, bad layout, n >= 2^28 or T or nnz >= 2^31,
 * no nonzeros, Jacobi with a zero or missing diagonal entry, unknown p1 bits, padding with
 * R > 255, col_slices outside [0, 64], single_block outside [-1, 1], stage_x outside [0, 1]),
 * CG_ENOMEM, CG_EDEVICE.
 */
int cg_create(const cg_tilecsc* A, const uint8_t* precision_map, const cg_options* opt,
              void* stream, cg_handle** out);

/* Free a handle and all its device memory; waits for the device first.
 * NULL is accepted. The handle must not be used afterwards. */
int cg_destroy(cg_handle* h);

/* Replace the active per-tile map (uint8[T], codes 0..2) without touching the
 * value planes (Sec. 3.3.2: switching reads another stream, nothing is
 * re-uploaded from the host). The SpMV reads a packed copy of the selected
 * values (each tile's values at its map precision, tile after tile), which is
 * rebuilt on the device from the planes, together with one 4-byte offset per
 * tile. on_device = 0: host pointer; 1: device pointer (copied through the
 * host and validated like a host map). Clears any schedule. Synchronous with
 * respect to the host. Errors: CG_EINVAL (NULL argument, a code > 2),
 * CG_EDEVICE. */
int cg_set_precision_map(cg_handle* h, const uint8_t* map, int32_t on_device);

/* Copy the active map to host uint8[T]. Under a uniform residual schedule the
 * map reported is that stage's precision for every tile. */
int cg_get_active_map(const cg_handle* h, uint8_t* out);

/* Static magnitude rule, computed on the device: ratio_t = max |a_ij| over the
 * tile / max |a_ii| over the whole diagonal (FP64 division); BF16 if
 * ratio_t < t_bf16, FP32 if ratio_t < t_fp32, else FP64. Sets the active map
 * and clears any schedule. Requires t_bf16 <= t_fp32. */
int cg_map_from_magnitude(cg_handle* h, double t_bf16, double t_fp32);

/* One-way residual schedule (uniform over tiles): precision prec[0] until
 * rho_k = ||r_k||/||r_0|| <= thresholds[0] has been seen, then prec[1] until
 * rho_k <= thresholds[1], ... ; a stage once reached is kept. nstage >= 1 is
 * the number of precisions; thresholds has nstage-1 entries. Applies to
 * cg_solve; cg_spmv uses prec[0]. */
int cg_set_schedule_residual(cg_handle* h, int32_t nstage, const double* thresholds,
                             const uint8_t* prec);

/* Per-segment max|p| rule (Sec. 4.7, the residual-threshold rule the paper
 * compares against; its setting is lo = eps/10, hi = eps for the tolerance
 * eps): each tile is given BF16 if the largest |p_j| of its column block's
 * segment of the multiplied vector is < lo, FP32 if it is < hi, else FP64.
 * In cg_solve the rule is evaluated on the direction p_k at every iteration k
 * that is a multiple of `period` and the map is reused in between (Sec. 3.4
 * "Interval Reuse Scheduling"); the map trace gets one entry per evaluation.
 * cg_spmv applies the rule to its input x. The value planes are read directly
 * (no repacking per evaluation). Requires lo <= hi, no NaN (infinities
 * allowed), period >= 1. Errors: CG_EINVAL, CG_ENOMEM, CG_EDEVICE. */
int cg_set_schedule_pmag(cg_handle* h, double lo, double hi, int32_t period);

/* With enable != 0, the next cg_solve under the max|p| rule keeps every
 * evaluation's column-block codes (uint8[ceil(n/C)] each, 0/1/2) in device
 * memory for cg_get_column_codes. */
int cg_record_column_codes(cg_handle* h, int32_t enable);

/* Copies up to `cap` recorded evaluations (row e = the codes used from
 * iteration e * period) into host out[cap][ceil(n/C)]; returns the number
 * recorded by the last solve (0 when nothing was recorded). */
int cg_get_column_codes(const cg_handle* h, int32_t cap, uint8_t* out);

/* Offline reuse interval K* (Sec. 3.4 "Interval Reuse Scheduling"), host only.
 * codes: host uint8[nrec][ncb], the column-block codes of a per-iteration run
 * (0 = FP64, 1 = FP32, 2 = BF16). An upward transition is a (k >= 1, J) with
 * codes[k][J] < codes[k-1][J]; reusing the window-start decision over windows
 * of K iterations delays it when codes[(k/K)*K][J] > codes[k][J]. For
 * K = 1, 2, 4, ... below max(nrec, 2) the delayed fraction (0 without upward
 * transitions) is written to intervals[c], fractions[c] for c < cap (either
 * may be NULL); *kstar = the largest K whose fraction is < max_fraction (the
 * paper uses 0.1). Returns the number of candidates. Errors: CG_EINVAL (NULL
 * codes or kstar, negative sizes, a code > 2). */
int cg_select_reuse_interval(const uint8_t* codes, int32_t nrec, int64_t ncb, double max_fraction,
                             int32_t* kstar, int32_t cap, int32_t* intervals, double* fractions);

/* Windowed per-tile rule (Sec. 3.4 "Interval Reuse Scheduling": a map chosen
 * at a window start is kept for the window). At every k with k % period == 0,
 * v_t = scores[t] * rho_k and tile t gets BF16 if v_t > hi, FP32 if v_t > lo,
 * else FP64. scores: host double[T], copied. Requires period >= 1, lo <= hi. */
int cg_set_schedule_tile_rule(cg_handle* h, int32_t period, const double* scores, double hi,
                              double lo);

/* Apply the tile rule of cg_set_schedule_tile_rule once at the given rho and
 * make the result the active map (the schedule stays set). */
int cg_eval_tile_rule(cg_handle* h, double rho);

/* Window maps of the windowed per-tile rule (Sec. 3.4: a map chosen at a
 * window start holds for the window), recorded by later solves for tests and
 * analysis. cg_record_window_maps(h, cap) keeps the map of each of the first
 * cap windows of every solve in cap * T bytes of device memory (cap = 0 stops
 * recording and frees them). cg_get_window_maps copies the first min(cap,
 * recorded) maps of the last solve to host uint8[windows][T] (canonical tile
 * order; out may be NULL) and returns the number recorded; 0 without the tile
 * rule or without recording. Errors: CG_EINVAL (NULL h, cap < 0), CG_ENOMEM. */
int cg_record_window_maps(cg_handle* h, int32_t cap);
int cg_get_window_maps(const cg_handle* h, int32_t cap, uint8_t* out);

/* Remove any schedule; the active map stays as it is. */
int cg_clear_schedule(cg_handle* h);

/*
 * y = (A + E(map)) x (Eq. (5)): each tile's values are read from the plane
 * its active map entry selects, widened exactly, and every product and sum is
 * formed in FP64. The map is the active map, or under a schedule: the first
 * stage's precision (residual schedule), the max|p| rule applied to x, the
 * tile rule's current map. With the handle's CG_P1_* options the product
 * follows them (x_j rounded to the tile's precision, column scale, padding).
 *   x, y : device double[n]; y must not overlap x. Asynchronous on stream.
 * Errors: CG_EINVAL on NULL or overlapping pointers.
 */
int cg_spmv(cg_handle* h, const double* x, double* y, void* stream);

/*
 * Solve A x = b by CG (or Jacobi-PCG when the handle was created with
 * opt.jacobi) with the mixed-precision SpMV under the active map or schedule.
 *   b          : device double[n].
 *   x0         : device double[n] initial guess, or NULL for zero.
 *                r0 = b - A x0 uses the exact FP64 values.
 *   tol        : stop when ||r_k||/||r_0|| <= tol (recurrence residual), tol >= 0.
 *   maxit      : iteration cap, maxit >= 0.
 *   x          : device double[n] receiving the last iterate; may equal x0.
 *                b, x0 and x need only the alignment of a double: the
 *                solve reads b and x0 and writes x entry by entry, and runs
 *                its iterations on the handle's own vectors.
 *   iterations : host int32, completed iterations K.
 *   res_hist   : host double[maxit+1] receiving rho_0 .. rho_K (rho_0 = 1;
 *                a zero r0 gives K = 0 and rho_0 = 0), or NULL.
 *   stream     : the solve is ordered after prior work on stream; the call
 *                returns when the solve has finished.
 * Returns CG_OK (converged), CG_NOT_CONVERGED (K = maxit), CG_BREAKDOWN
 * (p.q <= 0 or non-finite alpha/beta; x holds the last iterate; a NaN or an
 * infinity in b or x0 gives rho_0 = 1 and, past the tolerance and cap tests,
 * a breakdown with K = 0), or an error:
 * CG_EINVAL (NULL h, b, x or iterations, tol < 0, maxit < 0), CG_ENOMEM,
 * CG_EDEVICE.
 */
int cg_solve(cg_handle* h, const double* b, const double* x0, double tol, int32_t maxit,
             double* x, int32_t* iterations, double* res_hist, void* stream);

/*
 * True relative residual ||b - A x||_2 / ||b||_2 with the exact FP64 matrix
 * values (EvoCG paper Sec. 4.3: the final residual is recomputed in FP64
 * after the solve, outside the timed region), whatever the active map or
 * schedule; ||b - A x||_2 when b = 0.
 *   b, x   : device double[n] (any double alignment; not modified).
 *   out    : host double receiving the value.
 *   stream : the computation is ordered after prior work on stream; the call
 *            returns when the value is on the host.
 * The per-block partial sums live in the handle's memory (allocated by
 * cg_create). Errors: CG_EINVAL (NULL argument), CG_EDEVICE.
 */
int cg_true_residual(cg_handle* h, const double* b, const double* x, double* out, void* stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): cg_true_residual without
 * any allocation or host synchronisation. Same value as cg_true_residual,
 * from the same kernels, written to out, a caller-owned device double, and
 * enqueued on stream (the call returns at once; read out after the stream).
 * The per-block partial sums live in a static device array of 65,536 doubles
 * (512 KiB) per GPU, held until the process ends: every call on one GPU
 * shares it, so calls that overlap on one GPU (other streams, other host
 * threads) race. A launch needing more than 65,536 partial sums is rejected
 * with CG_EINVAL (no handle built by cg_create needs that many).
 * Errors: CG_EINVAL (NULL argument, too many partial sums), CG_EDEVICE.
 */
int cg_true_residual_noalloc(cg_handle* h, const double* b, const double* x, double* out, void* stream);

/*
 * Bandwidth references (measurement aids for benchmarks; no part of the
 * method): cg_stream_read reads `bytes` from src once with 16-byte
 * non-temporal loads and writes one sum per block to sink[blocks];
 * cg_stream_copy copies `bytes` from src to dst; cg_stream_mix reads
 * read_bytes from src as cg_stream_read does (same sink) and, interleaved
 * with the reads in proportion, writes write_bytes of running sums to dst
 * with 16-byte stores (a read stream with the share of writes of a kernel
 * under study). All are asynchronous on stream, with a grid of `blocks`
 * 256-thread blocks; sink must hold `blocks` doubles. Byte counts must be
 * multiples of 16 (read and copy sizes positive; write_bytes may be 0, and
 * dst NULL then) and the pointers 16-byte aligned device memory.
 * Errors: CG_EINVAL, CG_EDEVICE.
 */
int cg_stream_read(const void* src, int64_t bytes, double* sink, int32_t blocks, void* stream);
int cg_stream_copy(const void* src, void* dst, int64_t bytes, int32_t blocks, void* stream);
int cg_stream_mix(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, double* sink, int32_t blocks,
                  void* stream);

/* Map trace of the last cg_solve: one entry per map change (the first at
 * k = 0). Writes up to cap entries: k_out[i] (iteration the map took effect)
 * and counts_out[3*i + p] (tiles at precision p). Returns the number of
 * entries recorded (which may exceed cap), or a negative error. */
int cg_get_map_trace(const cg_handle* h, int32_t cap, int32_t* k_out, int64_t* counts_out);

/* Copy the device-resident layout back to host arrays in canonical form:
 * tile_row_ptr int64[ceil(n/R)+1], tile_col_idx int32[T], tile_nnz_ptr
 * int64[T+1], row_idx uint16[nnz], col_local uint8[nnz], and the three value
 * planes val64 double[nnz], val32 float[nnz], bf16 uint16[nnz] (bit
 * patterns). Any output pointer may be NULL to skip it. With
 * CG_P1_PAD_COLUMNS, nnz counts the sentinels (row offset R); with
 * CG_P1_COLUMN_SCALE, val32 and bf16 hold the scaled values fl(a / s_j). */
int cg_export_layout(const cg_handle* h, int64_t* tile_row_ptr, int32_t* tile_col_idx,
                     int64_t* tile_nnz_ptr, uint16_t* row_idx, uint8_t* col_local,
                     double* val64, float* val32, uint16_t* bf16);

/* Exponents e_j of the per-column scale s_j = 2^e_j (CG_P1_COLUMN_SCALE,
 * Sec. 3.3.2): host int32[n]. Without the option every e_j is 0. */
int cg_export_column_scale(const cg_handle* h, int32_t* out);

/* The options a handle runs with, after its automatic choices: col_slices
 * (the S in use, 1 for none), single_block (1 when cg_solve can run on one
 * workgroup for this handle, -1 otherwise), stage_x (1 when some batch is
 * staged), use_graph, window, jacobi and p1 as set. Errors: CG_EINVAL. */
int cg_get_options(const cg_handle* h, cg_options* out);

/* Sizes of a handle: n, T, nnz, R, C (any pointer may be NULL). */
int cg_get_sizes(const cg_handle* h, int64_t* n, int64_t* T, int64_t* nnz, int32_t* R,
                 int32_t* C);

/* Device-resident bytes held by the handle (matrix, planes, map, vectors). */
int64_t cg_device_bytes(const cg_handle* h);

/* Message of the calling thread's last failed call ("" when the last call
 * succeeded); owned by the library, valid until that thread's next call. */
const char* cg_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int cg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MPCG_H */
