// HIP runtime behind the C ABI: device-resident Tile-CSC matrix with its
// three value planes, the precision map and schedules, cg_spmv, and the
// cg_solve loop (device-resident scalars, window-wise stop polling, optional
// HIP-graph replay of each window, or one single-workgroup launch for small
// systems). Optional column slices reorder the tiles on the device; every
// map, trace and export is translated back to the canonical tile order.
//
// EvoCG paper: value-stream selection without re-quantisation (Sec. 3.3.2,
// Sec. 4.8), the per-iteration CG step (Sec. 2.1, Fig. 1), interval reuse of
// a map over a window (Sec. 3.4), device-side reductions and scalar broadcast
// plus graph replay of the solver backbone (Sec. 3.4 "Fused Execution and
// Graph Replay"), Jacobi-PCG (Sec. 4.6), stopping rule (Sec. 4.1).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "mpcg_internal.hpp"
#include "mpcg_kernels.hpp"

using mpcg::fail;
namespace dev = mpcg::dev;

namespace {

enum SchedKind { kSchedStatic = 0, kSchedResidual = 1, kSchedTileRule = 2, kSchedPMag = 3 };

struct DeviceBuffers {
    std::vector<void*> owned;
    ~DeviceBuffers() {
        for (void* p : owned) (void)hipFree(p);
    }
};

}  // namespace

struct cg_handle {
    int device = 0;
    hipStream_t stream = nullptr;  // internal stream for the solve loop
    int64_t n = 0, T = 0, nnz = 0, nrb = 0;  // canonical sizes (the caller's tiles)
    int32_t R = 0, C = 0, G = 0, rows_per_group = 0, ngroups = 0;
    // Device tiles: the canonical ones, or with R > 256 the non-empty pieces of
    // slabs of Rd rows (Rd the largest divisor of R not above 256).
    int64_t Td = 0, nrbd = 0;
    int32_t Rd = 0;
    int32_t S = 1;                 // column slices (cg_options.col_slices)
    int32_t single_block = 0;      // cg_options.single_block: 0 auto, 1 when supported, -1 never
    bool stage_x = false;          // cg_options.stage_x: vector segments staged in LDS per batch
    uint8_t* winmaps = nullptr;    // cg_record_window_maps: [winmap_cap][T] tile-rule window maps
    bool planes_map = false;       // a solve's tile rule changed the map: packed values stale until a repack
    int32_t winmap_cap = 0;
    int64_t nseg = 0;              // SpMV segments: S * ngroups (slice-major)
    std::vector<int32_t> dperm;    // device tile -> canonical tile (slices or slabs; empty: identity)
    uint8_t* dcount = nullptr;     // slabs: [Td] 1 on the first piece of every canonical tile (trace counts)
    int32_t* cptr = nullptr;       // slabs: [T + 1] pieces of canonical tile t are clist[cptr[t] .. cptr[t+1])
    int32_t* clist = nullptr;      // slabs: [Td]
    int32_t* trow = nullptr;       // [Td] device row block of every device tile
    double* qpart = nullptr;       // S > 1: [S][n_pad] partial products of the slices
    bool meta16 = false;
    bool nt_stores = false;        // CG vector stores stream past the caches (working set > kLastLevelCache)
    bool jacobi = false;
    int p1 = 0;                    // CG_P1_* options
    int16_t* colexp = nullptr;     // [n] per-column scale exponents (CG_P1_COLUMN_SCALE)
    int window = 16;
    bool use_graph = true;
    int64_t device_bytes = 0;

    // Matrix (device).
    uint64_t* win_mask = nullptr;  // [nwin]
    int32_t* win_tile = nullptr;   // [nwin]
    int64_t nwin = 0;
    int2* tent = nullptr;          // [T] SpMV tile entries: x byte offset, accumulator byte offset
    int32_t* btab = nullptr;       // [nbatch][8] SpMV batch table
    int32_t* gbatch = nullptr;     // [nseg+1] first batch of every segment (row group, slice)
    int64_t nbatch = 0;
    int32_t* xcb = nullptr;        // staged batches' distinct column blocks
    int64_t stage_doubles = 0;     // LDS vector stage of one SpMV wavefront (doubles)
    int32_t stage_shift = 0;       // log2(C / 2)
    int32_t* trp = nullptr;
    int32_t* tcol = nullptr;
    int32_t* tptr = nullptr;
    uint8_t* map = nullptr;
    void* meta = nullptr;
    double* v64 = nullptr;         // [nnz] FP64 values in storage order
    char* planes = nullptr;        // per-batch value segments (FP64, FP32, BF16)
    char* packed = nullptr;        // per-batch packed values of the active map (same offsets)
    int32_t* toff = nullptr;       // [T] packed start of every tile (see repack_kernel)
    int64_t planes_bytes = 0, packed_bytes = 0;
    std::vector<int32_t> btab_host;  // host copy of the batch table
    double* dinv = nullptr;

    // CG vectors and reduction scratch (device).
    double *x = nullptr, *r = nullptr, *p = nullptr, *q = nullptr, *z = nullptr;
    double* part_spmv = nullptr;  // one p.q partial per SpMV block
    double* part_vec = nullptr;   // two partials per vector-kernel block
    int spmv_blocks = 0, vec_blocks = 0, upd_blocks = 0;
    dev::State* st = nullptr;
    double* hist = nullptr;
    int64_t hist_cap = 0;
    int32_t* trace_k = nullptr;
    int32_t* trace_counts = nullptr;  // [entry][kTraceBlocks][3]
    int64_t trace_cap = 0;
    unsigned long long* scratch_u64 = nullptr;

    // Schedules.
    int sched = kSchedStatic;
    std::vector<double> thresholds;
    std::vector<int32_t> stage_prec;
    double* scores = nullptr;
    int32_t period = 0;
    double hi = 0.0, lo = 0.0;
    uint8_t* cbcode = nullptr;  // [ncb] max|p| rule: code per column block
    int32_t* tpcb = nullptr;    // [ncb] tiles per column block
    int64_t ncb = 0;
    double pm_lo = 0.0, pm_hi = 0.0;
    int32_t pm_period = 1;
    bool rec_cb = false;            // keep every evaluation's column-block codes
    uint8_t* cbhist = nullptr;      // [cbhist_rows][ncb]
    int64_t cbhist_rows = 0;

    // Host staging for polling.
    int32_t* pinned = nullptr;  // [2 windows][2 ints] (done, k)
    hipEvent_t ev[2] = {nullptr, nullptr};
    // The last cg_spmv / cg_true_residual launch on a caller's stream: calls
    // that rewrite the map, the packed values or the scalar state wait for it.
    hipEvent_t ev_user = nullptr;
    bool user_pending = false;  // a caller's stream: ev_user follows its last launch
    bool null_pending = false;  // the default stream: a launch since the last wait (no event needed)
    // cg_true_residual: (||r||^2, ||b||^2) partials per block and the result.
    double* part_res = nullptr;
    int64_t part_res_cap = 0;
    double* res_out = nullptr;
    double* res_host = nullptr;  // pinned

    // Captured window graph.
    hipGraphExec_t graph = nullptr;
    hipGraphExec_t graph_rule = nullptr;  // the window that ends with a max|p| evaluation (long periods)
    int graph_window = 0;
    int graph_period = 0;
    int graph_sched = -1;

    DeviceBuffers bufs;
};

namespace {

#define HIP_CHECK(expr)                                                                   \
    do {                                                                                  \
        hipError_t e_ = (expr);                                                           \
        if (e_ != hipSuccess)                                                             \
            return fail(CG_EDEVICE, std::string(#expr) + ": " + hipGetErrorString(e_));   \
    } while (0)

template <class Tp>
int dalloc(cg_handle* h, Tp** ptr, int64_t count) {
    *ptr = nullptr;
    if (count <= 0) count = 1;
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, sizeof(Tp) * (size_t)count);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(CG_ENOMEM, "device allocation of " + std::to_string(sizeof(Tp) * count) +
                                   " bytes failed: " + hipGetErrorString(e));
    }
    h->bufs.owned.push_back(p);
    h->device_bytes += (int64_t)(sizeof(Tp) * count);
    *ptr = static_cast<Tp*>(p);
    return CG_OK;
}

void dfree(cg_handle* h, void* p) {
    if (!p) return;
    auto it = std::find(h->bufs.owned.begin(), h->bufs.owned.end(), p);
    if (it != h->bufs.owned.end()) h->bufs.owned.erase(it);
    (void)hipFree(p);
}

int grid_for(int64_t work, int per_thread, int cap) {
    int64_t g = (work + (int64_t)dev::kBlock * per_thread - 1) / ((int64_t)dev::kBlock * per_thread);
    return (int)std::max<int64_t>(1, std::min<int64_t>(g, cap));
}

constexpr int kVecGridCap = 1024;
// Blocks of the update and direction kernels. Every block sums all of the
// previous kernel's partials, so fewer blocks read fewer of them: on the Q1
// 4096^2 workload 512 blocks took 575 us per iteration against 578 with 1024,
// and 594 with 256 (too few waves to keep the memory busy).
#ifndef MPCG_UPD_GRID_CAP
#define MPCG_UPD_GRID_CAP 512
#endif
constexpr int kUpdGridCap = MPCG_UPD_GRID_CAP;
#ifndef MPCG_SMALL_AUTO_NNZ
#define MPCG_SMALL_AUTO_NNZ 24576
#endif
#ifndef MPCG_SMALL_AUTO_N
#define MPCG_SMALL_AUTO_N 8192
#endif
#ifndef MPCG_SPMV_GRID_CAP
#define MPCG_SPMV_GRID_CAP 16384
#endif
constexpr int kSpmvGridCap = MPCG_SPMV_GRID_CAP;
constexpr int kResGridCap = 4096;
// MI355X's last-level (Infinity) cache. A CG iteration whose working set (the
// matrix stream at 10 bytes per nonzero and 12 per tile, and five vectors)
// exceeds it streams its vector accesses past the cache, except p's (see
// store_vec): 3-9 % faster per iteration on the 100^3 27-point and 4096^2 Q1
// workloads, and 5-6 % slower on the 128^3 Laplacian, whose 240 MB fit.
constexpr int64_t kLastLevelCache = int64_t(256) << 20;  // blocks of the column-slice residual-norm kernel
// SpMV grid: at most kSpmvPersist times the blocks the chip holds at once
// (0: one wavefront per segment up to the cap).
#ifndef MPCG_SPMV_PERSIST
#define MPCG_SPMV_PERSIST 0
#endif
constexpr int kSpmvPersist = MPCG_SPMV_PERSIST;

int vec_grid(const cg_handle* h) { return h->vec_blocks; }
int spmv_grid(const cg_handle* h) { return h->spmv_blocks; }
// Dynamic LDS of an SpMV block: one vector stage per wavefront.
size_t spmv_dyn_lds(const cg_handle* h) { return (size_t)h->stage_doubles * 8 * dev::kSpmvWaves; }

constexpr int64_t kSmallAutoNnz = MPCG_SMALL_AUTO_NNZ;
constexpr int64_t kSmallAutoN = MPCG_SMALL_AUTO_N;

// Whether the handle solves on one workgroup when its schedule allows it (the
// option, or automatically up to kSmallAutoNnz stored entries and kSmallAutoN
// rows, where one workgroup was measured no slower than three launches per
// iteration on 2D and 3D Laplacians); fixed when the handle is created, as its
// row groups are sized for it.
bool small_layout(const cg_handle* h) {
    if (h->single_block < 0 || h->S != 1 || h->p1 != 0) return false;
    if (dev::kSmallXLds && h->n > dev::kSmallMaxN) return false;  // p must fit the LDS copy
    return h->single_block > 0 || (h->nnz <= kSmallAutoNnz && h->n <= kSmallAutoN);
}

// Row-accumulator capacity of the SpMV instantiation a handle uses.
int spmv_maxrows(const cg_handle* h) { return h->rows_per_group > 128 ? 256 : h->rows_per_group > 64 ? 128 : 64; }

template <typename MetaT, int MODE, int MAXROWS, bool CB, bool P1>
const void* spmv_kernel_fn() {
    return reinterpret_cast<const void*>(&dev::spmv_tilecsc_kernel<MetaT, MODE, MAXROWS, CB, P1>);
}

// The SpMV grid: one wavefront per segment, but no more blocks than the chip
// holds at once (each XCD's wavefronts then take several segments each,
// interleaved; see spmv_tilecsc_kernel). Vector kernels use capped grids.
void plan_grids(cg_handle* h) {
    const int64_t want = std::max<int64_t>(1, (h->nseg + dev::kSpmvWaves - 1) / dev::kSpmvWaves);
    int64_t cap = kSpmvGridCap;
    if (kSpmvPersist) {
        const void* fn = h->meta16 ? (spmv_maxrows(h) == 256   ? spmv_kernel_fn<uint16_t, dev::kSpmvPlain, 256, false, false>()
                                      : spmv_maxrows(h) == 128 ? spmv_kernel_fn<uint16_t, dev::kSpmvPlain, 128, false, false>()
                                                               : spmv_kernel_fn<uint16_t, dev::kSpmvPlain, 64, false, false>())
                                   : (spmv_maxrows(h) == 256   ? spmv_kernel_fn<uint8_t, dev::kSpmvPlain, 256, false, false>()
                                      : spmv_maxrows(h) == 128 ? spmv_kernel_fn<uint8_t, dev::kSpmvPlain, 128, false, false>()
                                                               : spmv_kernel_fn<uint8_t, dev::kSpmvPlain, 64, false, false>());
        int per_cu = 0, cus = 0;
        hipDeviceProp_t prop;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, dev::kSpmvBlock, spmv_dyn_lds(h)) == hipSuccess &&
            hipGetDeviceProperties(&prop, h->device) == hipSuccess && per_cu > 0) {
            cus = prop.multiProcessorCount;
            cap = std::min<int64_t>(cap, (int64_t)per_cu * cus * kSpmvPersist);
        } else {
            (void)hipGetLastError();
        }
    }
    h->spmv_blocks = (int)std::max<int64_t>(1, std::min<int64_t>(want, cap));
    h->vec_blocks = grid_for(h->n, 8, kVecGridCap);
    const int64_t npairs = (h->n + 1) / 2;
    const int64_t per_block = (int64_t)dev::kVecBlock * dev::kVecPairs;
    // The fewest grid-stride rounds the cap allows, then the fewest blocks that
    // cover the vector in that many rounds, so the last round is not a ragged
    // one that leaves most threads idle (768 blocks on a 2^24-entry vector: 2.7
    // rounds, 591 against 575 us per Q1 iteration).
    const int64_t rounds = (npairs + per_block * kUpdGridCap - 1) / (per_block * kUpdGridCap);
    h->upd_blocks = (int)std::max<int64_t>(1, (npairs + per_block * rounds - 1) / (per_block * rounds));
}

dev::SpmvArgs spmv_args(cg_handle* h, const double* x, double* y, const int32_t* uprec) {
    dev::SpmvArgs a{};
    a.btab = h->btab;
    a.gbatch = h->gbatch;
    a.tent = h->tent;
    a.map = h->map;
    a.meta = h->meta;
    a.planes = h->planes;
    a.packed = h->packed;
    a.toff = h->toff;
    a.tcol = h->tcol;
    a.cbcode = h->sched == kSchedPMag ? h->cbcode : nullptr;
    a.win_mask = h->win_mask;
    a.win_tile = h->win_tile;
    a.x = x;
    a.y = y;
    a.b = nullptr;
    a.uprec = uprec;
    a.st = h->st;
    a.partials = h->part_spmv;
    a.n = (int32_t)h->n;
    a.rows_per_group = h->rows_per_group;
    a.ngroups = (int32_t)h->nseg;
    a.ystride = (int32_t)(h->n + (h->n & 1));
    a.nwin = (int32_t)h->nwin;
    a.colexp = (h->p1 & CG_P1_COLUMN_SCALE) ? h->colexp : nullptr;
    a.p1_round = (h->p1 & CG_P1_ROUND_VECTOR) ? 1 : 0;
    a.sentinel_row = (h->p1 & CG_P1_PAD_COLUMNS) ? h->R : -1;
    a.xcb = h->xcb;
    a.C = h->C;
    a.stage_shift = h->stage_shift;
    a.stage_doubles = (int32_t)h->stage_doubles;
    a.nt = h->nt_stores ? 1 : 0;
    // Under the windowed tile rule (and until the next repack after one of its
    // solves) each tile's values come from its precision's plane: the rule
    // changes the map every window, and reading the planes measured no slower
    // on its maps than a repack per window plus reading packed segments.
    a.planes_map = (h->sched == kSchedTileRule || h->planes_map) ? 1 : 0;
    return a;
}

template <typename MetaT, int MODE, int MAXROWS, bool CB, bool P1>
void launch_spmv_m(cg_handle* h, const dev::SpmvArgs& a, hipStream_t s) {
    if constexpr (!P1) {
        if (h->stage_doubles > 0) {  // vector segments staged in LDS (cg_options.stage_x)
            hipLaunchKernelGGL((dev::spmv_tilecsc_kernel<MetaT, MODE, MAXROWS, CB, false, true>), dim3(spmv_grid(h)),
                               dim3(dev::kSpmvBlock), spmv_dyn_lds(h), s, a, a.y, a.partials);
            return;
        }
    }
    hipLaunchKernelGGL((dev::spmv_tilecsc_kernel<MetaT, MODE, MAXROWS, CB, P1>), dim3(spmv_grid(h)),
                       dim3(dev::kSpmvBlock), 0, s, a, a.y, a.partials);
}

template <int MODE, bool CB, bool P1>
void launch_spmv_cb(cg_handle* h, const dev::SpmvArgs& a, hipStream_t s) {
    const int m = spmv_maxrows(h);
    if (h->meta16) {
        if (m == 256) launch_spmv_m<uint16_t, MODE, 256, CB, P1>(h, a, s);
        else if (m == 128) launch_spmv_m<uint16_t, MODE, 128, CB, P1>(h, a, s);
        else launch_spmv_m<uint16_t, MODE, 64, CB, P1>(h, a, s);
    } else {
        if (m == 256) launch_spmv_m<uint8_t, MODE, 256, CB, P1>(h, a, s);
        else if (m == 128) launch_spmv_m<uint8_t, MODE, 128, CB, P1>(h, a, s);
        else launch_spmv_m<uint8_t, MODE, 64, CB, P1>(h, a, s);
    }
}

// The max|p| rule's kernels take the tile precisions from the column-block
// codes; every other schedule uses the map (or a uniform precision). A handle
// with any of the paper's own numerics options runs the P1 kernels.
template <int MODE>
void launch_spmv(cg_handle* h, const dev::SpmvArgs& a, hipStream_t s) {
    if (h->p1) {
        if (a.cbcode)
            launch_spmv_cb<MODE, true, true>(h, a, s);
        else
            launch_spmv_cb<MODE, false, true>(h, a, s);
    } else if (a.cbcode) {
        launch_spmv_cb<MODE, true, false>(h, a, s);
    } else {
        launch_spmv_cb<MODE, false, false>(h, a, s);
    }
}

// Column slices: y = sum of the partial products in qpart (b - sum with b).
void launch_combine(cg_handle* h, const double* b, double* y, hipStream_t s) {
    hipLaunchKernelGGL(dev::combine_kernel, dim3(grid_for(h->n, 4, 4096)), dim3(dev::kBlock), 0, s, h->qpart,
                       h->S, (int64_t)(h->n + (h->n & 1)), b, y, h->n);
}

// Column-block codes of the max|p| rule from vector v (solve = 1: in-solve,
// trace entry k).
void launch_pmag(cg_handle* h, const double* v, int solve, hipStream_t s) {
    dev::PMagArgs a{};
    a.p = v;
    a.cbcode = h->cbcode;
    a.tpcb = h->tpcb;
    a.st = h->st;
    a.trace_k = h->trace_k;
    a.trace_counts = h->trace_counts;
    a.n = h->n;
    a.C = h->C;
    a.ncb = (int32_t)h->ncb;
    a.solve = solve;
    a.trace_cap = (int32_t)h->trace_cap;
    a.period = h->pm_period;
    a.history = solve && h->rec_cb ? h->cbhist : nullptr;
    a.lo = h->pm_lo;
    a.hi = h->pm_hi;
    // One thread per column block, one pass.
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((h->ncb + dev::kBlock - 1) / dev::kBlock, 16384));
    hipLaunchKernelGGL(dev::pmag_kernel, dim3((unsigned)blocks), dim3(dev::kBlock), 0, s, a);
}

dev::RepackArgs repack_args(const cg_handle* h) {
    dev::RepackArgs a{};
    a.btab = h->btab;
    a.tptr = h->tptr;
    a.map = h->map;
    a.planes = h->planes;
    a.packed = h->packed;
    a.toff = h->toff;
    a.win_mask = h->win_mask;
    a.win_tile = h->win_tile;
    a.nbatch = h->nbatch;
    return a;
}

// Packs the active map's values of every batch (every map change outside a solve).
void launch_repack(cg_handle* h, hipStream_t s) {
    const int64_t blocks = (h->nbatch + dev::kWavesPerBlock - 1) / dev::kWavesPerBlock;
    hipLaunchKernelGGL(dev::repack_kernel, dim3((unsigned)std::max<int64_t>(1, std::min<int64_t>(blocks, 16384))),
                       dim3(dev::kBlock), 0, s, repack_args(h));
}

// Repacks after a map written on the handle's stream; synchronous.
hipError_t repack(cg_handle* h) {
    launch_repack(h, h->stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = hipStreamSynchronize(h->stream);
    if (e == hipSuccess) h->planes_map = false;
    return e;
}

dev::VecArgs vec_args(cg_handle* h, const double* b, const double* x0) {
    dev::VecArgs a{};
    a.x = h->x;
    a.r = h->r;
    a.p = h->p;
    a.q = h->S > 1 ? h->qpart : h->q;  // with column slices the SpMV leaves partial products
    a.nq = h->S;
    a.qstride = h->n + (h->n & 1);
    a.z = h->z;
    a.dinv = h->dinv;
    a.b = b;
    a.x0 = x0;
    a.hist = h->hist;
    a.st = h->st;
    a.part_in = h->part_vec;
    a.nparts_in = vec_grid(h);
    a.part_out = h->part_vec;
    a.trace_k = h->trace_k;
    a.trace_counts = h->trace_counts;
    a.T = h->T;
    a.n = (int32_t)h->n;
    a.jacobi = h->jacobi ? 1 : 0;
    a.r_ready = 0;
    return a;
}

// Tile-rule grid: one wavefront per SpMV batch, at most 8192 blocks.
int tile_rule_grid(const cg_handle* h) {
    return (int)std::max<int64_t>(1, std::min<int64_t>((h->nbatch + dev::kWavesPerBlock - 1) / dev::kWavesPerBlock, 8192));
}

dev::MapArgs map_args(cg_handle* h, double rho, int solve) {
    dev::MapArgs a{};
    a.map = h->map;
    a.scores = h->scores;
    a.st = h->st;
    a.hist = h->hist;
    a.trace_k = h->trace_k;
    a.trace_counts = h->trace_counts;
    a.btab = h->btab;
    a.winmaps = h->winmaps;
    a.winmap_cap = h->winmap_cap;
    a.count_w = h->dcount;
    a.T = h->Td;
    a.nbatch = h->nbatch;
    a.rho = rho;
    a.solve = solve;
    return a;
}

// Writes the host-side schedule description into the device state.
int upload_schedule(cg_handle* h) {
    dev::State hs{};
    HIP_CHECK(hipMemcpy(&hs, h->st, sizeof(hs), hipMemcpyDeviceToHost));
    hs.nstage = 0;
    hs.period = 0;
    hs.spmv_uprec = -1;
    if (h->sched == kSchedResidual) {
        hs.nstage = (int32_t)h->stage_prec.size();
        for (size_t i = 0; i < h->thresholds.size(); ++i) hs.thresholds[i] = h->thresholds[i];
        for (size_t i = 0; i < h->stage_prec.size(); ++i) hs.stage_prec[i] = h->stage_prec[i];
        hs.spmv_uprec = h->stage_prec[0];
    } else if (h->sched == kSchedTileRule) {
        hs.period = h->period;
        hs.hi = h->hi;
        hs.lo = h->lo;
    }
    hs.zero_prec = 0;
    hs.uprec = hs.spmv_uprec;
    HIP_CHECK(hipMemcpy(h->st, &hs, sizeof(hs), hipMemcpyHostToDevice));
    return CG_OK;
}

void drop_graph(cg_handle* h) {
    if (h->graph) (void)hipGraphExecDestroy(h->graph);
    if (h->graph_rule) (void)hipGraphExecDestroy(h->graph_rule);
    h->graph = nullptr;
    h->graph_rule = nullptr;
    h->graph_window = 0;
    h->graph_sched = -1;
}

// Iterations per enqueued window. Under a tile rule it is a multiple of the
// rule's period, so the map steps fall on the same iterations of every window.
// A max|p| rule whose period is a multiple of the window: windows stay short
// and only the windows that end just before a multiple of the period run the
// rule (a second captured graph), so a long period does not lengthen the
// windows and with them the no-op iterations after convergence.
bool pmag_split(const cg_handle* h) {
    return h->sched == kSchedPMag && h->pm_period > h->window && h->pm_period % h->window == 0;
}

int solve_window(const cg_handle* h) {
    if (pmag_split(h)) return h->window;
    const int period = h->sched == kSchedTileRule ? h->period : h->sched == kSchedPMag ? h->pm_period : 1;
    return std::max(1, h->window / period) * period;
}

// The update (UPDATE = true) or direction kernel in the handle's instantiation:
// Jacobi or not, streaming vector accesses or not.
template <bool UPDATE>
void launch_vec_kernel(cg_handle* h, const dev::VecArgs& va, hipStream_t s) {
    const dim3 g(h->upd_blocks), b(dev::kVecBlock);
    if (UPDATE) {
        if (h->jacobi && h->nt_stores) hipLaunchKernelGGL((dev::cg_update_kernel<true, true>), g, b, 0, s, va);
        else if (h->jacobi) hipLaunchKernelGGL((dev::cg_update_kernel<true, false>), g, b, 0, s, va);
        else if (h->nt_stores) hipLaunchKernelGGL((dev::cg_update_kernel<false, true>), g, b, 0, s, va);
        else hipLaunchKernelGGL((dev::cg_update_kernel<false, false>), g, b, 0, s, va);
    } else {
        if (h->jacobi && h->nt_stores) hipLaunchKernelGGL((dev::cg_direction_kernel<true, true>), g, b, 0, s, va);
        else if (h->jacobi) hipLaunchKernelGGL((dev::cg_direction_kernel<true, false>), g, b, 0, s, va);
        else if (h->nt_stores) hipLaunchKernelGGL((dev::cg_direction_kernel<false, true>), g, b, 0, s, va);
        else hipLaunchKernelGGL((dev::cg_direction_kernel<false, false>), g, b, 0, s, va);
    }
}

// One CG iteration: [map window step] -> SpMV with fused p.q and alpha ->
// x/r update with fused r.r (r.z), beta, rho and stop flag -> new direction.
// i is the iteration's index in its window (the solve's k modulo the window
// length while the solve runs). rule_at_end: under a split max|p| rule, this
// window's last iteration is followed by the rule's evaluation.
void enqueue_iteration(cg_handle* h, int i, hipStream_t s, bool rule_at_end = false) {
    if (h->sched == kSchedTileRule && i % h->period == 0) {
        dev::MapArgs ma = map_args(h, 0.0, 1);
        hipLaunchKernelGGL(dev::tile_rule_kernel, dim3(tile_rule_grid(h)), dim3(dev::kBlock), 0, s, ma);
    }
    dev::SpmvArgs sa = spmv_args(h, h->p, h->S > 1 ? h->qpart : h->q, &h->st->uprec);
    launch_spmv<dev::kSpmvCg>(h, sa, s);
    dev::VecArgs va = vec_args(h, nullptr, nullptr);
    va.part_in = h->part_spmv;
    va.nparts_in = spmv_grid(h);
    va.part_out = h->part_vec;
    launch_vec_kernel<true>(h, va, s);  // update
    va.part_in = h->part_vec;
    va.nparts_in = h->upd_blocks;
    launch_vec_kernel<false>(h, va, s);  // direction
    if (h->sched == kSchedPMag) {  // the map of the next window (iteration i + 1 starts it)
        if (pmag_split(h) ? (rule_at_end && i == h->window - 1) : (i + 1) % h->pm_period == 0)
            launch_pmag(h, h->p, 1, s);
    }
}

// The single-workgroup solver runs schedules whose per-tile map is fixed for
// the whole solve (static maps and the residual stages, which are uniform),
// on handles whose row groups were sized for it (small_layout).

bool single_block_solve(const cg_handle* h) {
    const bool supported = h->S == 1 && h->p1 == 0 && (h->sched == kSchedStatic || h->sched == kSchedResidual);
    return supported && small_layout(h);
}

template <typename MetaT, int MAXROWS>
void launch_small_m(cg_handle* h, const dev::SpmvArgs& sa, const dev::VecArgs& va, hipStream_t s) {
    if (h->jacobi)
        hipLaunchKernelGGL((dev::cg_small_kernel<MetaT, MAXROWS, true>), dim3(1), dim3(dev::kSmallBlock), 0, s, sa, va);
    else
        hipLaunchKernelGGL((dev::cg_small_kernel<MetaT, MAXROWS, false>), dim3(1), dim3(dev::kSmallBlock), 0, s, sa,
                           va);
}

// Every iteration of the solve in one launch of one workgroup.
void launch_small(cg_handle* h, hipStream_t s) {
    const dev::SpmvArgs sa = spmv_args(h, h->p, h->q, &h->st->uprec);
    const dev::VecArgs va = vec_args(h, nullptr, nullptr);
    const bool wide = h->rows_per_group > 64;
    if (h->meta16) {
        if (wide)
            launch_small_m<uint16_t, dev::kMaxRows>(h, sa, va, s);
        else
            launch_small_m<uint16_t, 64>(h, sa, va, s);
    } else if (wide) {
        launch_small_m<uint8_t, dev::kMaxRows>(h, sa, va, s);
    } else {
        launch_small_m<uint8_t, 64>(h, sa, va, s);
    }
}

// ||b - A x|| / ||b|| with the exact FP64 values into out[0] (device),
// asynchronously on s; partials: 2 doubles per block of the launch (at most
// 2 * max(SpMV grid, kResGridCap)).
int launch_true_residual(cg_handle* h, const double* b, const double* x, double* partials, double* out,
                         hipStream_t s) {
    dev::SpmvArgs sa = spmv_args(h, x, nullptr, &h->st->zero_prec);
    sa.cbcode = nullptr;  // exact FP64 values, whatever the schedule
    sa.p1_round = 0;
    sa.b = b;
    int nparts = 0;
    if (h->S > 1) {  // the slices' partial products, then the residual and its norms
        sa.y = h->qpart;
        launch_spmv<dev::kSpmvPlain>(h, sa, s);
        nparts = grid_for(h->n, 4, kResGridCap);
        hipLaunchKernelGGL(dev::combine_resnorm_kernel, dim3(nparts), dim3(dev::kBlock), 0, s, h->qpart, h->S,
                           (int64_t)(h->n + (h->n & 1)), b, (int64_t)h->n, partials);
    } else {
        sa.partials = partials;
        launch_spmv<dev::kSpmvResNorm>(h, sa, s);
        nparts = spmv_grid(h);
    }
    hipLaunchKernelGGL(dev::resnorm_finish_kernel, dim3(1), dim3(dev::kBlock), 0, s, partials, nparts, out);
    HIP_CHECK(hipGetLastError());
    return CG_OK;
}

int ensure_graph(cg_handle* h) {
    const int W = solve_window(h);
    const int period = h->sched == kSchedPMag ? h->pm_period : h->period;
    if (h->graph && h->graph_window == W && h->graph_sched == h->sched && h->graph_period == period)
        return CG_OK;
    drop_graph(h);
    for (int variant = 0; variant < (pmag_split(h) ? 2 : 1); ++variant) {
        hipGraph_t g = nullptr;
        HIP_CHECK(hipStreamBeginCapture(h->stream, hipStreamCaptureModeThreadLocal));
        for (int i = 0; i < W; ++i) enqueue_iteration(h, i, h->stream, variant == 1);
        hipError_t e = hipStreamEndCapture(h->stream, &g);
        if (e != hipSuccess) {
            if (g) (void)hipGraphDestroy(g);
            drop_graph(h);
            return fail(CG_EDEVICE, std::string("graph capture failed: ") + hipGetErrorString(e));
        }
        hipGraphExec_t* dst = variant == 1 ? &h->graph_rule : &h->graph;
        e = hipGraphInstantiate(dst, g, nullptr, nullptr, 0);
        (void)hipGraphDestroy(g);
        if (e != hipSuccess) {
            *dst = nullptr;
            drop_graph(h);
            return fail(CG_EDEVICE, std::string("graph instantiation failed: ") + hipGetErrorString(e));
        }
    }
    h->graph_window = W;
    h->graph_period = period;
    h->graph_sched = h->sched;
    return CG_OK;
}

// Scratch of cg_true_residual_noalloc: the per-block partial sums (two per
// block of the residual-norm launch) live in this file-scope device array, one
// copy per GPU, held until the process ends. In host code `scratch` only names
// the symbol; its address on each device comes from hipGetSymbolAddress, taken
// once per device (with that device current) by the first cg_create there.
constexpr int64_t kNoAllocScratchDoubles = 2 * (int64_t)std::max(kSpmvGridCap, kResGridCap);
static __device__ __align__(256) double scratch[kNoAllocScratchDoubles];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
double* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (device d), looked
// up the first time and kept.
int scratch_address(int d, double** out) {
    *out = nullptr;
    if (d < 0 || d >= kMaxDevices) return fail(CG_EDEVICE, "device index " + std::to_string(d) + " out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[d]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(CG_EDEVICE, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
        }
        g_scratch_ptr[d] = static_cast<double*>(p);
    }
    *out = g_scratch_ptr[d];
    return CG_OK;
}

// Waits until the last launch made on a caller's stream (cg_spmv,
// cg_true_residual) has finished, before a call rewrites what it reads (the
// map, the packed values, the column codes, the scalar state). Those calls
// use the handle's own stream or blocking copies, which are not ordered after
// a caller's non-blocking stream. Launches on the default stream are waited
// for by synchronising that stream, so they need no event of their own (an
// event recorded after every cg_spmv costs a few microseconds per call).
hipError_t order_after_user(cg_handle* h) {
    hipError_t e = hipSuccess;
    if (h->null_pending) {
        h->null_pending = false;
        e = hipStreamSynchronize(nullptr);
    }
    if (e == hipSuccess && h->user_pending) {
        h->user_pending = false;
        e = hipEventSynchronize(h->ev_user);
    }
    return e;
}

// Notes a launch on a caller's stream for order_after_user.
hipError_t note_user_launch(cg_handle* h, hipStream_t s) {
    if (!s) {
        h->null_pending = true;
        return hipSuccess;
    }
    h->user_pending = true;
    return hipEventRecord(h->ev_user, s);
}

bool ranges_overlap(const void* a, const void* b, size_t bytes) {
    const char* pa = static_cast<const char*>(a);
    const char* pb = static_cast<const char*>(b);
    return pa < pb + bytes && pb < pa + bytes;
}

}  // namespace

namespace {

// The canonical layout with every odd-length local column closed by a
// sentinel entry (row offset R, value +0.0), as drawn in Fig. 4(b). Canonical
// order is kept: the sentinel follows its column's last nonzero.
void pad_columns(const cg_tilecsc& A, cg_tilecsc& P) {
    const int64_t T = A.T();
    P.n = A.n;
    P.R = A.R;
    P.C = A.C;
    P.nrb = A.nrb;
    P.tile_row_ptr = A.tile_row_ptr;
    P.tile_col_idx = A.tile_col_idx;
    std::vector<int64_t> extra(T + 1, 0);
    mpcg::parallel_for(T, [&](int64_t lo, int64_t hi) {
        for (int64_t t = lo; t < hi; ++t) {
            int64_t e = 0, run = 0;
            for (int64_t k = A.tile_nnz_ptr[t]; k < A.tile_nnz_ptr[t + 1]; ++k) {
                ++run;
                if (k + 1 == A.tile_nnz_ptr[t + 1] || A.col_local[k + 1] != A.col_local[k]) {
                    e += run & 1;
                    run = 0;
                }
            }
            extra[t] = e;
        }
    });
    P.tile_nnz_ptr.assign(T + 1, 0);
    int64_t added = 0;
    for (int64_t t = 0; t < T; ++t) {
        P.tile_nnz_ptr[t] = A.tile_nnz_ptr[t] + added;
        added += extra[t];
    }
    P.tile_nnz_ptr[T] = A.tile_nnz_ptr[T] + added;
    const int64_t nnz = P.tile_nnz_ptr[T];
    P.row_idx.resize(nnz);
    P.col_local.resize(nnz);
    P.val.resize(nnz);
    P.perm.assign(nnz, -1);
    mpcg::parallel_for(T, [&](int64_t lo, int64_t hi) {
        for (int64_t t = lo; t < hi; ++t) {
            int64_t o = P.tile_nnz_ptr[t], run = 0;
            for (int64_t k = A.tile_nnz_ptr[t]; k < A.tile_nnz_ptr[t + 1]; ++k, ++o) {
                P.row_idx[o] = A.row_idx[k];
                P.col_local[o] = A.col_local[k];
                P.val[o] = A.val[k];
                P.perm[o] = A.perm.empty() ? -1 : A.perm[k];
                ++run;
                if (k + 1 == A.tile_nnz_ptr[t + 1] || A.col_local[k + 1] != A.col_local[k]) {
                    if (run & 1) {
                        ++o;
                        P.row_idx[o] = (uint16_t)A.R;
                        P.col_local[o] = A.col_local[k];
                        P.val[o] = 0.0;
                    }
                    run = 0;
                }
            }
        }
    });
}

// Per-column scale exponents e_j (s_j = 2^e_j, e_j the binary exponent of the
// column's largest |a_ij|, 0 for a column without a nonzero value) and the
// scaled values a / s_j in storage order (Sec. 3.3.2).
void column_scale(const cg_tilecsc& A, std::vector<int16_t>& e, std::vector<double>& scaled) {
    std::vector<double> colmax(A.n, 0.0);
    for (int64_t t = 0; t < A.T(); ++t) {
        const int64_t c0 = (int64_t)A.tile_col_idx[t] * A.C;
        for (int64_t k = A.tile_nnz_ptr[t]; k < A.tile_nnz_ptr[t + 1]; ++k)
            colmax[c0 + A.col_local[k]] = std::max(colmax[c0 + A.col_local[k]], std::fabs(A.val[k]));
    }
    e.assign(A.n, 0);
    for (int64_t j = 0; j < A.n; ++j) {
        int ej = 0;
        if (colmax[j] != 0.0) (void)std::frexp(colmax[j], &ej);
        e[j] = (int16_t)ej;
    }
    scaled.resize(A.nnz());
    mpcg::parallel_for(A.T(), [&](int64_t lo, int64_t hi) {
        for (int64_t t = lo; t < hi; ++t) {
            const int64_t c0 = (int64_t)A.tile_col_idx[t] * A.C;
            for (int64_t k = A.tile_nnz_ptr[t]; k < A.tile_nnz_ptr[t + 1]; ++k)
                scaled[k] = std::ldexp(A.val[k], -(int)e[c0 + A.col_local[k]]);
        }
    });
}

// Slabs of a layout whose row blocks are taller than a wavefront's
// accumulators: row block I (R rows) becomes slabs I*k .. I*k+k-1 of Rs = R / k
// rows, and tile t = (I, J) becomes the non-empty Rs x C pieces of its slabs.
// B lists the pieces slab by slab, column blocks ascending in a slab (the
// canonical order of an Rs x C layout); a piece keeps its tile's entries in
// their order (column by column, rows ascending) with row offsets from the
// slab's first row. parent[d] is the canonical tile of piece d.
void split_slabs(const cg_tilecsc& A, int Rs, cg_tilecsc& B, std::vector<int32_t>& parent) {
    const int64_t k = A.R / Rs, nrb = A.nrb, nslab = nrb * k;
    std::vector<int64_t> pieces(nslab + 1, 0), nz(nslab + 1, 0);
    mpcg::parallel_for(nrb, [&](int64_t lo, int64_t hi) {
        std::vector<int64_t> stamp(k, -1);  // last tile with an entry in slab s
        for (int64_t I = lo; I < hi; ++I)
            for (int64_t t = A.tile_row_ptr[I]; t < A.tile_row_ptr[I + 1]; ++t)
                for (int64_t e = A.tile_nnz_ptr[t]; e < A.tile_nnz_ptr[t + 1]; ++e) {
                    const int64_t sl = A.row_idx[e] / Rs;
                    ++nz[I * k + sl + 1];
                    if (stamp[sl] != t) {
                        stamp[sl] = t;
                        ++pieces[I * k + sl + 1];
                    }
                }
    });
    for (int64_t v = 0; v < nslab; ++v) {
        pieces[v + 1] += pieces[v];
        nz[v + 1] += nz[v];
    }
    const int64_t Td = pieces[nslab], nnz = nz[nslab];
    B.n = A.n;
    B.R = Rs;
    B.C = A.C;
    B.nrb = (A.n + Rs - 1) / Rs;  // slabs past the last row hold nothing
    B.tile_row_ptr.assign(pieces.begin(), pieces.begin() + B.nrb + 1);
    B.tile_col_idx.assign(Td, 0);
    B.tile_nnz_ptr.assign(Td + 1, nnz);
    B.row_idx.assign(nnz, 0);
    B.col_local.assign(nnz, 0);
    B.val.assign(nnz, 0.0);
    B.perm.clear();
    parent.assign(Td, 0);
    mpcg::parallel_for(nrb, [&](int64_t lo, int64_t hi) {
        std::vector<int64_t> pnext(k), znext(k), cur(k, -1), stamp(k, -1);
        for (int64_t I = lo; I < hi; ++I) {
            for (int64_t sl = 0; sl < k; ++sl) {
                pnext[sl] = pieces[I * k + sl];
                znext[sl] = nz[I * k + sl];
            }
            for (int64_t t = A.tile_row_ptr[I]; t < A.tile_row_ptr[I + 1]; ++t)
                for (int64_t e = A.tile_nnz_ptr[t]; e < A.tile_nnz_ptr[t + 1]; ++e) {
                    const int64_t sl = A.row_idx[e] / Rs;
                    if (stamp[sl] != t) {  // tile t's piece in slab sl starts here
                        stamp[sl] = t;
                        cur[sl] = pnext[sl]++;
                        B.tile_col_idx[cur[sl]] = A.tile_col_idx[t];
                        B.tile_nnz_ptr[cur[sl]] = znext[sl];
                        parent[cur[sl]] = (int32_t)t;
                    }
                    const int64_t o = znext[sl]++;
                    B.row_idx[o] = (uint16_t)(A.row_idx[e] - sl * Rs);
                    B.col_local[o] = A.col_local[e];
                    B.val[o] = A.val[e];
                }
        }
    });
}

// Automatic column slices: S = ceil(8n / L2) (at most 64) when x is larger
// than one XCD's L2 and at least half of the nonzeros lie more than L2 / 16
// entries from the diagonal (their gathers leave an L2-sized window around
// the rows being swept); else 1.
int auto_slices(const cg_tilecsc& A, int device) {
    int64_t l2 = 4 << 20;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) == hipSuccess && prop.l2CacheSize > 0) l2 = prop.l2CacheSize;
    else (void)hipGetLastError();
    if (8 * A.n <= l2 || A.nnz() == 0) return 1;
    const int64_t near = l2 / 16;
    std::atomic<int64_t> far{0};
    mpcg::parallel_for(A.nrb, [&](int64_t lo, int64_t hi) {
        int64_t f = 0;
        for (int64_t I = lo; I < hi; ++I)
            for (int64_t t = A.tile_row_ptr[I]; t < A.tile_row_ptr[I + 1]; ++t) {
                const int64_t c0 = (int64_t)A.tile_col_idx[t] * A.C;
                for (int64_t k = A.tile_nnz_ptr[t]; k < A.tile_nnz_ptr[t + 1]; ++k) {
                    const int64_t i = I * A.R + A.row_idx[k], j = c0 + A.col_local[k];
                    f += (i > j ? i - j : j - i) > near;
                }
            }
        far += f;
    });
    if (2 * far.load() < A.nnz()) return 1;
    return (int)std::min<int64_t>(64, (8 * A.n + l2 - 1) / l2);
}

// Device order of the tiles with S column slices: slice s holds the column
// blocks [ceil(s ncb / S), ceil((s+1) ncb / S)); the tiles are listed slice by
// slice, then row group by row group (segment s * ngroups + g), then in
// canonical order. D receives the layout in that order (tile_row_ptr left
// canonical), trb the row block of every device tile, seg_t0 the first device
// tile of every segment (nseg + 1 entries), dperm device tile -> canonical.
void build_slices(const cg_tilecsc& A, int S, int G, int64_t ngroups, cg_tilecsc& D, std::vector<int32_t>& trb,
                  std::vector<int64_t>& seg_t0, std::vector<int32_t>& dperm) {
    const int64_t T = A.T(), nrb = A.nrb, ncb = (A.n + A.C - 1) / A.C;
    auto jlo = [&](int64_t s) { return (s * ncb + S - 1) / S; };
    // Tiles of row block I in slice s: [lb(I, jlo(s)), lb(I, jlo(s+1))).
    auto lb = [&](int64_t I, int64_t j) {
        const int32_t* b = A.tile_col_idx.data() + A.tile_row_ptr[I];
        const int32_t* e = A.tile_col_idx.data() + A.tile_row_ptr[I + 1];
        return (int64_t)(std::lower_bound(b, e, (int32_t)j) - A.tile_col_idx.data());
    };
    const int64_t nseg = (int64_t)S * ngroups;
    std::vector<int64_t> cnt(nseg, 0);
    mpcg::parallel_for(ngroups, [&](int64_t lo, int64_t hi) {
        for (int64_t g = lo; g < hi; ++g)
            for (int64_t I = g * G; I < std::min<int64_t>((g + 1) * G, nrb); ++I)
                for (int64_t s = 0; s < S; ++s) cnt[s * ngroups + g] += lb(I, jlo(s + 1)) - lb(I, jlo(s));
    });
    seg_t0.assign(nseg + 1, 0);
    for (int64_t v = 0; v < nseg; ++v) seg_t0[v + 1] = seg_t0[v] + cnt[v];
    dperm.assign(T, 0);
    trb.assign(std::max<int64_t>(T, 1), 0);
    mpcg::parallel_for(ngroups, [&](int64_t lo, int64_t hi) {
        for (int64_t g = lo; g < hi; ++g)
            for (int64_t s = 0; s < S; ++s) {
                int64_t d = seg_t0[s * ngroups + g];
                for (int64_t I = g * G; I < std::min<int64_t>((g + 1) * G, nrb); ++I)
                    for (int64_t t = lb(I, jlo(s)); t < lb(I, jlo(s + 1)); ++t, ++d) {
                        dperm[d] = (int32_t)t;
                        trb[d] = (int32_t)I;
                    }
            }
    });
    D.n = A.n;
    D.R = A.R;
    D.C = A.C;
    D.nrb = A.nrb;
    D.tile_row_ptr = A.tile_row_ptr;
    D.tile_col_idx.resize(T);
    D.tile_nnz_ptr.assign(T + 1, 0);
    for (int64_t d = 0; d < T; ++d) {
        const int64_t t = dperm[d];
        D.tile_col_idx[d] = A.tile_col_idx[t];
        D.tile_nnz_ptr[d + 1] = D.tile_nnz_ptr[d] + (A.tile_nnz_ptr[t + 1] - A.tile_nnz_ptr[t]);
    }
    const int64_t nnz = A.nnz();
    D.row_idx.resize(nnz);
    D.col_local.resize(nnz);
    D.val.resize(nnz);
    mpcg::parallel_for(T, [&](int64_t lo, int64_t hi) {
        for (int64_t d = lo; d < hi; ++d) {
            const int64_t t = dperm[d], k0 = A.tile_nnz_ptr[t], len = A.tile_nnz_ptr[t + 1] - k0;
            const int64_t o = D.tile_nnz_ptr[d];
            std::memcpy(&D.row_idx[o], &A.row_idx[k0], sizeof(uint16_t) * len);
            std::memcpy(&D.col_local[o], &A.col_local[k0], len);
            std::memcpy(&D.val[o], &A.val[k0], sizeof(double) * len);
        }
    });
}

}  // namespace

extern "C" int cg_create(const cg_tilecsc* A, const uint8_t* precision_map, const cg_options* opt,
                         void* stream, cg_handle** out) {
    mpcg::clear_error();
    if (!out) return fail(CG_EINVAL, "cg_create: out is NULL");
    *out = nullptr;
    if (!A) return fail(CG_EINVAL, "cg_create: A is NULL");
    const int p1 = opt ? opt->p1 : 0;
    if (p1 & ~(CG_P1_ROUND_VECTOR | CG_P1_COLUMN_SCALE | CG_P1_PAD_COLUMNS))
        return fail(CG_EINVAL, "cg_create: opt->p1 has unknown bits");
    if ((p1 & CG_P1_PAD_COLUMNS) && A->R > 255)
        return fail(CG_EINVAL, "cg_create: column padding needs R <= 255 (the sentinel row offset is R)");
    cg_tilecsc padded;
    if (p1 & CG_P1_PAD_COLUMNS) {
        pad_columns(*A, padded);
        A = &padded;
    }
    const int64_t T = A->T(), nnz = A->nnz(), n = A->n;
    if (n > INT32_MAX || T > INT32_MAX || nnz > INT32_MAX)
        return fail(CG_EINVAL, "cg_create: n, T and nnz must be below 2^31");
    if (n >= (int64_t(1) << 28))
        return fail(CG_EINVAL, "cg_create: n must be below 2^28 (x is addressed with 32-bit byte offsets)");
    if (nnz == 0) return fail(CG_EINVAL, "cg_create: the matrix has no nonzeros (it cannot be SPD)");
    if (precision_map) {
        for (int64_t t = 0; t < T; ++t)
            if (precision_map[t] > 2)
                return fail(CG_EINVAL, "cg_create: precision_map[" + std::to_string(t) +
                                           "] is not 0, 1 or 2");
    }
    cg_handle* h = new (std::nothrow) cg_handle();
    if (!h) return fail(CG_ENOMEM, "cg_create: out of host memory");
    auto bail = [&](int rc) {
        if (h->graph) (void)hipGraphExecDestroy(h->graph);
        for (auto& e : h->ev)
            if (e) (void)hipEventDestroy(e);
        if (h->pinned) (void)hipHostFree(h->pinned);
        if (h->res_host) (void)hipHostFree(h->res_host);
        if (h->ev_user) (void)hipEventDestroy(h->ev_user);
        if (h->stream) (void)hipStreamDestroy(h->stream);
        delete h;
        return rc;
    };
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipGetDevice(&h->device) != hipSuccess) return bail(fail(CG_EDEVICE, "cg_create: no HIP device"));
    {
        double* sp = nullptr;  // the static scratch of cg_true_residual_noalloc on this device
        const int rc = scratch_address(h->device, &sp);
        if (rc != CG_OK) return bail(rc);
    }
    h->n = n;
    h->T = T;
    h->nnz = nnz;
    h->R = A->R;
    h->C = A->C;
    h->nrb = A->nrb;
    h->p1 = p1;
    // Row blocks taller than one wavefront's row accumulators run as slabs:
    // B is the layout of the pieces (split_slabs), or the canonical one.
    cg_tilecsc slabs;
    std::vector<int32_t> sparent;
    const cg_tilecsc* B = A;
    if (A->R > dev::kMaxRows) {
        int Rs = dev::kMaxRows;
        while (A->R % Rs) --Rs;
        try {
            split_slabs(*A, Rs, slabs, sparent);
        } catch (const std::bad_alloc&) {
            return bail(fail(CG_ENOMEM, "cg_create: out of host memory"));
        }
        B = &slabs;
    }
    h->Td = B->T();
    h->Rd = B->R;
    h->nrbd = B->nrb;
    const int64_t Td = h->Td;
    if (Td > INT32_MAX) return bail(fail(CG_EINVAL, "cg_create: more than 2^31 - 1 device tiles"));
    // Padding stores the sentinel row offset R, which needs the 16-bit form.
    h->meta16 = !(B->R <= 16 && B->C <= 16) || (p1 & CG_P1_PAD_COLUMNS);
    h->S = 0;  // automatic unless opt says otherwise
    if (opt) {
        h->jacobi = opt->jacobi != 0;
        if (opt->window > 0) h->window = std::min(opt->window, 4096);
        if (opt->use_graph >= 0) h->use_graph = opt->use_graph != 0;
        if (opt->col_slices < 0 || opt->col_slices > 64)
            return bail(fail(CG_EINVAL, "cg_create: col_slices must lie in [0, 64]"));
        h->S = opt->col_slices;
        if (opt->single_block < -1 || opt->single_block > 1)
            return bail(fail(CG_EINVAL, "cg_create: single_block must be -1, 0 or 1"));
        h->single_block = opt->single_block;
        if (opt->stage_x < 0 || opt->stage_x > 1) return bail(fail(CG_EINVAL, "cg_create: stage_x must be 0 or 1"));
        h->stage_x = opt->stage_x != 0;
    }
    if (h->S == 0) h->S = auto_slices(*A, h->device);
    // Row blocks per wavefront: the largest of 32, 64, 128, 256 rows whose row
    // groups hold at most one batch of tiles on average (at least one row block).
    // A small matrix would then leave too few groups (wavefronts) to spread its
    // product over the chip: below kMinGroups groups the group shrinks to the
    // largest size that reaches kMinGroups, down to one row block.
    auto group_rb = [&](int rows) { return std::max(1, std::min(dev::kMaxGroupRB, rows / B->R)); };
    auto groups_of = [&](int G) { return (h->nrbd + G - 1) / G; };
    if (dev::kGroupRows > 0) {
        h->G = group_rb(dev::kGroupRows);
    } else if (small_layout(h)) {
        // A handle that solves on one workgroup: about one group of up to 256
        // rows per wavefront, so that each wavefront pays the latency of a
        // batch over many windows.
        h->G = std::min<int>(group_rb(256),
                             (int)std::max<int64_t>(1, (h->nrbd + dev::kSmallWaves - 1) / dev::kSmallWaves));
    } else {
        h->G = group_rb(32);
        for (int rows : {64, 128, 256}) {
            const int G = group_rb(rows);
            if (groups_of(G) > 0 && Td <= (int64_t)dev::kTileBatch * groups_of(G)) h->G = G;
        }
        constexpr int64_t kMinGroups = 1024;
        if (groups_of(h->G) < kMinGroups) {
            int G = h->G;
            while (G > 1 && groups_of(G) < kMinGroups) G = std::max(1, G / 2);
            h->G = G;
        }
    }
    h->rows_per_group = h->G * B->R;
    h->ngroups = (int32_t)((h->nrbd + h->G - 1) / h->G);

    // Device order of the tiles: that of B, or slice by slice (col_slices).
    // D is the layout in device order; segment v (slice v / ngroups, row group
    // v % ngroups) owns device tiles [seg_t0[v], seg_t0[v + 1]); trb holds the
    // row block (of B) of every device tile.
    h->nseg = (int64_t)h->S * h->ngroups;
    cg_tilecsc sliced;
    const cg_tilecsc* D = B;
    std::vector<int32_t> trb;
    std::vector<int64_t> seg_t0;
    if (h->S > 1) {
        std::vector<int32_t> dslice;  // device tile -> tile of B
        build_slices(*B, h->S, h->G, h->ngroups, sliced, trb, seg_t0, dslice);
        D = &sliced;
        h->dperm.resize(Td);
        for (int64_t d = 0; d < Td; ++d) h->dperm[d] = sparent.empty() ? dslice[d] : sparent[dslice[d]];
    } else {
        trb.assign(std::max<int64_t>(Td, 1), 0);
        mpcg::parallel_for(h->nrbd, [&](int64_t lo, int64_t hi) {
            for (int64_t I = lo; I < hi; ++I)
                for (int64_t t = B->tile_row_ptr[I]; t < B->tile_row_ptr[I + 1]; ++t) trb[t] = (int32_t)I;
        });
        seg_t0.assign(h->nseg + 1, 0);
        for (int64_t g = 0; g <= h->ngroups; ++g)
            seg_t0[g] = B->tile_row_ptr[std::min<int64_t>(g * h->G, h->nrbd)];
        h->dperm = sparent;
    }
    // Slabs: the pieces of every canonical tile (device order), and which
    // piece counts for its tile in the map trace.
    std::vector<int32_t> cptr_h, clist_h;
    std::vector<uint8_t> dcount_h;
    if (!sparent.empty()) {
        cptr_h.assign(T + 1, 0);
        for (int64_t d = 0; d < Td; ++d) ++cptr_h[h->dperm[d] + 1];
        for (int64_t t = 0; t < T; ++t) cptr_h[t + 1] += cptr_h[t];
        clist_h.assign(Td, 0);
        dcount_h.assign(Td, 0);
        std::vector<int32_t> fill(cptr_h.begin(), cptr_h.end() - 1);
        for (int64_t d = 0; d < Td; ++d) {
            const int32_t t = h->dperm[d];
            dcount_h[d] = fill[t] == cptr_h[t];
            clist_h[fill[t]++] = (int32_t)d;
        }
    }
    auto seg_group = [&](int64_t v) { return v % h->ngroups; };
    auto seg_slice = [&](int64_t v) { return v / h->ngroups; };
    // Host-side packing of the device layout: 32-bit offsets and packed (row, col).
    std::vector<int32_t> trp(h->nrb + 1), tptr(Td + 1);
    for (int64_t i = 0; i <= h->nrb; ++i) trp[i] = (int32_t)A->tile_row_ptr[i];  // canonical
    for (int64_t i = 0; i <= Td; ++i) tptr[i] = (int32_t)D->tile_nnz_ptr[i];
    std::vector<uint8_t> meta8;
    std::vector<uint16_t> meta16;
    if (h->meta16) {
        meta16.resize(nnz);
        mpcg::parallel_for(nnz, [&](int64_t lo, int64_t hi) {
            for (int64_t k = lo; k < hi; ++k)
                meta16[k] = (uint16_t)((D->row_idx[k] << 8) | D->col_local[k]);
        });
    } else {
        meta8.resize(nnz);
        mpcg::parallel_for(nnz, [&](int64_t lo, int64_t hi) {
            for (int64_t k = lo; k < hi; ++k) meta8[k] = (uint8_t)((D->row_idx[k] << 4) | D->col_local[k]);
        });
    }
    // Batches: a segment's tiles are taken kTileBatch at a time; a segment
    // without tiles gets one batch without tiles so that its rows are written.
    std::vector<int32_t> gbatch(h->nseg + 1, 0);
    {
        int64_t nb = 0;
        for (int64_t v = 0; v < h->nseg; ++v) {
            gbatch[v] = (int32_t)nb;
            const int64_t ntile = seg_t0[v + 1] - seg_t0[v];
            nb += std::max<int64_t>(1, (ntile + dev::kTileBatch - 1) / dev::kTileBatch);
            if (nb > INT32_MAX) return bail(fail(CG_EINVAL, "cg_create: too many SpMV batches"));
        }
        gbatch[h->nseg] = (int32_t)nb;
        h->nbatch = nb;
    }
    const int64_t nb = h->nbatch;
    std::vector<int32_t> btab((size_t)nb * dev::kBtFields, 0);
    // First tile, tiles and nonzeros of every batch, and whether its vector
    // segments are staged in LDS: the handle supports it (multi-launch
    // product, C a power of two, none of the paper's numerics options), the
    // batch's distinct column blocks fit the stage and hold no more entries
    // than the batch has nonzeros (each staged entry is used once or more on
    // average), and its padded records fit one chunk of 64.
    const bool stage_ok = h->stage_x && dev::kStageMaxBytes > 0 && !small_layout(h) && p1 == 0 && A->C >= 2 &&
                          (A->C & (A->C - 1)) == 0;
    std::vector<int32_t> bnx(nb, 0);  // distinct column blocks of a staged batch (0: not staged)
    mpcg::parallel_for(h->nseg, [&](int64_t lo, int64_t hi) {
        int32_t cols[dev::kTileBatch];
        for (int64_t v = lo; v < hi; ++v) {
            const int64_t t0 = seg_t0[v], t1 = seg_t0[v + 1];
            int64_t tb = t0;
            for (int64_t b = gbatch[v]; b < gbatch[v + 1]; ++b, tb += dev::kTileBatch) {
                int32_t* e = &btab[(size_t)b * dev::kBtFields];
                const int64_t nt = std::max<int64_t>(0, std::min<int64_t>(dev::kTileBatch, t1 - tb));
                const int64_t len = nt ? D->tile_nnz_ptr[tb + nt] - D->tile_nnz_ptr[tb] : 0;
                e[dev::kBtTile] = nt ? (int32_t)tb : 0;
                e[dev::kBtTiles] = (int32_t)nt;
                e[dev::kBtFirstNnz] = nt ? (int32_t)D->tile_nnz_ptr[tb] : 0;
                e[dev::kBtLen] = (int32_t)len;
                e[dev::kBtGroup] = (int32_t)seg_group(v);
                e[dev::kBtFlags] = (b == gbatch[v] ? dev::kBatchFirstOfGroup : 0) |
                                   (b == gbatch[v + 1] - 1 ? dev::kBatchLastOfGroup : 0) |
                                   (int32_t)(seg_slice(v) << dev::kBatchSliceShift);
                if (!stage_ok || nt == 0) continue;
                for (int64_t k = 0; k < nt; ++k) cols[k] = D->tile_col_idx[tb + k];
                std::sort(cols, cols + nt);
                const int64_t nx = std::unique(cols, cols + nt) - cols;
                const int64_t entries = nx * A->C;
                if (entries * 8 <= dev::kStageMaxBytes && entries * 100 <= len * dev::kStageRatioPct &&
                    dev::batch_records((int)len, true) <= dev::kWave) {
                    bnx[b] = (int32_t)nx;
                    e[dev::kBtFlags] |= dev::kBatchStaged;
                }
            }
        }
    });
    // Stage lists (xcb) and window records, in batch order.
    std::vector<int64_t> xbase(nb + 1, 0);
    int64_t nwin = 0;
    for (int64_t b = 0; b < nb; ++b) {
        int32_t* e = &btab[(size_t)b * dev::kBtFields];
        xbase[b + 1] = xbase[b] + bnx[b];
        e[dev::kBtXList] = (int32_t)xbase[b];
        e[dev::kBtXCount] = bnx[b];
        e[dev::kBtRecords] = (int32_t)nwin;
        if (e[dev::kBtTiles]) nwin += dev::batch_records(e[dev::kBtLen], bnx[b] > 0);
        if (nwin > INT32_MAX) return bail(fail(CG_EINVAL, "cg_create: too many SpMV windows"));
    }
    h->nwin = nwin;
    if (h->nwin >= (int64_t(1) << 28)) return bail(fail(CG_EINVAL, "cg_create: too many SpMV windows"));
    if (xbase[nb] > INT32_MAX) return bail(fail(CG_EINVAL, "cg_create: too many staged column blocks"));
    std::vector<int32_t> xcb(std::max<int64_t>(xbase[nb], 1), 0);
    h->stage_doubles = 0;
    for (int64_t b = 0; b < nb; ++b) h->stage_doubles = std::max<int64_t>(h->stage_doubles, (int64_t)bnx[b] * A->C);
    h->stage_shift = 0;
    while ((2 << h->stage_shift) < A->C) ++h->stage_shift;
    // Value segments (three planes) and packed parts (the active map's
    // values), each in batch order, in 16-byte units.
    {
        int64_t off = 0, poff = 0;
        for (int64_t b = 0; b < nb; ++b) {
            int32_t* e = &btab[(size_t)b * dev::kBtFields];
            e[dev::kBtSegment] = (int32_t)(off / 16);
            e[dev::kBtPacked] = (int32_t)(poff / 16);
            off += e[dev::kBtLen] ? dev::segment_bytes(e[dev::kBtLen]) : 0;
            poff += e[dev::kBtLen] ? dev::packed_bytes(e[dev::kBtLen]) : 0;
            if (off / 16 > INT32_MAX) return bail(fail(CG_EINVAL, "cg_create: value planes above 32 GiB"));
        }
        h->planes_bytes = std::max<int64_t>(off, 16);
        h->packed_bytes = std::max<int64_t>(poff, 16);
    }
    // Tile entries and window records. A tile entry holds the byte offset of
    // its column block's segment (in x, or in the stage of a staged batch:
    // slot * C * 8 with the slot the block's rank among the batch's distinct
    // blocks) and of its rows in the row-group accumulators. A record holds
    // the batch tile of the window's first nonzero and a mask whose bit q says
    // that nonzero q+1 of the window starts a tile; the batch's end counts as
    // the start of the sentinel (tile index nt), which is also where padding
    // records point.
    std::vector<int2> tent(std::max<int64_t>(Td, 1), make_int2(0, 0));
    std::vector<uint64_t> win_mask(std::max<int64_t>(h->nwin, 1), 0);
    std::vector<int32_t> win_tile(std::max<int64_t>(h->nwin, 1), 0);
    mpcg::parallel_for(h->nbatch, [&](int64_t lo, int64_t hi) {
        for (int64_t b = lo; b < hi; ++b) {
            const int32_t* e = &btab[(size_t)b * dev::kBtFields];
            const int64_t tb = e[dev::kBtTile], nt = e[dev::kBtTiles], len = e[dev::kBtLen];
            if (!nt) continue;
            const bool staged = bnx[b] > 0;
            int32_t list[dev::kTileBatch];
            if (staged) {
                for (int64_t k = 0; k < nt; ++k) list[k] = D->tile_col_idx[tb + k];
                std::sort(list, list + nt);
                (void)std::unique(list, list + nt);  // the first bnx[b] entries
                std::copy(list, list + bnx[b], xcb.data() + xbase[b]);
            }
            for (int64_t t = tb; t < tb + nt; ++t) {
                int xoff = (int)(D->tile_col_idx[t] * A->C * 8);
                if (staged)
                    xoff = (int)((std::lower_bound(list, list + bnx[b], D->tile_col_idx[t]) - list) * A->C * 8);
                tent[t] = make_int2(xoff, (int)((trb[t] % h->G) * B->R * 8));
            }
            const int64_t kb = D->tile_nnz_ptr[tb], nw = (len + 63) / 64, E = dev::batch_records((int)len, staged);
            int64_t j = 0;
            for (int64_t v = 0; v < E; ++v) {
                const int64_t wi = e[dev::kBtRecords] + v;
                if (v >= nw) {
                    win_tile[wi] = (int32_t)nt;
                    continue;
                }
                const int64_t w0 = v * 64;
                while (j + 1 < nt && D->tile_nnz_ptr[tb + j + 1] - kb <= w0) ++j;
                win_tile[wi] = (int32_t)j;
                uint64_t m = 0;
                for (int64_t jn = j + 1; jn <= nt; ++jn) {
                    const int64_t start = (jn < nt ? D->tile_nnz_ptr[tb + jn] - kb : len);
                    if (start >= w0 + 64) break;
                    m |= 1ull << (start - w0 - 1);
                }
                win_mask[wi] = m;
            }
        }
    });
    h->btab_host = btab;
    std::vector<double> dinv_h;
    if (h->jacobi) {
        dinv_h.assign(n, 0.0);
        std::vector<uint8_t> seen(n, 0);
        for (int64_t I = 0; I < h->nrb; ++I)
            for (int64_t t = A->tile_row_ptr[I]; t < A->tile_row_ptr[I + 1]; ++t)
                for (int64_t k = A->tile_nnz_ptr[t]; k < A->tile_nnz_ptr[t + 1]; ++k) {
                    if (A->row_idx[k] >= A->R) continue;  // padding sentinel
                    int64_t row = I * A->R + A->row_idx[k];
                    int64_t col = (int64_t)A->tile_col_idx[t] * A->C + A->col_local[k];
                    if (row == col) {
                        dinv_h[row] = 1.0 / A->val[k];
                        seen[row] = A->val[k] != 0.0;
                    }
                }
        for (int64_t i = 0; i < n; ++i)
            if (!seen[i])
                return bail(fail(CG_EINVAL, "cg_create: Jacobi needs a nonzero diagonal; row " +
                                                std::to_string(i) + " has none"));
    }

    int rc = CG_OK;
#define TRY(expr)                       \
    do {                                \
        rc = (expr);                    \
        if (rc != CG_OK) return bail(rc); \
    } while (0)
    TRY(dalloc(h, &h->trp, h->nrb + 1));
    TRY(dalloc(h, &h->win_mask, h->nwin));
    TRY(dalloc(h, &h->win_tile, h->nwin));
    TRY(dalloc(h, &h->tent, std::max<int64_t>(Td, 1)));
    TRY(dalloc(h, &h->btab, (int64_t)btab.size()));
    TRY(dalloc(h, &h->gbatch, h->nseg + 1));
    TRY(dalloc(h, &h->xcb, (int64_t)xcb.size()));
    TRY(dalloc(h, &h->tcol, Td));
    TRY(dalloc(h, &h->tptr, Td + 1));
    TRY(dalloc(h, &h->map, Td));
    TRY(dalloc(h, &h->trow, std::max<int64_t>(Td, 1)));
    if (!cptr_h.empty()) {
        TRY(dalloc(h, &h->cptr, T + 1));
        TRY(dalloc(h, &h->clist, Td));
        TRY(dalloc(h, &h->dcount, Td));
    }
    if (h->meta16) {
        uint16_t* m = nullptr;
        TRY(dalloc(h, &m, nnz));
        h->meta = m;
    } else {
        uint8_t* m = nullptr;
        TRY(dalloc(h, &m, nnz));
        h->meta = m;
    }
    TRY(dalloc(h, &h->v64, nnz));
    std::vector<int16_t> colexp_h;
    std::vector<double> scaled_h;
    double* vlow = nullptr;  // set-up only: the scaled values the reduced planes are rounded from
    if (p1 & CG_P1_COLUMN_SCALE) {
        column_scale(*D, colexp_h, scaled_h);
        TRY(dalloc(h, &h->colexp, n));
        if (hipMalloc(&vlow, sizeof(double) * (size_t)std::max<int64_t>(nnz, 1)) != hipSuccess) {
            (void)hipGetLastError();
            return bail(fail(CG_ENOMEM, "cg_create: device allocation of the scaled values failed"));
        }
    }
    struct FreeLater {
        double* p;
        ~FreeLater() {
            if (p) (void)hipFree(p);
        }
    } free_vlow{vlow};
    TRY(dalloc(h, &h->planes, h->planes_bytes));
    TRY(dalloc(h, &h->packed, h->packed_bytes));
    TRY(dalloc(h, &h->toff, std::max<int64_t>(Td, 1)));
    // CG vectors padded with zeros to an even length (the vector kernels work
    // in 16-byte pairs); the padding entry stays zero, as every update of it
    // combines zeros (q's padding is never written by the SpMV).
    const int64_t n_pad = n + (n & 1);
    TRY(dalloc(h, &h->x, n_pad));
    TRY(dalloc(h, &h->r, n_pad));
    TRY(dalloc(h, &h->p, n_pad));
    TRY(dalloc(h, &h->q, n_pad));
    if (h->S > 1) TRY(dalloc(h, &h->qpart, (int64_t)h->S * n_pad));
    if (h->jacobi) {
        TRY(dalloc(h, &h->z, n_pad));
        TRY(dalloc(h, &h->dinv, n_pad));
    }
    plan_grids(h);
    h->nt_stores = 10 * nnz + 12 * Td + 40 * n > kLastLevelCache;
    TRY(dalloc(h, &h->part_spmv, spmv_grid(h)));
    TRY(dalloc(h, &h->part_vec, 2 * std::max(vec_grid(h), h->upd_blocks)));
    h->part_res_cap = 2 * (int64_t)std::max(spmv_grid(h), kResGridCap);
    TRY(dalloc(h, &h->part_res, h->part_res_cap));
    TRY(dalloc(h, &h->res_out, 4));
    TRY(dalloc(h, &h->st, 1));
    TRY(dalloc(h, &h->scratch_u64, 4));
    h->trace_cap = 16;
    TRY(dalloc(h, &h->trace_k, h->trace_cap));
    TRY(dalloc(h, &h->trace_counts, 3 * dev::kTraceBlocks * h->trace_cap));
#undef TRY

    auto dev_err = [&](hipError_t e, const char* what) {
        return bail(fail(CG_EDEVICE, std::string("cg_create: ") + what + ": " + hipGetErrorString(e)));
    };
    hipError_t e;
    if ((e = hipStreamCreateWithFlags(&h->stream, hipStreamNonBlocking)) != hipSuccess)
        return dev_err(e, "stream");
    for (auto& ev : h->ev)
        if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess)
            return dev_err(e, "event");
    if ((e = hipHostMalloc((void**)&h->pinned, 4 * sizeof(int32_t), hipHostMallocDefault)) != hipSuccess)
        return dev_err(e, "pinned host memory");
    if ((e = hipHostMalloc((void**)&h->res_host, 4 * sizeof(double), hipHostMallocDefault)) != hipSuccess)
        return dev_err(e, "pinned host memory");
    if ((e = hipEventCreateWithFlags(&h->ev_user, hipEventDisableTiming)) != hipSuccess) return dev_err(e, "event");

    for (double* v : {h->x, h->r, h->p, h->q, h->z, h->dinv})
        if (v && (e = hipMemsetAsync(v, 0, sizeof(double) * (size_t)n_pad, s))) return dev_err(e, "vectors");
    // The SpMV never writes a slice's padding entry n, which the pair-wise
    // update kernel reads: it stays zero.
    if (h->qpart && (e = hipMemsetAsync(h->qpart, 0, sizeof(double) * (size_t)n_pad * h->S, s)))
        return dev_err(e, "vectors");
    if ((e = hipMemcpyAsync(h->win_mask, win_mask.data(), sizeof(uint64_t) * win_mask.size(), hipMemcpyHostToDevice, s)) ||
        (e = hipMemcpyAsync(h->win_tile, win_tile.data(), sizeof(int32_t) * win_tile.size(), hipMemcpyHostToDevice, s)) ||
        (e = hipMemcpyAsync(h->tent, tent.data(), sizeof(int2) * tent.size(), hipMemcpyHostToDevice, s)) ||
        (e = hipMemcpyAsync(h->trp, trp.data(), sizeof(int32_t) * trp.size(), hipMemcpyHostToDevice, s)) ||
        (e = hipMemcpyAsync(h->btab, btab.data(), sizeof(int32_t) * btab.size(), hipMemcpyHostToDevice, s)) ||
        (e = hipMemcpyAsync(h->gbatch, gbatch.data(), sizeof(int32_t) * gbatch.size(), hipMemcpyHostToDevice, s)) ||
        (e = hipMemcpyAsync(h->xcb, xcb.data(), sizeof(int32_t) * xcb.size(), hipMemcpyHostToDevice, s)) ||
        (e = hipMemcpyAsync(h->tcol, D->tile_col_idx.data(), sizeof(int32_t) * Td, hipMemcpyHostToDevice, s)) ||
        (e = hipMemcpyAsync(h->trow, trb.data(), sizeof(int32_t) * Td, hipMemcpyHostToDevice, s)) ||
        (e = hipMemcpyAsync(h->tptr, tptr.data(), sizeof(int32_t) * tptr.size(), hipMemcpyHostToDevice, s)) ||
        (e = hipMemcpyAsync(h->meta, h->meta16 ? (const void*)meta16.data() : (const void*)meta8.data(),
                            (h->meta16 ? 2 : 1) * (size_t)nnz, hipMemcpyHostToDevice, s)) ||
        (e = hipMemcpyAsync(h->v64, D->val.data(), sizeof(double) * nnz, hipMemcpyHostToDevice, s)))
        return dev_err(e, "upload");
    if (vlow &&
        ((e = hipMemcpyAsync(h->colexp, colexp_h.data(), sizeof(int16_t) * n, hipMemcpyHostToDevice, s)) ||
         (e = hipMemcpyAsync(vlow, scaled_h.data(), sizeof(double) * nnz, hipMemcpyHostToDevice, s))))
        return dev_err(e, "upload");
    if (h->jacobi &&
        (e = hipMemcpyAsync(h->dinv, dinv_h.data(), sizeof(double) * n, hipMemcpyHostToDevice, s)))
        return dev_err(e, "upload");
    if (!cptr_h.empty() &&
        ((e = hipMemcpyAsync(h->cptr, cptr_h.data(), sizeof(int32_t) * cptr_h.size(), hipMemcpyHostToDevice, s)) ||
         (e = hipMemcpyAsync(h->clist, clist_h.data(), sizeof(int32_t) * Td, hipMemcpyHostToDevice, s)) ||
         (e = hipMemcpyAsync(h->dcount, dcount_h.data(), Td, hipMemcpyHostToDevice, s))))
        return dev_err(e, "upload");
    if (precision_map) {
        if (!h->dperm.empty()) {
            std::vector<uint8_t> dm(Td);
            for (int64_t d = 0; d < Td; ++d) dm[d] = precision_map[h->dperm[d]];
            if ((e = hipMemcpyAsync(h->map, dm.data(), Td, hipMemcpyHostToDevice, s)) ||
                (e = hipStreamSynchronize(s)))
                return dev_err(e, "upload");
        } else if ((e = hipMemcpyAsync(h->map, precision_map, T, hipMemcpyHostToDevice, s))) {
            return dev_err(e, "upload");
        }
    } else if ((e = hipMemsetAsync(h->map, 0, Td, s))) {
        return dev_err(e, "map");
    }
    if ((e = hipMemsetAsync(h->planes, 0, h->planes_bytes, s)) ||
        (e = hipMemsetAsync(h->packed, 0, h->packed_bytes, s)))
        return dev_err(e, "planes");
    hipLaunchKernelGGL(dev::build_segments_kernel,
                       dim3((unsigned)std::max<int64_t>(1, std::min<int64_t>((h->nbatch + 3) / 4, 8192))),
                       dim3(dev::kBlock), 0, s, h->btab, h->nbatch, h->v64, vlow ? vlow : h->v64, h->planes);
    if ((e = hipGetLastError()) != hipSuccess) return dev_err(e, "plane kernel");
    dev::State hs{};
    hs.uprec = -1;
    hs.spmv_uprec = -1;
    hs.trace_cap = (int32_t)h->trace_cap;
    if ((e = hipMemcpyAsync(h->st, &hs, sizeof(hs), hipMemcpyHostToDevice, s))) return dev_err(e, "state");
    launch_repack(h, s);
    if ((e = hipGetLastError()) != hipSuccess) return dev_err(e, "repack kernel");
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return dev_err(e, "set-up");
    *out = h;
    return CG_OK;
}

extern "C" int cg_destroy(cg_handle* h) {
    mpcg::clear_error();
    if (!h) return CG_OK;
    (void)hipDeviceSynchronize();
    drop_graph(h);
    for (auto& e : h->ev)
        if (e) (void)hipEventDestroy(e);
    if (h->pinned) (void)hipHostFree(h->pinned);
    if (h->res_host) (void)hipHostFree(h->res_host);
    if (h->ev_user) (void)hipEventDestroy(h->ev_user);
    if (h->stream) (void)hipStreamDestroy(h->stream);
    delete h;  // frees device buffers
    return CG_OK;
}

extern "C" int cg_get_options(const cg_handle* h, cg_options* out) {
    mpcg::clear_error();
    if (!h || !out) return fail(CG_EINVAL, "cg_get_options: NULL argument");
    *out = cg_options{};
    out->jacobi = h->jacobi ? 1 : 0;
    out->window = h->window;
    out->use_graph = h->use_graph ? 1 : 0;
    out->p1 = h->p1;
    out->col_slices = h->S;
    out->single_block = small_layout(h) ? 1 : -1;
    out->stage_x = h->stage_doubles > 0 ? 1 : 0;
    return CG_OK;
}

extern "C" int cg_get_sizes(const cg_handle* h, int64_t* n, int64_t* T, int64_t* nnz, int32_t* R,
                            int32_t* C) {
    mpcg::clear_error();
    if (!h) return fail(CG_EINVAL, "cg_get_sizes: h is NULL");
    if (n) *n = h->n;
    if (T) *T = h->T;
    if (nnz) *nnz = h->nnz;
    if (R) *R = h->R;
    if (C) *C = h->C;
    return CG_OK;
}

extern "C" int64_t cg_device_bytes(const cg_handle* h) { return h ? h->device_bytes : 0; }

extern "C" int cg_set_precision_map(cg_handle* h, const uint8_t* map, int32_t on_device) {
    mpcg::clear_error();
    if (!h || !map) return fail(CG_EINVAL, "cg_set_precision_map: NULL argument");
    HIP_CHECK(order_after_user(h));
    // A device map is staged through the host so that it is validated like a host map.
    std::vector<uint8_t> staged;
    if (on_device) {
        staged.resize(h->T);
        HIP_CHECK(hipMemcpy(staged.data(), map, h->T, hipMemcpyDeviceToHost));
        map = staged.data();
    }
    for (int64_t t = 0; t < h->T; ++t)
        if (map[t] > 2)
            return fail(CG_EINVAL, "cg_set_precision_map: map[" + std::to_string(t) + "] is not 0, 1 or 2");
    if (!h->dperm.empty()) {  // device order of the tiles
        std::vector<uint8_t> dm(h->Td);
        for (int64_t d = 0; d < h->Td; ++d) dm[d] = map[h->dperm[d]];
        HIP_CHECK(hipMemcpy(h->map, dm.data(), h->Td, hipMemcpyHostToDevice));
    } else {
        HIP_CHECK(hipMemcpy(h->map, map, h->T, hipMemcpyHostToDevice));
    }
    HIP_CHECK(repack(h));
    h->sched = kSchedStatic;
    return upload_schedule(h);
}

extern "C" int cg_get_active_map(const cg_handle* h, uint8_t* out) {
    mpcg::clear_error();
    if (!h || !out) return fail(CG_EINVAL, "cg_get_active_map: NULL argument");
    dev::State hs{};
    HIP_CHECK(hipMemcpy(&hs, h->st, sizeof(hs), hipMemcpyDeviceToHost));
    if (hs.uprec >= 0) {
        std::memset(out, hs.uprec, h->T);
        return CG_OK;
    }
    if (h->sched == kSchedPMag) {  // the column-block codes last computed, per tile
        std::vector<uint8_t> code(std::max<int64_t>(h->ncb, 1));
        std::vector<int32_t> tcol(std::max<int64_t>(h->Td, 1));
        HIP_CHECK(hipMemcpy(code.data(), h->cbcode, h->ncb, hipMemcpyDeviceToHost));
        if (h->Td) HIP_CHECK(hipMemcpy(tcol.data(), h->tcol, sizeof(int32_t) * h->Td, hipMemcpyDeviceToHost));
        for (int64_t d = 0; d < h->Td; ++d) out[h->dperm.empty() ? d : h->dperm[d]] = code[tcol[d]];
        return CG_OK;
    }
    if (!h->dperm.empty()) {  // device order of the tiles (the pieces of a tile agree)
        std::vector<uint8_t> dm(h->Td);
        HIP_CHECK(hipMemcpy(dm.data(), h->map, h->Td, hipMemcpyDeviceToHost));
        for (int64_t d = 0; d < h->Td; ++d) out[h->dperm[d]] = dm[d];
        return CG_OK;
    }
    HIP_CHECK(hipMemcpy(out, h->map, h->T, hipMemcpyDeviceToHost));
    return CG_OK;
}

extern "C" int cg_map_from_magnitude(cg_handle* h, double t_bf16, double t_fp32) {
    mpcg::clear_error();
    if (!h) return fail(CG_EINVAL, "cg_map_from_magnitude: h is NULL");
    HIP_CHECK(order_after_user(h));
    if (!(t_bf16 <= t_fp32)) return fail(CG_EINVAL, "cg_map_from_magnitude: need t_bf16 <= t_fp32");
    HIP_CHECK(hipMemset(h->scratch_u64, 0, sizeof(unsigned long long)));
    hipLaunchKernelGGL(dev::diag_absmax_kernel, dim3(grid_for(h->Td, 1, 8192)), dim3(dev::kBlock), 0, h->stream,
                       h->trow, h->tcol, h->tptr, (const void*)h->meta, h->meta16 ? 1 : 0, h->v64,
                       (int32_t)h->Td, h->Rd, h->C, h->scratch_u64);
    // Per canonical tile over its pieces (slabs), else per device tile.
    const int64_t units = h->cptr ? h->T : h->Td;
    hipLaunchKernelGGL(dev::magnitude_map_kernel, dim3(grid_for(units, 1, 8192)), dim3(dev::kBlock), 0, h->stream,
                       h->tptr, h->v64, (int32_t)units, (const int32_t*)h->cptr, (const int32_t*)h->clist,
                       (const unsigned long long*)h->scratch_u64, t_bf16, t_fp32, h->map);
    HIP_CHECK(hipGetLastError());
    HIP_CHECK(repack(h));
    h->sched = kSchedStatic;
    return upload_schedule(h);
}

extern "C" int cg_set_schedule_residual(cg_handle* h, int32_t nstage, const double* thresholds,
                                        const uint8_t* prec) {
    mpcg::clear_error();
    if (!h || !prec) return fail(CG_EINVAL, "cg_set_schedule_residual: NULL argument");
    HIP_CHECK(order_after_user(h));
    if (nstage < 1 || nstage > 8) return fail(CG_EINVAL, "cg_set_schedule_residual: nstage must lie in [1, 8]");
    if (nstage > 1 && !thresholds) return fail(CG_EINVAL, "cg_set_schedule_residual: thresholds is NULL");
    // Checked in full before the handle changes: a rejected call leaves the schedule as it was.
    for (int i = 0; i < nstage; ++i)
        if (prec[i] > 2) return fail(CG_EINVAL, "cg_set_schedule_residual: prec values must be 0, 1 or 2");
    for (int i = 0; i + 1 < nstage; ++i)
        if (!std::isfinite(thresholds[i]))
            return fail(CG_EINVAL, "cg_set_schedule_residual: thresholds must be finite");
    h->thresholds.assign(thresholds, thresholds + (nstage - 1));
    h->stage_prec.assign(prec, prec + nstage);
    h->sched = kSchedResidual;
    return upload_schedule(h);
}

extern "C" int cg_set_schedule_tile_rule(cg_handle* h, int32_t period, const double* scores, double hi,
                                         double lo) {
    mpcg::clear_error();
    if (!h || !scores) return fail(CG_EINVAL, "cg_set_schedule_tile_rule: NULL argument");
    HIP_CHECK(order_after_user(h));
    if (period < 1) return fail(CG_EINVAL, "cg_set_schedule_tile_rule: period must be >= 1");
    if (!(lo <= hi)) return fail(CG_EINVAL, "cg_set_schedule_tile_rule: need lo <= hi");
    if (!h->scores) {
        int rc = dalloc(h, &h->scores, std::max<int64_t>(h->Td, 1));
        if (rc != CG_OK) return rc;
    }
    if (!h->dperm.empty()) {  // every device tile takes its canonical tile's score
        std::vector<double> ds(h->Td);
        for (int64_t d = 0; d < h->Td; ++d) ds[d] = scores[h->dperm[d]];
        HIP_CHECK(hipMemcpy(h->scores, ds.data(), sizeof(double) * h->Td, hipMemcpyHostToDevice));
    } else {
        HIP_CHECK(hipMemcpy(h->scores, scores, sizeof(double) * h->T, hipMemcpyHostToDevice));
    }
    h->period = period;
    h->hi = hi;
    h->lo = lo;
    h->sched = kSchedTileRule;
    return upload_schedule(h);
}

extern "C" int cg_set_schedule_pmag(cg_handle* h, double lo, double hi, int32_t period) {
    mpcg::clear_error();
    if (!h) return fail(CG_EINVAL, "cg_set_schedule_pmag: h is NULL");
    HIP_CHECK(order_after_user(h));
    if (std::isnan(lo) || std::isnan(hi) || !(lo <= hi))
        return fail(CG_EINVAL, "cg_set_schedule_pmag: need lo <= hi (no NaN)");
    if (period < 1) return fail(CG_EINVAL, "cg_set_schedule_pmag: period must be >= 1");
    if (!h->cbcode) {
        h->ncb = (h->n + h->C - 1) / h->C;
        std::vector<int32_t> tcol(std::max<int64_t>(h->Td, 1));
        if (h->Td) HIP_CHECK(hipMemcpy(tcol.data(), h->tcol, sizeof(int32_t) * h->Td, hipMemcpyDeviceToHost));
        std::vector<uint8_t> dcount(h->dcount ? h->Td : 0);
        if (h->dcount) HIP_CHECK(hipMemcpy(dcount.data(), h->dcount, h->Td, hipMemcpyDeviceToHost));
        std::vector<int32_t> tpcb(h->ncb, 0);  // canonical tiles per column block
        for (int64_t d = 0; d < h->Td; ++d)
            if (!h->dcount || dcount[d]) ++tpcb[tcol[d]];
        int rc = dalloc(h, &h->cbcode, h->ncb);
        if (rc == CG_OK) rc = dalloc(h, &h->tpcb, h->ncb);
        if (rc != CG_OK) return rc;
        HIP_CHECK(hipMemcpy(h->tpcb, tpcb.data(), sizeof(int32_t) * h->ncb, hipMemcpyHostToDevice));
        HIP_CHECK(hipMemset(h->cbcode, 0, h->ncb));
    }
    h->pm_lo = lo;
    h->pm_hi = hi;
    h->pm_period = period;
    h->sched = kSchedPMag;
    drop_graph(h);  // the thresholds are baked into the captured launches
    return upload_schedule(h);
}

extern "C" int cg_record_column_codes(cg_handle* h, int32_t enable) {
    mpcg::clear_error();
    if (!h) return fail(CG_EINVAL, "cg_record_column_codes: h is NULL");
    HIP_CHECK(order_after_user(h));
    h->rec_cb = enable != 0;
    drop_graph(h);
    return CG_OK;
}

extern "C" int cg_get_column_codes(const cg_handle* h, int32_t cap, uint8_t* out) {
    mpcg::clear_error();
    if (!h) return fail(CG_EINVAL, "cg_get_column_codes: h is NULL");
    if (h->sched != kSchedPMag || !h->cbhist) return 0;
    dev::State hs{};
    HIP_CHECK(hipMemcpy(&hs, h->st, sizeof(hs), hipMemcpyDeviceToHost));
    const int64_t n = std::min<int64_t>(std::min<int64_t>(hs.ntrace, h->cbhist_rows), std::max(cap, 0));
    if (n > 0 && out) HIP_CHECK(hipMemcpy(out, h->cbhist, (size_t)(n * h->ncb), hipMemcpyDeviceToHost));
    return (int)std::min<int64_t>(hs.ntrace, h->cbhist_rows);
}

extern "C" int cg_record_window_maps(cg_handle* h, int32_t cap) {
    mpcg::clear_error();
    if (!h) return fail(CG_EINVAL, "cg_record_window_maps: h is NULL");
    HIP_CHECK(order_after_user(h));
    if (cap < 0) return fail(CG_EINVAL, "cg_record_window_maps: cap must be >= 0");
    if (h->winmaps) {
        HIP_CHECK(hipDeviceSynchronize());
        dfree(h, h->winmaps);
        h->winmaps = nullptr;
        h->winmap_cap = 0;
    }
    if (cap > 0) {
        const int rc = dalloc(h, &h->winmaps, (int64_t)cap * h->Td);
        if (rc != CG_OK) return rc;
        h->winmap_cap = cap;
    }
    drop_graph(h);  // the captured tile-rule launches carry the buffer
    return CG_OK;
}

extern "C" int cg_get_window_maps(const cg_handle* h, int32_t cap, uint8_t* out) {
    mpcg::clear_error();
    if (!h) return fail(CG_EINVAL, "cg_get_window_maps: h is NULL");
    if (h->sched != kSchedTileRule || !h->winmaps) return 0;
    dev::State hs{};
    HIP_CHECK(hipMemcpy(&hs, h->st, sizeof(hs), hipMemcpyDeviceToHost));
    const int64_t avail = std::min<int64_t>(hs.ntrace, h->winmap_cap);
    const int64_t m = std::min<int64_t>(avail, std::max(cap, 0));
    if (m > 0 && out) {
        if (!h->dperm.empty()) {  // device order of the tiles (the pieces of a tile agree)
            std::vector<uint8_t> dm((size_t)(m * h->Td));
            HIP_CHECK(hipMemcpy(dm.data(), h->winmaps, dm.size(), hipMemcpyDeviceToHost));
            for (int64_t w = 0; w < m; ++w)
                for (int64_t d = 0; d < h->Td; ++d) out[w * h->T + h->dperm[d]] = dm[w * h->Td + d];
        } else {
            HIP_CHECK(hipMemcpy(out, h->winmaps, (size_t)(m * h->T), hipMemcpyDeviceToHost));
        }
    }
    return (int)avail;
}

extern "C" int cg_eval_tile_rule(cg_handle* h, double rho) {
    mpcg::clear_error();
    if (!h) return fail(CG_EINVAL, "cg_eval_tile_rule: h is NULL");
    HIP_CHECK(order_after_user(h));
    if (h->sched != kSchedTileRule) return fail(CG_EINVAL, "cg_eval_tile_rule: no tile rule is set");
    dev::MapArgs ma = map_args(h, rho, 0);
    hipLaunchKernelGGL(dev::tile_rule_kernel, dim3(tile_rule_grid(h)), dim3(dev::kBlock), 0, h->stream, ma);
    HIP_CHECK(hipGetLastError());
    HIP_CHECK(repack(h));
    return CG_OK;
}

extern "C" int cg_clear_schedule(cg_handle* h) {
    mpcg::clear_error();
    if (!h) return fail(CG_EINVAL, "cg_clear_schedule: h is NULL");
    HIP_CHECK(order_after_user(h));
    h->sched = kSchedStatic;
    return upload_schedule(h);
}

extern "C" int cg_spmv(cg_handle* h, const double* x, double* y, void* stream) {
    mpcg::clear_error();
    if (!h || !x || !y) return fail(CG_EINVAL, "cg_spmv: NULL argument");
    if (ranges_overlap(x, y, sizeof(double) * h->n)) return fail(CG_EINVAL, "cg_spmv: y overlaps x");
    if (h->sched == kSchedPMag) launch_pmag(h, x, 0, static_cast<hipStream_t>(stream));  // map from x
    if (h->S > 1) {  // the slices' partial products, then their sum
        dev::SpmvArgs a = spmv_args(h, x, h->qpart, &h->st->spmv_uprec);
        launch_spmv<dev::kSpmvPlain>(h, a, static_cast<hipStream_t>(stream));
        launch_combine(h, nullptr, y, static_cast<hipStream_t>(stream));
    } else {
        dev::SpmvArgs a = spmv_args(h, x, y, &h->st->spmv_uprec);
        launch_spmv<dev::kSpmvPlain>(h, a, static_cast<hipStream_t>(stream));
    }
    HIP_CHECK(hipGetLastError());
    HIP_CHECK(note_user_launch(h, static_cast<hipStream_t>(stream)));
    return CG_OK;
}

extern "C" int cg_true_residual(cg_handle* h, const double* b, const double* x, double* out, void* stream) {
    mpcg::clear_error();
    if (!h || !b || !x || !out) return fail(CG_EINVAL, "cg_true_residual: NULL argument");
    hipStream_t s = static_cast<hipStream_t>(stream);
    HIP_CHECK(order_after_user(h));  // the result is copied through the handle's pinned buffer
    int rc = launch_true_residual(h, b, x, h->part_res, h->res_out, s);
    if (rc != CG_OK) return rc;
    HIP_CHECK(hipMemcpyAsync(h->res_host, h->res_out, sizeof(double), hipMemcpyDeviceToHost, s));
    HIP_CHECK(hipStreamSynchronize(s));
    *out = h->res_host[0];
    return CG_OK;
}

extern "C" int cg_true_residual_noalloc(cg_handle* h, const double* b, const double* x, double* out, void* stream) {
    mpcg::clear_error();
    if (!h || !b || !x || !out) return fail(CG_EINVAL, "cg_true_residual_noalloc: NULL argument");
    double* sp = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (h->device >= 0 && h->device < kMaxDevices) sp = g_scratch_ptr[h->device];
    }
    if (!sp) return fail(CG_EDEVICE, "cg_true_residual_noalloc: no scratch address for the handle's device");
    const int64_t parts = h->S > 1 ? grid_for(h->n, 4, kResGridCap) : spmv_grid(h);
    if (2 * parts > kNoAllocScratchDoubles)
        return fail(CG_EINVAL, "cg_true_residual_noalloc: " + std::to_string(2 * parts) +
                                   " partial sums exceed the static scratch of " +
                                   std::to_string(kNoAllocScratchDoubles));
    return launch_true_residual(h, b, x, sp, out, static_cast<hipStream_t>(stream));
}

extern "C" int cg_solve(cg_handle* h, const double* b, const double* x0, double tol, int32_t maxit,
                        double* x, int32_t* iterations, double* res_hist, void* stream) {
    mpcg::clear_error();
    if (!h || !b || !x || !iterations) return fail(CG_EINVAL, "cg_solve: NULL argument");
    if (!(tol >= 0.0)) return fail(CG_EINVAL, "cg_solve: tol must be >= 0");
    if (maxit < 0) return fail(CG_EINVAL, "cg_solve: maxit must be >= 0");
    hipStream_t user = static_cast<hipStream_t>(stream);
    hipStream_t s = h->stream;

    // History and trace capacity.
    if (h->hist_cap < (int64_t)maxit + 1) {
        dfree(h, h->hist);
        h->hist = nullptr;
        int rc = dalloc(h, &h->hist, (int64_t)maxit + 1);
        if (rc != CG_OK) return rc;
        h->hist_cap = (int64_t)maxit + 1;
        drop_graph(h);
    }
    int64_t need_trace = 16;
    if (h->sched == kSchedTileRule) {
        need_trace = maxit / h->period + 2;
        h->planes_map = true;  // the windows change the map without repacking it
    }
    if (h->sched == kSchedResidual) need_trace = (int64_t)h->stage_prec.size() + 1;
    if (h->sched == kSchedPMag) need_trace = (int64_t)maxit / h->pm_period + 2;
    if (need_trace > h->trace_cap) {
        dfree(h, h->trace_k);
        dfree(h, h->trace_counts);
        h->trace_k = nullptr;
        h->trace_counts = nullptr;
        int rc = dalloc(h, &h->trace_k, need_trace);
        if (rc == CG_OK) rc = dalloc(h, &h->trace_counts, 3 * dev::kTraceBlocks * need_trace);
        if (rc != CG_OK) return rc;
        h->trace_cap = need_trace;
        drop_graph(h);
    }
    if (h->sched == kSchedPMag && h->rec_cb && h->cbhist_rows < h->trace_cap) {
        dfree(h, h->cbhist);
        h->cbhist = nullptr;
        h->cbhist_rows = 0;
        int rc = dalloc(h, &h->cbhist, h->trace_cap * h->ncb);
        if (rc != CG_OK) return rc;
        h->cbhist_rows = h->trace_cap;
        drop_graph(h);
    }

    // Order after the caller's prior work (and a cg_spmv on another stream).
    HIP_CHECK(order_after_user(h));
    HIP_CHECK(hipEventRecord(h->ev[0], user));
    HIP_CHECK(hipStreamWaitEvent(s, h->ev[0], 0));

    dev::State hs{};
    HIP_CHECK(hipMemcpyAsync(&hs, h->st, sizeof(hs), hipMemcpyDeviceToHost, s));
    HIP_CHECK(hipStreamSynchronize(s));
    hs.tol = tol;
    hs.maxit = maxit;
    hs.done = 0;
    hs.k = 0;
    hs.trace_cap = (int32_t)h->trace_cap;
    hs.ntrace = 0;
    HIP_CHECK(hipMemcpyAsync(h->st, &hs, sizeof(hs), hipMemcpyHostToDevice, s));

    const int64_t ncount = 3 * dev::kTraceBlocks * h->trace_cap;
    hipLaunchKernelGGL(dev::fill_i32_kernel, dim3(grid_for(ncount, 4, 1024)), dim3(dev::kBlock), 0, s,
                       h->trace_counts, (int32_t)0, ncount);
    dev::VecArgs va = vec_args(h, b, x0);
    if (x0) {
        // r0 = b - A x0 with the exact FP64 values.
        if (h->S > 1) {
            dev::SpmvArgs sa = spmv_args(h, x0, h->qpart, &h->st->zero_prec);
            sa.p1_round = 0;
            launch_spmv<dev::kSpmvPlain>(h, sa, s);
            launch_combine(h, b, h->r, s);
        } else {
            dev::SpmvArgs sa = spmv_args(h, x0, h->r, &h->st->zero_prec);
            sa.b = b;
            sa.p1_round = 0;
            launch_spmv<dev::kSpmvResidual>(h, sa, s);
        }
        va.r_ready = 1;
    }
    hipLaunchKernelGGL(dev::cg_init_kernel, dim3(vec_grid(h)), dim3(dev::kBlock), 0, s, va);
    hipLaunchKernelGGL(dev::cg_init_finish_kernel, dim3(1), dim3(dev::kBlock), 0, s, va);
    if (h->sched == kSchedPMag) launch_pmag(h, h->p, 1, s);  // the map of iteration 0 from p_0
    HIP_CHECK(hipGetLastError());
    const bool static_map = h->sched == kSchedStatic;
    if (static_map) {
        hipLaunchKernelGGL(dev::map_count_kernel, dim3(dev::kTraceBlocks), dim3(dev::kBlock), 0, s, h->map,
                           (const uint8_t*)h->dcount, h->Td, h->trace_k, h->trace_counts);
    }

    // Small systems: every iteration in one launch. Otherwise iterate in
    // windows and poll the device stop flag of the previous window while the
    // current one runs.
    const bool small = single_block_solve(h);
    if (small) {
        launch_small(h, s);
        HIP_CHECK(hipGetLastError());
    }
    int polled = 0;
    if (h->use_graph && !small) {
        int rc = ensure_graph(h);
        if (rc != CG_OK) return rc;
    }
    int64_t windows = 0;
    int32_t done = 0, kdone = 0;
    const int W = solve_window(h);
    const int64_t max_windows = (int64_t)maxit / W + 2;
    while (!small) {
        if (windows < max_windows) {
            // Split max|p| rule: window w ends at k = (w + 1) W; evaluate when that is a
            // multiple of the period.
            const bool rule_at_end = pmag_split(h) && ((windows + 1) * W) % h->pm_period == 0;
            if (h->use_graph) {
                HIP_CHECK(hipGraphLaunch(rule_at_end ? h->graph_rule : h->graph, s));
            } else {
                for (int i = 0; i < W; ++i) enqueue_iteration(h, i, s, rule_at_end);
                HIP_CHECK(hipGetLastError());
            }
            const int slot = (int)(windows & 1);
            HIP_CHECK(hipMemcpyAsync(h->pinned + 2 * slot, &h->st->done, sizeof(int32_t) * 2,
                                     hipMemcpyDeviceToHost, s));
            HIP_CHECK(hipEventRecord(h->ev[slot], s));
            ++windows;
        }
        if (windows - polled >= 2 || windows >= max_windows) {
            const int slot = (int)(polled & 1);
            HIP_CHECK(hipEventSynchronize(h->ev[slot]));
            done = h->pinned[2 * slot];
            kdone = h->pinned[2 * slot + 1];
            ++polled;
            if (done || polled >= windows) break;
        }
    }
    HIP_CHECK(hipStreamSynchronize(s));

    HIP_CHECK(hipMemcpy(&hs, h->st, sizeof(hs), hipMemcpyDeviceToHost));
    if (static_map) {
        // One trace entry: the static map at k = 0.
        hs.ntrace = 1;
        HIP_CHECK(hipMemcpy(&h->st->ntrace, &hs.ntrace, sizeof(int32_t), hipMemcpyHostToDevice));
    }
    (void)kdone;
    *iterations = hs.k;
    if (res_hist) HIP_CHECK(hipMemcpy(res_hist, h->hist, sizeof(double) * (hs.k + 1), hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpyAsync(x, h->x, sizeof(double) * h->n, hipMemcpyDeviceToDevice, s));
    HIP_CHECK(hipEventRecord(h->ev[0], s));
    HIP_CHECK(hipStreamWaitEvent(user, h->ev[0], 0));
    HIP_CHECK(hipStreamSynchronize(s));
    if (hs.done == 1) return CG_OK;
    if (hs.done == 3) return CG_BREAKDOWN;
    return CG_NOT_CONVERGED;
}

extern "C" int cg_get_map_trace(const cg_handle* h, int32_t cap, int32_t* k_out, int64_t* counts_out) {
    mpcg::clear_error();
    if (!h) return fail(CG_EINVAL, "cg_get_map_trace: h is NULL");
    dev::State hs{};
    HIP_CHECK(hipMemcpy(&hs, h->st, sizeof(hs), hipMemcpyDeviceToHost));
    int64_t n = std::min<int64_t>(hs.ntrace, h->trace_cap);
    int64_t m = std::min<int64_t>(n, cap);
    if (m > 0 && k_out) HIP_CHECK(hipMemcpy(k_out, h->trace_k, sizeof(int32_t) * m, hipMemcpyDeviceToHost));
    if (m > 0 && counts_out) {
        std::vector<int32_t> per_block((size_t)m * dev::kTraceBlocks * 3);
        HIP_CHECK(hipMemcpy(per_block.data(), h->trace_counts, sizeof(int32_t) * per_block.size(),
                            hipMemcpyDeviceToHost));
        for (int64_t i = 0; i < m; ++i)
            for (int p = 0; p < 3; ++p) {
                int64_t sum = 0;
                for (int b = 0; b < dev::kTraceBlocks; ++b) sum += per_block[((size_t)i * dev::kTraceBlocks + b) * 3 + p];
                counts_out[3 * i + p] = sum;
            }
    }
    return hs.ntrace;
}

extern "C" int cg_export_column_scale(const cg_handle* h, int32_t* out) {
    mpcg::clear_error();
    if (!h || !out) return fail(CG_EINVAL, "cg_export_column_scale: NULL argument");
    std::vector<int16_t> e(h->n, 0);
    if (h->colexp) HIP_CHECK(hipMemcpy(e.data(), h->colexp, sizeof(int16_t) * h->n, hipMemcpyDeviceToHost));
    for (int64_t j = 0; j < h->n; ++j) out[j] = e[j];
    return CG_OK;
}

extern "C" int cg_export_layout(const cg_handle* h, int64_t* tile_row_ptr, int32_t* tile_col_idx,
                                int64_t* tile_nnz_ptr, uint16_t* row_idx, uint8_t* col_local, double* val64,
                                float* val32, uint16_t* bf16) {
    mpcg::clear_error();
    if (!h) return fail(CG_EINVAL, "cg_export_layout: h is NULL");
    const int64_t T = h->T, Td = h->Td, nnz = h->nnz;
    std::vector<int32_t> trp(h->nrb + 1);  // canonical tile row pointers
    HIP_CHECK(hipMemcpy(trp.data(), h->trp, sizeof(int32_t) * trp.size(), hipMemcpyDeviceToHost));
    if (tile_row_ptr)
        for (size_t i = 0; i < trp.size(); ++i) tile_row_ptr[i] = trp[i];
    std::vector<int32_t> dt(Td + 1), tcol(std::max<int64_t>(Td, 1)), trow(std::max<int64_t>(Td, 1));
    HIP_CHECK(hipMemcpy(dt.data(), h->tptr, sizeof(int32_t) * dt.size(), hipMemcpyDeviceToHost));
    if (Td) {
        HIP_CHECK(hipMemcpy(tcol.data(), h->tcol, sizeof(int32_t) * Td, hipMemcpyDeviceToHost));
        HIP_CHECK(hipMemcpy(trow.data(), h->trow, sizeof(int32_t) * Td, hipMemcpyDeviceToHost));
    }
    // Row offsets (from the device tile's row block) and local columns.
    std::vector<uint16_t> r(std::max<int64_t>(nnz, 1));
    std::vector<uint8_t> c(std::max<int64_t>(nnz, 1));
    if (h->meta16) {
        std::vector<uint16_t> m(std::max<int64_t>(nnz, 1));
        HIP_CHECK(hipMemcpy(m.data(), h->meta, 2 * (size_t)nnz, hipMemcpyDeviceToHost));
        for (int64_t k = 0; k < nnz; ++k) {
            r[k] = (uint16_t)(m[k] >> 8);
            c[k] = (uint8_t)(m[k] & 255);
        }
    } else {
        std::vector<uint8_t> m(std::max<int64_t>(nnz, 1));
        HIP_CHECK(hipMemcpy(m.data(), h->meta, (size_t)nnz, hipMemcpyDeviceToHost));
        for (int64_t k = 0; k < nnz; ++k) {
            r[k] = (uint16_t)(m[k] >> 4);
            c[k] = (uint8_t)(m[k] & 15);
        }
    }
    // Device order of tiles and nonzeros; with column slices or slabs it is
    // mapped back to the canonical order: device tile d is (a piece of)
    // canonical tile dperm[d]; a piece's rows move by its slab's offset in the
    // row block, and the pieces of a tile merge column by column.
    const bool reordered = !h->dperm.empty();
    std::vector<int64_t> ct;   // canonical tile pointers
    std::vector<int64_t> pos;  // canonical position of every device nonzero
    if (reordered) {
        ct.assign(T + 1, 0);
        std::vector<int32_t> cp(T + 1, 0), cl(Td), crb(std::max<int64_t>(T, 1), 0);
        for (int64_t d = 0; d < Td; ++d) {
            ct[h->dperm[d] + 1] += dt[d + 1] - dt[d];
            ++cp[h->dperm[d] + 1];
        }
        for (int64_t t = 0; t < T; ++t) {
            ct[t + 1] += ct[t];
            cp[t + 1] += cp[t];
        }
        {
            std::vector<int32_t> fill(cp.begin(), cp.end() - 1);
            for (int64_t d = 0; d < Td; ++d) cl[fill[h->dperm[d]]++] = (int32_t)d;
        }
        for (int64_t I = 0; I < h->nrb; ++I)
            for (int64_t t = trp[I]; t < trp[I + 1]; ++t) crb[t] = (int32_t)I;
        pos.assign(std::max<int64_t>(nnz, 1), 0);
        mpcg::parallel_for(T, [&](int64_t lo, int64_t hi) {
            std::vector<std::pair<int64_t, int64_t>> ent;  // (local column, canonical row offset) key, device index
            for (int64_t t = lo; t < hi; ++t) {
                ent.clear();
                for (int32_t q = cp[t]; q < cp[t + 1]; ++q) {
                    const int64_t d = cl[q];
                    const int64_t off = (int64_t)trow[d] * h->Rd - (int64_t)crb[t] * h->R;
                    for (int64_t k = dt[d]; k < dt[d + 1]; ++k) {
                        r[k] = (uint16_t)(r[k] + off);
                        ent.emplace_back(((int64_t)c[k] << 20) | r[k], k);
                    }
                }
                std::sort(ent.begin(), ent.end());
                for (size_t i = 0; i < ent.size(); ++i) pos[ent[i].second] = ct[t] + (int64_t)i;
            }
        });
    }
    // Copies a per-nonzero array from device order into canonical order.
    auto to_canonical = [&](const char* src, char* dst, size_t w) {
        if (!reordered) {
            std::memcpy(dst, src, w * (size_t)nnz);
            return;
        }
        for (int64_t k = 0; k < nnz; ++k) std::memcpy(dst + w * (size_t)pos[k], src + w * (size_t)k, w);
    };
    if (tile_col_idx)
        for (int64_t d = 0; d < Td; ++d) tile_col_idx[reordered ? h->dperm[d] : d] = tcol[d];
    if (tile_nnz_ptr)
        for (int64_t t = 0; t <= T; ++t) tile_nnz_ptr[t] = reordered ? ct[t] : dt[t];
    if (row_idx) to_canonical((const char*)r.data(), (char*)row_idx, 2);
    if (col_local) to_canonical((const char*)c.data(), (char*)col_local, 1);
    if (val64) {
        std::vector<double> v(std::max<int64_t>(nnz, 1));
        HIP_CHECK(hipMemcpy(v.data(), h->v64, sizeof(double) * nnz, hipMemcpyDeviceToHost));
        to_canonical((const char*)v.data(), (char*)val64, sizeof(double));
    }
    if (val32 || bf16) {
        // The reduced planes live in the per-batch segments.
        std::vector<char> seg(h->planes_bytes);
        HIP_CHECK(hipMemcpy(seg.data(), h->planes, seg.size(), hipMemcpyDeviceToHost));
        std::vector<float> v32(std::max<int64_t>(nnz, 1));
        std::vector<uint16_t> v16(std::max<int64_t>(nnz, 1));
        for (int64_t b = 0; b < h->nbatch; ++b) {
            const int32_t* e = &h->btab_host[(size_t)b * dev::kBtFields];
            const int64_t first = e[dev::kBtFirstNnz], len = e[dev::kBtLen];
            const char* base = seg.data() + (int64_t)e[dev::kBtSegment] * 16;
            std::memcpy(v32.data() + first, base + 8 * len, 4 * len);
            std::memcpy(v16.data() + first, base + 12 * len, 2 * len);
        }
        if (val32) to_canonical((const char*)v32.data(), (char*)val32, 4);
        if (bf16) to_canonical((const char*)v16.data(), (char*)bf16, 2);
    }
    return CG_OK;
}
