// Device code for gfx950: value-plane builder, mixed-precision Tile-CSC SpMV,
// fused CG vector updates with single-pass grid reductions, a single-workgroup
// CG loop for small systems, the column-slice combine, and map kernels.
//
// Method: EvoCG paper ("EvoCG: Self-Evolving Precision Control for Faster
// Conjugate Gradient"): Tile-CSC and value streams (Sec. 3.3, Fig. 4), the
// perturbed product (A + E(a)) p (Eq. (2), Eq. (5)), the CG recurrence
// (Sec. 2.1, Eq. (1), Fig. 1), Jacobi-PCG (Sec. 4.6), fused reductions with
// scalars kept on the device (Sec. 3.4 "Fused Execution and Graph Replay").
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mpcg {
namespace dev {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kTileBatch = 64;   // tile descriptors staged in LDS per pass
constexpr int kMaxRows = 256;    // rows owned by one wavefront (taller row blocks run as slabs of at most this)
constexpr int kMaxGroupRB = 63;  // row blocks per wavefront at most (boundaries fit one wave)

// Solver scalars, resident on the device for the whole solve. Each field has
// one writer per kernel launch (thread 0 of block 0) and no other block of
// that launch reads it, except `done` (see cg_direction_kernel). In the
// single-workgroup loop thread 0 writes them and reads back only its own
// stores (stage and trace counters through atomic loads; cg_small_kernel).
struct State {
    double rz;        // r.z of the current iterate (r.r for plain CG)
    double rz_prev;   // r.z before the current update (copied by the update kernel)
    double rr;        // r.r of the current iterate
    double norm0;     // ||r_0||
    double alpha;
    double beta;
    double pq;
    double tol;
    double thresholds[7];
    int32_t done;     // 0 running, 1 converged, 2 iteration cap, 3 breakdown
    int32_t k;        // completed iterations (kept next to done: polled together)
    int32_t maxit;
    int32_t bd;       // breakdown found by the update kernel of this iteration
    int32_t uprec;    // precision used by the solver's SpMV: -1 = per-tile map, else uniform
    int32_t spmv_uprec;  // the same for cg_spmv
    int32_t zero_prec;   // always 0: exact FP64 products (initial residual)
    int32_t stage;
    int32_t nstage;
    int32_t stage_prec[8];
    int32_t ntrace;
    int32_t trace_cap;
    int32_t period;      // tile-rule window length (0: no tile rule)
    int32_t live;        // set by the update kernel: this iteration runs (the direction kernel's gate)
    double hi, lo;       // tile-rule thresholds
};

// Map-trace counts are kept per block of the map kernels: [entry][kTraceBlocks][3].
constexpr int kTraceBlocks = 256;

__device__ inline int load_done(const State* st) {
    return __hip_atomic_load(&st->done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void store_done(State* st, int v) {
    __hip_atomic_store(&st->done, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Rounding FP64 -> small binary formats with an 8-bit exponent (bias 127):
// FP32 (m = 23 fraction bits) and BF16 (m = 7). IEEE round-to-nearest-even,
// one step from the FP64 value, subnormals kept, overflow to infinity, NaN to
// the canonical quiet NaN. Integer arithmetic only, so the result does not
// depend on the floating-point mode of the device.
// ---------------------------------------------------------------------------
template <int M>
__host__ __device__ inline uint32_t round_f64_to_e8(uint64_t u) {
    const uint32_t sign = (uint32_t)(u >> 63) << (8 + M);
    const int e = (int)((u >> 52) & 0x7FF);
    const uint64_t frac = u & ((1ull << 52) - 1);
    const uint32_t inf = 255u << M;
    if (e == 0x7FF) return frac ? (inf | (1u << (M - 1))) : (sign | inf);
    if (e == 0) return sign;  // FP64 zeros and subnormals are far below half the smallest target value
    const int E = e - 1023;
    const uint64_t s = (1ull << 52) | frac;  // value = s * 2^(E-52)
    const int qe = (E - M > -126 - M) ? (E - M) : (-126 - M);  // exponent of one target ulp
    const int shift = qe - (E - 52);                            // low bits of s that are dropped
    if (shift > 63) return sign;
    uint64_t q = s >> shift;
    const uint64_t rem = s & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    uint64_t bits;
    if (qe == -126 - M) {
        bits = q;  // subnormal; q = 2^M becomes the smallest normal through the exponent carry
    } else {
        bits = ((uint64_t)(E + 126) << M) + q;  // q in [2^M, 2^(M+1)]: the carry lands in the exponent
    }
    if (bits >= inf) bits = inf;
    return sign | (uint32_t)bits;
}

// ---------------------------------------------------------------------------
// Reduction helpers.
// ---------------------------------------------------------------------------
__device__ inline double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Block sum in a fixed order over NW wavefronts; the result is valid in
// every thread.
template <int NW = kWavesPerBlock>
__device__ inline double block_sum(double v, double* s_tmp) {
    v = wave_sum(v);
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    __syncthreads();
    if (lane == 0) s_tmp[w] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < NW; ++i) t += s_tmp[i];
    return t;
}

// Sum of nparts per-block partials (NV values each) in a fixed order: every
// thread of the block gets the same value, and every block that calls this on
// the same data gets the same bits. A thread takes
// partials threadIdx.x + k * blockDim.x; it loads eight of them at once (eight
// independent loads in flight instead of one at a time) into eight running
// sums, adds the rest one by one into the first, and the block reduces.
template <int NV, int NW = kWavesPerBlock>
__device__ inline void sum_partials(const double* partials, int nparts, double (&out)[NV],
                                    double* s_tmp) {
    constexpr int kLoads = 8;
    double acc[kLoads][NV];
#pragma unroll
    for (int u = 0; u < kLoads; ++u)
#pragma unroll
        for (int j = 0; j < NV; ++j) acc[u][j] = 0.0;
    const int stride = blockDim.x;
    int i = threadIdx.x;
    for (; i + (kLoads - 1) * stride < nparts; i += kLoads * stride) {
        double v[kLoads][NV];
#pragma unroll
        for (int u = 0; u < kLoads; ++u)
#pragma unroll
            for (int j = 0; j < NV; ++j) v[u][j] = partials[(size_t)(i + u * stride) * NV + j];
#pragma unroll
        for (int u = 0; u < kLoads; ++u)
#pragma unroll
            for (int j = 0; j < NV; ++j) acc[u][j] += v[u][j];
    }
    for (; i < nparts; i += stride) {
#pragma unroll
        for (int j = 0; j < NV; ++j) acc[0][j] += partials[(size_t)i * NV + j];
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        double s = acc[0][j];
#pragma unroll
        for (int u = 1; u < kLoads; ++u) s += acc[u][j];
        out[j] = block_sum<NW>(s, s_tmp);
    }
}

// Logical block index that gives every XCD a contiguous range of the work:
// the hardware hands out consecutive workgroups round-robin over the 8 XCDs.
__device__ inline int xcd_contiguous_block(int b, int nb) {
    const int q = nb >> 3, r = nb & 7, x = b & 7, i = b >> 3;
    return x * q + (x < r ? x : r) + i;
}

__device__ inline void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Vector accesses of the CG loop. nt: streaming (non-temporal) loads and
// stores, for solves whose working set exceeds the last-level cache. There
// they keep the cache for p, which the next product gathers: every vector
// access but p's streams, and p is stored plainly. Per iteration, a 4096^2
// Q1 solve takes 582 us (597 with plain accesses, 590 with streaming stores
// only), a 100^3 27-point one 71.4 us (78.7, 77.1). A solve that fits the
// cache keeps plain accesses (streaming ones made the 128^3 Laplacian 5-6 %
// slower). One more exception: the update stores plainly the vector that the
// direction kernel reads right after it (r, or z with Jacobi), which then
// comes from the cache: 581 -> 576 us on the Q1 solve, no change on the
// 27-point and power-law ones.
typedef double f64x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ double2 load_vec(const double2* p, bool nt) {
    if (!nt) return *p;
    const f64x2 w = __builtin_nontemporal_load(reinterpret_cast<const f64x2*>(p));
    double2 v;
    v.x = w.x;
    v.y = w.y;
    return v;
}
__device__ __forceinline__ void store_vec(double2* p, double2 v, bool nt) {
    if (nt) {
        f64x2 w;
        w.x = v.x;
        w.y = v.y;
        __builtin_nontemporal_store(w, reinterpret_cast<f64x2*>(p));
    } else {
        *p = v;
    }
}
__device__ __forceinline__ void store_vec(double* p, double v, bool nt) {
    if (nt) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// ---------------------------------------------------------------------------
// Mixed-precision Tile-CSC SpMV.
//
// One wavefront owns a run of row groups; a row group is G consecutive row
// blocks (at most 256 rows; G is chosen per handle when it is created). With
// column slices the unit is a segment, the tiles of one row group within one
// slice, and each segment writes its own partial product.
// Its tiles are taken in batches of up to 64 in storage order, and the 64
// lanes sweep a batch's nonzeros 64 at a time ("windows"), several windows
// at once. Products of the widened stored value and the FP64 vector entry are
// accumulated in FP64 into the group's row accumulators in LDS; the group's
// rows are written once.
//
// Lane t of a batch stages tile t's entry in LDS: column base in x, row
// offset in the group's accumulators, and where its precision's values start
// in the batch's value segment together with their width, both taken from
// the active map when the batch is staged. A lane finds its tile from a
// record per window built with the layout (the tile of the window's first
// nonzero and a bit mask of the tiles that start inside the window, so the
// lookup is a prefix popcount). Each lane then reads its value with one
// 8-byte load, from its precision's plane under a uniform precision or from
// the map's packed segment (rebuilt by repack_kernel when the map changes):
// no branch on the precision. Lanes past a batch's end land on a sentinel
// entry whose offsets are past the end of every buffer; the hardware answers
// those loads with zero and no memory access.
//
// A wavefront loads the next batch's header, tile entries and window records
// while it sweeps the current one. A block of kSpmvWaves wavefronts handles a
// contiguous range of row groups (blocks are spread so that each XCD gets a
// contiguous part of the matrix); in CG mode each block also writes its part
// of p.q. The single-workgroup solver runs the same per-wavefront code
// (spmv_wave) on its 16 wavefronts.
// ---------------------------------------------------------------------------
// Plain: y = A x. Cg: y = A p and per-block partials of p.q. Residual:
// y = b - A x. ResNorm: no y; per-block partials of ||b - A x||^2 and ||b||^2.
enum SpmvMode { kSpmvPlain = 0, kSpmvCg = 1, kSpmvResidual = 2, kSpmvResNorm = 3 };
#ifndef MPCG_SPMV_UNROLL
#define MPCG_SPMV_UNROLL 4
#endif
#ifndef MPCG_SPMV_WAVES
#define MPCG_SPMV_WAVES 4
#endif
#ifndef MPCG_GROUP_ROWS
#define MPCG_GROUP_ROWS 0  // 0: chosen per matrix
#endif
constexpr int kUnroll = MPCG_SPMV_UNROLL;      // windows per full sweep (a power of two)
constexpr int kSpmvWaves = MPCG_SPMV_WAVES;    // wavefronts per SpMV block
constexpr int kSpmvBlock = kSpmvWaves * kWave;
constexpr int kGroupRows = MPCG_GROUP_ROWS;    // fixed rows per wavefront, or 0
constexpr uint32_t kBufferConfig = 0x00020000u;  // raw buffer, dword3 for the gfx9 family
constexpr int kDescSlots = kTileBatch + 1;      // batch tiles + the sentinel
constexpr int kSentinelPlane = 1 << 28;         // plane start: past every value segment
constexpr int kSentinelColumn = 0x7fffff00;     // x byte offset: past every x

// Window records a batch executes: whole sweeps of kUnroll windows, then one
// sweep of the smallest power of two that covers the rest.
__host__ __device__ inline int sweep_windows(int nw) {
    const int full = nw / kUnroll * kUnroll;
    int r = nw - full, t = r > 0 ? 1 : 0;
    while (t < r) t <<= 1;
    return full + t;
}
// Batches whose vector segments are staged in LDS run pipelined sweeps of
// kStagedU windows each: their records are padded to a multiple of kStagedU
// and fit one chunk of 64 records.
constexpr int kStagedU = 4;
// Largest LDS vector stage of one wavefront (bytes; 0 turns staging off), and
// the largest staged entries per nonzero of a batch, in percent.
#ifndef MPCG_STAGE_MAX_BYTES
#define MPCG_STAGE_MAX_BYTES 8192
#endif
#ifndef MPCG_STAGE_RATIO_PCT
#define MPCG_STAGE_RATIO_PCT 100
#endif
constexpr int kStageMaxBytes = MPCG_STAGE_MAX_BYTES;
// Sweeps of a staged batch in flight at once (1 or 2).
#ifndef MPCG_STAGED_PIPE
#define MPCG_STAGED_PIPE 2
#endif
constexpr int kStagedPipe = MPCG_STAGED_PIPE;
constexpr int kStageRatioPct = MPCG_STAGE_RATIO_PCT;
// Window records of a batch of len nonzeros.
__host__ __device__ inline int batch_records(int len, bool staged = false) {
    const int nw = (len + kWave - 1) / kWave;
    return staged ? (nw + kStagedU - 1) / kStagedU * kStagedU : sweep_windows(nw);
}

// Batch table entry (int32 fields, scalar loads): the wave's work is a run of
// consecutive batches covering whole row groups (segments, with column
// slices). A segment without tiles has one entry with no tiles, so its rows
// are still written. A staged batch (flag kBatchStaged) lists the distinct
// column blocks its tiles touch in xcb[kBtXList .. kBtXList + kBtXCount);
// its tiles' vector offsets then point into the LDS copy of those segments.
enum BatchField {
    kBtTile = 0, kBtTiles, kBtFirstNnz, kBtLen, kBtRecords, kBtGroup, kBtFlags, kBtSegment, kBtPacked, kBtXList,
    kBtXCount, kBtFields
};
constexpr int kBatchFirstOfGroup = 1, kBatchLastOfGroup = 2, kBatchStaged = 4;
// Bits from kBatchSliceShift up: the column slice of the batch's segment,
// whose rows go to partial product number slice (stride SpmvArgs.ystride).
constexpr int kBatchSliceShift = 8;

// Value planes, stored per batch: one 16-byte aligned segment holds the
// batch's FP64 values (8*len bytes), then its FP32 values (4*len), then its
// BF16 values (2*len), all in storage order, and 16 spare bytes. Plane code p
// starts at byte p*(10-2p)*len of the segment.
__host__ __device__ inline int64_t segment_bytes(int64_t len) { return (14 * len + 16 + 15) / 16 * 16; }
// The active map's values of a batch (see repack_kernel) take at most 8 bytes
// per value: each tile starts on 8 bytes and its values are 8, 4 or 2 bytes
// wide. They sit in a buffer of their own, batch after batch (kBtPacked, in
// 16-byte units), with 16 spare bytes each for the 8-byte loads of the last
// values.
__host__ __device__ inline int64_t packed_bytes(int64_t len) { return (8 * len + 16 + 15) / 16 * 16; }

// Builds every batch's segment from the FP64 values, rounding to nearest even
// (one wavefront per batch). The FP32 and BF16 planes are rounded from vlow:
// the FP64 values themselves, or the per-column scaled values a / s_j.
__global__ __launch_bounds__(kBlock) void build_segments_kernel(const int32_t* __restrict__ btab, int64_t nbatch,
                                                               const double* __restrict__ v64,
                                                               const double* __restrict__ vlow,
                                                               char* __restrict__ planes) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x / kWave);
    for (int64_t b = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave; b < nbatch; b += waves) {
        const int32_t* e = btab + b * kBtFields;
        const int first = e[kBtFirstNnz], len = e[kBtLen];
        char* seg = planes + (int64_t)e[kBtSegment] * 16;
        double* s64 = reinterpret_cast<double*>(seg);
        uint32_t* s32 = reinterpret_cast<uint32_t*>(seg + 8 * (int64_t)len);
        uint16_t* s16 = reinterpret_cast<uint16_t*>(seg + 12 * (int64_t)len);
        for (int i = lane; i < len; i += kWave) {
            const uint64_t u = (uint64_t)__double_as_longlong(vlow[first + i]);
            s64[i] = v64[first + i];
            s32[i] = round_f64_to_e8<23>(u);
            s16[i] = (uint16_t)round_f64_to_e8<7>(u);
        }
    }
}

// Packed values of a per-tile map: inside every batch's packed part (its own
// buffer, packed_bytes apart), tile after tile in storage order, each tile's values at its precision, every
// tile starting on an 8-byte boundary; toff[t] = start of tile t's values
// minus (its position in the batch << log2 of its value width). One
// wavefront per batch: lane l sizes tile l and a wave prefix sum places it,
// then the lanes copy the batch's values 64 at a time, each finding its tile
// from the window records. Rerun at every map change: repack_kernel rebuilds
// every batch; in a solve the tile-rule kernel rebuilds, at the start of each
// window, only the batches in which a tile changed precision (each batch's part
// is self-contained).
struct RepackArgs {
    const int32_t* btab;
    const int32_t* tptr;
    const uint8_t* map;
    const char* planes;
    char* packed;
    int32_t* toff;
    const uint64_t* win_mask;
    const int32_t* win_tile;
    int64_t nbatch;
};

// One batch by one wavefront: lane l holds p, the precision code of the
// batch's tile l (lanes past the batch's nt tiles hold nothing). s_toff and
// s_prec are the wavefront's LDS slots (kTileBatch each).
__device__ inline void repack_batch(const RepackArgs& a, const int32_t* e, int lane, int p, int* s_toff,
                                    int* s_prec) {
    const int tb = e[kBtTile], nt = e[kBtTiles], first = e[kBtFirstNnz], len = e[kBtLen];
    const bool valid = lane < nt;
    const int sh = 3 - p;
    const int start = valid ? a.tptr[tb + lane] - first : 0;
    const int bytes = valid ? ((a.tptr[tb + lane + 1] - a.tptr[tb + lane]) << sh) : 0;
    int incl = (bytes + 7) & ~7;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int t = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += t;
    }
    const int base = incl - ((bytes + 7) & ~7);
    if (valid) {
        const int to = base - (start << sh);
        a.toff[tb + lane] = to;
        s_toff[lane] = to;
        s_prec[lane] = p;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const char* src = a.planes + (int64_t)e[kBtSegment] * 16;
    char* dst = a.packed + (int64_t)e[kBtPacked] * 16;
    for (int o = 0, v = e[kBtRecords]; o < len; o += kWave, ++v) {
        const uint64_t m = a.win_mask[v];
        const int j = a.win_tile[v] + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        const int i = o + lane;
        if (i < len) {
            const int pj = s_prec[j];
            const int shj = 3 - pj;
            const int64_t from = (int64_t)pj * (10 - 2 * pj) * len + ((int64_t)i << shj);
            const int64_t to = (int64_t)s_toff[j] + ((int64_t)i << shj);
            if (pj == 0)
                *reinterpret_cast<uint64_t*>(dst + to) = *reinterpret_cast<const uint64_t*>(src + from);
            else if (pj == 1)
                *reinterpret_cast<uint32_t*>(dst + to) = *reinterpret_cast<const uint32_t*>(src + from);
            else
                *reinterpret_cast<uint16_t*>(dst + to) = *reinterpret_cast<const uint16_t*>(src + from);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(kBlock) void repack_kernel(RepackArgs a) {
    __shared__ int s_toff[kWavesPerBlock][kTileBatch];
    __shared__ int s_prec[kWavesPerBlock][kTileBatch];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int64_t waves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t b = (int64_t)blockIdx.x * kWavesPerBlock + w; b < a.nbatch; b += waves) {
        const int32_t* e = a.btab + b * kBtFields;
        const int tb = e[kBtTile], nt = e[kBtTiles];
        if (nt == 0) continue;
        const int p = lane < nt ? min((int)a.map[tb + lane], 2) : 0;
        repack_batch(a, e, lane, p, s_toff[w], s_prec[w]);
    }
}

struct SpmvArgs {
    const int32_t* btab;    // [nbatch][8] batch table
    const int32_t* gbatch;  // [ngroups+1] first batch of every segment (a row group, per column slice)
    const int2* tent;       // [T] per tile: x byte offset of its column block, accumulator byte offset of its rows
    const uint8_t* map;     // [T] active precision map
    const int32_t* toff;    // [T] per tile: its values' start in the packed segment minus position << width shift
    const int32_t* tcol;    // [T] column block of every tile
    const uint8_t* cbcode;  // per column block precision (max|p| rule kernels only)
    const void* meta;       // per nonzero (row, col) packed: u8 (R, C <= 16) or u16
    const char* planes;     // value segments, one per batch
    const char* packed;     // packed value segments of the active map, same offsets
    const uint64_t* win_mask;  // per window: bit q = nonzero q+1 of the window starts a tile
    const int32_t* win_tile;   // per window: batch tile of the window's first nonzero
    const double* x;
    double* y;
    const double* b;       // residual mode: y = b - A x
    const int32_t* uprec;  // -1 per-tile map, else uniform code
    const State* st;
    double* partials;      // CG mode: one p.q partial per block
    const int16_t* colexp;  // P1 kernels: per column e_j of the scale 2^e_j (NULL: no scale)
    const int32_t* xcb;     // staged batches: their distinct column blocks (see kBtXList)
    int32_t n, rows_per_group, ngroups, nwin;
    int32_t ystride;       // column slices: distance between two slices' partial products
    int32_t p1_round;      // P1 kernels: round the vector entry to the tile's precision
    int32_t sentinel_row;  // P1 kernels: row offset of padding entries (R), or -1
    int32_t C;             // tile width
    int32_t stage_shift;   // staged batches: log2 of the 16-byte chunks per column block (C / 2)
    int32_t stage_doubles; // LDS doubles of one wavefront's vector stage (0: no staged batch)
    int32_t nt;            // CG mode: streaming stores of q (see store_vec)
    int32_t planes_map;    // per-tile map: values from the precision planes, not the packed segments
};

template <typename MetaT>
__device__ inline void decode_meta(uint32_t m, int& r, int& c);
template <>
__device__ inline void decode_meta<uint8_t>(uint32_t m, int& r, int& c) {
    r = (int)(m >> 4);
    c = (int)(m & 15u);
}
template <>
__device__ inline void decode_meta<uint16_t>(uint32_t m, int& r, int& c) {
    r = (int)(m >> 8);
    c = (int)(m & 255u);
}

// A buffer resource over a batch's part of a stream. Its fields come from
// wave-uniform values; reading them through readfirstlane says so, so that
// the loads through it stay single instructions (a resource the compiler
// cannot prove uniform is used in a loop over its distinct values).
__device__ inline __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    char* q = reinterpret_cast<char*>((uintptr_t)(((uint64_t)hi << 32) | lo));
    return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, __builtin_amdgcn_readfirstlane(bytes), (int)kBufferConfig);
}

__device__ inline __amdgpu_buffer_rsrc_t batch_rsrc(const void* base, int64_t first, int width, int count) {
    return uniform_rsrc(static_cast<const char*>(base) + first * width, count * width);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Cache policy of the streamed value and index loads. The non-temporal hint
// (2) suits bytes read once per product, but it measured slower on every
// workload on MI355X, so the default policy (0) is used.
#ifndef MPCG_SPMV_NT
#define MPCG_SPMV_NT 0
#endif
constexpr int kStreamAux = MPCG_SPMV_NT ? 2 : 0;

// Packed (row, column) of the nonzero at batch position q (buffer loads: past
// the batch they return zero).
template <typename MetaT>
__device__ __forceinline__ uint32_t load_meta(__amdgpu_buffer_rsrc_t r, int q) {
    return sizeof(MetaT) == 1 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, q, 0, kStreamAux)
                              : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, 2 * q, 0, kStreamAux);
}

// Wave-uniform reads of data no kernel here writes while the SpMV runs: read
// through the constant address space so they become scalar loads.
template <typename T>
__device__ inline T uniform_load(const T* p, int i) {
    return ((const __attribute__((address_space(4))) T*)(uintptr_t)p)[i];
}

// One batch's header in scalar registers.
struct BatchHdr {
    int tile, tiles, first, len, records, group, flags, segment, packed, xlist, xcount;
};
__device__ __forceinline__ BatchHdr load_hdr(const int32_t* btab, int b) {
    const int32_t* e = btab + (size_t)b * kBtFields;
    BatchHdr h;
    h.tile = uniform_load(e, kBtTile);
    h.tiles = uniform_load(e, kBtTiles);
    h.first = uniform_load(e, kBtFirstNnz);
    h.len = uniform_load(e, kBtLen);
    h.records = uniform_load(e, kBtRecords);
    h.group = uniform_load(e, kBtGroup);
    h.flags = uniform_load(e, kBtFlags);
    h.segment = uniform_load(e, kBtSegment);
    h.packed = uniform_load(e, kBtPacked);
    h.xlist = uniform_load(e, kBtXList);
    h.xcount = uniform_load(e, kBtXCount);
    return h;
}

// A batch's per-lane data: tile `lane`'s entry and precision code (lane <
// tiles) and window record `lane` of a chunk of 64 windows.
struct BatchRegs {
    int2 entry;
    int prec, toff;
    uint32_t mlo, mhi;
    int rec;
    int xcb;  // staged batch: column block of stage slot `lane` (lane < kBtXCount)
};

struct SweepCtx {
    __amdgpu_buffer_rsrc_t rv, rmt, rx, rmask, rrec;  // rv: this batch's value segment
    __amdgpu_buffer_rsrc_t rexp;                       // P1: per-column scale exponents
    const int4* desc;  // this wave's plan entries in LDS
    char* acc;         // this wave's row accumulators in LDS
    const int2* tent;
    const uint8_t* map;
    const int32_t* toff;
    const int32_t* tcol;
    const uint8_t* cbcode;
    const int32_t* xcb;
    const double* xs;  // XL sweeps: the vector in LDS (entries 0 .. xmax); staged batches: the stage
    int xmax;
    int len, lane;
    int spare;  // byte offset of this lane's spare accumulator
    int round_p, scale, sentinel_row;  // P1 options (wave-uniform)
};

// A vector entry rounded to FP32 and, in one step from FP64, to BF16 (both
// round-to-nearest-even, returned widened). FP32: the conversion instruction.
// BF16: x is first rounded to FP32 by round-to-odd (truncation toward zero,
// last bit set when inexact), then to BF16 to nearest even; FP32 keeps 16 more
// bits than BF16 over the whole shared exponent range, so the odd bit only
// breaks false ties and the result equals the direct rounding of x.
__device__ __forceinline__ void round_vector_entry(double x, double& x32, double& x16) {
    const float f = (float)x;
    const double fd = (double)f;
    x32 = fd;
    uint32_t u = __float_as_uint(f);
    u -= (fabs(fd) > fabs(x)) ? 1u : 0u;  // rounded away from zero: step back to the truncation
    u |= (fd != x) ? 1u : 0u;             // inexact (NaN stays NaN)
    const uint32_t b = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    x16 = (double)__uint_as_float(b);
}

// Issues the loads of a batch's tile entries and of its window records
// [chunk, chunk+64) (out-of-range record reads return zero). CB: the tile's
// precision is its column block's code (max|p| rule), else the map's.
template <bool CB>
__device__ __forceinline__ void load_batch_regs(const SweepCtx& c, const BatchHdr& h, int chunk, bool with_entry,
                                                BatchRegs& r) {
    if (with_entry) {
        const int t = h.tile + min(c.lane, max(h.tiles - 1, 0));
        r.entry = c.tent[t];
        if (CB) {
            r.prec = c.cbcode[c.tcol[t]];
            r.toff = 0;
        } else {
            r.prec = c.map[t];
            r.toff = c.toff[t];
        }
        r.xcb = 0;
        if (h.flags & kBatchStaged) r.xcb = c.xcb[h.xlist + min(c.lane, h.xcount - 1)];
    }
    const int wi = h.records + chunk + c.lane;
    const u32x2 m = __builtin_amdgcn_raw_buffer_load_b64(c.rmask, 8 * wi, 0, 0);
    r.mlo = m.x;
    r.mhi = m.y;
    r.rec = (int)__builtin_amdgcn_raw_buffer_load_b32(c.rrec, 4 * wi, 0, 0);
}

// U consecutive windows of one batch, starting at batch window wi (records in
// lanes of R) and batch position o0. Loads are issued for all U windows
// before any is consumed. With next = true the next batch's tile entries and
// first records (header Hn) are loaded into Rn once the value loads are issued.
//
// A lane's value is one 8-byte load at its tile's entry shift plus its
// position times the value width, rounded down to 4 bytes (a BF16 lane then
// takes the half its byte offset selects); the widening is a bitwise blend.
// Lanes past the batch add their zero product to a private spare accumulator.
//
// XL: the vector entries come from the LDS copy c.xs (lanes on a sentinel
// entry read its last entry, and add their zero product to the spare).
template <typename MetaT, int U, bool CB, bool P1, bool XL = false>
__device__ __forceinline__ void spmv_sweep(const SweepCtx& c, const BatchRegs& R, int wi, int o0, bool next,
                                           const BatchHdr& Hn, BatchRegs& Rn) {
    int q[U];
    int4 d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int l = (wi + u) & (kWave - 1);
        const uint32_t mlo = __builtin_amdgcn_readlane(R.mlo, l);
        const uint32_t mhi = __builtin_amdgcn_readlane(R.mhi, l);
        const int j = __builtin_amdgcn_readlane(R.rec, l) +
                      (int)__builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, 0u));
        d[u] = c.desc[j];
        q[u] = o0 + u * kWave + c.lane;  // position in the batch
    }
    uint32_t mt[U];
#pragma unroll
    for (int u = 0; u < U; ++u) mt[u] = load_meta<MetaT>(c.rmt, q[u]);
    // Stored values, issued before the vector gathers (which wait for the
    // packed indices).
    u32x2 raw[U];
    int hs[U];  // BF16: 16 when the value is the high half of its 4-byte word
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int off = d[u].z + (q[u] << d[u].w);
        hs[u] = (off & 2) << 3;
        raw[u] = __builtin_amdgcn_raw_buffer_load_b64(c.rv, off & ~3, 0, kStreamAux);
    }
    if (next) load_batch_regs<CB>(c, Hn, 0, true, Rn);
    double xv[U];
    int racc[U];
    int ex[U];  // P1: scale exponent of the lane's column (sentinel lanes read past the end: 0)
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int r, col;
        decode_meta<MetaT>(mt[u], r, col);
        const bool real = q[u] < c.len && (!P1 || r != c.sentinel_row);
        racc[u] = real ? d[u].y + 8 * r : c.spare;
        if (XL) {
            xv[u] = c.xs[min((d[u].x >> 3) + col, c.xmax)];
        } else {
            const u32x2 xb = __builtin_amdgcn_raw_buffer_load_b64(c.rx, d[u].x + 8 * col, 0, 0);
            xv[u] = __longlong_as_double(((long long)xb.y << 32) | xb.x);
        }
        ex[u] = 0;
        if (P1 && c.scale)
            ex[u] = (int)(int16_t)__builtin_amdgcn_raw_buffer_load_b16(c.rexp, 2 * ((d[u].x >> 3) + col), 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        // FP32: the low word. BF16 (width shift 1): the half holding the value
        // (little endian), moved to the high half of an FP32 word. FP64: width
        // shift 3.
        const uint32_t h = (raw[u].x >> hs[u]) << 16;
        const uint32_t f = d[u].w == 1 ? h : raw[u].x;
        double v32 = (double)__uint_as_float(f);
        // Materialise the widened value in every lane (an empty statement that
        // emits nothing), so that the choice below stays two selects: left to
        // itself the compiler branches around the conversion, which costs five
        // scalar and control instructions per window in an issue-bound loop.
        asm volatile("" : "+v"(v32));
        double v = d[u].w == 3 ? __longlong_as_double(((long long)raw[u].y << 32) | raw[u].x) : v32;
        double xu = xv[u];
        if (P1) {
            // Reduced-precision values carry their column's scale 2^e (exact).
            if (c.scale) v = d[u].w == 3 ? v : ldexp(v, ex[u]);
            if (c.round_p) {
                double x32, x16;
                round_vector_entry(xu, x32, x16);
                xu = d[u].w == 3 ? xu : d[u].w == 2 ? x32 : x16;
            }
        }
        atomicAdd(reinterpret_cast<double*>(c.acc + racc[u]), v * xu);
    }
    // Every load of the sweep has been consumed; saying so keeps the compiler
    // from guarding the next sweep's loads against this one's.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

// All window records of one batch on the gather path (vector entries loaded
// from x, or from the LDS copy with XL): whole sweeps of U windows, leftover
// whole kUnroll sweeps, then one sweep of the power of two that covers the
// rest. The first sweep also starts the loads of the next batch (header Hn)
// into Rn when `more`.
template <typename MetaT, bool CB, bool P1, int U, bool XL>
__device__ __forceinline__ void sweep_batch_gather(const SweepCtx& c, const BatchHdr& H, BatchRegs& R, bool more,
                                                   const BatchHdr& Hn, BatchRegs& Rn) {
    const int E = batch_records(H.len);
    int left = E, wi = 0, o0 = 0;
    for (; left >= U; left -= U, wi += U, o0 += U * kWave) {
        if (wi > 0 && (wi & (kWave - 1)) == 0) load_batch_regs<CB>(c, H, wi, false, R);  // next 64 records
        spmv_sweep<MetaT, U, CB, P1, XL>(c, R, wi, o0, more && wi == 0, Hn, Rn);
    }
    if (U > kUnroll) {
        for (; left >= kUnroll; left -= kUnroll, wi += kUnroll, o0 += kUnroll * kWave) {
            if (wi > 0 && (wi & (kWave - 1)) == 0) load_batch_regs<CB>(c, H, wi, false, R);
            spmv_sweep<MetaT, kUnroll, CB, P1, XL>(c, R, wi, o0, more && wi == 0, Hn, Rn);
        }
    }
    // The rest is 0 or one power of two below kUnroll (never crossing a record chunk).
    if (wi > 0 && (wi & (kWave - 1)) == 0 && left > 0) load_batch_regs<CB>(c, H, wi, false, R);
    const bool first = more && wi == 0;
    if (kUnroll > 8 && left == 8)
        spmv_sweep<MetaT, (kUnroll > 8 ? 8 : 1), CB, P1, XL>(c, R, wi, o0, first, Hn, Rn);
    if (kUnroll > 4 && left == 4)
        spmv_sweep<MetaT, (kUnroll > 4 ? 4 : 1), CB, P1, XL>(c, R, wi, o0, first, Hn, Rn);
    if (kUnroll > 2 && left == 2)
        spmv_sweep<MetaT, (kUnroll > 2 ? 2 : 1), CB, P1, XL>(c, R, wi, o0, first, Hn, Rn);
    if (kUnroll > 1 && left == 1) spmv_sweep<MetaT, 1, CB, P1, XL>(c, R, wi, o0, first, Hn, Rn);
    if (more && E == 0) load_batch_regs<CB>(c, Hn, 0, true, Rn);  // a batch without windows
}

// Staged batches. At the batch start the x segments of the batch's distinct
// column blocks (C entries each, listed in xcb) are copied into the wave's
// LDS stage by LDS-direct buffer loads (16 bytes per lane, no registers), in
// slot order: the tile entries of such a batch hold their block's slot
// offset in the stage instead of an offset in x. The sweeps then read every
// vector entry from LDS, so a sweep waits on one round trip to memory (the
// packed indices and the values, issued together) instead of two.
//
// The sweeps are pipelined: the loads of sweep s + 1 are issued before sweep
// s is accumulated, so every wave keeps two sweeps of stream loads in flight.
struct StagedSweep {
    uint32_t mt[kStagedU];
    u32x2 raw[kStagedU];
    uint32_t cw[kStagedU];  // stage offset | accumulator offset << 16 | width shift << 28 | BF16 high half << 30
};

template <typename MetaT>
__device__ __forceinline__ void staged_issue(const SweepCtx& c, const BatchRegs& R, int s, StagedSweep& S) {
#pragma unroll
    for (int u = 0; u < kStagedU; ++u) {
        const int wi = s * kStagedU + u;  // < 64: a staged batch's records fit one chunk
        const uint32_t mlo = __builtin_amdgcn_readlane(R.mlo, wi);
        const uint32_t mhi = __builtin_amdgcn_readlane(R.mhi, wi);
        const int j = __builtin_amdgcn_readlane(R.rec, wi) +
                      (int)__builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, 0u));
        const int4 d = c.desc[j];
        const int q = wi * kWave + c.lane;
        S.mt[u] = load_meta<MetaT>(c.rmt, q);
        const int off = d.z + (q << d.w);
        S.raw[u] = __builtin_amdgcn_raw_buffer_load_b64(c.rv, off & ~3, 0, kStreamAux);
        S.cw[u] = (uint32_t)d.x | ((uint32_t)d.y << 16) | ((uint32_t)d.w << 28) | ((uint32_t)(off & 2) << 29);
    }
}

template <typename MetaT>
__device__ __forceinline__ void staged_consume(const SweepCtx& c, const StagedSweep& S, int s) {
    double xv[kStagedU];
    int racc[kStagedU];
#pragma unroll
    for (int u = 0; u < kStagedU; ++u) {
        int r, col;
        decode_meta<MetaT>(S.mt[u], r, col);
        const int q = (s * kStagedU + u) * kWave + c.lane;
        racc[u] = q < c.len ? (int)((S.cw[u] >> 16) & 0xFFFu) + 8 * r : c.spare;
        xv[u] = c.xs[(int)((S.cw[u] & 0xFFFFu) >> 3) + col];
    }
#pragma unroll
    for (int u = 0; u < kStagedU; ++u) {
        const int w = (int)((S.cw[u] >> 28) & 3u);
        const uint32_t h = (S.raw[u].x >> ((S.cw[u] >> 26) & 16u)) << 16;
        const uint32_t f = w == 1 ? h : S.raw[u].x;
        double v32 = (double)__uint_as_float(f);
        asm volatile("" : "+v"(v32));  // keep the choice below two selects (see spmv_sweep)
        const double v = w == 3 ? __longlong_as_double(((long long)S.raw[u].y << 32) | S.raw[u].x) : v32;
        atomicAdd(reinterpret_cast<double*>(c.acc + racc[u]), v * xv[u]);
    }
}

// The x segments of a staged batch into the stage: chunk i (16 bytes) of the
// stage is chunk i & (C/2 - 1) of column block xcb[i >> stage_shift]; lanes
// past the batch's chunks are masked off.
__device__ __forceinline__ void stage_x(const SweepCtx& c, const BatchRegs& R, int xcount, int shift, int C8,
                                        double* stage) {
    const int chunks = xcount << shift;
    const int mask = (1 << shift) - 1;
    for (int j = 0; j < chunks; j += kWave) {
        const int i = j + c.lane;
        const int blk = __builtin_amdgcn_ds_bpermute(4 * min(i >> shift, kWave - 1), R.xcb);
        if (i < chunks)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rx, (__attribute__((address_space(3))) void*)(stage + 2 * j),
                                                     16, blk * C8 + ((i & mask) << 4), 0, 0, 0);
    }
}

// A staged batch: stage the vector segments, then the pipelined sweeps. The
// first sweep's loads are issued together with the staging; the next batch's
// loads (header Hn) go out after the second sweep's.
template <typename MetaT, bool CB>
__device__ __forceinline__ void sweep_batch_staged(const SweepCtx& c, const SpmvArgs& a, const BatchHdr& H,
                                                   const BatchRegs& R, bool more, const BatchHdr& Hn, BatchRegs& Rn) {
    stage_x(c, R, H.xcount, a.stage_shift, a.C * 8, const_cast<double*>(c.xs));
    const int nsw = batch_records(H.len, true) / kStagedU;
    if (nsw == 0) {
        if (more) load_batch_regs<CB>(c, Hn, 0, true, Rn);
        return;
    }
    StagedSweep A, B;
    staged_issue<MetaT>(c, R, 0, A);
    if (kStagedPipe == 1) {  // one sweep in flight at a time
        if (more) load_batch_regs<CB>(c, Hn, 0, true, Rn);
        for (int s = 0;;) {
            staged_consume<MetaT>(c, A, s);
            if (++s >= nsw) break;
            staged_issue<MetaT>(c, R, s, A);
        }
        return;
    }
    if (nsw > 1) staged_issue<MetaT>(c, R, 1, B);
    if (more) load_batch_regs<CB>(c, Hn, 0, true, Rn);
    for (int s = 0;;) {
        staged_consume<MetaT>(c, A, s);
        if (++s >= nsw) break;
        if (s + 1 < nsw) staged_issue<MetaT>(c, R, s + 1, A);
        staged_consume<MetaT>(c, B, s);
        if (++s >= nsw) break;
        if (s + 1 < nsw) staged_issue<MetaT>(c, R, s + 1, B);
    }
}

// The outputs are separate restrict arguments: the compiler may then treat
// every other array as read-only for the whole launch.
//
// CB = true: the max|p| rule's kernels, where a tile's precision is its column
// block's code for this product (values from the precision planes).
//
// P1 = true: the paper's own numerics as options (vector entry rounded to the
// tile's precision, per-column scale of the reduced values, padding entries
// at row offset R skipped).
//
// spmv_wave is one wavefront's share: the batches of row groups (segments)
// [g0, g1), with the wave's LDS row accumulators `acc` (MAXROWS + kWave
// doubles: the rows, then one spare per lane for lanes on a sentinel entry)
// and tile descriptors `desc` (kDescSlots). uprec is the uniform precision, or
// -1 for the per-tile map. Returns the lane's part of p.q in CG mode, else 0.
// U: windows per full sweep (kUnroll, or a larger power of two for latency-
// bound callers; a batch's leftover whole kUnroll sweeps then run one by one).
// XL: vector entries from the LDS copy xs[0 .. n-1] instead of a.x.
template <typename MetaT, int MODE, int MAXROWS, bool CB, bool P1, int U = kUnroll, bool XL = false>
__device__ __forceinline__ double spmv_wave(const SpmvArgs& a, double* __restrict__ y, int g0, int g1, int uprec,
                                            double* acc, int4* desc, int lane, const double* xs = nullptr) {
    // The sweep-ordered indices are laid out for sweeps of kUnroll windows.
    static_assert(U == kUnroll, "sweep size");
    SweepCtx c;
    c.lane = lane;
    c.xs = xs;
    c.xmax = a.n - 1;
    c.tent = a.tent;
    c.map = a.map;
    c.toff = a.toff;
    c.tcol = a.tcol;
    c.cbcode = a.cbcode;
    c.xcb = a.xcb;
    // Values come from the precision planes under a uniform precision or the
    // max|p| rule (which changes the map every iteration), else from the map's
    // packed segment.
    const bool from_planes = CB || uprec >= 0 || a.planes_map != 0;
    c.desc = desc;
    c.acc = reinterpret_cast<char*>(acc);
    c.spare = (MAXROWS + lane) * 8;
    // Byte offsets are 32-bit: n < 2^28 and the record count < 2^28 are
    // checked when the handle is created.
    c.rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<double*>(a.x), (short)0, a.n * 8, (int)kBufferConfig);
    c.rmask = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint64_t*>(a.win_mask), (short)0, a.nwin * 8,
                                                (int)kBufferConfig);
    c.rrec = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(a.win_tile), (short)0, a.nwin * 4,
                                               (int)kBufferConfig);
    c.round_p = P1 ? a.p1_round : 0;
    c.scale = P1 && a.colexp != nullptr;
    c.sentinel_row = P1 ? a.sentinel_row : -1;
    if (P1)
        c.rexp = __builtin_amdgcn_make_buffer_rsrc(const_cast<int16_t*>(a.colexp), (short)0,
                                                   a.colexp ? a.n * 2 : 0, (int)kBufferConfig);
    // CG mode, groups of at most 64 rows: the lane's own p entry, loaded when
    // the group starts (larger groups reload p at the group's end: holding
    // four entries per lane costs more occupancy than the reload).
    double dot = 0.0, p_own = 0.0;

    int b = uniform_load(a.gbatch, g0);
    const int b_end = uniform_load(a.gbatch, g1);
    BatchHdr H{};
    BatchRegs R{};
    if (b < b_end) {
        H = load_hdr(a.btab, b);
        load_batch_regs<CB>(c, H, 0, true, R);
    }
    for (; b < b_end; ++b) {
        const bool more = b + 1 < b_end;
        BatchHdr Hn{};
        if (more) Hn = load_hdr(a.btab, b + 1);
        const int row0 = H.group * a.rows_per_group;
        const int nrows = min(a.rows_per_group, a.n - row0);
        if (H.flags & kBatchFirstOfGroup) {
            for (int i = lane; i < a.rows_per_group; i += kWave) acc[i] = 0.0;
            if (MODE == kSpmvCg && MAXROWS <= kWave && lane < nrows) p_own = a.x[row0 + lane];
        }
        // Tile entries, the sentinel past the batch's tiles.
        {
            const int p = uprec >= 0 ? uprec : R.prec;
            const bool tile = lane < H.tiles;
            int4 e;
            e.x = tile ? R.entry.x : kSentinelColumn;
            e.y = R.entry.y;
            e.z = !tile ? kSentinelPlane : from_planes ? p * (10 - 2 * p) * H.len : R.toff;
            e.w = tile ? 3 - p : 3;
            desc[lane] = e;
            if (lane == 0) desc[kTileBatch] = make_int4(kSentinelColumn, 0, kSentinelPlane, 3);
        }
        c.rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(from_planes ? a.planes + (int64_t)H.segment * 16 : a.packed + (int64_t)H.packed * 16),
            (short)0, (int)(from_planes ? segment_bytes(H.len) : packed_bytes(H.len)), (int)kBufferConfig);
        c.rmt = batch_rsrc(a.meta, H.first, (int)sizeof(MetaT), H.len);
        c.len = H.len;
        wave_lds_sync();
        BatchRegs Rn{};
        sweep_batch_gather<MetaT, CB, P1, U, XL>(c, H, R, more, Hn, Rn);
        wave_lds_sync();
        if (H.flags & kBatchLastOfGroup) {
            // This segment's partial product (the product itself without column slices).
            double* __restrict__ yo = y + (size_t)(H.flags >> kBatchSliceShift) * a.ystride;
            for (int i = lane; i < nrows; i += kWave) {
                const double v = acc[i];
                if (MODE == kSpmvPlain) {
                    yo[row0 + i] = v;
                } else if (MODE == kSpmvCg) {
                    yo[row0 + i] = v;
                    dot += (MAXROWS <= kWave ? p_own : a.x[row0 + i]) * v;
                } else {
                    yo[row0 + i] = a.b[row0 + i] - v;
                }
            }
            wave_lds_sync();
        }
        H = Hn;
        R = Rn;
    }
    return dot;
}

// One wavefront's share in the multi-launch product: the segments g, g +
// gstride, ... below gend (the kernel interleaves an XCD's segments over its
// wavefronts), each a run of batches. The next batch's header, tile entries,
// window records and stage list are loaded while the current batch is swept,
// also across segments. Batches flagged kBatchStaged run the staged,
// pipelined sweeps with the vector segments in LDS (`stage`); the others
// gather the vector from memory. Returns the lane's part of p.q in CG mode.
template <typename MetaT, int MODE, int MAXROWS, bool CB, bool P1, bool STAGE>
__device__ __forceinline__ double spmv_wave_multi(const SpmvArgs& a, double* __restrict__ y, int g, int gstride,
                                                  int gend, int uprec, double* acc, int4* desc, double* stage,
                                                  double* pown, int lane, double& dot2) {
    SweepCtx c;
    c.lane = lane;
    c.xs = stage;
    c.xmax = a.n - 1;
    c.tent = a.tent;
    c.map = a.map;
    c.toff = a.toff;
    c.tcol = a.tcol;
    c.cbcode = a.cbcode;
    c.xcb = a.xcb;
    const bool from_planes = CB || uprec >= 0 || a.planes_map != 0;
    c.desc = desc;
    c.acc = reinterpret_cast<char*>(acc);
    c.spare = (MAXROWS + lane) * 8;
    c.rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<double*>(a.x), (short)0, a.n * 8, (int)kBufferConfig);
    c.rmask = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint64_t*>(a.win_mask), (short)0, a.nwin * 8,
                                                (int)kBufferConfig);
    c.rrec = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(a.win_tile), (short)0, a.nwin * 4,
                                               (int)kBufferConfig);
    c.round_p = P1 ? a.p1_round : 0;
    c.scale = P1 && a.colexp != nullptr;
    c.sentinel_row = P1 ? a.sentinel_row : -1;
    if (P1)
        c.rexp = __builtin_amdgcn_make_buffer_rsrc(const_cast<int16_t*>(a.colexp), (short)0,
                                                   a.colexp ? a.n * 2 : 0, (int)kBufferConfig);
    double dot = 0.0, p_own = 0.0;
    dot2 = 0.0;
    if (g >= gend) return 0.0;
    int b = uniform_load(a.gbatch, g);
    int bend = uniform_load(a.gbatch, g + 1);
    BatchHdr H = load_hdr(a.btab, b);
    BatchRegs R{};
    load_batch_regs<CB>(c, H, 0, true, R);
    for (;;) {
        // The successor: the next batch of this segment, else the first batch
        // of this wave's next segment.
        int bn = b + 1, bendn = bend, gn = g;
        bool more = true;
        if (bn >= bend) {
            gn = g + gstride;
            more = gn < gend;
            if (more) {
                bn = uniform_load(a.gbatch, gn);
                bendn = uniform_load(a.gbatch, gn + 1);
            }
        }
        BatchHdr Hn{};
        if (more) Hn = load_hdr(a.btab, bn);
        const int row0 = H.group * a.rows_per_group;
        const int nrows = min(a.rows_per_group, a.n - row0);
        if (H.flags & kBatchFirstOfGroup) {
            for (int i = lane; i < a.rows_per_group; i += kWave) acc[i] = 0.0;
            if (MODE == kSpmvCg && MAXROWS <= kWave && lane < nrows) p_own = a.x[row0 + lane];
            if (MODE == kSpmvCg && MAXROWS > kWave) {
                // The group's own p entries (for p.q at the group's end) go to LDS
                // now, 16 bytes per lane by LDS-direct loads; the sweeps' waits
                // cover them. An odd group (R odd) takes one pair more, whose
                // second entry is the next group's and is not used; entries past
                // n read as zero.
                const int npairs = (a.rows_per_group + 1) / 2;
                for (int j = 0; j < npairs; j += kWave)
                    if (j + lane < npairs)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rx, (__attribute__((address_space(3))) void*)(pown + 2 * j),
                                                                 16, row0 * 8 + (j + lane) * 16, 0, 0, 0);
            }
        }
        const bool staged = STAGE && (H.flags & kBatchStaged) != 0;
        {
            const int p = uprec >= 0 ? uprec : R.prec;
            const bool tile = lane < H.tiles;
            const int none = staged ? 0 : kSentinelColumn;  // a staged sentinel reads stage entry 0
            int4 e;
            e.x = tile ? R.entry.x : none;
            e.y = R.entry.y;
            e.z = !tile ? kSentinelPlane : from_planes ? p * (10 - 2 * p) * H.len : R.toff;
            e.w = tile ? 3 - p : 3;
            desc[lane] = e;
            if (lane == 0) desc[kTileBatch] = make_int4(none, 0, kSentinelPlane, 3);
        }
        c.rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(from_planes ? a.planes + (int64_t)H.segment * 16 : a.packed + (int64_t)H.packed * 16),
            (short)0, (int)(from_planes ? segment_bytes(H.len) : packed_bytes(H.len)), (int)kBufferConfig);
        c.rmt = batch_rsrc(a.meta, H.first, (int)sizeof(MetaT), H.len);
        c.len = H.len;
        wave_lds_sync();
        BatchRegs Rn{};
        if (STAGE && staged)
            sweep_batch_staged<MetaT, CB>(c, a, H, R, more, Hn, Rn);
        else
            sweep_batch_gather<MetaT, CB, P1, kUnroll, false>(c, H, R, more, Hn, Rn);
        wave_lds_sync();
        if (H.flags & kBatchLastOfGroup) {
            // This segment's partial product (the product itself without column slices).
            double* __restrict__ yo = y + (size_t)(H.flags >> kBatchSliceShift) * a.ystride;
            for (int i = lane; i < nrows; i += kWave) {
                const double v = acc[i];
                if (MODE == kSpmvPlain) {
                    yo[row0 + i] = v;
                } else if (MODE == kSpmvCg) {
                    store_vec(&yo[row0 + i], v, a.nt != 0);
                    dot += (MAXROWS <= kWave ? p_own : pown[i]) * v;
                } else if (MODE == kSpmvResidual) {
                    yo[row0 + i] = a.b[row0 + i] - v;
                } else {
                    const double bi = a.b[row0 + i], ri = bi - v;
                    dot += ri * ri;
                    dot2 += bi * bi;
                }
            }
            wave_lds_sync();
        }
        if (!more) break;
        H = Hn;
        R = Rn;
        b = bn;
        bend = bendn;
        g = gn;
    }
    return dot;
}

// The multi-launch product. Blocks are dealt to the XCDs round robin; XCD x
// takes a contiguous range of segments in proportion to its blocks and
// interleaves it over its wavefronts (wavefront i takes segments i, i + W,
// ... of the range), so that the XCD's wavefronts sweep neighbouring
// segments together (shared vector segments stay in its L2) and finish
// together whatever the grid size. The grid is at most what the chip holds
// at once. Dynamic LDS: a vector stage of a.stage_doubles per wavefront.
template <typename MetaT, int MODE, int MAXROWS, bool CB = false, bool P1 = false, bool STAGE = false>
__global__ __launch_bounds__(kSpmvBlock) void spmv_tilecsc_kernel(SpmvArgs a, double* __restrict__ y,
                                                                  double* __restrict__ partials) {
    __shared__ double s_acc[kSpmvWaves][MAXROWS + kWave];
    __shared__ int4 s_desc[kSpmvWaves][kDescSlots];
    __shared__ double s_tmp[kSpmvWaves];
    // CG mode, groups above 64 rows: each wavefront's copy of its group's p entries.
    constexpr int kPown = (MODE == kSpmvCg && MAXROWS > kWave) ? MAXROWS : 2;
    __shared__ __attribute__((aligned(16))) double s_pown[kSpmvWaves][kPown];
    extern __shared__ __attribute__((aligned(16))) double s_stage[];

    if (MODE == kSpmvCg && load_done(a.st)) return;

    const int lane = threadIdx.x & (kWave - 1);
    // The wavefront index is uniform across the wave; saying so keeps every
    // per-batch and per-window quantity in scalar registers.
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nb = gridDim.x, bx = blockIdx.x;
    const int xcd = bx & 7, q = nb >> 3, r = nb & 7;
    const int nbx = q + (xcd < r ? 1 : 0);          // blocks on this XCD
    const int b0 = xcd * q + (xcd < r ? xcd : r);   // its first block in XCD-contiguous order
    const int s0 = (int)((int64_t)a.ngroups * b0 / nb);
    const int s1 = (int)((int64_t)a.ngroups * (b0 + nbx) / nb);
    const int wx = (bx >> 3) * kSpmvWaves + w;
    double dot2;
    double dot = spmv_wave_multi<MetaT, MODE, MAXROWS, CB, P1, STAGE>(a, y, s0 + wx, nbx * kSpmvWaves, s1, *a.uprec,
                                                              &s_acc[w][0], &s_desc[w][0],
                                                              s_stage + (size_t)w * a.stage_doubles, &s_pown[w][0],
                                                              lane, dot2);
    if (MODE == kSpmvCg) {
        dot = wave_sum(dot);
        __syncthreads();
        if (lane == 0) s_tmp[w] = dot;
        __syncthreads();
        if (threadIdx.x == 0) {
            double t = 0.0;
            for (int i = 0; i < kSpmvWaves; ++i) t += s_tmp[i];
            partials[blockIdx.x] = t;
        }
    } else if (MODE == kSpmvResNorm) {
        const double t1 = block_sum<kSpmvWaves>(dot, s_tmp);
        const double t2 = block_sum<kSpmvWaves>(dot2, s_tmp);
        if (threadIdx.x == 0) {
            partials[2 * blockIdx.x] = t1;
            partials[2 * blockIdx.x + 1] = t2;
        }
    }
}

// The relative true residual from nparts (||b - A x||^2, ||b||^2) partials:
// out[0] = ||b - A x|| / ||b|| (||b - A x|| when b = 0), summed in a fixed
// order (one block).
__global__ __launch_bounds__(kBlock) void resnorm_finish_kernel(const double* __restrict__ partials, int nparts,
                                                               double* __restrict__ out) {
    __shared__ double s_tmp[kWavesPerBlock];
    double tot[2];
    sum_partials<2>(partials, nparts, tot, s_tmp);
    if (threadIdx.x == 0) out[0] = tot[1] > 0.0 ? sqrt(tot[0]) / sqrt(tot[1]) : sqrt(tot[0]);
}

// Column slices: the residual from the slices' partial products (r_i = b_i -
// their sum) straight into (||r||^2, ||b||^2) block partials.
__global__ __launch_bounds__(kBlock) void combine_resnorm_kernel(const double* __restrict__ parts, int nparts,
                                                                int64_t stride, const double* __restrict__ b,
                                                                int64_t n, double* __restrict__ partials) {
    __shared__ double s_tmp[kWavesPerBlock];
    double rr = 0.0, bb = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        double acc = parts[i];
        for (int s = 1; s < nparts; ++s) acc += parts[s * stride + i];
        const double r = b[i] - acc;
        rr += r * r;
        bb += b[i] * b[i];
    }
    const double t1 = block_sum(rr, s_tmp);
    const double t2 = block_sum(bb, s_tmp);
    if (threadIdx.x == 0) {
        partials[2 * blockIdx.x] = t1;
        partials[2 * blockIdx.x + 1] = t2;
    }
}

// ---------------------------------------------------------------------------
// CG vector kernels. No atomics and no grid-wide fences: every kernel writes
// one partial per block for each quantity it reduces, and the next kernel
// sums those partials in a fixed order in every block (kernel boundaries
// make them visible across XCDs). Scalar state is committed by thread 0 of
// block 0 into fields the other blocks of the same launch do not read.
// ---------------------------------------------------------------------------
struct VecArgs {
    double* x;
    double* r;
    double* p;
    const double* q;      // the product q, or its column-slice partial products (nq of them)
    double* z;            // Jacobi only (z = dinv .* r)
    const double* dinv;   // Jacobi only
    const double* b;
    const double* x0;     // may be null
    double* hist;
    State* st;
    const double* part_in;   // partials written by the previous kernel
    int32_t nparts_in;
    double* part_out;        // this kernel's partials
    int32_t* trace_k;
    int32_t* trace_counts;   // [entry][kTraceBlocks][3]
    int64_t T;
    int32_t n;
    int32_t jacobi;
    int32_t r_ready;         // init: r already holds b - A x0
    int32_t nq;              // partial products summed into q (column slices), >= 1
    int64_t qstride;         // distance between two partial products
};

// st->ntrace and st->stage are read with atomic loads: the single-workgroup
// solver writes them and reads them back within one launch, and such loads
// are never served by the scalar cache, which does not see vector stores.
__device__ inline int load_i32(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void trace_uniform(State* st, int32_t* trace_k, int32_t* trace_counts, int k,
                                     int prec, int64_t T) {
    const int i = load_i32(&st->ntrace);
    if (i < st->trace_cap) {
        trace_k[i] = k;
        for (int p = 0; p < 3; ++p) trace_counts[(size_t)i * kTraceBlocks * 3 + p] = (p == prec) ? (int32_t)T : 0;
    }
    st->ntrace = i + 1;
}

// Advances the one-way residual schedule for the residual rho of iteration k.
__device__ inline void advance_stage(State* st, int32_t* trace_k, int32_t* trace_counts, int k,
                                     double rho, int64_t T, bool first) {
    if (st->nstage <= 0) return;
    const int s0 = load_i32(&st->stage);
    int s = s0;
    while (s < st->nstage - 1 && rho <= st->thresholds[s]) ++s;
    if (s != s0 || first) {
        st->stage = s;
        st->uprec = st->stage_prec[s];
        trace_uniform(st, trace_k, trace_counts, k, st->uprec, T);
    }
}

// Initial vectors: x = x0 (or 0), r = b - A x0 (computed beforehand when x0 is
// given), z = dinv .* r, p = z; partials of r.r and r.z.
__global__ __launch_bounds__(kBlock) void cg_init_kernel(VecArgs a) {
    __shared__ double s_tmp[kWavesPerBlock];
    double rr = 0.0, rz = 0.0;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < a.n; i += gridDim.x * blockDim.x) {
        const double ri = a.r_ready ? a.r[i] : a.b[i];
        a.x[i] = a.x0 ? a.x0[i] : 0.0;
        if (!a.r_ready) a.r[i] = ri;
        double zi = ri;
        if (a.jacobi) {
            zi = a.dinv[i] * ri;
            a.z[i] = zi;
        }
        a.p[i] = zi;
        rr += ri * ri;
        rz += ri * zi;
    }
    const double prr = block_sum(rr, s_tmp);
    const double prz = block_sum(rz, s_tmp);
    if (threadIdx.x == 0) {
        a.part_out[2 * blockIdx.x] = prr;
        a.part_out[2 * blockIdx.x + 1] = prz;
    }
}

// One block: ||r0||, r.z, rho_0, the stop decision at k = 0, the first stage.
__global__ __launch_bounds__(kBlock) void cg_init_finish_kernel(VecArgs a) {
    __shared__ double s_tmp[kWavesPerBlock];
    double tot[2];
    sum_partials<2>(a.part_in, a.nparts_in, tot, s_tmp);
    if (threadIdx.x == 0) {
        State* st = a.st;
        st->rr = tot[0];
        st->rz = a.jacobi ? tot[1] : tot[0];
        st->rz_prev = st->rz;
        st->norm0 = sqrt(tot[0]);
        st->k = 0;
        st->bd = 0;
        st->ntrace = 0;
        st->stage = 0;
        st->alpha = 0.0;
        st->beta = 0.0;
        // A non-finite r0 (b or x0 holds a NaN or an infinity) starts at rho_0 = 1
        // and, past the tolerance and iteration-cap tests, stops as a breakdown
        // before the first update: its p.q would not be finite.
        const bool finite = isfinite(st->norm0);
        const double rho0 = (st->norm0 > 0.0 || !finite) ? 1.0 : 0.0;
        a.hist[0] = rho0;
        if (st->nstage > 0) advance_stage(st, a.trace_k, a.trace_counts, 0, rho0, a.T, true);
        int done = 0;
        if (st->norm0 == 0.0 || rho0 <= st->tol) done = 1;
        else if (st->maxit <= 0) done = 2;
        else if (!finite) done = 3;
        store_done(st, done);
    }
}

// Update and direction kernels: blocks of kVecBlock threads; thread t of a
// grid of S threads handles the 16-byte pairs t, t+S, ... (kVecPairs of them
// per chunk). The handle's vectors are padded with zeros to an even length,
// so pairs need no tail handling. Each kernel issues its first chunk's loads
// before it sums the previous kernel's partials, which hides that sum.
#ifndef MPCG_VEC_BLOCK
#define MPCG_VEC_BLOCK 512
#endif
constexpr int kVecBlock = MPCG_VEC_BLOCK;
constexpr int kVecWaves = kVecBlock / kWave;
#ifndef MPCG_VEC_PAIRS
#define MPCG_VEC_PAIRS 4
#endif
constexpr int kVecPairs = MPCG_VEC_PAIRS;

// alpha = r.z / p.q (p.q summed from the SpMV partials in every block);
// r -= alpha q; [z = dinv .* r]; partials of r.r [and r.z]. x += alpha p is
// left to the direction kernel, which reads p anyway. On p.q <= 0 or a
// non-finite alpha nothing is updated and the breakdown is flagged for the
// direction kernel. `done` does not change during this launch, so every block
// takes the same decision, and block 0 records it in `live` for the direction
// kernel.
template <bool JAC, bool NT>
__global__ __launch_bounds__(kVecBlock) void cg_update_kernel(VecArgs a) {
    __shared__ double s_tmp[kVecWaves];
    State* st = a.st;
    const bool live = load_done(st) == 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) st->live = live ? 1 : 0;
    if (!live) return;
    const int64_t npairs = ((int64_t)a.n + 1) / 2;
    const int64_t stride = (int64_t)gridDim.x * kVecBlock;
    const int64_t tid = (int64_t)blockIdx.x * kVecBlock + threadIdx.x;
    double2* __restrict__ r2 = reinterpret_cast<double2*>(a.r);
    double2* __restrict__ z2 = reinterpret_cast<double2*>(a.z);
    const double2* __restrict__ q2 = reinterpret_cast<const double2*>(a.q);
    const double2* __restrict__ d2 = reinterpret_cast<const double2*>(a.dinv);
    double2 rv[kVecPairs], qv[kVecPairs], dv[kVecPairs];
    auto load = [&](int64_t base) {
#pragma unroll
        for (int j = 0; j < kVecPairs; ++j) {
            const int64_t i = base + j * stride + tid;
            if (i < npairs) {
                rv[j] = load_vec(&r2[i], NT);
                qv[j] = load_vec(&q2[i], NT);
                for (int s = 1; s < a.nq; ++s) {  // column slices: q is the sum of the partials
                    const double2 qs = q2[s * (a.qstride / 2) + i];
                    qv[j].x += qs.x;
                    qv[j].y += qs.y;
                }
                if (JAC) dv[j] = d2[i];
            }
        }
    };
    load(0);
    double tot[1];
    sum_partials<1, kVecWaves>(a.part_in, a.nparts_in, tot, s_tmp);
    const double pq = tot[0];
    const double alpha = st->rz / pq;
    const bool bd = !(pq > 0.0) || !isfinite(pq) || !isfinite(alpha);
    double rr = 0.0, rz = 0.0;
    if (!bd) {
        for (int64_t base = 0; base < npairs; base += stride * kVecPairs) {
            if (base > 0) load(base);
#pragma unroll
            for (int j = 0; j < kVecPairs; ++j) {
                const int64_t i = base + j * stride + tid;
                if (i < npairs) {
                    double2 rn;
                    rn.x = rv[j].x - alpha * qv[j].x;
                    rn.y = rv[j].y - alpha * qv[j].y;
                    store_vec(&r2[i], rn, NT && JAC);  // r is read next unless z is
                    rr += rn.x * rn.x + rn.y * rn.y;
                    if (JAC) {
                        double2 zn;
                        zn.x = dv[j].x * rn.x;
                        zn.y = dv[j].y * rn.y;
                        z2[i] = zn;  // read next by the direction kernel
                        rz += rn.x * zn.x + rn.y * zn.y;
                    }
                }
            }
        }
    }
    const double prr = block_sum<kVecWaves>(rr, s_tmp);
    const double prz = JAC ? block_sum<kVecWaves>(rz, s_tmp) : prr;
    if (threadIdx.x == 0) {
        a.part_out[2 * blockIdx.x] = prr;
        a.part_out[2 * blockIdx.x + 1] = prz;
        if (blockIdx.x == 0) {
            st->pq = pq;
            st->alpha = alpha;
            st->rz_prev = st->rz;
            st->bd = bd ? 1 : 0;
        }
    }
}

// x += alpha p; beta = (r.z)_new / (r.z)_old from the update partials (in
// every block); p = z + beta p (z = r for plain CG). Thread 0 of block 0
// commits rho_{k+1}, the history entry, the stop flag and the schedule stage.
// The launch runs when the update kernel of this iteration ran (`live`, which
// no block of this launch writes); `done` may be set by block 0 while other
// blocks still run, and they must still apply this iteration's x update.
template <bool JAC, bool NT>
__global__ __launch_bounds__(kVecBlock) void cg_direction_kernel(VecArgs a) {
    __shared__ double s_tmp[kVecWaves];
    State* st = a.st;
    if (!st->live) return;
    if (st->bd) {
        if (blockIdx.x == 0 && threadIdx.x == 0) store_done(st, 3);
        return;
    }
    const int64_t npairs = ((int64_t)a.n + 1) / 2;
    const int64_t stride = (int64_t)gridDim.x * kVecBlock;
    const int64_t tid = (int64_t)blockIdx.x * kVecBlock + threadIdx.x;
    double2* __restrict__ p2 = reinterpret_cast<double2*>(a.p);
    double2* __restrict__ x2 = reinterpret_cast<double2*>(a.x);
    const double2* __restrict__ z2 = reinterpret_cast<const double2*>(JAC ? a.z : a.r);
    double2 pv[kVecPairs], zv[kVecPairs], xv[kVecPairs];
    auto load = [&](int64_t base) {
#pragma unroll
        for (int j = 0; j < kVecPairs; ++j) {
            const int64_t i = base + j * stride + tid;
            if (i < npairs) {
                pv[j] = p2[i];
                zv[j] = load_vec(&z2[i], NT);
                xv[j] = load_vec(&x2[i], NT);
            }
        }
    };
    load(0);
    double tot[2];
    sum_partials<2, kVecWaves>(a.part_in, a.nparts_in, tot, s_tmp);
    const double rr_new = tot[0];
    const double rz_new = tot[1];
    const double beta = rz_new / st->rz_prev;
    const double alpha = st->alpha;
    for (int64_t base = 0; base < npairs; base += stride * kVecPairs) {
        if (base > 0) load(base);
#pragma unroll
        for (int j = 0; j < kVecPairs; ++j) {
            const int64_t i = base + j * stride + tid;
            if (i < npairs) {
                double2 pn, xn;
                xn.x = xv[j].x + alpha * pv[j].x;
                xn.y = xv[j].y + alpha * pv[j].y;
                pn.x = zv[j].x + beta * pv[j].x;
                pn.y = zv[j].y + beta * pv[j].y;
                store_vec(&x2[i], xn, NT);
                p2[i] = pn;  // p stays cached for the next product's gathers
            }
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        const int k = st->k + 1;
        const double rho = sqrt(rr_new) / st->norm0;
        a.hist[k] = rho;
        st->k = k;
        st->rr = rr_new;
        st->rz = rz_new;
        st->beta = beta;
        int done = 0;
        if (!isfinite(beta) || !isfinite(rho)) done = 3;
        else if (rho <= st->tol) done = 1;
        else if (k >= st->maxit) done = 2;
        else if (st->nstage > 0) advance_stage(st, a.trace_k, a.trace_counts, k, rho, a.T, false);
        if (done) store_done(st, done);
    }
}

// ---------------------------------------------------------------------------
// Single-workgroup CG for small systems. One launch of kSmallBlock threads
// runs the iterations that the SpMV, update and direction kernels run one
// launch each, with workgroup barriers between the phases; small systems are
// bound by launch latency, not bandwidth. Same state, history, stop tests,
// breakdown rule and residual schedule as those kernels; the per-tile map is
// fixed during the launch (static maps, uniform stages). Wavefront w takes the
// row groups [w G / W, (w + 1) G / W). Scalars that change during the launch
// are passed through LDS: the scalar cache does not see vector stores.
constexpr int kSmallWaves = 16;
constexpr int kSmallBlock = kSmallWaves * kWave;
#ifndef MPCG_SMALL_UNROLL
#define MPCG_SMALL_UNROLL 4
#endif
#ifndef MPCG_SMALL_XLDS
#define MPCG_SMALL_XLDS 1
#endif
constexpr int kSmallUnroll = MPCG_SMALL_UNROLL;  // windows per sweep: a latency-bound SpMV
constexpr bool kSmallXLds = MPCG_SMALL_XLDS != 0;  // gather p from an LDS copy
// Rows the LDS copy of p holds: with the widest accumulators the workgroup
// then uses 154 of gfx950's 160 KB of LDS.
constexpr int kSmallMaxN = 12288;

template <typename MetaT, int MAXROWS, bool JAC>
__global__ __launch_bounds__(kSmallBlock) void cg_small_kernel(SpmvArgs sa, VecArgs va) {
    __shared__ double s_acc[kSmallWaves][MAXROWS + kWave];
    __shared__ int4 s_desc[kSmallWaves][kDescSlots];
    __shared__ double s_tmp[kSmallWaves];
    __shared__ double s_p[kSmallXLds ? kSmallMaxN : 1];  // p, for the SpMV's gathers
    __shared__ int s_done, s_uprec, s_k;
    State* st = va.st;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int g0 = (int)((int64_t)sa.ngroups * w / kSmallWaves);
    const int g1 = (int)((int64_t)sa.ngroups * (w + 1) / kSmallWaves);
    const int64_t npairs = ((int64_t)va.n + 1) / 2;
    double2* r2 = reinterpret_cast<double2*>(va.r);
    double2* z2 = reinterpret_cast<double2*>(va.z);
    double2* p2 = reinterpret_cast<double2*>(va.p);
    double2* x2 = reinterpret_cast<double2*>(va.x);
    const double2* q2 = reinterpret_cast<const double2*>(va.q);
    const double2* d2 = reinterpret_cast<const double2*>(va.dinv);
    if (threadIdx.x == 0) {
        s_done = load_done(st);
        s_uprec = st->uprec;
        s_k = st->k;
    }
    if (kSmallXLds)
        for (int i = threadIdx.x; i < va.n; i += kSmallBlock) s_p[i] = va.p[i];
    __syncthreads();
    const int maxit = st->maxit;
    double rz_old = st->rz;  // then carried in registers (every thread gets the same sums)
    // Every thread leaves the loop at the same iteration: the exit reads LDS
    // values written before the barrier that ends the previous iteration.
    for (int k = s_k; k < maxit && s_done == 0; k = s_k) {
        // q = A p and p.q.
        const double pq = block_sum<kSmallWaves>(
            spmv_wave<MetaT, kSpmvCg, MAXROWS, false, false, kSmallUnroll, kSmallXLds>(
                sa, sa.y, g0, g1, s_uprec, &s_acc[w][0], &s_desc[w][0], lane, s_p),
            s_tmp);
        const double alpha = rz_old / pq;
        if (!(pq > 0.0) || !isfinite(pq) || !isfinite(alpha)) {  // breakdown: nothing is updated
            if (threadIdx.x == 0) {
                st->pq = pq;
                st->bd = 1;
                store_done(st, 3);
            }
            break;
        }
        // r -= alpha q; [z = dinv .* r]; r.r [and r.z].
        double rr = 0.0, rz = 0.0;
        for (int64_t i = threadIdx.x; i < npairs; i += kSmallBlock) {
            const double2 qv = q2[i];
            double2 rn = r2[i];
            rn.x -= alpha * qv.x;
            rn.y -= alpha * qv.y;
            r2[i] = rn;
            rr += rn.x * rn.x + rn.y * rn.y;
            if (JAC) {
                const double2 dv = d2[i];
                double2 zn;
                zn.x = dv.x * rn.x;
                zn.y = dv.y * rn.y;
                z2[i] = zn;
                rz += rn.x * zn.x + rn.y * zn.y;
            }
        }
        const double rr_new = block_sum<kSmallWaves>(rr, s_tmp);
        const double rz_new = JAC ? block_sum<kSmallWaves>(rz, s_tmp) : rr_new;
        const double beta = rz_new / rz_old;
        // x += alpha p; p = z + beta p (z = r for plain CG): each thread reads
        // back only the r or z entries it has just written.
        const double2* zsrc = reinterpret_cast<const double2*>(JAC ? va.z : va.r);
        for (int64_t i = threadIdx.x; i < npairs; i += kSmallBlock) {
            const double2 pv = p2[i], zv = zsrc[i];
            double2 xv = x2[i], pn;
            xv.x += alpha * pv.x;
            xv.y += alpha * pv.y;
            pn.x = zv.x + beta * pv.x;
            pn.y = zv.y + beta * pv.y;
            x2[i] = xv;
            p2[i] = pn;
            if (kSmallXLds) {  // 2i < n always; for odd n the padding entry n has no slot
                s_p[2 * i] = pn.x;
                if (2 * i + 1 < va.n) s_p[2 * i + 1] = pn.y;
            }
        }
        if (threadIdx.x == 0) {
            const int kn = k + 1;
            const double rho = sqrt(rr_new) / st->norm0;
            va.hist[kn] = rho;
            st->pq = pq;
            st->alpha = alpha;
            st->rz_prev = rz_old;
            st->k = kn;
            st->rr = rr_new;
            st->rz = rz_new;
            st->beta = beta;
            int done = 0;
            if (!isfinite(beta) || !isfinite(rho)) done = 3;
            else if (rho <= st->tol) done = 1;
            else if (kn >= maxit) done = 2;
            else if (st->nstage > 0) advance_stage(st, va.trace_k, va.trace_counts, kn, rho, va.T, false);
            if (done) store_done(st, done);
            s_done = done;
            s_uprec = load_i32(&st->uprec);
            s_k = kn;
        }
        rz_old = rz_new;
        __syncthreads();
    }
}

// Column slices: y = sum of the nparts partial products (or b minus it).
__global__ __launch_bounds__(kBlock) void combine_kernel(const double* __restrict__ parts, int nparts, int64_t stride,
                                                        const double* __restrict__ b, double* __restrict__ y,
                                                        int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        double acc = parts[i];
        for (int s = 1; s < nparts; ++s) acc += parts[s * stride + i];
        y[i] = b ? b[i] - acc : acc;
    }
}

// ---------------------------------------------------------------------------
// Map kernels. Launched with exactly kTraceBlocks blocks; per-block precision
// counts go to the trace (summed on the host), so no atomics are needed.
// ---------------------------------------------------------------------------
__device__ inline int tile_rule_code(double s, double rho, double hi, double lo) {
    const double v = s * rho;
    return v > hi ? 2 : (v > lo ? 1 : 0);
}

struct MapArgs {
    uint8_t* map;
    const double* scores;
    State* st;
    const double* hist;
    int32_t* trace_k;
    int32_t* trace_counts;
    const int32_t* btab;  // tile rule: batches of the SpMV (a partition of the tiles)
    uint8_t* winmaps;     // tile rule, recording on: [window][T] map of every window (else NULL)
    const uint8_t* count_w;  // per tile: 1 if it counts in the trace (one piece per tile of R > 256), or NULL: all
    int64_t T;
    int64_t nbatch;
    double rho;          // explicit rho (eval mode)
    int32_t solve;       // 1: in-solve window step (reads k and rho_k from the state)
    int32_t winmap_cap;  // windows winmaps holds
};

// The block's totals of three per-thread counts, returned in thread c for
// count c (c < 3; other threads get 0). Each wavefront sums with shuffles and
// leaves one slot per count in LDS: an LDS atomic from every lane on one
// address would run its 64 lanes one after another.
__device__ inline unsigned block_count3(unsigned c0, unsigned c1, unsigned c2) {
    __shared__ unsigned s_part[kWavesPerBlock][3];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        c0 += __shfl_xor(c0, off, kWave);
        c1 += __shfl_xor(c1, off, kWave);
        c2 += __shfl_xor(c2, off, kWave);
    }
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
        s_part[w][0] = c0;
        s_part[w][1] = c1;
        s_part[w][2] = c2;
    }
    __syncthreads();
    unsigned t = 0;
    if (threadIdx.x < 3)
        for (int v = 0; v < (int)(blockDim.x / kWave); ++v) t += s_part[v][threadIdx.x];
    return t;
}

__device__ inline void block_counts_out(unsigned c0, unsigned c1, unsigned c2, int32_t* out) {
    const unsigned t = block_count3(c0, c1, c2);
    if (threadIdx.x < 3) out[threadIdx.x] = (int32_t)t;
}

// Windowed tile rule: at k % period == 0 every tile's precision is re-selected
// from its score and rho_k, and the window's precision counts are recorded.
// One wavefront per SpMV batch (lane l: the batch's tile l). The grid is sized
// to the batches; block b adds its counts to slot b % kTraceBlocks of the
// entry. Nothing is repacked: while the tile rule owns the map, the SpMV reads
// each tile's values from its precision's plane.
__global__ __launch_bounds__(kBlock) void tile_rule_kernel(MapArgs a) {
    State* st = a.st;
    double rho = a.rho;
    int slot = -1;
    if (a.solve) {
        if (load_done(st)) return;
        const int k = st->k;
        if (k % st->period != 0) return;
        rho = a.hist[k];
        slot = k / st->period;
        if (slot >= st->trace_cap) slot = -1;
    }
    unsigned c0 = 0, c1 = 0, c2 = 0;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int64_t waves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t b = (int64_t)blockIdx.x * kWavesPerBlock + w; b < a.nbatch; b += waves) {
        const int32_t* e = a.btab + b * kBtFields;
        const int tb = e[kBtTile], nt = e[kBtTiles];
        if (lane < nt) {
            const int64_t t = (int64_t)tb + lane;
            const int code = tile_rule_code(a.scores[t], rho, st->hi, st->lo);
            a.map[t] = (uint8_t)code;
            if (slot >= 0 && slot < a.winmap_cap) a.winmaps[(size_t)slot * a.T + t] = (uint8_t)code;
            const bool counted = !a.count_w || a.count_w[t];
            c0 += counted && code == 0;
            c1 += counted && code == 1;
            c2 += counted && code == 2;
        }
    }
    if (slot >= 0) {
        const unsigned t = block_count3(c0, c1, c2);
        if (threadIdx.x < 3)
            atomicAdd(a.trace_counts + ((size_t)slot * kTraceBlocks + blockIdx.x % kTraceBlocks) * 3 + threadIdx.x,
                      (int32_t)t);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            a.trace_k[slot] = st->k;
            st->ntrace = slot + 1;
        }
    }
}

// Per-segment max|p| rule (Sec. 4.7): the code of every column block from the
// largest |p_j| in its segment (BF16 below lo, FP32 below hi, else FP64), and
// counts of tiles per code into the trace. One thread per column block; a
// whole block of even width is read with 16-byte loads (unrolled, so they are
// all in flight together) when the vector is 16-byte aligned. Block b adds its
// counts to the entry's slot b % kTraceBlocks (atomics on addresses shared by
// a few blocks only). In a solve (solve = 1) the rule is evaluated at the
// iterations k that are multiples of the period, for the direction p_k, into
// trace entry k / period (with the codes themselves kept in `history` when it
// is set); it does nothing once the solve has stopped.
struct PMagArgs {
    const double* p;
    uint8_t* cbcode;
    const int32_t* tpcb;  // tiles in every column block
    State* st;
    int32_t* trace_k;
    int32_t* trace_counts;
    uint8_t* history;  // [trace_cap][ncb] or null
    int64_t n;
    int32_t C, ncb, solve, trace_cap, period;
    double lo, hi;
};

__device__ inline double nan_max(double a, double b) { return (a > b || a != a) ? a : b; }
__device__ inline int pmag_code(double m, double lo, double hi) { return m < lo ? 2 : (m < hi ? 1 : 0); }

// In a solve the rule runs at iterations k that are multiples of the period
// and writes trace entry k / period; returns false where this launch has
// nothing to do (the solve has stopped, or k is not a multiple).
__device__ inline bool pmag_slot(const PMagArgs& a, int& k, int& slot) {
    slot = -1;
    k = 0;
    if (!a.solve) return true;
    if (load_done(a.st)) return false;
    k = a.st->k;
    if (k % a.period != 0) return false;
    slot = k / a.period;
    if (slot >= a.trace_cap) slot = -1;
    return true;
}

// The block's tile counts per code into the trace entry (slot b % kTraceBlocks
// of entry `slot`); block 0 also records the entry's iteration.
__device__ inline void pmag_counts_out(const PMagArgs& a, const unsigned (&cnt)[3], int slot, int k) {
    if (slot < 0) return;
    const unsigned t = block_count3(cnt[0], cnt[1], cnt[2]);
    if (threadIdx.x < 3) {
        int32_t* out = a.trace_counts + ((size_t)slot * kTraceBlocks + blockIdx.x % kTraceBlocks) * 3;
        atomicAdd(&out[threadIdx.x], (int32_t)t);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.trace_k[slot] = k;
        a.st->ntrace = slot + 1;
    }
}

// One thread per column block.
__global__ __launch_bounds__(kBlock) void pmag_kernel(PMagArgs a) {
    int k, slot;
    if (!pmag_slot(a, k, slot)) return;
    uint8_t* hist = slot >= 0 && a.history ? a.history + (size_t)slot * a.ncb : nullptr;
    unsigned cnt[3] = {0u, 0u, 0u};
    const bool pairs = (a.C & 1) == 0 && ((uintptr_t)a.p & 15) == 0;
    for (int64_t J = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; J < a.ncb;
         J += (int64_t)gridDim.x * blockDim.x) {
        const int64_t j0 = J * a.C, j1 = min(j0 + a.C, a.n);
        const unsigned tiles = (unsigned)a.tpcb[J];  // issued with the vector loads
        double m = 0.0;
        if (pairs && j1 - j0 == a.C) {
            const double2* q = reinterpret_cast<const double2*>(a.p + j0);
#pragma unroll 8
            for (int e = 0; e < a.C / 2; ++e) {
                const double2 v = q[e];
                m = nan_max(m, nan_max(fabs(v.x), fabs(v.y)));
            }
        } else {
            for (int64_t j = j0; j < j1; ++j) m = nan_max(m, fabs(a.p[j]));
        }
        const int code = pmag_code(m, a.lo, a.hi);
        a.cbcode[J] = (uint8_t)code;
        if (hist) hist[J] = (uint8_t)code;
        cnt[code] += tiles;
    }
    pmag_counts_out(a, cnt, slot, k);
}

// Precision counts of the active map into trace entry 0 (static maps); with
// count_w only the tiles it flags count.
__global__ __launch_bounds__(kBlock) void map_count_kernel(const uint8_t* map, const uint8_t* count_w, int64_t T,
                                                           int32_t* trace_k, int32_t* counts) {
    unsigned c[3] = {0, 0, 0};
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < T;
         t += (int64_t)gridDim.x * blockDim.x)
        if (!count_w || count_w[t]) c[map[t] < 3 ? map[t] : 0]++;
    block_counts_out(c[0], c[1], c[2], counts + (size_t)blockIdx.x * 3);
    if (blockIdx.x == 0 && threadIdx.x == 0) trace_k[0] = 0;
}

// Fills n int32 values (a device-side clear that is safe inside captured graphs).
__global__ void fill_i32_kernel(int32_t* p, int32_t v, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// Magnitude rule, part 1: max |a_ii| over the diagonal entries (atomic max on
// the bit pattern, which orders non-negative doubles like unsigned integers).
// trow[t]: the row block of tile t (height R), in any tile order.
__global__ __launch_bounds__(kBlock) void diag_absmax_kernel(const int32_t* trow, const int32_t* tcol,
                                                             const int32_t* tptr, const void* meta,
                                                             int meta16, const double* v64,
                                                             int32_t T, int32_t R,
                                                             int32_t C, unsigned long long* out) {
    for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < T; t += gridDim.x * blockDim.x) {
        const int64_t row_base = (int64_t)trow[t] * R, col_base = (int64_t)tcol[t] * C;
        double m = 0.0;
        for (int k = tptr[t]; k < tptr[t + 1]; ++k) {
            int r, c;
            if (meta16) decode_meta<uint16_t>(static_cast<const uint16_t*>(meta)[k], r, c);
            else decode_meta<uint8_t>(static_cast<const uint8_t*>(meta)[k], r, c);
            if (row_base + r == col_base + c) m = fmax(m, fabs(v64[k]));
        }
        if (m > 0.0) atomicMax(out, (unsigned long long)__double_as_longlong(m));
    }
}

// Magnitude rule, part 2: ratio_t = max |a| in tile / max |a_ii|; BF16 below
// t16, FP32 below t32, else FP64. One thread per tile t < T. With cptr, tile
// t is stored as the pieces clist[cptr[t] .. cptr[t+1]) (row blocks taller
// than the device's slabs): the maximum runs over all of them and every piece
// gets the tile's code. Without, tile t is device tile t.
__global__ __launch_bounds__(kBlock) void magnitude_map_kernel(const int32_t* tptr, const double* v64,
                                                               int32_t T, const int32_t* cptr,
                                                               const int32_t* clist,
                                                               const unsigned long long* dmax_bits,
                                                               double t16, double t32, uint8_t* map) {
    const double dmax = __longlong_as_double((long long)*dmax_bits);
    for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < T; t += gridDim.x * blockDim.x) {
        const int c0 = cptr ? cptr[t] : t, c1 = cptr ? cptr[t + 1] : t + 1;
        double m = 0.0;
        for (int c = c0; c < c1; ++c) {
            const int d = cptr ? clist[c] : c;
            for (int k = tptr[d]; k < tptr[d + 1]; ++k) m = fmax(m, fabs(v64[k]));
        }
        const double ratio = m / dmax;
        const uint8_t code = ratio < t16 ? 2 : (ratio < t32 ? 1 : 0);
        for (int c = c0; c < c1; ++c) map[cptr ? clist[c] : c] = code;
    }
}

}  // namespace dev
}  // namespace mpcg
