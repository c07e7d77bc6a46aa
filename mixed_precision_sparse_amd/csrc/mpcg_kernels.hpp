// Device code for gfx950: value-plane builder, mixed-precision Tile-CSC SpMV,
// fused CG vector updates with single-pass grid reductions, and map kernels.
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
constexpr int kMaxRows = 256;    // rows owned by one wavefront (R <= 256)
constexpr int kMaxGroupRB = 63;  // row blocks per wavefront at most (boundaries fit one wave)

// Solver scalars, resident on the device for the whole solve. Each field has
// one writer per kernel launch (thread 0 of block 0) and no other block of
// that launch reads it, except `done` (see cg_direction_kernel).
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
    int32_t pad;
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

__global__ void build_planes_kernel(const double* __restrict__ v64, float* __restrict__ v32,
                                    uint16_t* __restrict__ v16, int64_t nnz) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nnz;
         i += (int64_t)gridDim.x * blockDim.x) {
        uint64_t u = (uint64_t)__double_as_longlong(v64[i]);
        v32[i] = __uint_as_float(round_f64_to_e8<23>(u));
        v16[i] = (uint16_t)round_f64_to_e8<7>(u);
    }
}

// ---------------------------------------------------------------------------
// Reduction helpers.
// ---------------------------------------------------------------------------
__device__ inline double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ inline int wave_sum_int(int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Block sum in a fixed order; the result is valid in every thread.
__device__ inline double block_sum(double v, double* s_tmp) {
    v = wave_sum(v);
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    __syncthreads();
    if (lane == 0) s_tmp[w] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < kWavesPerBlock; ++i) t += s_tmp[i];
    return t;
}

// Fixed-order sum of nparts partials (component j of NV per part); every
// thread of the block gets the same value, and every block that calls this
// on the same data gets the same bits.
template <int NV>
__device__ inline void sum_partials(const double* partials, int nparts, double (&out)[NV],
                                    double* s_tmp) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        double a = 0.0;
        for (int i = threadIdx.x; i < nparts; i += blockDim.x) a += partials[(size_t)i * NV + j];
        out[j] = block_sum(a, s_tmp);
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

// ---------------------------------------------------------------------------
// Mixed-precision Tile-CSC SpMV.
//
// One wavefront owns a row group: G consecutive row blocks (G*R rows, at most
// kGroupRows, or one row block when R is larger). It walks the group's tiles
// in batches of up to 64 and the 64 lanes sweep a batch's nonzeros 64 at a
// time ("windows"), several windows at once. Products of the widened stored
// value and the FP64 vector entry are accumulated in FP64 into the group's
// row accumulators in LDS; the group's rows are written once.
//
// The sweep follows a plan built on the device whenever the map changes
// (spmv_plan_kernel). Inside a batch the tiles are taken grouped by
// precision (FP64 tiles, then FP32, then BF16, each group in storage order)
// and every group starts on a window boundary, so each window reads exactly
// one value plane: its precision is a scalar and the plane is read with one
// load per lane. The plan has one entry per tile (column base in x, row offset
// in the group's accumulators, the shift from its position in the sweep to
// its storage position, and its precision) and one record per window (the
// entry of the window's first nonzero, a bit mask of the entries that start
// inside the window -- a lane's entry is then a prefix popcount -- the
// window's precision, and the batch's window count). The lanes past the end
// of a precision group land on a sentinel entry whose offsets are past the
// end of every buffer: the hardware answers those loads with zero and no
// memory access.
//
// A block of kSpmvWaves wavefronts handles a contiguous range of row groups
// (blocks are spread so that each XCD gets a contiguous part of the matrix);
// in CG mode each block also writes its part of p.q.
// ---------------------------------------------------------------------------
enum SpmvMode { kSpmvPlain = 0, kSpmvCg = 1, kSpmvResidual = 2 };
#ifndef MPCG_SPMV_UNROLL
#define MPCG_SPMV_UNROLL 8
#endif
#ifndef MPCG_SPMV_WAVES
#define MPCG_SPMV_WAVES 4
#endif
#ifndef MPCG_GROUP_ROWS
#define MPCG_GROUP_ROWS 64
#endif
constexpr int kUnroll = MPCG_SPMV_UNROLL;      // windows per full sweep (a power of two)
constexpr int kSpmvWaves = MPCG_SPMV_WAVES;    // wavefronts per SpMV block
constexpr int kSpmvBlock = kSpmvWaves * kWave;
constexpr int kGroupRows = MPCG_GROUP_ROWS;    // rows per wavefront when R <= kGroupRows
constexpr uint32_t kBufferConfig = 0x00020000u;  // raw buffer, dword3 for the gfx9 family
constexpr int kDescSlots = kTileBatch + 3;      // batch tiles + a sentinel after each precision group
constexpr int kSentinelShift = 1 << 27;         // storage shift: past every batch plane
constexpr int kSentinelColumn = 0x7fffff00;     // x byte offset: past every x

// Window records a batch executes: whole sweeps of kUnroll windows, then one
// sweep of the smallest power of two that covers the rest.
__host__ __device__ inline int sweep_windows(int nw) {
    const int full = nw / kUnroll * kUnroll;
    int r = nw - full, t = r > 0 ? 1 : 0;
    while (t < r) t <<= 1;
    return full + t;
}
// Records reserved for a batch of len nonzeros: at most two windows are added
// by starting the FP32 and BF16 groups on window boundaries.
__host__ __device__ inline int batch_records(int len) { return sweep_windows((len + kWave - 1) / kWave + 2); }

// Window record bit fields (int32): entry of the first nonzero, precision, and
// the batch's window count (the same in every record of the batch).
constexpr int kRecSlotBits = 8, kRecPrecShift = 8, kRecCountShift = 10;

struct SpmvArgs {
    const int32_t* trp;   // tile_row_ptr [nrb+1]
    const int32_t* tptr;  // tile_nnz_ptr [T+1]
    const int4* plan;     // [T] per tile, in plan order
    const void* meta;     // per nonzero (row, col) packed: u8 (R, C <= 16) or u16
    const double* v64;
    const float* v32;
    const uint16_t* v16;
    const int32_t* win_base;   // [ngroups+1] first window record of every row group
    const uint64_t* win_mask;  // per window: bit q = nonzero q+1 of the window starts a new entry
    const int32_t* win_tile;   // per window: packed record (see kRec*)
    const double* x;
    double* y;
    const double* b;       // residual mode: y = b - A x
    const int32_t* uprec;  // -1 per-tile map, else uniform code
    const State* st;
    double* partials;      // CG mode: one p.q partial per block
    int32_t n, nrb, R, C, G, rows_per_group, ngroups, groups_per_block;
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

__device__ inline __amdgpu_buffer_rsrc_t batch_rsrc(const void* base, int64_t first, int width, int count) {
    const char* p = static_cast<const char*>(base) + first * width;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, count * width, (int)kBufferConfig);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Wave-uniform reads of data no kernel here writes while the SpMV runs
// (window records, tile ranges): read through the constant address space so
// they become scalar loads.
template <typename T>
__device__ inline T uniform_load(const T* p, int i) {
    return ((const __attribute__((address_space(4))) T*)(uintptr_t)p)[i];
}

struct SweepCtx {
    __amdgpu_buffer_rsrc_t r64, r32, r16, rmt, rx;
    const uint64_t* win_mask;
    const int32_t* win_tile;
    const int4* desc;  // this wave's plan entries in LDS
    char* acc;         // this wave's row accumulators in LDS
    int uprec, len, lane;
};

// U consecutive windows of one batch, starting at record wi and sweep
// position o0. Loads are issued for all U windows before any is consumed.
template <typename MetaT, int U>
__device__ __forceinline__ void spmv_sweep(const SweepCtx& c, int wi, int o0) {
    uint64_t mask[U];
    int wp[U], q[U];
    int4 d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        mask[u] = uniform_load(c.win_mask, wi + u);
        const int rec = uniform_load(c.win_tile, wi + u);
        wp[u] = c.uprec >= 0 ? c.uprec : (rec >> kRecPrecShift) & 3;
        const int j = (rec & ((1 << kRecSlotBits) - 1)) +
                      (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask[u] >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask[u], 0u));
        d[u] = c.desc[j];
        q[u] = o0 + u * kWave + c.lane + d[u].z;  // storage position in the batch
    }
    uint32_t mt[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        mt[u] = sizeof(MetaT) == 1 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(c.rmt, q[u], 0, 0)
                                   : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(c.rmt, 2 * q[u], 0, 0);
    // Stored values, issued before the vector gathers (which wait for the
    // packed indices); the raw bits are widened after every load is issued.
    u32x2 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (wp[u] == 0)
            raw[u] = __builtin_amdgcn_raw_buffer_load_b64(c.r64, 8 * q[u], 0, 0);
        else if (wp[u] == 1)
            raw[u].x = __builtin_amdgcn_raw_buffer_load_b32(c.r32, 4 * q[u], 0, 0);
        else
            raw[u].x = __builtin_amdgcn_raw_buffer_load_b16(c.r16, 2 * q[u], 0, 0);
    }
    double xv[U];
    int racc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int r, col;
        decode_meta<MetaT>(mt[u], r, col);
        racc[u] = d[u].y + 8 * r;
        const u32x2 xb = __builtin_amdgcn_raw_buffer_load_b64(c.rx, d[u].x + 8 * col, 0, 0);
        xv[u] = __longlong_as_double(((long long)xb.y << 32) | xb.x);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        double v;
        if (wp[u] == 0)
            v = __longlong_as_double(((long long)raw[u].y << 32) | raw[u].x);
        else if (wp[u] == 1)
            v = (double)__uint_as_float(raw[u].x);
        else
            v = (double)__uint_as_float(raw[u].x << 16);
        // Sentinel lanes have storage positions past the batch: nothing to add.
        if (q[u] < c.len) atomicAdd(reinterpret_cast<double*>(c.acc + racc[u]), v * xv[u]);
    }
}

// The outputs are separate restrict arguments: the compiler may then treat
// every other array as read-only for the whole launch.
template <typename MetaT, int MODE, int MAXROWS>
__global__ __launch_bounds__(kSpmvBlock) void spmv_tilecsc_kernel(SpmvArgs a, double* __restrict__ y,
                                                                  double* __restrict__ partials) {
    // One spare accumulator per wave: the sentinel entry's row (never added to).
    __shared__ double s_acc[kSpmvWaves][MAXROWS + 1];
    __shared__ int4 s_desc[kSpmvWaves][kDescSlots];
    __shared__ double s_tmp[kSpmvWaves];

    if (MODE == kSpmvCg && load_done(a.st)) return;

    const int lane = threadIdx.x & (kWave - 1);
    // The wavefront index is uniform across the wave; saying so keeps every
    // per-group and per-window quantity in scalar registers and scalar loads.
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int blk = xcd_contiguous_block(blockIdx.x, gridDim.x);
    const int g_begin = blk * a.groups_per_block;
    const int g_end = min(g_begin + a.groups_per_block, a.ngroups);
    SweepCtx c;
    c.uprec = *a.uprec;
    c.lane = lane;
    c.win_mask = a.win_mask;
    c.win_tile = a.win_tile;
    c.desc = &s_desc[w][0];
    c.acc = reinterpret_cast<char*>(&s_acc[w][0]);
    // x through a buffer resource with 32-bit byte offsets (n < 2^28 is
    // checked when the handle is created).
    c.rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<double*>(a.x), (short)0, a.n * 8, (int)kBufferConfig);
    double dot = 0.0;

    for (int g = g_begin + w; g < g_end; g += kSpmvWaves) {
        const int rb0 = g * a.G;
        const int nrbg = min(rb0 + a.G, a.nrb) - rb0;
        const int row0 = rb0 * a.R;
        const int nrows = min(a.rows_per_group, a.n - row0);
        for (int i = lane; i < a.rows_per_group; i += kWave) s_acc[w][i] = 0.0;
        const int t_begin = uniform_load(a.trp, rb0);
        const int t_end = uniform_load(a.trp, rb0 + nrbg);
        double p_own = 0.0;
        if (MODE == kSpmvCg && MAXROWS <= kWave && lane < nrows) p_own = a.x[row0 + lane];
        int win = uniform_load(a.win_base, g);
        for (int tb = t_begin; tb < t_end; tb += kTileBatch) {
            const int nt = min(kTileBatch, t_end - tb);
            const int kb = uniform_load(a.tptr, tb);
            const int len = uniform_load(a.tptr, tb + nt) - kb;
            // Every entry starts as the sentinel; tile entries then go to their
            // slot (plan position + precision: one sentinel after each group).
            const int4 sentinel = make_int4(kSentinelColumn, MAXROWS * 8, kSentinelShift, 0);
            s_desc[w][lane] = sentinel;
            if (lane < kDescSlots - kWave) s_desc[w][kWave + lane] = sentinel;
            if (lane < nt) {
                const int4 e = a.plan[tb + lane];
                s_desc[w][lane + e.w] = e;
            }
            c.r64 = batch_rsrc(a.v64, kb, 8, len);
            c.r32 = batch_rsrc(a.v32, kb, 4, len);
            c.r16 = batch_rsrc(a.v16, kb, 2, len);
            c.rmt = batch_rsrc(a.meta, kb, (int)sizeof(MetaT), len);
            c.len = len;
            const int w0 = win;
            win += batch_records(len);
            int left = sweep_windows(uniform_load(a.win_tile, w0) >> kRecCountShift);
            wave_lds_sync();
            int wi = w0, o0 = 0;
            for (; left >= kUnroll; left -= kUnroll, wi += kUnroll, o0 += kUnroll * kWave)
                spmv_sweep<MetaT, kUnroll>(c, wi, o0);
            // The rest is 0 or one power of two below kUnroll.
            if (kUnroll > 8 && left == 8) spmv_sweep<MetaT, (kUnroll > 8 ? 8 : 1)>(c, wi, o0);
            if (kUnroll > 4 && left == 4) spmv_sweep<MetaT, (kUnroll > 4 ? 4 : 1)>(c, wi, o0);
            if (kUnroll > 2 && left == 2) spmv_sweep<MetaT, (kUnroll > 2 ? 2 : 1)>(c, wi, o0);
            if (kUnroll > 1 && left == 1) spmv_sweep<MetaT, 1>(c, wi, o0);
            wave_lds_sync();
        }
        for (int i = lane; i < nrows; i += kWave) {
            const double acc = s_acc[w][i];
            if (MODE == kSpmvPlain) {
                y[row0 + i] = acc;
            } else if (MODE == kSpmvCg) {
                y[row0 + i] = acc;
                dot += (MAXROWS <= kWave ? p_own : a.x[row0 + i]) * acc;
            } else {
                y[row0 + i] = a.b[row0 + i] - acc;
            }
        }
        wave_lds_sync();
    }

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
    }
}

// ---------------------------------------------------------------------------
// SpMV plan for the active map (one wavefront per row group, same batches as
// the SpMV). Lane l holds tile tb+l. A tile's plan position is its rank in
// (precision, storage order), found with one ballot per precision; prefix
// sums of the tile lengths in plan order, with each precision group rounded
// up to whole windows, give every entry's first sweep position. Lane v then
// writes the records of windows v, v+64, ...; records past the batch's
// windows (the rest of the last sweep) point at a sentinel.
// uniform = 1 plans every tile as FP64 (storage order, no gaps): used while a
// uniform precision overrides the map.
// ---------------------------------------------------------------------------
struct PlanArgs {
    const int32_t* trp;
    const int32_t* tptr;
    const int32_t* tcol;
    const uint8_t* trow;  // [T] row block of every tile inside its row group
    const uint8_t* map;
    const int32_t* win_base;
    int4* plan;
    uint64_t* win_mask;
    int32_t* win_tile;
    const State* st;
    int32_t solve;    // 1: run only at the start of a tile-rule window of a running solve
    int32_t uniform;  // 1: ignore the map
    int32_t nrb, R, C, G, ngroups;
};

__device__ inline int wave_prefix_incl(int v, int lane) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int t = __shfl_up(v, off, kWave);
        if (lane >= off) v += t;
    }
    return v;
}

__global__ __launch_bounds__(kBlock) void spmv_plan_kernel(PlanArgs a) {
    __shared__ int s_len[kWavesPerBlock][kTileBatch];
    __shared__ int s_tile[kWavesPerBlock][kTileBatch];
    __shared__ int s_start[kWavesPerBlock][kTileBatch];
    if (a.solve) {
        if (load_done(a.st)) return;
        if (a.st->k % a.st->period != 0) return;
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    auto rank_in = [&](uint64_t m) {
        return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    };
    for (int g = blockIdx.x * kWavesPerBlock + w; g < a.ngroups; g += gridDim.x * kWavesPerBlock) {
        const int rb0 = g * a.G;
        const int t_begin = a.trp[rb0];
        const int t_end = a.trp[min(rb0 + a.G, a.nrb)];
        int wb = a.win_base[g];
        for (int tb = t_begin; tb < t_end; tb += kTileBatch) {
            const int nt = min(kTileBatch, t_end - tb);
            const int kb = a.tptr[tb];
            const int len = a.tptr[tb + nt] - kb;
            const bool valid = lane < nt;
            // Every map writer stores 0..2; the clamp only keeps the plan a permutation.
            const int p = !valid ? -1 : a.uniform ? 0 : min((int)a.map[tb + lane], 2);
            const int tlen = valid ? a.tptr[tb + lane + 1] - a.tptr[tb + lane] : 0;
            const uint64_t b0 = __ballot(p == 0), b1 = __ballot(p == 1), b2 = __ballot(p == 2);
            const int n0 = __popcll(b0), n1 = __popcll(b1), n2 = __popcll(b2);
            // Nonzeros of each precision group and the sweep position where it starts.
            const int l0 = wave_sum_int(p == 0 ? tlen : 0), l1 = wave_sum_int(p == 1 ? tlen : 0);
            const int l2 = len - l0 - l1;
            const int P1 = (l0 + kWave - 1) / kWave * kWave;
            const int P2 = P1 + (l1 + kWave - 1) / kWave * kWave;
            const int nw = (P2 + l2 + kWave - 1) / kWave;
            if (valid) {
                const int slot = p == 0 ? rank_in(b0) : p == 1 ? n0 + rank_in(b1) : n0 + n1 + rank_in(b2);
                s_len[w][slot] = tlen;
                s_tile[w][slot] = lane;
            }
            wave_lds_sync();
            // Entry q (plan order) of precision c = (q >= n0) + (q >= n0 + n1).
            const int ql = valid ? s_len[w][lane] : 0;
            const int qc = (lane >= n0) + (lane >= n0 + n1);
            const int incl = wave_prefix_incl(ql, lane);
            const int before = qc == 0 ? 0 : qc == 1 ? l0 : l0 + l1;  // nonzeros of earlier groups
            const int gstart = qc == 0 ? 0 : qc == 1 ? P1 : P2;       // sweep position of the group
            const int first = gstart + (incl - ql - before);
            if (valid) {
                const int t = tb + s_tile[w][lane];
                a.plan[tb + lane] = make_int4(a.tcol[t] * a.C * 8, (int)a.trow[t] * a.R * 8,
                                              (a.tptr[t] - kb) - first, qc);
                s_start[w][lane] = first;
            }
            wave_lds_sync();
            const int E = sweep_windows(nw);
            for (int v = lane; v < E; v += kWave) {
                uint64_t m = 0;
                int rec = nt + 2;  // padding record: the sentinel after the last group, FP64
                if (v < nw) {
                    const int w0 = v * kWave;
                    const int c = w0 >= P2 ? 2 : (w0 >= P1 ? 1 : 0);
                    const int lo_q = c == 0 ? 0 : c == 1 ? n0 : n0 + n1;  // entries of group c
                    const int hi_q = lo_q + (c == 0 ? n0 : c == 1 ? n1 : n2) - 1;
                    const int gend = (c == 0 ? 0 : c == 1 ? P1 : P2) + (c == 0 ? l0 : c == 1 ? l1 : l2);
                    int lo_s = lo_q, hi_s = hi_q;  // last entry of the group starting at or before w0
                    while (lo_s < hi_s) {
                        const int mid = (lo_s + hi_s + 1) >> 1;
                        if (s_start[w][mid] <= w0) lo_s = mid; else hi_s = mid - 1;
                    }
                    for (int jj = lo_s + 1; jj <= hi_q && s_start[w][jj] < w0 + kWave; ++jj)
                        m |= 1ull << (s_start[w][jj] - w0 - 1);
                    if (gend < w0 + kWave) m |= 1ull << (gend - w0 - 1);  // the group's sentinel
                    rec = (lo_s + c) | (c << kRecPrecShift);
                }
                a.win_mask[wb + v] = m;
                a.win_tile[wb + v] = rec | (nw << kRecCountShift);
            }
            wb += batch_records(len);
            wave_lds_sync();
        }
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
    const double* q;
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
};

__device__ inline void trace_uniform(State* st, int32_t* trace_k, int32_t* trace_counts, int k,
                                     int prec, int64_t T) {
    const int i = st->ntrace;
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
    int s = st->stage;
    while (s < st->nstage - 1 && rho <= st->thresholds[s]) ++s;
    if (s != st->stage || first) {
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
        const double rho0 = st->norm0 > 0.0 ? 1.0 : 0.0;
        a.hist[0] = rho0;
        if (st->nstage > 0) advance_stage(st, a.trace_k, a.trace_counts, 0, rho0, a.T, true);
        int done = 0;
        if (st->norm0 == 0.0 || rho0 <= st->tol) done = 1;
        else if (st->maxit <= 0) done = 2;
        store_done(st, done);
    }
}

// alpha = r.z / p.q (p.q summed from the SpMV partials in every block);
// x += alpha p; r -= alpha q; [z = dinv .* r]; partials of r.r [and r.z].
// On p.q <= 0 or a non-finite alpha nothing is updated and the breakdown is
// flagged for the direction kernel.
__global__ __launch_bounds__(kBlock) void cg_update_kernel(VecArgs a) {
    __shared__ double s_tmp[kWavesPerBlock];
    State* st = a.st;
    if (load_done(st)) return;
    double tot[1];
    sum_partials<1>(a.part_in, a.nparts_in, tot, s_tmp);
    const double pq = tot[0];
    const double alpha = st->rz / pq;
    const bool bd = !(pq > 0.0) || !isfinite(pq) || !isfinite(alpha);
    double rr = 0.0, rz = 0.0;
    if (!bd) {
        for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < a.n; i += gridDim.x * blockDim.x) {
            a.x[i] += alpha * a.p[i];
            const double ri = a.r[i] - alpha * a.q[i];
            a.r[i] = ri;
            rr += ri * ri;
            if (a.jacobi) {
                const double zi = a.dinv[i] * ri;
                a.z[i] = zi;
                rz += ri * zi;
            }
        }
    }
    const double prr = block_sum(rr, s_tmp);
    const double prz = a.jacobi ? block_sum(rz, s_tmp) : prr;
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

// beta = (r.z)_new / (r.z)_old from the update partials (in every block);
// p = z + beta p (z = r for plain CG). Thread 0 of block 0 commits
// rho_{k+1}, the history entry, the stop flag and the schedule stage.
// Other blocks may read `done` before or after that commit within the final
// iteration; either way the direction update they skip or make is unused.
__global__ __launch_bounds__(kBlock) void cg_direction_kernel(VecArgs a) {
    __shared__ double s_tmp[kWavesPerBlock];
    State* st = a.st;
    if (load_done(st)) return;
    if (st->bd) {
        if (blockIdx.x == 0 && threadIdx.x == 0) store_done(st, 3);
        return;
    }
    double tot[2];
    sum_partials<2>(a.part_in, a.nparts_in, tot, s_tmp);
    const double rr_new = tot[0];
    const double rz_new = tot[1];
    const double beta = rz_new / st->rz_prev;
    const double* z = a.jacobi ? a.z : a.r;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < a.n; i += gridDim.x * blockDim.x)
        a.p[i] = z[i] + beta * a.p[i];
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
    int64_t T;
    double rho;     // explicit rho (eval mode)
    int32_t solve;  // 1: in-solve window step (reads k and rho_k from the state)
};

__device__ inline void block_counts_out(unsigned c0, unsigned c1, unsigned c2, int32_t* out) {
    __shared__ unsigned s_cnt[3];
    if (threadIdx.x < 3) s_cnt[threadIdx.x] = 0;
    __syncthreads();
    atomicAdd(&s_cnt[0], c0);  // LDS atomics
    atomicAdd(&s_cnt[1], c1);
    atomicAdd(&s_cnt[2], c2);
    __syncthreads();
    if (threadIdx.x < 3) out[threadIdx.x] = (int32_t)s_cnt[threadIdx.x];
}

// Windowed tile rule: at k % period == 0 every tile's precision is re-selected
// from its score and rho_k, and the window's precision counts are recorded.
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
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < a.T;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int code = tile_rule_code(a.scores[t], rho, st->hi, st->lo);
        a.map[t] = (uint8_t)code;
        c0 += code == 0;
        c1 += code == 1;
        c2 += code == 2;
    }
    if (slot >= 0) {
        block_counts_out(c0, c1, c2, a.trace_counts + ((size_t)slot * kTraceBlocks + blockIdx.x) * 3);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            a.trace_k[slot] = st->k;
            st->ntrace = slot + 1;
        }
    }
}

// Precision counts of the active map into trace entry 0 (static maps).
__global__ __launch_bounds__(kBlock) void map_count_kernel(const uint8_t* map, int64_t T,
                                                           int32_t* trace_k, int32_t* counts) {
    unsigned c[3] = {0, 0, 0};
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < T;
         t += (int64_t)gridDim.x * blockDim.x)
        c[map[t] < 3 ? map[t] : 0]++;
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
__global__ __launch_bounds__(kBlock) void diag_absmax_kernel(const int32_t* trp, const int32_t* tcol,
                                                             const int32_t* tptr, const void* meta,
                                                             int meta16, const double* v64,
                                                             int32_t nrb, int32_t T, int32_t R,
                                                             int32_t C, unsigned long long* out) {
    for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < T; t += gridDim.x * blockDim.x) {
        int lo = 0, hi = nrb;  // row block of tile t: last I with trp[I] <= t
        while (hi - lo > 1) {
            const int mid = (lo + hi) / 2;
            if (trp[mid] <= t) lo = mid; else hi = mid;
        }
        const int64_t row_base = (int64_t)lo * R, col_base = (int64_t)tcol[t] * C;
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
// t16, FP32 below t32, else FP64.
__global__ __launch_bounds__(kBlock) void magnitude_map_kernel(const int32_t* tptr, const double* v64,
                                                               int32_t T,
                                                               const unsigned long long* dmax_bits,
                                                               double t16, double t32, uint8_t* map) {
    const double dmax = __longlong_as_double((long long)*dmax_bits);
    for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < T; t += gridDim.x * blockDim.x) {
        double m = 0.0;
        for (int k = tptr[t]; k < tptr[t + 1]; ++k) m = fmax(m, fabs(v64[k]));
        const double ratio = m / dmax;
        map[t] = ratio < t16 ? 2 : (ratio < t32 ? 1 : 0);
    }
}

}  // namespace dev
}  // namespace mpcg
