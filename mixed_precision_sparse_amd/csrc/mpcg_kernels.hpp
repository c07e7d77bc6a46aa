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
constexpr int kMaxGroupRB = 65;  // row blocks per wavefront + 1 (R = 1 gives 64)

// Solver scalars, resident on the device for the whole solve.
struct State {
    double rz;        // r.z of the current iterate (r.r for plain CG)
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
    uint32_t ticket[4];  // arrival counters of the single-pass reductions
};

enum TicketSlot { kTicketSpmv = 0, kTicketUpdate = 1, kTicketInit = 2, kTicketMisc = 3 };

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

// Publishes this block's partials and returns true in every thread of the
// block that arrives last. The last block then reads all partials.
template <int NV>
__device__ inline bool arrive_last(const double (&vals)[NV], double* partials, uint32_t* ticket,
                                   bool* s_flag) {
    if (threadIdx.x == 0) {
#pragma unroll
        for (int j = 0; j < NV; ++j) partials[(size_t)blockIdx.x * NV + j] = vals[j];
        __threadfence();
        uint32_t t = atomicAdd(ticket, 1u);
        *s_flag = (t == gridDim.x - 1);
    }
    __syncthreads();
    bool last = *s_flag;
    if (last) __threadfence();
    return last;
}

// Fixed-order sum of the partials of all blocks (called by the last block).
template <int NV>
__device__ inline void reduce_partials(const double* partials, int nblocks, double (&out)[NV],
                                       double* s_tmp) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        double a = 0.0;
        for (int i = threadIdx.x; i < nblocks; i += blockDim.x)
            a += partials[(size_t)i * NV + j];
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
// One wavefront owns a row group: G consecutive row blocks (G*R <= 64 rows,
// or one row block when R > 64). It walks the group's tiles in batches of up
// to 64: lane j stages tile j's descriptor (first nonzero, column base,
// precision, row offset inside the group) in LDS; then the 64 lanes sweep the
// batch's nonzeros 64 at a time in storage order, so every value plane is
// read with contiguous, coalesced loads and only from the plane the tile's
// map entry selects. A lane finds its tile from the tile starts that fall in
// the current 64-nonzero window (ballot + prefix popcount). The product of
// the widened stored value and the FP64 vector entry is accumulated in FP64
// into the group's row accumulators in LDS; the group's rows are written once.
// ---------------------------------------------------------------------------
enum SpmvMode { kSpmvPlain = 0, kSpmvCg = 1, kSpmvResidual = 2 };

struct SpmvArgs {
    const int32_t* trp;   // tile_row_ptr [nrb+1]
    const int32_t* tcol;  // tile_col_idx [T]
    const int32_t* tptr;  // tile_nnz_ptr [T+1]
    const uint8_t* map;   // [T]
    const void* meta;     // per nonzero (row, col) packed: u8 (R, C <= 16) or u16
    const double* v64;
    const float* v32;
    const uint16_t* v16;
    const double* x;
    double* y;
    const double* b;       // residual mode: y = b - A x
    const int32_t* uprec;  // -1 per-tile map, else uniform code
    State* st;
    double* partials;
    int32_t n, nrb, R, C, G, rows_per_group, ngroups;
};

template <typename MetaT>
__device__ inline void decode_meta(MetaT m, int& r, int& c);
template <>
__device__ inline void decode_meta<uint8_t>(uint8_t m, int& r, int& c) {
    r = m >> 4;
    c = m & 15;
}
template <>
__device__ inline void decode_meta<uint16_t>(uint16_t m, int& r, int& c) {
    r = m >> 8;
    c = m & 255;
}

__device__ inline double load_stored_value(const SpmvArgs& a, int prec, int k) {
    if (prec == 0) return __builtin_nontemporal_load(&a.v64[k]);
    if (prec == 1) return (double)__builtin_nontemporal_load(&a.v32[k]);
    uint32_t h = __builtin_nontemporal_load(&a.v16[k]);
    return (double)__uint_as_float(h << 16);
}

template <typename MetaT, int MODE>
__global__ __launch_bounds__(kBlock) void spmv_tilecsc_kernel(SpmvArgs a) {
    __shared__ double s_acc[kWavesPerBlock][kMaxRows];
    __shared__ int32_t s_cbase[kWavesPerBlock][kTileBatch];
    __shared__ int32_t s_pr[kWavesPerBlock][kTileBatch];
    __shared__ int32_t s_trp[kWavesPerBlock][kMaxGroupRB];
    __shared__ uint8_t s_flag[kWavesPerBlock][kWave];
    __shared__ double s_tmp[kWavesPerBlock];
    __shared__ bool s_last;

    if (MODE == kSpmvCg && a.st->done) return;

    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int blk = xcd_contiguous_block(blockIdx.x, gridDim.x);
    const int g = blk * kWavesPerBlock + w;
    const MetaT* meta = static_cast<const MetaT*>(a.meta);
    double dot = 0.0;

    if (g < a.ngroups) {
        const int rb0 = g * a.G;
        const int rb1 = min(rb0 + a.G, a.nrb);
        const int nrbg = rb1 - rb0;
        const int row0 = rb0 * a.R;
        const int nrows = min(a.rows_per_group, a.n - row0);
        for (int i = lane; i < a.rows_per_group; i += kWave) s_acc[w][i] = 0.0;
        for (int i = lane; i <= nrbg; i += kWave) s_trp[w][i] = a.trp[rb0 + i];
        const int uprec = *a.uprec;
        wave_lds_sync();
        const int t_begin = s_trp[w][0];
        const int t_end = s_trp[w][nrbg];
        for (int tb = t_begin; tb < t_end; tb += kTileBatch) {
            const int nt = min(kTileBatch, t_end - tb);
            int my_start = 0x7fffffff;
            if (lane < nt) {
                const int t = tb + lane;
                my_start = a.tptr[t];
                int rbi = 0;
                while (rbi + 1 < nrbg && s_trp[w][rbi + 1] <= t) ++rbi;
                const int prec = uprec >= 0 ? uprec : (int)a.map[t];
                s_cbase[w][lane] = a.tcol[t] * a.C;
                s_pr[w][lane] = prec | ((rbi * a.R) << 2);
            }
            const int kb = __shfl(my_start, 0, kWave);
            const int ke = a.tptr[tb + nt];
            int jprev = -1;
            for (int k0 = kb; k0 < ke; k0 += kWave) {
                s_flag[w][lane] = 0;
                wave_lds_sync();
                const int pos = my_start - k0;
                if (pos >= 0 && pos < kWave) s_flag[w][pos] = 1;
                wave_lds_sync();
                const int f = s_flag[w][lane];
                const uint64_t mask = __ballot(f);
                const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
                const int j = jprev + below + f;
                jprev += __popcll(mask);
                const int k = k0 + lane;
                if (k < ke) {
                    int r, c;
                    decode_meta<MetaT>(__builtin_nontemporal_load(&meta[k]), r, c);
                    const int pr = s_pr[w][j];
                    const int cb = s_cbase[w][j];
                    const double v = load_stored_value(a, pr & 3, k);
                    const double xv = a.x[cb + c];
                    atomicAdd(&s_acc[w][(pr >> 2) + r], v * xv);
                }
            }
        }
        wave_lds_sync();
        for (int i = lane; i < nrows; i += kWave) {
            const double acc = s_acc[w][i];
            if (MODE == kSpmvPlain) {
                a.y[row0 + i] = acc;
            } else if (MODE == kSpmvCg) {
                a.y[row0 + i] = acc;
                dot += a.x[row0 + i] * acc;
            } else {
                a.y[row0 + i] = a.b[row0 + i] - acc;
            }
        }
    }

    if (MODE == kSpmvCg) {
        double part[1] = {block_sum(dot, s_tmp)};
        if (arrive_last<1>(part, a.partials, &a.st->ticket[kTicketSpmv], &s_last)) {
            double tot[1];
            reduce_partials<1>(a.partials, gridDim.x, tot, s_tmp);
            if (threadIdx.x == 0) {
                State* st = a.st;
                const double pq = tot[0];
                const double alpha = st->rz / pq;
                st->pq = pq;
                st->alpha = alpha;
                if (!(pq > 0.0) || !isfinite(pq) || !isfinite(alpha)) st->done = 3;
                st->ticket[kTicketSpmv] = 0;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// CG vector kernels. Grid-stride loops; every block publishes one partial per
// reduced quantity and the last block to arrive finishes the reduction in a
// fixed order, computes the scalars and updates the solver state.
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
    double* partials;
    int32_t* trace_k;
    int64_t* trace_counts;
    int64_t T;
    int32_t n;
    int32_t jacobi;
    int32_t r_ready;      // init: r already holds b - A x0
};

__device__ inline void trace_uniform(State* st, int32_t* trace_k, int64_t* trace_counts, int k,
                                     int prec, int64_t T) {
    const int i = st->ntrace;
    if (i < st->trace_cap) {
        trace_k[i] = k;
        for (int p = 0; p < 3; ++p) trace_counts[3 * i + p] = (p == prec) ? T : 0;
    }
    st->ntrace = i + 1;
}

// Advances the one-way residual schedule for the residual rho of iteration k.
__device__ inline void advance_stage(State* st, int32_t* trace_k, int64_t* trace_counts, int k,
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

// Initial state: x = x0 (or 0), r = b - A x0 (computed beforehand when x0 is
// given), z = dinv .* r, p = z, then ||r0||, r.z and the stop decision at k = 0.
__global__ __launch_bounds__(kBlock) void cg_init_kernel(VecArgs a) {
    __shared__ double s_tmp[kWavesPerBlock];
    __shared__ bool s_last;
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
    double part[2] = {block_sum(rr, s_tmp), block_sum(rz, s_tmp)};
    if (arrive_last<2>(part, a.partials, &a.st->ticket[kTicketInit], &s_last)) {
        double tot[2];
        reduce_partials<2>(a.partials, gridDim.x, tot, s_tmp);
        if (threadIdx.x == 0) {
            State* st = a.st;
            st->rr = tot[0];
            st->rz = a.jacobi ? tot[1] : tot[0];
            st->norm0 = sqrt(tot[0]);
            st->k = 0;
            st->ntrace = 0;
            st->stage = 0;
            st->alpha = 0.0;
            st->beta = 0.0;
            const double rho0 = st->norm0 > 0.0 ? 1.0 : 0.0;
            a.hist[0] = rho0;
            if (st->nstage > 0) advance_stage(st, a.trace_k, a.trace_counts, 0, rho0, a.T, true);
            if (st->norm0 == 0.0 || rho0 <= st->tol) st->done = 1;
            else if (st->maxit <= 0) st->done = 2;
            else st->done = 0;
            st->ticket[kTicketInit] = 0;
        }
    }
}

// x += alpha p; r -= alpha q; [z = dinv .* r]; partials of r.r [and r.z];
// the last block forms beta, rho_{k+1}, the history entry and the stop flag.
__global__ __launch_bounds__(kBlock) void cg_update_kernel(VecArgs a) {
    __shared__ double s_tmp[kWavesPerBlock];
    __shared__ bool s_last;
    State* st = a.st;
    if (st->done) return;
    const double alpha = st->alpha;
    double rr = 0.0, rz = 0.0;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < a.n; i += gridDim.x * blockDim.x) {
        const double pi = a.p[i];
        a.x[i] += alpha * pi;
        const double ri = a.r[i] - alpha * a.q[i];
        a.r[i] = ri;
        rr += ri * ri;
        if (a.jacobi) {
            const double zi = a.dinv[i] * ri;
            a.z[i] = zi;
            rz += ri * zi;
        }
    }
    double part[2] = {block_sum(rr, s_tmp), a.jacobi ? block_sum(rz, s_tmp) : 0.0};
    if (arrive_last<2>(part, a.partials, &st->ticket[kTicketUpdate], &s_last)) {
        double tot[2];
        reduce_partials<2>(a.partials, gridDim.x, tot, s_tmp);
        if (threadIdx.x == 0) {
            const double rr_new = tot[0];
            const double rz_new = a.jacobi ? tot[1] : rr_new;
            const double beta = rz_new / st->rz;
            const int k = st->k + 1;
            const double rho = sqrt(rr_new) / st->norm0;
            a.hist[k] = rho;
            st->k = k;
            st->rr = rr_new;
            st->rz = rz_new;
            st->beta = beta;
            if (!isfinite(beta) || !isfinite(rho)) st->done = 3;
            else if (rho <= st->tol) st->done = 1;
            else if (k >= st->maxit) st->done = 2;
            else if (st->nstage > 0) advance_stage(st, a.trace_k, a.trace_counts, k, rho, a.T, false);
            st->ticket[kTicketUpdate] = 0;
        }
    }
}

// p = z + beta p (z = r for plain CG).
__global__ __launch_bounds__(kBlock) void cg_direction_kernel(VecArgs a) {
    const State* st = a.st;
    if (st->done) return;
    const double beta = st->beta;
    const double* z = a.jacobi ? a.z : a.r;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < a.n; i += gridDim.x * blockDim.x)
        a.p[i] = z[i] + beta * a.p[i];
}

// ---------------------------------------------------------------------------
// Map kernels.
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
    int64_t* trace_counts;
    int64_t T;
    double rho;     // explicit rho (eval mode)
    int32_t solve;  // 1: in-solve window step (reads k and rho_k from the state)
};

// Windowed tile rule: at k % period == 0 every tile's precision is re-selected
// from its score and rho_k, and the window's precision counts are recorded.
__global__ __launch_bounds__(kBlock) void tile_rule_kernel(MapArgs a) {
    __shared__ unsigned long long s_cnt[3];
    State* st = a.st;
    double rho = a.rho;
    int slot = -1;
    if (a.solve) {
        if (st->done) return;
        const int k = st->k;
        if (k % st->period != 0) return;
        rho = a.hist[k];
        slot = k / st->period;
        if (slot >= st->trace_cap) slot = -1;
    }
    if (threadIdx.x < 3) s_cnt[threadIdx.x] = 0;
    __syncthreads();
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
        atomicAdd(&s_cnt[0], (unsigned long long)c0);
        atomicAdd(&s_cnt[1], (unsigned long long)c1);
        atomicAdd(&s_cnt[2], (unsigned long long)c2);
        __syncthreads();
        if (threadIdx.x < 3)
            atomicAdd((unsigned long long*)&a.trace_counts[3 * slot + threadIdx.x], s_cnt[threadIdx.x]);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            a.trace_k[slot] = st->k;
            st->ntrace = slot + 1;
        }
    }
}

// Precision counts of the active map into trace entry 0 (static maps).
__global__ __launch_bounds__(kBlock) void map_count_kernel(const uint8_t* map, int64_t T,
                                                           int64_t* counts) {
    __shared__ unsigned long long s_cnt[3];
    if (threadIdx.x < 3) s_cnt[threadIdx.x] = 0;
    __syncthreads();
    unsigned c[3] = {0, 0, 0};
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < T;
         t += (int64_t)gridDim.x * blockDim.x)
        c[map[t] < 3 ? map[t] : 0]++;
    for (int p = 0; p < 3; ++p) atomicAdd(&s_cnt[p], (unsigned long long)c[p]);
    __syncthreads();
    if (threadIdx.x < 3) atomicAdd((unsigned long long*)&counts[threadIdx.x], s_cnt[threadIdx.x]);
}

// Fills n int64 values (device-side clear that is safe inside captured graphs).
__global__ void fill_i64_kernel(int64_t* p, int64_t v, int64_t n) {
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
