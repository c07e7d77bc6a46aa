// Bandwidth references for the benchmark: a read-only stream and a copy over
// device buffers, so that the SpMV's bytes per second can be set against what
// the memory system delivers on the same GPU in the same run. 16-byte loads
// per lane, several in flight per thread, grid-stride over the buffer.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mpcg_internal.hpp"

using mpcg::fail;

namespace {

constexpr int kStreamBlock = 256;
constexpr int kStreamUnroll = 4;

// Sums every double of src (n2 pairs) and writes the block sums to sink[block]
// (the loads cannot be dropped). Non-temporal loads: each byte is read once.
__global__ __launch_bounds__(kStreamBlock) void stream_read_kernel(const double2* __restrict__ src, int64_t n2,
                                                                  double* __restrict__ sink) {
    typedef double d2v __attribute__((ext_vector_type(2)));
    const int64_t stride = (int64_t)gridDim.x * kStreamBlock;
    int64_t i = (int64_t)blockIdx.x * kStreamBlock + threadIdx.x;
    double s = 0.0;
    for (; i + (kStreamUnroll - 1) * stride < n2; i += kStreamUnroll * stride) {
        d2v v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u)
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const d2v*>(src + i + u * stride));
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) s += v[u].x + v[u].y;
    }
    for (; i < n2; i += stride) s += src[i].x + src[i].y;
    __shared__ double part[kStreamBlock / 64];
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

__global__ __launch_bounds__(kStreamBlock) void stream_copy_kernel(const double2* __restrict__ src,
                                                                  double2* __restrict__ dst, int64_t n2) {
    const int64_t stride = (int64_t)gridDim.x * kStreamBlock;
    int64_t i = (int64_t)blockIdx.x * kStreamBlock + threadIdx.x;
    for (; i + (kStreamUnroll - 1) * stride < n2; i += kStreamUnroll * stride) {
        double2 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) dst[i + u * stride] = v[u];
    }
    for (; i < n2; i += stride) dst[i] = src[i];
}

// A read stream with a share of writes: thread t reads pairs t, t + stride,
// ... of src (non-temporal, as stream_read_kernel) and writes pairs t,
// t + stride, ... of dst, interleaved so that its writes keep pace with its
// reads (after its k-th read, floor(nw * k / nr) of its nw writes are out).
// The written values are running sums; sink[block] gets the block's sum of
// src, as from stream_read_kernel.
__global__ __launch_bounds__(kStreamBlock) void stream_mix_kernel(const double2* __restrict__ src, int64_t r2,
                                                                 double2* __restrict__ dst, int64_t w2,
                                                                 double* __restrict__ sink) {
    typedef double d2v __attribute__((ext_vector_type(2)));
    const int64_t stride = (int64_t)gridDim.x * kStreamBlock;
    const int64_t t = (int64_t)blockIdx.x * kStreamBlock + threadIdx.x;
    const int64_t nr = t < r2 ? (r2 - t + stride - 1) / stride : 0;
    const int64_t nw = t < w2 ? (w2 - t + stride - 1) / stride : 0;
    double s = 0.0;
    int64_t k = 0, kw = 0;
    for (; k + kStreamUnroll <= nr; k += kStreamUnroll) {
        d2v v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u)
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const d2v*>(src + t + (k + u) * stride));
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) s += v[u].x + v[u].y;
        const int64_t due = nw * (k + kStreamUnroll) / nr;
        for (; kw < due; ++kw) dst[t + kw * stride] = make_double2(s, s);
    }
    for (; k < nr; ++k) s += src[t + k * stride].x + src[t + k * stride].y;
    for (; kw < nw; ++kw) dst[t + kw * stride] = make_double2(s, s);
    __shared__ double part[kStreamBlock / 64];
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

}  // namespace

extern "C" int cg_stream_read(const void* src, int64_t bytes, double* sink, int32_t blocks, void* stream) {
    mpcg::clear_error();
    if (!src || !sink) return fail(CG_EINVAL, "cg_stream_read: NULL argument");
    if (bytes < 16 || (bytes & 15) || ((uintptr_t)src & 15))
        return fail(CG_EINVAL, "cg_stream_read: bytes must be a positive multiple of 16 and src 16-byte aligned");
    if (blocks < 1) return fail(CG_EINVAL, "cg_stream_read: blocks must be >= 1");
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kStreamBlock), 0, static_cast<hipStream_t>(stream),
                       static_cast<const double2*>(src), bytes / 16, sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(CG_EDEVICE, std::string("cg_stream_read: ") + hipGetErrorString(e));
    return CG_OK;
}

extern "C" int cg_stream_copy(const void* src, void* dst, int64_t bytes, int32_t blocks, void* stream) {
    mpcg::clear_error();
    if (!src || !dst) return fail(CG_EINVAL, "cg_stream_copy: NULL argument");
    if (bytes < 16 || (bytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15))
        return fail(CG_EINVAL, "cg_stream_copy: bytes must be a positive multiple of 16, pointers 16-byte aligned");
    if (blocks < 1) return fail(CG_EINVAL, "cg_stream_copy: blocks must be >= 1");
    hipLaunchKernelGGL(stream_copy_kernel, dim3(blocks), dim3(kStreamBlock), 0, static_cast<hipStream_t>(stream),
                       static_cast<const double2*>(src), static_cast<double2*>(dst), bytes / 16);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(CG_EDEVICE, std::string("cg_stream_copy: ") + hipGetErrorString(e));
    return CG_OK;
}

extern "C" int cg_stream_mix(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, double* sink,
                             int32_t blocks, void* stream) {
    mpcg::clear_error();
    if (!src || !sink || (write_bytes > 0 && !dst)) return fail(CG_EINVAL, "cg_stream_mix: NULL argument");
    if (read_bytes < 16 || (read_bytes & 15) || write_bytes < 0 || (write_bytes & 15) || ((uintptr_t)src & 15) ||
        ((uintptr_t)dst & 15))
        return fail(CG_EINVAL,
                    "cg_stream_mix: read_bytes must be a positive and write_bytes a non-negative multiple of 16, "
                    "pointers 16-byte aligned");
    if (blocks < 1) return fail(CG_EINVAL, "cg_stream_mix: blocks must be >= 1");
    hipLaunchKernelGGL(stream_mix_kernel, dim3(blocks), dim3(kStreamBlock), 0, static_cast<hipStream_t>(stream),
                       static_cast<const double2*>(src), read_bytes / 16, static_cast<double2*>(dst), write_bytes / 16,
                       sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(CG_EDEVICE, std::string("cg_stream_mix: ") + hipGetErrorString(e));
    return CG_OK;
}
