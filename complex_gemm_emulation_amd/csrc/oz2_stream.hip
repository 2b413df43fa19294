// oz2_stream.hip -- HBM stream kernels of known size: the bandwidth ceilings
// against which the memory-bound phases (scan reads, encode and reconstruct
// read and write) are judged.  A measurement aid, not part of the method.
//
// Three kinds over a buffer of n 16-byte words: read (every word loaded
// once, folded into one word per thread so the loads cannot be dropped),
// write (every word stored once with a value that depends on its index, so
// the data is not a constant pattern) and copy (load, store).  Each thread
// handles `unroll` words per trip, their loads issued before any use, in a
// grid-stride loop; plain or nontemporal accesses.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "oz2_stream.h"

namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

template <int U, bool NT>
__global__ __launch_bounds__(256) void read_kernel(const u4* __restrict__ src, int64_t n, u4* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    u4 acc = {0u, 0u, 0u, 0u};
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        u4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    for (; i < n; i += stride) acc ^= src[i];
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__device__ __forceinline__ u4 pattern(int64_t i) {
    const uint32_t x = (uint32_t)i * 2654435761u;
    return u4{x, x ^ 0x9e3779b9u, x + 0x7f4a7c15u, ~x};
}

template <int U, bool NT>
__global__ __launch_bounds__(256) void write_kernel(u4* __restrict__ dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < n; i += U * stride) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const u4 v = pattern(i + u * stride);
            if (NT)
                __builtin_nontemporal_store(v, dst + i + u * stride);
            else
                dst[i + u * stride] = v;
        }
    }
    for (; i < n; i += stride) dst[i] = pattern(i);
}

template <int U, bool NT>
__global__ __launch_bounds__(256) void copy_kernel(const u4* __restrict__ src, u4* __restrict__ dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        u4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (NT)
                __builtin_nontemporal_store(v[u], dst + i + u * stride);
            else
                dst[i + u * stride] = v[u];
        }
    }
    for (; i < n; i += stride) dst[i] = src[i];
}

template <int U, bool NT>
hipError_t go(int kind, const void* src, void* dst, int64_t n, int blocks, hipStream_t st) {
    const dim3 grid((unsigned)blocks), block(256);
    if (kind == OZ2_STREAM_READ)
        hipLaunchKernelGGL((read_kernel<U, NT>), grid, block, 0, st, (const u4*)src, n, (u4*)dst);
    else if (kind == OZ2_STREAM_WRITE)
        hipLaunchKernelGGL((write_kernel<U, NT>), grid, block, 0, st, (u4*)dst, n);
    else
        hipLaunchKernelGGL((copy_kernel<U, NT>), grid, block, 0, st, (const u4*)src, (u4*)dst, n);
    return hipGetLastError();
}

}  // namespace

extern "C" int oz2_stream_run(int kind, const void* src, void* dst, int64_t bytes, int blocks, int unroll,
                              int nontemporal, void* stream) {
    if (kind < OZ2_STREAM_READ || kind > OZ2_STREAM_COPY) return -1;
    if (kind != OZ2_STREAM_WRITE && !src) return -2;
    if (!dst) return -3;
    if (bytes <= 0 || bytes % 16) return -4;
    if (blocks < 1) return -5;
    if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return -6;
    const int64_t n = bytes / 16;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    const bool nt = nontemporal != 0;
    switch (unroll) {
        case 1: e = nt ? go<1, true>(kind, src, dst, n, blocks, st) : go<1, false>(kind, src, dst, n, blocks, st); break;
        case 2: e = nt ? go<2, true>(kind, src, dst, n, blocks, st) : go<2, false>(kind, src, dst, n, blocks, st); break;
        case 4: e = nt ? go<4, true>(kind, src, dst, n, blocks, st) : go<4, false>(kind, src, dst, n, blocks, st); break;
        default: e = nt ? go<8, true>(kind, src, dst, n, blocks, st) : go<8, false>(kind, src, dst, n, blocks, st); break;
    }
    return e == hipSuccess ? 0 : 2;
}
