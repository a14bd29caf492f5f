// Read-only streaming kernel: the HBM read ceiling that the decode kernels
// are measured against.  It reads a buffer once with 16-byte non-temporal
// loads, eight per thread in flight per iteration, XOR-folds the words so the
// loads cannot be dropped, and writes one word per workgroup.  No part of the
// attention step uses it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "kernels.hpp"

namespace gqa {

namespace {

constexpr int SR_THREADS = 256;
constexpr int SR_UNROLL = 8;

__global__ __launch_bounds__(SR_THREADS) void stream_read_kernel(const u32x4_t* __restrict__ src, size_t n16,
                                                                 uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    const size_t step = (size_t)gridDim.x * SR_THREADS * SR_UNROLL;
    for (size_t base = (size_t)blockIdx.x * SR_THREADS * SR_UNROLL + threadIdx.x; base < n16; base += step) {
        u32x4_t v[SR_UNROLL];
#pragma unroll
        for (int k = 0; k < SR_UNROLL; ++k) {
            const size_t i = base + (size_t)k * SR_THREADS;
            v[k] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < SR_UNROLL; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    __shared__ uint32_t s_acc[SR_THREADS / 64];
    if ((threadIdx.x & 63) == 0) s_acc[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t a = 0;
        for (int k = 0; k < SR_THREADS / 64; ++k) a ^= s_acc[k];
        sink[blockIdx.x] = a;
    }
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups, hipStream_t st) {
    prof_begin(K_STREAM_READ, st);
    hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(SR_THREADS), 0, st,
                       static_cast<const u32x4_t*>(buf), bytes / 16, sink);
    prof_end(K_STREAM_READ, st);
    return hipGetLastError();
}

}  // namespace gqa
