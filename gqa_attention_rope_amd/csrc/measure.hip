// Measurement probes; no part of the attention step uses them.
//  * Read-only streaming kernel: the HBM read ceiling that the decode kernels
//    are measured against.  It reads a buffer once with 16-byte non-temporal
//    loads, eight per thread in flight per iteration, XOR-folds the words so
//    the loads cannot be dropped, and writes one word per workgroup.
//  * Matrix-rate kernel: the sustained rate of v_mfma_f32_16x16x32_bf16, the
//    prefill kernel's instruction, with every wave of the grid issuing it
//    back to back on data-dependent operands.  Under a full-chip matrix load
//    the shader clock falls below its nominal 2.4 GHz (the chip holds its
//    power limit), so this rate, not the datasheet peak, is what a
//    matrix-bound kernel can reach on the same box; the kernel also records
//    the clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "kernels.hpp"
#include "measure.hpp"

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

// Operands: random bits with the exponents of values in [-4, 4), so the
// multipliers switch as they do on real data (constant operands draw less
// power and would overstate the rate).
__device__ __forceinline__ uint32_t mr_hash(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}
__device__ __forceinline__ bf16x8_t mr_operand(uint32_t seed) {
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t h = mr_hash(seed * 4u + (uint32_t)i);
        const uint32_t lo = (h & 0x807Fu) | ((126u + ((h >> 7) & 1u) + ((h >> 8) & 1u)) << 7);
        const uint32_t hi = ((h >> 16) & 0x807Fu) | ((126u + ((h >> 23) & 1u) + ((h >> 24) & 1u)) << 7);
        v[i] = lo | (hi << 16);
    }
    return __builtin_bit_cast(bf16x8_t, v);
}

// Each wave keeps 8 A and 8 B operands in registers and issues 8 MFMAs per
// iteration onto 4 accumulator chains (two dependent MFMAs per chain and
// iteration, which the matrix pipe overlaps).  Per workgroup, sink receives
// the folded accumulators of its 4 waves (words 0..3, so no MFMA is dead) and
// wave 0's shader-clock and 100 MHz counter deltas over the loop (words 4, 5).
__global__ __launch_bounds__(MFMA_RATE_THREADS) void mfma_rate_kernel(unsigned long long* __restrict__ sink,
                                                                      int iters) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t seed = ((uint32_t)blockIdx.x * MFMA_RATE_THREADS + (uint32_t)tid) * 16u;
    bf16x8_t a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = mr_operand(seed + (uint32_t)i);
        b[i] = mr_operand(seed + 8u + (uint32_t)i);
    }
    f32x4_t c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const unsigned long long m0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < MFMA_RATE_PER_ITER; ++u)
            c[u & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[(u + 3) & 7], c[u & 3], 0, 0, 0);
    }
    const unsigned long long m1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    unsigned long long* w = sink + (size_t)blockIdx.x * MFMA_RATE_SINK_WORDS;
    if (lane == 0) w[wave] = (unsigned long long)__float_as_uint(s);
    if (tid == 0) {
        w[4] = m1 - m0;
        w[5] = r1 - r0;
        w[6] = 0;
        w[7] = 0;
    }
}

}  // namespace

hipError_t launch_mfma_rate(unsigned long long* sink, int workgroups, int iters, hipStream_t st) {
    hipLaunchKernelGGL(mfma_rate_kernel, dim3(workgroups), dim3(MFMA_RATE_THREADS), 0, st, sink, iters);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups, hipStream_t st) {
    prof_begin(K_STREAM_READ, st);
    hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(SR_THREADS), 0, st,
                       static_cast<const u32x4_t*>(buf), bytes / 16, sink);
    prof_end(K_STREAM_READ, st);
    return hipGetLastError();
}

}  // namespace gqa
