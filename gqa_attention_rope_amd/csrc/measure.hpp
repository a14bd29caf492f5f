// Measurement probes that no part of the attention step uses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// The sustained rate of the prefill's matrix instruction (bf16 16x16x32 MFMA)
// on every CU; see measure.hip.
constexpr int MFMA_RATE_THREADS = 256;
constexpr int MFMA_RATE_PER_ITER = 8;     // MFMAs per wave and iteration
constexpr int MFMA_RATE_SINK_WORDS = 8;   // 64-bit words written per workgroup
hipError_t launch_mfma_rate(unsigned long long* sink, int workgroups, int iters, hipStream_t st);

}  // namespace gqa
