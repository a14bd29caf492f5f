// Loads from HBM straight into LDS, and the transposing LDS read, on gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// LDS address of a __shared__ object, as the loads below take it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(size_t)(const lds_void_t*)p; }

// A range-checked 16-byte-per-lane buffer load whose data goes to LDS: lane i
// writes lds_addr + 16 i (the address is uniform, in m0), and lanes past the
// descriptor's range write zeros.  Issued as inline asm: through the builtin
// the compiler guards later transposed LDS reads of another buffer with a wait
// for these loads, which would expose their latency.  The caller waits for
// them itself (vmcnt(0)) before the barrier that publishes the data.  The
// instruction has no register result.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_addr, int voff, int soff) {
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr)
                 : "memory");
}
// The same with the non-temporal cache policy, for data read once per launch.
__device__ __forceinline__ void load_lds16_nt(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_addr, int voff, int soff) {
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen nt lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr)
                 : "memory");
}

// Transposing read of 4 bf16 per lane: within each group of 16 lanes, lanes
// 4i .. 4i+3 name row i (4 consecutive values each, 16 in all) and lane n
// receives value n of rows 0..3.
__device__ __forceinline__ i16x4_t read_tr16(const unsigned char* lds_ptr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)lds_ptr);
}

}  // namespace gqa
