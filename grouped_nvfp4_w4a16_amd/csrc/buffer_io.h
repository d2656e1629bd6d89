// Raw buffer loads for gfx950 (a gfx9 buffer resource with word 3 = 0x00020000).
//
// Offsets past num_records read as zero without touching memory, which masks padded and
// invalid rows at no cost. The range check covers the vector offset, not the scalar one,
// so row offsets always go in the vector offset.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Past-the-end offset: the load returns zeros and moves no data.
constexpr uint32_t kNoLoad = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0,
                                           static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ u32x4_t load16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                          uint32_t soff) {
  return __builtin_bit_cast(
      u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff),
                                                     static_cast<int>(soff), 0));
}

}  // namespace moe
