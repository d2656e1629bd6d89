// The clamped SwiGLU of one element, shared by the standalone swiglu_clamp kernel and the
// grouped GEMM's fused epilogue so both give the same bits:
//   silu(min(g, L)) * clamp(u, -L, L),   silu(x) = x / (1 + exp(-x)),   in FP32
// (swiglu_rows on the 2026-09-25 glm5next_mlp forward.rs page; the gate is clamped from
// above only).
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

__device__ __forceinline__ float swiglu_clamp1(float g, float u, float limit) {
  const float gc = fminf(g, limit);
  const float uc = fminf(fmaxf(u, -limit), limit);
  return gc / (1.0f + __expf(-gc)) * uc;
}

}  // namespace moe
