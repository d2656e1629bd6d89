// The clamped SwiGLU of one element, shared by the standalone swiglu_clamp kernel and the
// grouped GEMM's fused epilogue so both give the same bits:
//   silu(min(g, L)) * clamp(u, -L, L),   silu(x) = x / (1 + exp(-x)),   in FP32
// (swiglu_rows on the 2026-09-25 glm5next_mlp forward.rs page; the gate is clamped from
// above only).
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

// The clamps are selects, not fminf/fmaxf, so that a NaN gate or up value stays NaN (the
// minimum of NaN and the limit is NaN; fminf would return the limit and hide it).
// silu(x) = x / (1 + e^-x) for x >= 0, and the same value as x e^x / (1 + e^x) for x < 0,
// where e^-x would overflow FP32 below about -88.7 and turn a small but representable
// result into zero. One exponential, e = e^-|x|: the hardware exponential where e is a
// normal FP32 number, the full-range expf below x = -87 (e subnormal, x e^x possibly
// still normal); that rare branch costs nothing where no lane takes it.
__device__ __forceinline__ float swiglu_clamp1(float g, float u, float limit) {
  const float gc = g > limit ? limit : g;
  const float uc = u > limit ? limit : (u < -limit ? -limit : u);
  float e = __expf(-fabsf(gc));
  if (gc < -87.0f) e = expf(gc);
  const float num = gc >= 0.0f ? gc : gc * e;
  return num / (1.0f + e) * uc;
}

}  // namespace moe
