// Shared host-side plumbing of the C ABI: error state, argument checks, kernel launch.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <tuple>
#include <utility>

#include "moe_w4a16.h"

namespace moe {

// Records the message returned by moe_w4a16_last_error() on this thread.
void set_error(const char *fmt, ...);
void clear_error();

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define MOE_REQUIRE(cond, ...)                 \
  do {                                         \
    if (!(cond)) {                             \
      ::moe::set_error(__VA_ARGS__);           \
      return MOE_EINVAL;                       \
    }                                          \
  } while (0)

#define MOE_REQUIRE_CODE(cond, code, ...)      \
  do {                                         \
    if (!(cond)) {                             \
      ::moe::set_error(__VA_ARGS__);           \
      return (code);                           \
    }                                          \
  } while (0)

template <typename Tuple, size_t... I>
void arg_pointers(Tuple &t, void **out, std::index_sequence<I...>) {
  ((out[I] = static_cast<void *>(&std::get<I>(t))), ...);
}

// Launches `kern` through hipLaunchKernel so that a refused launch is reported by this
// call's own return code (not by a later hipGetLastError that other code may own).
template <typename... KArgs, typename... Args>
int launch(const char *name, void (*kern)(KArgs...), dim3 grid, dim3 block, size_t lds_bytes,
           void *stream, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> vals(static_cast<KArgs>(args)...);
  void *ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
  arg_pointers(vals, ptrs, std::index_sequence_for<KArgs...>{});
  hipError_t err = hipLaunchKernel(reinterpret_cast<const void *>(kern), grid, block, ptrs,
                                   lds_bytes, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    set_error("%s: launch failed: %s", name, hipGetErrorString(err));
    return MOE_ELAUNCH;
  }
  return MOE_OK;
}

}  // namespace moe
