// moe_hbm_read_probe: a pure streaming read of device memory, the practical HBM ceiling
// the weight-streaming kernels are measured against (next to the 8 TB/s datasheet
// figure), and the cache-evicting stream run between timed iterations of small
// workloads.
//
// Each wave reads 1 KB of contiguous bytes per load instruction (16 bytes per lane),
// kUnroll instructions in flight per wave before it folds the words into a running XOR;
// blocks stride over the buffer. The XOR of a block is written to sink[block] so that no
// load can be dropped; the values written mean nothing.
#include "common.h"

namespace {

constexpr int kThreads = 256;

template <int kUnroll>
__global__ __launch_bounds__(kThreads) void read_probe_kernel(const uint4 *__restrict__ p,
                                                              int64_t n16,
                                                              uint32_t *__restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads * kUnroll;
  uint32_t acc = 0;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kUnroll + threadIdx.x;
       base < n16; base += stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * kThreads;
      v[u] = i < n16 ? p[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t part[kThreads / 64];
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) acc ^= __shfl_xor(acc, d, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) r ^= part[w];
    sink[blockIdx.x] = r;
  }
}

}  // namespace

extern "C" int moe_hbm_read_probe(const void *buf, int64_t bytes, uint32_t *sink,
                                  int32_t blocks, int32_t unroll, void *stream) {
  moe::clear_error();
  MOE_REQUIRE(buf && sink, "hbm_read_probe: a required pointer is NULL");
  MOE_REQUIRE(moe::aligned16(buf), "hbm_read_probe: buf must be 16-byte aligned");
  MOE_REQUIRE(bytes > 0 && bytes % 16 == 0, "hbm_read_probe: bytes must be a positive multiple of 16");
  MOE_REQUIRE(blocks >= 1 && blocks <= (1 << 20), "hbm_read_probe: blocks must be in [1, 2^20]");
  const int64_t n16 = bytes / 16;
  switch (unroll) {
    case 4:
      return moe::launch("moe_hbm_read_probe", read_probe_kernel<4>, dim3(blocks), dim3(kThreads),
                         0, stream, static_cast<const uint4 *>(buf), n16, sink);
    case 8:
      return moe::launch("moe_hbm_read_probe", read_probe_kernel<8>, dim3(blocks), dim3(kThreads),
                         0, stream, static_cast<const uint4 *>(buf), n16, sink);
    case 16:
      return moe::launch("moe_hbm_read_probe", read_probe_kernel<16>, dim3(blocks),
                         dim3(kThreads), 0, stream, static_cast<const uint4 *>(buf), n16, sink);
    default:
      MOE_REQUIRE(false, "hbm_read_probe: unroll must be 4, 8 or 16 (got %d)", unroll);
  }
}
