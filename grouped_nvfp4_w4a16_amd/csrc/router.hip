// moe_router_topk: the routed layer's top-k expert selection on the device.
//
// The router launch of forward_moe (both glm5next_mlp forward.rs pages) takes FP32
// logits [rows, E], an optional per-expert bias, top_k, n_group = 1, routed_scale and a
// renormalize flag, one row per block. The pages do not print the kernel's arithmetic;
// this follows the plainest reading (the oracle's router_topk states it):
//   scores = softmax(logits row)
//   key(e) = scores[e] + bias[e] with a bias, else logits[e] (the same selection as the
//            score, without ties created by rounding the scores)
//   the top_k largest keys in descending order, equal keys to the lower id
//   weight = score, / (sum of the selected scores) when renormalize, * routed_scale
//
// gfx950 design: one wave64 per row, four rows per block. Lane l holds logits
// l, l + 64, ... in registers: kPL of them, the smallest of 4, 8, 16, 32 that covers E
// (E <= 2048), so that the per-round scans do no work for absent experts. The max and the softmax sum
// are wave reductions; each of the top_k rounds is a local argmax over the lane's values
// followed by a wave-wide (key, id) reduction, and lane r keeps the r-th pick. The
// weights then take one expf per selected logit.
#include "common.h"

namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kThreads = 64 * kRowsPerBlock;
static_assert(MOE_ROUTER_MAX_EXPERTS % 64 == 0 && MOE_ROUTER_MAX_EXPERTS <= 32 * 64,
              "whole lanes, at most 32 values per lane");

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// (key, id) of the larger key; equal keys: the lower id. id -1 (nothing) always loses.
__device__ __forceinline__ void better(float &k, int &i, float k2, int i2) {
  const bool take = i2 >= 0 && (i < 0 || k2 > k || (k2 == k && i2 < i));
  k = take ? k2 : k;
  i = take ? i2 : i;
}

template <int kPL>
__global__ __launch_bounds__(kThreads) void router_topk_kernel(
    const float *__restrict__ logits, int64_t ld, int32_t rows, int32_t E,
    const float *__restrict__ bias, int32_t top_k, float routed_scale, int32_t renormalize,
    int32_t *__restrict__ ids, float *__restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole waves leave together (no barriers below)
  const float *lg = logits + static_cast<size_t>(row) * ld;

  float l[kPL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPL; ++i) {
    const int e = lane + 64 * i;
    l[i] = e < E ? lg[e] : -INFINITY;
    m = fmaxf(m, l[i]);
  }
  m = wave_max(m);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) sum += __expf(l[i] - m);
  }
  sum = wave_sum(sum);

  // Selection keys; a taken entry has its bit cleared in `avail`.
  float key[kPL];
  unsigned avail = 0;  // bit i: entry lane + 64 i is still selectable
#pragma unroll
  for (int i = 0; i < kPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      avail |= 1u << i;
      key[i] = bias != nullptr ? __expf(l[i] - m) / sum + bias[e] : l[i];
    } else {
      key[i] = -INFINITY;
    }
  }

  int my_id = -1;  // lane r: the r-th pick
  float my_l = 0.f;
  for (int r = 0; r < top_k; ++r) {
    float bk = 0.f;
    int bi = -1, bslot = -1;
#pragma unroll
    for (int i = 0; i < kPL; ++i) {
      const int e = lane + 64 * i;
      const bool ok = (avail >> i) & 1u;
      const bool take = ok && (bi < 0 || key[i] > bk);  // ids rise with i: keep the first
      bk = take ? key[i] : bk;
      bi = take ? e : bi;
      bslot = take ? i : bslot;
    }
    // wave-wide winner
    float wk = bk;
    int wi = bi;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const float ok2 = __shfl_xor(wk, d, 64);
      const int oi2 = __shfl_xor(wi, d, 64);
      better(wk, wi, ok2, oi2);
    }
    if (wi < 0) break;  // fewer than top_k experts: the rest stay -1 (wave-uniform)
    if (bi == wi) avail &= ~(1u << bslot);  // the owner retires its entry
    // the winning logit: owner lane (wi % 64), slot wi / 64
    const int owner = wi & 63, oslot = wi >> 6;
    float ol = 0.f;
#pragma unroll
    for (int i = 0; i < kPL; ++i) ol = i == oslot ? l[i] : ol;
    ol = __shfl(ol, owner, 64);
    if (lane == r) {
      my_id = wi;
      my_l = ol;
    }
  }

  const bool picked = my_id >= 0;
  const float p = picked ? __expf(my_l - m) : 0.f;
  const float denom = renormalize ? wave_sum(p) : sum;
  if (lane < top_k) {
    ids[static_cast<size_t>(row) * top_k + lane] = my_id;
    wts[static_cast<size_t>(row) * top_k + lane] = picked ? p / denom * routed_scale : 0.f;
  }
}

}  // namespace

extern "C" int moe_router_topk(const float *logits, int64_t ld_logits, int32_t rows,
                               int32_t num_experts, const float *bias, int32_t top_k,
                               float routed_scale, int32_t renormalize, int32_t *topk_ids,
                               float *topk_weights, void *stream) {
  moe::clear_error();
  MOE_REQUIRE(rows >= 0, "router_topk: rows must be >= 0 (got %d)", rows);
  MOE_REQUIRE(num_experts >= 1 && num_experts <= MOE_ROUTER_MAX_EXPERTS,
              "router_topk: num_experts must be in [1, %d] (got %d)", MOE_ROUTER_MAX_EXPERTS,
              num_experts);
  MOE_REQUIRE(top_k >= 1 && top_k <= MOE_ROUTER_MAX_TOPK,
              "router_topk: top_k must be in [1, %d] (got %d)", MOE_ROUTER_MAX_TOPK, top_k);
  MOE_REQUIRE(ld_logits >= num_experts, "router_topk: ld_logits must be >= num_experts");
  MOE_REQUIRE(routed_scale == routed_scale && routed_scale > -INFINITY && routed_scale < INFINITY,
              "router_topk: routed_scale must be finite");
  if (rows == 0) return MOE_OK;
  MOE_REQUIRE(logits && topk_ids && topk_weights, "router_topk: a required pointer is NULL");
  const dim3 grid(static_cast<unsigned>((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  const auto go = [&](auto kern) {
    return moe::launch("moe_router_topk", kern, grid, dim3(kThreads), 0, stream, logits,
                       ld_logits, rows, num_experts, bias, top_k, routed_scale, renormalize,
                       topk_ids, topk_weights);
  };
  const int per_lane = (num_experts + 63) / 64;
  if (per_lane <= 4) return go(router_topk_kernel<4>);
  if (per_lane <= 8) return go(router_topk_kernel<8>);
  if (per_lane <= 16) return go(router_topk_kernel<16>);
  return go(router_topk_kernel<32>);
}
