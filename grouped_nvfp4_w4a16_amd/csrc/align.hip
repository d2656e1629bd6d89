// moe_align: stable counting sort of the routed slots by expert, in one workgroup.
//
// Produces the grouped path's routing buffers as the 2026-09-25 glm5next_mlp forward.rs
// page documents them (Glm5NextMlpWorkspace fields sorted_token_ids, sorted_expert_ids,
// expert_offsets, token_to_perm): expert_offsets is the prefix sum over the
// expert-sorted rows, sorted_token_ids maps a sorted row back to its token, and
// token_to_perm maps a slot to its sorted row.
//
// Design (gfx950, wave64): the slots are split into 16 contiguous ranges, one per wave.
//   1. Each wave counts its range into a private LDS histogram: per chunk of 64 slots,
//      the lowest lane of each group of equal ids adds the group's size.
//   2. Per expert (a thread each), the 16 per-wave counts become per-wave starting
//      positions within the expert; then one wave scans the experts' counts, each lane
//      summing a contiguous range of experts, for expert_offsets and the active-expert
//      list (two barriers in all, where a block-wide scan needs three per scan).
//   3. Each wave walks its range again in order, 64 slots at a time. The lanes holding
//      the same expert id are found with one ballot per id bit; a lane's rank in its
//      group is the number of lower lanes in it, so positions follow slot order: the
//      sort is stable and the result is deterministic (no atomics decide an order).
//      The group's lowest lane advances the wave's running position of that expert.
//   The ids and group masks of the first two chunks of 64 slots of a wave stay in
//   registers between passes 1 and 3.
// At most 64 slots (a few decode rows) take a one-wave form of the same steps.
#include "common.h"

#include <algorithm>

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// Lanes of the wave whose valid id equals this lane's: one ballot per id bit.
// `bits` (wave-uniform) covers every valid id.
__device__ inline uint64_t same_id_lanes(int id, bool valid, int bits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < bits; ++b) {
    const bool bit = (id >> b) & 1;
    const uint64_t ones = __ballot(valid && bit);
    m &= bit ? ones : ~ones;
  }
  return valid ? m : 0ull;
}

__device__ inline int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

// Workgroups past the first of a moe_align_zero launch: forward_moe's zero-first step on
// rows [0, n_rows) x columns [0, cols) of `zero`, 16 bytes per thread, beside the sort.
__device__ __forceinline__ void zero_rows_part(uint16_t *__restrict__ zero, int64_t ld,
                                               int32_t n_rows, int32_t cols) {
  const int64_t per_row = cols / 8, units = per_row * n_rows;
  const int64_t stride = static_cast<int64_t>(gridDim.x - 1) * blockDim.x;
  for (int64_t u = static_cast<int64_t>(blockIdx.x - 1) * blockDim.x + threadIdx.x; u < units;
       u += stride) {
    const int64_t row = u / per_row, col8 = u - row * per_row;
    *reinterpret_cast<uint4 *>(zero + row * ld + col8 * 8) = make_uint4(0u, 0u, 0u, 0u);
  }
}

__global__ __launch_bounds__(kThreads) void moe_align_kernel(
    const int32_t *__restrict__ ids, int32_t n_slots, int32_t top_k, int32_t num_experts,
    int32_t *__restrict__ sorted_token_ids, int32_t *__restrict__ sorted_expert_ids,
    int32_t *__restrict__ expert_offsets, int32_t *__restrict__ token_to_perm,
    int32_t *__restrict__ active_experts, int32_t *__restrict__ counters,
    uint16_t *__restrict__ zero, int64_t ld_zero, int32_t zero_cols) {
  if (blockIdx.x != 0) {  // uniform: a zeroing workgroup
    zero_rows_part(zero, ld_zero, n_slots, zero_cols);
    return;
  }
  extern __shared__ int lds[];
  const int E = num_experts;
  int *hist = lds;                  // [kWaves][E]: counts, then positions within the expert
  int *first = lds + kWaves * E;    // [E]: slots per expert, then the expert's first row
  int *misc = first + E;            // [0] invalid slots, [1] valid slots, [2] active experts

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kWaves * E; i += kThreads) hist[i] = 0;
  if (tid == 0) misc[0] = 0;
  __syncthreads();

  // Contiguous slot range of this wave, a multiple of 64 long.
  const int per_wave = ((n_slots + kWaves - 1) / kWaves + 63) & ~63;
  const int begin = min(wave * per_wave, n_slots);
  const int end = min(begin + per_wave, n_slots);
  int *my_hist = hist + wave * E;

  const int bits = E > 1 ? 32 - __clz(E - 1) : 1;
  const uint64_t lower = (1ull << lane) - 1ull;

  // 1. per-wave histograms: each group's lowest lane adds the group size (the groups of
  //    a chunk have distinct ids, so the updates do not collide). The ids and group masks
  //    of the first two chunks stay in registers for step 3.
  int cache_id[2] = {-1, -1};
  uint64_t cache_grp[2] = {0ull, 0ull};
  int invalid = 0;
  for (int c = 0, base = begin; base < end; ++c, base += 64) {
    const int t = base + lane;
    const bool in = t < end;
    const int id = in ? ids[t] : -1;
    const bool valid = in && id >= 0 && id < E;
    const uint64_t grp = same_id_lanes(id, valid, bits);
    if (c < 2) {
      cache_id[c] = id;
      cache_grp[c] = grp;
    }
    if (valid && (grp & lower) == 0) my_hist[id] += __popcll(grp);
    invalid += __popcll(__ballot(in && !valid));
  }
  if (lane == 0 && invalid) atomicAdd(&misc[0], invalid);
  __syncthreads();

  // 2. Each expert's count and its waves' starting positions within the expert (a
  //    thread per expert), then the experts' first rows: one wave scans the counts,
  //    each lane taking a contiguous range of experts (no block-wide scan).
  for (int e = tid; e < E; e += kThreads) {
    int cnt = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int h = hist[w * E + e];
      hist[w * E + e] = cnt;
      cnt += h;
    }
    first[e] = cnt;
  }
  __syncthreads();
  if (wave == 0) {
    const int per = (E + 63) / 64;
    const int e0 = lane * per;
    int n_mine = 0, act_mine = 0;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      const int c = e < E ? first[e] : 0;
      n_mine += c;
      act_mine += c > 0;
    }
    const int run0 = wave_inclusive_scan(n_mine) - n_mine;
    const int act0 = wave_inclusive_scan(act_mine) - act_mine;
    int run = run0, act = act0;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        const int c = first[e];
        expert_offsets[e] = run;
        first[e] = run;
        if (active_experts != nullptr && c > 0) active_experts[act++] = e;
        run += c;
      }
    }
    if (lane == 63) {
      misc[1] = run;
      misc[2] = act;
      expert_offsets[E] = run;
      if (counters != nullptr) {
        counters[0] = act;
        counters[1] = misc[0];
      }
    }
  }
  __syncthreads();
  const int n_valid = misc[1], n_active = misc[2];
  if (active_experts != nullptr)
    for (int i = n_active + tid; i < E; i += kThreads) active_experts[i] = -1;

  // 3. stable scatter: an expert's first row, plus the wave's start within the expert,
  //    plus the lane's rank in its group.
  for (int c = 0, base = begin; base < end; ++c, base += 64) {
    const int t = base + lane;
    const bool in = t < end;
    const int id = c < 2 ? cache_id[c] : (in ? ids[t] : -1);
    const bool valid = in && id >= 0 && id < E;
    const uint64_t grp = c < 2 ? cache_grp[c] : same_id_lanes(id, valid, bits);
    int pos = -1;
    if (valid) {
      const int start = my_hist[id];  // read by every lane of the group first
      pos = first[id] + start + __popcll(grp & lower);
      if ((grp & lower) == 0) my_hist[id] = start + __popcll(grp);
    }
    if (in) {
      token_to_perm[t] = pos;
      if (valid) {
        sorted_token_ids[pos] = t / top_k;
        sorted_expert_ids[pos] = id;
      }
    }
  }
  for (int p = n_valid + tid; p < n_slots; p += kThreads) {
    sorted_token_ids[p] = -1;
    sorted_expert_ids[p] = -1;
  }
}

// The same sort for at most 64 slots (a few decode rows), in one wave with no block-wide
// scans: lane t holds slot t; the lanes of one expert come from same_id_lanes, a lane's
// rank among them is its stable position, and the expert offsets are a wave scan over
// the per-expert counts, each lane summing a contiguous range of experts.
__global__ __launch_bounds__(64) void moe_align_wave_kernel(
    const int32_t *__restrict__ ids, int32_t n_slots, int32_t top_k, int32_t num_experts,
    int32_t *__restrict__ sorted_token_ids, int32_t *__restrict__ sorted_expert_ids,
    int32_t *__restrict__ expert_offsets, int32_t *__restrict__ token_to_perm,
    int32_t *__restrict__ active_experts, int32_t *__restrict__ counters,
    uint16_t *__restrict__ zero, int64_t ld_zero, int32_t zero_cols) {
  if (blockIdx.x != 0) {  // uniform: a zeroing workgroup
    zero_rows_part(zero, ld_zero, n_slots, zero_cols);
    return;
  }
  extern __shared__ int lds[];
  const int E = num_experts;
  int *cnt = lds;  // [E]: slots per expert, then each expert's first position
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  const bool in = lane < n_slots;
  const int id = in ? ids[lane] : -1;
  const bool valid = in && id >= 0 && id < E;
  const int bits = E > 1 ? 32 - __clz(E - 1) : 1;
  const uint64_t lower = (1ull << lane) - 1ull;
  const uint64_t grp = same_id_lanes(id, valid, bits);
  const int n_invalid = __popcll(__ballot(in && !valid));
  __syncthreads();
  if (valid && (grp & lower) == 0) cnt[id] = __popcll(grp);  // one writer per expert
  __syncthreads();
  // Lane l owns experts [l per, (l + 1) per): its slot and active-expert counts, then
  // their exclusive wave prefix sums.
  const int per = (E + 63) / 64;
  const int e0 = lane * per;
  int n_mine = 0, act_mine = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    const int c = e < E ? cnt[e] : 0;
    n_mine += c;
    act_mine += c > 0;
  }
  const int run0 = wave_inclusive_scan(n_mine) - n_mine;
  const int act0 = wave_inclusive_scan(act_mine) - act_mine;
  const int n_valid = __shfl(run0 + n_mine, 63, 64);
  const int n_active = __shfl(act0 + act_mine, 63, 64);
  int run = run0, act = act0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      const int c = cnt[e];
      expert_offsets[e] = run;
      cnt[e] = run;
      if (active_experts != nullptr && c > 0) active_experts[act++] = e;
      run += c;
    }
  }
  __syncthreads();
  if (in) {
    const int pos = valid ? cnt[id] + __popcll(grp & lower) : -1;
    token_to_perm[lane] = pos;
    if (valid) {
      sorted_token_ids[pos] = lane / top_k;
      sorted_expert_ids[pos] = id;
    }
  }
  for (int p = n_valid + lane; p < n_slots; p += 64) {
    sorted_token_ids[p] = -1;
    sorted_expert_ids[p] = -1;
  }
  if (active_experts != nullptr)
    for (int i = n_active + lane; i < E; i += 64) active_experts[i] = -1;
  if (lane == 0) {
    expert_offsets[E] = n_valid;
    if (counters != nullptr) {
      counters[0] = n_active;
      counters[1] = n_invalid;
    }
  }
}

}  // namespace

namespace {

// moe_align, with the zeroing workgroups of moe_align_zero when `zero` is given.
int align_launch(const char *name, const int32_t *topk_ids, int32_t rows, int32_t top_k,
                 int32_t num_experts, int32_t *sorted_token_ids, int32_t *sorted_expert_ids,
                 int32_t *expert_offsets, int32_t *token_to_perm, int32_t *active_experts,
                 int32_t *counters, uint16_t *zero, int64_t ld_zero, int32_t zero_cols,
                 void *stream) {
  MOE_REQUIRE(rows >= 0, "%s: rows must be >= 0 (got %d)", name, rows);
  MOE_REQUIRE(top_k >= 1, "%s: top_k must be >= 1 (got %d)", name, top_k);
  MOE_REQUIRE(num_experts >= 1 && num_experts <= MOE_ALIGN_MAX_EXPERTS,
              "%s: num_experts must be in [1, %d] (got %d)", name, MOE_ALIGN_MAX_EXPERTS,
              num_experts);
  const int64_t n_slots = static_cast<int64_t>(rows) * top_k;
  MOE_REQUIRE(n_slots <= INT32_MAX, "%s: rows * top_k overflows int32", name);
  MOE_REQUIRE(expert_offsets != nullptr, "%s: expert_offsets is NULL", name);
  if (n_slots > 0) {
    MOE_REQUIRE(topk_ids && sorted_token_ids && sorted_expert_ids && token_to_perm,
                "%s: a required pointer is NULL", name);
  }
  // Zeroing workgroups: enough to cover the rows in a few passes, none without a buffer.
  int64_t zero_blocks = 0;
  const bool wave_form = n_slots > 0 && n_slots <= 64;
  const int threads = wave_form ? 64 : kThreads;
  if (zero != nullptr && n_slots > 0 && zero_cols > 0) {
    const int64_t units = n_slots * (zero_cols / 8);
    zero_blocks = std::min<int64_t>((units + threads - 1) / threads, wave_form ? 4096 : 1024);
  }
  if (wave_form)
    return moe::launch(name, moe_align_wave_kernel, dim3(static_cast<unsigned>(1 + zero_blocks)),
                       dim3(64), static_cast<size_t>(num_experts) * sizeof(int), stream,
                       topk_ids, static_cast<int32_t>(n_slots), top_k, num_experts,
                       sorted_token_ids, sorted_expert_ids, expert_offsets, token_to_perm,
                       active_experts, counters, zero, ld_zero, zero_cols);
  const size_t lds = ((static_cast<size_t>(kWaves) + 1) * num_experts + 4) * sizeof(int);
  // Histograms of large expert counts exceed the default 64 KiB of dynamic LDS.
  static const hipError_t attr_err = hipFuncSetAttribute(
      reinterpret_cast<const void *>(moe_align_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
      static_cast<int>(((kWaves + 1) * MOE_ALIGN_MAX_EXPERTS + 4) * sizeof(int)));
  if (lds > 65536 && attr_err != hipSuccess) {
    moe::set_error("%s: cannot raise the LDS limit: %s", name, hipGetErrorString(attr_err));
    return MOE_ELAUNCH;
  }
  return moe::launch(name, moe_align_kernel, dim3(static_cast<unsigned>(1 + zero_blocks)),
                     dim3(kThreads), lds, stream, topk_ids, static_cast<int32_t>(n_slots), top_k,
                     num_experts, sorted_token_ids, sorted_expert_ids, expert_offsets,
                     token_to_perm, active_experts, counters, zero, ld_zero, zero_cols);
}

}  // namespace

extern "C" int moe_align(const int32_t *topk_ids, int32_t rows, int32_t top_k,
                         int32_t num_experts, int32_t *sorted_token_ids,
                         int32_t *sorted_expert_ids, int32_t *expert_offsets,
                         int32_t *token_to_perm, int32_t *active_experts, int32_t *counters,
                         void *stream) {
  moe::clear_error();
  return align_launch("moe_align", topk_ids, rows, top_k, num_experts, sorted_token_ids,
                      sorted_expert_ids, expert_offsets, token_to_perm, active_experts, counters,
                      nullptr, 0, 0, stream);
}

extern "C" int moe_align_zero(const int32_t *topk_ids, int32_t rows, int32_t top_k,
                              int32_t num_experts, int32_t *sorted_token_ids,
                              int32_t *sorted_expert_ids, int32_t *expert_offsets,
                              int32_t *token_to_perm, int32_t *active_experts,
                              int32_t *counters, uint16_t *zero, int64_t ld_zero,
                              int32_t zero_cols, void *stream) {
  moe::clear_error();
  MOE_REQUIRE(zero_cols >= 0 && zero_cols % 8 == 0,
              "moe_align_zero: zero_cols must be >= 0 and a multiple of 8 (got %d)", zero_cols);
  MOE_REQUIRE(ld_zero >= zero_cols && ld_zero % 8 == 0,
              "moe_align_zero: ld_zero must be >= zero_cols and a multiple of 8");
  if (static_cast<int64_t>(rows) * top_k > 0 && zero_cols > 0)
    MOE_REQUIRE(zero != nullptr && moe::aligned16(zero),
                "moe_align_zero: zero must be non-NULL and 16-byte aligned");
  return align_launch("moe_align_zero", topk_ids, rows, top_k, num_experts, sorted_token_ids,
                      sorted_expert_ids, expert_offsets, token_to_perm, active_experts, counters,
                      zero, ld_zero, zero_cols, stream);
}
