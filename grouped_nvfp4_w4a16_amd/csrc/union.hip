// Decode / verify path for a few rows: moe_row_union and moe_w4a16_gemv_union (and its
// SwiGLU-fused form).
//
// What it computes follows "glm5next_mlp/forward.rs" (2026-09-25): the workspace fields
// u_eid (union expert ids, -1 = entry unused) and u_slot (slot per union entry per row, -1
// = row absent), the row-batched GEMV that sweeps each expert of the rows' union once and
// writes C[rows, top_k, N], and moe_row_groups' statement that which rows share a sweep
// never changes what a row adds. The union is found by pairwise scans in one workgroup, no
// sort; the outputs are laid out by (row, slot), so the combine reads them back through
// slot_perm without an expert-sorted permutation.
//
// gfx950 design of the GEMV (the pages' mma-less GEMV tiers are not used):
//   - A union entry has at most one activation row per routed row, so with rows <= 16 all
//     of its rows fit one MFMA tile (v_mfma_f32_16x16x32_bf16, weights as A, the entry's
//     rows as B): each weight is decoded once per launch, whatever the rows.
//   - Few rows means few experts and little work per expert, so blocks are small: a block
//     of 4 waves owns 32 * (4 / kKSplit) weight rows of one entry, and the kKSplit waves of
//     each 32-row group split K (wave kw takes the 256-k steps kw, kw + kKSplit, ...).
//     The partial FP32 tiles are summed in LDS in wave order (deterministic) and stored as
//     BF16. The split keeps each wave's weight stream a few steps long while the grid
//     still covers the chip when only tens of experts are live.
//   - Weights: raw buffer loads, 16 rows x 2 x 16 bytes per wave instruction pair, one
//     step ahead in a two-slot register ring, decoded in registers by the exact per-code
//     byte tables (nvfp4_decode.h, one 256-code LUT per block) straight into A.
//   - Lane (r16, kb) takes k in [64 kb, 64 kb + 64) of each step, so its four block
//     scales are one aligned dword of the row's 16 scale bytes, and its activation bytes
//     are 128 contiguous bytes loaded straight from the input row (no LDS staging: each
//     wave reads different steps), one step ahead, put in the decoder's k order.
//   - SwiGLU-fused form: a wave's two tiles are 16 gate rows and the matching 16 up rows,
//     rounded to BF16 and passed through the clamped SwiGLU in the epilogue (as the grouped
//     GEMM's fused form).
#include "buffer_io.h"
#include "common.h"
#include "nvfp4_decode.h"
#include "swiglu.h"
#include "w4a16_mma.h"

namespace {

using moe::bf16x8_t;
using moe::f32x4_t;
using moe::kNoLoad;
using moe::load16;
using moe::make_rsrc;
using moe::u32x4_t;

// ------------------------------------------------------------------------- row union

constexpr int kUnionMaxIds = 1024;  // rows * top_k: one thread per id, one workgroup

__global__ __launch_bounds__(kUnionMaxIds) void row_union_kernel(
    const int32_t *__restrict__ ids, int32_t rows, int32_t top_k, int32_t num_experts,
    int32_t *__restrict__ u_eid, int32_t *__restrict__ u_slot, int32_t *__restrict__ slot_perm,
    int32_t *__restrict__ counters) {
  __shared__ int32_t s_id[kUnionMaxIds];    // id of a covered slot, else -1
  __shared__ int32_t s_uid[kUnionMaxIds];   // union entries in order
  __shared__ int32_t s_wave_first[kUnionMaxIds / 64];
  const int n_ids = rows * top_k;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r = t / top_k, j = t - r * top_k;

  // 1. A slot is covered when its id is in range and no lower slot of its row has it.
  int id = -1;
  if (t < n_ids) {
    const int v = ids[t];
    if (v >= 0 && v < num_experts) id = v;
  }
  s_id[t] = id;
  __syncthreads();
  if (id >= 0) {
    for (int jj = 0; jj < j; ++jj) {
      if (s_id[r * top_k + jj] == id) {
        id = -1;  // a repeat in the row
        break;
      }
    }
  }
  __syncthreads();
  s_id[t] = id;
  __syncthreads();

  // 2. The union in order of first appearance: slot t opens an entry when no lower
  //    covered slot has its id; entries are numbered by a block-wide count of openers.
  bool opens = id >= 0;
  for (int q = 0; opens && q < t; ++q) opens = s_id[q] != id;
  const uint64_t ballot = __ballot(opens);
  if (lane == 0) s_wave_first[wave] = __popcll(ballot);
  s_uid[t] = -1;
  __syncthreads();
  int base = 0, n_union = 0;
  for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) {
    if (w < wave) base += s_wave_first[w];
    n_union += s_wave_first[w];
  }
  if (opens) s_uid[base + __popcll(ballot & ((1ull << lane) - 1ull))] = id;
  __syncthreads();

  // 3. Outputs, each entry written by exactly one thread.
  if (t < n_ids) {
    u_eid[t] = s_uid[t];
    if (slot_perm != nullptr) slot_perm[t] = id >= 0 ? t : -1;
  }
  for (int q = t; q < n_ids * rows; q += blockDim.x) {
    const int p = q / rows, rr = q - p * rows;
    const int e = s_uid[p];
    int slot = -1;
    if (e >= 0) {
      for (int jj = 0; jj < top_k; ++jj) {
        if (s_id[rr * top_k + jj] == e) {
          slot = jj;
          break;
        }
      }
    }
    u_slot[q] = slot;
  }
  if (counters != nullptr && t == 0) {
    int covered = 0;
    for (int q = 0; q < n_ids; ++q) covered += s_id[q] >= 0;
    counters[0] = n_union;
    counters[1] = n_ids - covered;
  }
}

// ------------------------------------------------------------------------- union GEMV

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kChunkK = 256;       // k per step
constexpr int kMaxRows = 16;       // routed rows a launch may have: one MFMA tile of B
static_assert(kThreads == 256, "build_code_table_lut: one E4M3 code per thread");

// One lane's data of one step: packed weights of its two tiles (k in [64 kb, 64 kb + 32)
// and [64 kb + 32, 64 kb + 64)), the four block-scale codes of each tile, and its
// activation row's 64 k in eight 16-byte pieces.
struct StepRegs {
  u32x4_t wa[2], wb[2];
  uint32_t sc[2];
  u32x4_t x[8];
};

template <bool kSwiglu, int kKSplit>
__global__ __launch_bounds__(kThreads, 3) void gemv_union_kernel(
    const uint16_t *__restrict__ a, int64_t lda, int32_t a_rows, int32_t a_per_slot,
    const uint64_t *__restrict__ packed_ptrs, const uint64_t *__restrict__ scale_ptrs,
    const float *__restrict__ scale2s, const int32_t *__restrict__ u_eid,
    const int32_t *__restrict__ u_slot, int32_t rows, int32_t top_k, int32_t num_experts,
    uint16_t *__restrict__ c, int64_t ldc, int32_t N, int32_t K, float limit) {
  constexpr int kGroups = kWaves / kKSplit;  // 32-row groups per block
  __shared__ __attribute__((aligned(16))) uint8_t lut[256 * 16];
  __shared__ __attribute__((aligned(16))) f32x4_t red[kWaves][2][64];

  const int p = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave % kKSplit, nw = wave / kKSplit;
  const int r16 = lane & 15, kb = lane >> 4;

  // The entry's expert and its rows: lane l < rows reads u_slot[p, l].
  const int e = u_eid[p];
  const int my_slot_of_lane = lane < rows ? u_slot[static_cast<int64_t>(p) * rows + lane] : -1;
  if (e < 0 || e >= num_experts) return;
  const uint64_t packed_u = packed_ptrs[e], scales_u = scale_ptrs[e];
  const float scale2 = scale2s[e];
  asm volatile("" ::"s"(packed_u), "s"(scales_u), "s"(scale2));
  if (packed_u == 0) return;  // expert not present: its rows keep the caller's values
  const uint64_t present = __ballot(my_slot_of_lane >= 0);
  if (present == 0) return;
  // Token r16 of the tile: the r16-th routed row present in the entry.
  int tok_row = -1;
  {
    uint64_t m = present;
    for (int i = 0; i < kMaxRows && m != 0; ++i) {
      const int b = __builtin_ctzll(m);
      if (i == r16) tok_row = b;
      m &= m - 1;
    }
  }
  const int tok_slot = __shfl(my_slot_of_lane, tok_row < 0 ? 0 : tok_row);
  const bool tok_on = tok_row >= 0;
  const int dst_row = tok_row * top_k + tok_slot;
  const int src_row = a_per_slot ? dst_row : tok_row;

  const uint8_t *packed = reinterpret_cast<const uint8_t *>(packed_u);
  const uint8_t *scales = reinterpret_cast<const uint8_t *>(scales_u);
  const int mi = N / 2;
  // This wave's two tiles of 16 weight rows. Plain: the group's 32 consecutive rows.
  // Fused: 16 gate rows and the matching 16 up rows.
  const int n_t0 = kSwiglu ? (blockIdx.x * kGroups + nw) * 16 : (blockIdx.x * kGroups + nw) * 32;
  const int n_t1 = kSwiglu ? mi + n_t0 : n_t0 + 16;
  const int row_end0 = kSwiglu ? mi : N;
  const bool t0_on = n_t0 < row_end0, t1_on = n_t1 < N && (!kSwiglu || t0_on);

  const uint32_t row_bytes = static_cast<uint32_t>(K) / 2, srow_bytes = static_cast<uint32_t>(K) / 16;
  const int n_steps = K / kChunkK;
  const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(packed, static_cast<uint32_t>(N) * row_bytes);
  const __amdgpu_buffer_rsrc_t s_rsrc = make_rsrc(scales, static_cast<uint32_t>(N) * srow_bytes);
  const __amdgpu_buffer_rsrc_t x_rsrc =
      make_rsrc(a, static_cast<uint32_t>(a_rows) * static_cast<uint32_t>(lda) * 2u);
  // Rows past N lie past the buffer end and read zeros; out-of-range inputs read zeros.
  const uint32_t w_voff[2] = {static_cast<uint32_t>(n_t0 + r16) * row_bytes + 32u * kb,
                              static_cast<uint32_t>(n_t1 + r16) * row_bytes + 32u * kb};
  const uint32_t s_voff[2] = {static_cast<uint32_t>(n_t0 + r16) * srow_bytes + 4u * kb,
                              static_cast<uint32_t>(n_t1 + r16) * srow_bytes + 4u * kb};
  const bool x_on = tok_on && src_row >= 0 && src_row < a_rows;
  const uint32_t x_voff =
      x_on ? (static_cast<uint32_t>(src_row) * static_cast<uint32_t>(lda) + 64u * kb) * 2u : kNoLoad;

  // Step s of this wave's share (kw, kw + kKSplit, ...); past the last one the loads read
  // nothing, so every load stays unconditional.
  const int n_mine = n_steps > kw ? (n_steps - kw + kKSplit - 1) / kKSplit : 0;
  const auto load_step = [&](StepRegs &st, int i) {
    const bool live = i < n_mine;
    const int step = kw + i * kKSplit;
    const uint32_t wsoff = static_cast<uint32_t>(step) * (kChunkK / 2);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t v = live ? w_voff[t] : kNoLoad;
      st.wa[t] = load16(w_rsrc, v, wsoff);
      st.wb[t] = load16(w_rsrc, v + 16, wsoff);
      st.sc[t] = __builtin_amdgcn_raw_buffer_load_b32(
          s_rsrc, static_cast<int>(live ? s_voff[t] : kNoLoad), static_cast<int>(step * 16), 0);
    }
    const uint32_t xv = live ? x_voff : kNoLoad;
    const uint32_t xsoff = static_cast<uint32_t>(step) * (kChunkK * 2);
#pragma unroll
    for (int q = 0; q < 8; ++q) st.x[q] = load16(x_rsrc, xv + 16u * q, xsoff);
  };

  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  const auto run_step = [&](const StepRegs &st) {
    moe::Fp4Table blk0[4], blk1[4];
    moe::lut_blocks(st.sc[0], lut, blk0);
    moe::lut_blocks(st.sc[1], lut, blk1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8_t B[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) B[q] = __builtin_bit_cast(bf16x8_t, moe::permute_k8(st.x[4 * h + q]));
      const u32x4_t &x0 = h ? st.wb[0] : st.wa[0];
      const uint32_t w0w[4] = {x0[0], x0[1], x0[2], x0[3]};
      moe::mfma4(w0w, blk0[2 * h], blk0[2 * h + 1], B, acc[0]);
      if (t1_on) {
        const u32x4_t &x1 = h ? st.wb[1] : st.wa[1];
        const uint32_t w1w[4] = {x1[0], x1[1], x1[2], x1[3]};
        moe::mfma4(w1w, blk1[2 * h], blk1[2 * h + 1], B, acc[1]);
      }
    }
  };

  StepRegs s0, s1;
  load_step(s0, 0);
  moe::build_code_table_lut(lut, tid, scale2);
  __syncthreads();  // the LUT is complete
  if (t0_on) {
    for (int i = 0; i < n_mine; i += 2) {
      load_step(s1, i + 1);
      run_step(s0);
      load_step(s0, i + 2);
      if (i + 1 < n_mine) run_step(s1);
    }
  }

  // Sum the kKSplit partial tiles of each 32-row group in wave order.
  if (kKSplit > 1) {
    if (kw > 0) {
      red[wave][0][lane] = acc[0];
      red[wave][1][lane] = acc[1];
    }
    __syncthreads();
    if (kw > 0) return;
#pragma unroll
    for (int q = 1; q < kKSplit; ++q) {
      acc[0] += red[wave + q][0][lane];
      acc[1] += red[wave + q][1][lane];
    }
  }
  // acc[t][i] = result for weight row n_t + 4 kb + i and the entry's row r16.
  if (!tok_on || !t0_on) return;
  uint16_t *crow = c + static_cast<size_t>(dst_row) * ldc;
  if (kSwiglu) {
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t gu = moe::pack_bf16x2(acc[0][i], acc[1][i]);
      o[i] = moe::swiglu_clamp1(__uint_as_float(gu << 16), __uint_as_float(gu & 0xFFFF0000u),
                                limit);
    }
    uint2 v;
    v.x = moe::pack_bf16x2(o[0], o[1]);
    v.y = moe::pack_bf16x2(o[2], o[3]);
    *reinterpret_cast<uint2 *>(crow + n_t0 + 4 * kb) = v;
  } else {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t == 0 || t1_on) {
        uint2 v;
        v.x = moe::pack_bf16x2(acc[t][0], acc[t][1]);
        v.y = moe::pack_bf16x2(acc[t][2], acc[t][3]);
        *reinterpret_cast<uint2 *>(crow + (t == 0 ? n_t0 : n_t1) + 4 * kb) = v;
      }
    }
  }
}

// K split across the waves of a 32-row group: each wave keeps at least a few steps.
int k_split(int32_t k) {
  const int n_steps = k / kChunkK;
  return n_steps >= 16 ? 4 : (n_steps >= 8 ? 2 : 1);
}

template <bool kSwiglu>
int launch_gemv_union(const char *name, int split, dim3 grid, void *stream, const uint16_t *a,
                      int64_t lda, int32_t a_rows, int32_t a_per_slot,
                      const uint64_t *packed_ptrs, const uint64_t *scale_ptrs,
                      const float *scale2, const int32_t *u_eid, const int32_t *u_slot,
                      int32_t rows, int32_t top_k, int32_t num_experts, uint16_t *c,
                      int64_t ldc, int32_t n, int32_t k, float limit) {
  const auto go = [&](auto kern) {
    return moe::launch(name, kern, grid, dim3(kThreads), 0, stream, a, lda, a_rows, a_per_slot,
                       packed_ptrs, scale_ptrs, scale2, u_eid, u_slot, rows, top_k, num_experts,
                       c, ldc, n, k, limit);
  };
  if (split == 4) return go(gemv_union_kernel<kSwiglu, 4>);
  if (split == 2) return go(gemv_union_kernel<kSwiglu, 2>);
  return go(gemv_union_kernel<kSwiglu, 1>);
}

int check_union_gemv_args(const char *name, const uint16_t *a, int64_t lda, int32_t a_rows,
                          const uint64_t *packed_ptrs, const uint64_t *scale_ptrs,
                          const float *scale2, const int32_t *u_eid, const int32_t *u_slot,
                          int32_t rows, int32_t top_k, int32_t num_experts, const uint16_t *c,
                          int64_t ldc, int32_t n, int32_t n_out, int32_t k) {
  MOE_REQUIRE(rows >= 0 && rows <= kMaxRows, "%s: rows must be in [0, %d] (got %d)", name,
              kMaxRows, rows);
  MOE_REQUIRE(top_k >= 1 && static_cast<int64_t>(rows) * top_k <= kUnionMaxIds,
              "%s: need top_k >= 1 and rows * top_k <= %d", name, kUnionMaxIds);
  MOE_REQUIRE(k > 0 && k % kChunkK == 0, "%s: k must be a positive multiple of %d (got %d)",
              name, kChunkK, k);
  MOE_REQUIRE(n > 0 && n % 16 == 0, "%s: n must be a positive multiple of 16 (got %d)", name, n);
  MOE_REQUIRE(lda >= k && lda % 8 == 0, "%s: lda must be >= k and a multiple of 8", name);
  MOE_REQUIRE(ldc >= n_out && ldc % 4 == 0, "%s: ldc must be >= %d and a multiple of 4", name,
              n_out);
  MOE_REQUIRE(num_experts >= 1, "%s: num_experts must be >= 1", name);
  MOE_REQUIRE(a && packed_ptrs && scale_ptrs && scale2 && u_eid && u_slot && c,
              "%s: a required pointer is NULL", name);
  MOE_REQUIRE(moe::aligned16(a), "%s: a must be 16-byte aligned", name);
  MOE_REQUIRE((reinterpret_cast<uintptr_t>(c) & 7u) == 0, "%s: c must be 8-byte aligned", name);
  MOE_REQUIRE(a_rows >= 1 && static_cast<uint64_t>(a_rows) * lda * 2 < (1ull << 31),
              "%s: need a_rows >= 1 and an activation buffer smaller than 2 GiB", name);
  MOE_REQUIRE(static_cast<uint64_t>(n) * k / 2 < (1ull << 32),
              "%s: one expert's packed weights must be smaller than 4 GiB", name);
  return MOE_OK;
}

}  // namespace

extern "C" int moe_row_union(const int32_t *topk_ids, int32_t rows, int32_t top_k,
                             int32_t num_experts, int32_t *u_eid, int32_t *u_slot,
                             int32_t *slot_perm, int32_t *counters, void *stream) {
  moe::clear_error();
  MOE_REQUIRE(rows >= 0 && top_k >= 1 && num_experts >= 1,
              "row_union: need rows >= 0, top_k >= 1, num_experts >= 1");
  MOE_REQUIRE(static_cast<int64_t>(rows) * top_k <= kUnionMaxIds,
              "row_union: rows * top_k must be <= %d (got %lld)", kUnionMaxIds,
              static_cast<long long>(rows) * top_k);
  if (rows == 0) return MOE_OK;
  MOE_REQUIRE(topk_ids && u_eid && u_slot, "row_union: a required pointer is NULL");
  const int n_ids = rows * top_k;
  const int threads = (n_ids + 63) / 64 * 64;
  return moe::launch("moe_row_union", row_union_kernel, dim3(1), dim3(threads), 0, stream,
                     topk_ids, rows, top_k, num_experts, u_eid, u_slot, slot_perm, counters);
}

extern "C" int moe_w4a16_gemv_union(const uint16_t *a, int64_t lda, int32_t a_rows,
                                    int32_t a_per_slot, const uint64_t *packed_ptrs,
                                    const uint64_t *scale_ptrs, const float *scale2,
                                    const int32_t *u_eid, const int32_t *u_slot, int32_t rows,
                                    int32_t top_k, int32_t num_experts, uint16_t *c,
                                    int64_t ldc, int32_t n, int32_t k, void *stream) {
  moe::clear_error();
  const int rc = check_union_gemv_args("gemv_union", a, lda, a_rows, packed_ptrs, scale_ptrs,
                                       scale2, u_eid, u_slot, rows, top_k, num_experts, c, ldc,
                                       n, n, k);
  if (rc != MOE_OK || rows == 0) return rc;
  const int split = k_split(k);
  const int rows_per_block = 32 * (kWaves / split);
  const dim3 grid((n + rows_per_block - 1) / rows_per_block, rows * top_k);
  return launch_gemv_union<false>("moe_w4a16_gemv_union", split, grid, stream, a, lda, a_rows,
                                  a_per_slot != 0, packed_ptrs, scale_ptrs, scale2, u_eid, u_slot,
                                  rows, top_k, num_experts, c, ldc, n, k, 0.0f);
}

extern "C" int moe_w4a16_gemv_union_swiglu(const uint16_t *a, int64_t lda, int32_t a_rows,
                                           int32_t a_per_slot, const uint64_t *packed_ptrs,
                                           const uint64_t *scale_ptrs, const float *scale2,
                                           const int32_t *u_eid, const int32_t *u_slot,
                                           int32_t rows, int32_t top_k, int32_t num_experts,
                                           uint16_t *act, int64_t ld_act, int32_t mi,
                                           int32_t k, float limit, void *stream) {
  moe::clear_error();
  MOE_REQUIRE(mi > 0 && mi % 16 == 0 && mi <= (1 << 29),
              "gemv_union_swiglu: mi must be a positive multiple of 16 (got %d)", mi);
  MOE_REQUIRE(limit > 0.0f, "gemv_union_swiglu: limit must be > 0");
  const int rc = check_union_gemv_args("gemv_union_swiglu", a, lda, a_rows, packed_ptrs,
                                       scale_ptrs, scale2, u_eid, u_slot, rows, top_k,
                                       num_experts, act, ld_act, 2 * mi, mi, k);
  if (rc != MOE_OK || rows == 0) return rc;
  const int split = k_split(k);
  const int gate_rows_per_block = 16 * (kWaves / split);
  const dim3 grid((mi + gate_rows_per_block - 1) / gate_rows_per_block, rows * top_k);
  return launch_gemv_union<true>("moe_w4a16_gemv_union_swiglu", split, grid, stream, a, lda,
                                 a_rows, a_per_slot != 0, packed_ptrs, scale_ptrs, scale2, u_eid,
                                 u_slot, rows, top_k, num_experts, act, ld_act, 2 * mi, k, limit);
}
