// Decode / verify path for a few rows: moe_row_union and moe_w4a16_gemv_union (and its
// SwiGLU-fused form).
//
// What it computes follows "glm5next_mlp/forward.rs" (2026-09-25): the workspace fields
// u_eid (union expert ids, -1 = entry unused) and u_slot (slot per union entry per row, -1
// = row absent), the row-batched GEMV that sweeps each expert of the rows' union once and
// writes C[rows, top_k, N], and moe_row_groups' statement that which rows share a sweep
// never changes what a row adds. The union is found in one workgroup without a sort (one
// wave's ballots up to 64 ids; above, a per-expert LDS map, or pairwise scans for expert
// ids past the map); the outputs are laid out by (row, slot), so the combine reads them
// back through slot_perm without an expert-sorted permutation.
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
//     scales are one aligned dword of the row's 16 scale bytes, and its B operand is 128
//     contiguous bytes of the entry's token r16, put in the decoder's k order. The
//     activations are loaded one step ahead. With at most 16 rows a launch loads them
//     straight into the B layout (8 loads per lane and step); with at most 8 rows each
//     wave stages its step's tokens in a private piece of LDS instead: one 16-byte load
//     per lane covers two tokens' 512 bytes, so a step takes rows / 2 loads (rounded up
//     to 1, 2 or 4), and the B operands are read back from LDS. Each wave reads different
//     steps, so the staging is per wave, with no barrier.
//   - SwiGLU-fused form: a wave's two tiles are 16 gate rows and the matching 16 up rows,
//     rounded to BF16 and passed through the clamped SwiGLU in the epilogue (as the grouped
//     GEMM's fused form).
#include "buffer_io.h"
#include "common.h"
#include "nvfp4_decode.h"
#include "swiglu.h"
#include "w4a16_mma.h"

#include <type_traits>

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
    const uint64_t *__restrict__ present, int32_t *__restrict__ u_eid,
    int32_t *__restrict__ u_slot, int32_t *__restrict__ slot_perm,
    int32_t *__restrict__ counters) {
  __shared__ int32_t s_id[kUnionMaxIds];    // id of a covered slot, else -1
  __shared__ int32_t s_uid[kUnionMaxIds];   // union entries in order
  __shared__ int32_t s_wave_first[kUnionMaxIds / 64];
  const int n_ids = rows * top_k;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r = t / top_k, j = t - r * top_k;

  // 1. A slot is covered when its id is in range, its expert present and no lower slot
  //    of its row has it.
  int id = -1;
  if (t < n_ids) {
    const int v = ids[t];
    if (v >= 0 && v < num_experts && (present == nullptr || present[v] != 0)) id = v;
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

// The same table for 65 to 1024 ids when the expert ids fit a table in LDS: instead of
// pairwise scans, each expert's lowest covered slot comes from an LDS atomic minimum (the
// minimum does not depend on the order of the atomics), the openers are numbered by a
// block-wide count in slot order, and every covered slot writes its one u_slot entry
// over a table first filled with -1.
constexpr int kUnionMapExperts = 8192;  // experts an LDS map covers (32 KB)

__global__ __launch_bounds__(kUnionMaxIds) void row_union_map_kernel(
    const int32_t *__restrict__ ids, int32_t rows, int32_t top_k, int32_t num_experts,
    const uint64_t *__restrict__ present, int32_t *__restrict__ u_eid,
    int32_t *__restrict__ u_slot, int32_t *__restrict__ slot_perm,
    int32_t *__restrict__ counters) {
  __shared__ int32_t s_id[kUnionMaxIds];          // valid id of a slot, else -1
  __shared__ int32_t s_map[kUnionMapExperts];     // expert -> lowest covered slot -> entry
  __shared__ int32_t s_wave_open[kUnionMaxIds / 64], s_wave_cov[kUnionMaxIds / 64];
  const int n_ids = rows * top_k;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n_waves = static_cast<int>(blockDim.x >> 6);
  const int r = t / top_k, j = t - r * top_k;

  int id = -1;
  if (t < n_ids) {
    const int v = ids[t];
    if (v >= 0 && v < num_experts && (present == nullptr || present[v] != 0)) id = v;
  }
  s_id[t] = id;
  for (int e = t; e < num_experts; e += blockDim.x) s_map[e] = INT32_MAX;
  __syncthreads();
  // 1. Covered: valid and no lower slot of the row holds the same id.
  bool covered = id >= 0;
  for (int jj = 0; covered && jj < j; ++jj) covered = s_id[r * top_k + jj] != id;
  if (covered) atomicMin(&s_map[id], t);
  __syncthreads();
  // 2. An opener is its expert's lowest covered slot; entries are numbered in slot order.
  const bool opens = covered && s_map[id] == t;
  const uint64_t m_open = __ballot(opens), m_cov = __ballot(covered);
  if (lane == 0) {
    s_wave_open[wave] = __popcll(m_open);
    s_wave_cov[wave] = __popcll(m_cov);
  }
  __syncthreads();
  int base = 0, n_union = 0, n_cov = 0;
  for (int w = 0; w < n_waves; ++w) {
    if (w < wave) base += s_wave_open[w];
    n_union += s_wave_open[w];
    n_cov += s_wave_cov[w];
  }
  const int p_open = base + __popcll(m_open & ((1ull << lane) - 1ull));
  if (opens) s_map[id] = p_open;  // the expert's entry, for every covered slot
  // 3. Outputs: u_eid and slot_perm directly; u_slot filled with -1, then each covered
  //    slot's entry (the barrier orders the two writes of an element).
  if (t < n_ids) {
    if (opens) u_eid[p_open] = id;
    if (t >= n_union) u_eid[t] = -1;
    if (slot_perm != nullptr) slot_perm[t] = covered ? t : -1;
  }
  for (int q = t; q < n_ids * rows; q += blockDim.x) u_slot[q] = -1;
  __syncthreads();
  if (covered) u_slot[static_cast<int64_t>(s_map[id]) * rows + r] = j;
  if (counters != nullptr && t == 0) {
    counters[0] = n_union;
    counters[1] = n_ids - n_cov;
  }
}

// The same table for at most 64 ids, in one wave and without scans: lane t holds slot t.
// The lanes holding the same valid id are found with one ballot per id bit; a slot is
// covered when no lower lane of its row has its id, and opens an entry when no lower
// covered lane has it. An entry's number is the count of openers below its opener.
__global__ __launch_bounds__(64) void row_union_wave_kernel(
    const int32_t *__restrict__ ids, int32_t rows, int32_t top_k, int32_t num_experts,
    const uint64_t *__restrict__ present, int32_t *__restrict__ u_eid,
    int32_t *__restrict__ u_slot, int32_t *__restrict__ slot_perm,
    int32_t *__restrict__ counters) {
  __shared__ int32_t s_slot[64 * 64];  // u_slot: [n_ids][rows], n_ids * rows <= 64 * 64
  const int n_ids = rows * top_k;
  const int t = threadIdx.x;
  const int r = t / top_k, j = t - r * top_k;
  int id = -1;
  if (t < n_ids) {
    const int v = ids[t];
    if (v >= 0 && v < num_experts && (present == nullptr || present[v] != 0)) id = v;
  }
  const bool valid = id >= 0;
  const int bits = num_experts > 1 ? 32 - __clz(num_experts - 1) : 1;
  uint64_t same = __ballot(valid);
  for (int b = 0; b < bits; ++b) {  // lanes whose valid id has the same bits as this one
    const bool bit = (id >> b) & 1;
    const uint64_t ones = __ballot(valid && bit);
    same &= bit ? ones : ~ones;
  }
  const uint64_t below = (1ull << t) - 1ull;
  const uint64_t row_below = below & ~((1ull << (t - j)) - 1ull);  // lower lanes of the row
  const bool covered = valid && (same & row_below) == 0;
  const uint64_t cov = __ballot(covered);
  const bool opens = covered && (same & cov & below) == 0;
  const uint64_t openers = __ballot(opens);
  const int n_union = __popcll(openers);
  for (int q = t; q < n_ids * rows; q += 64) s_slot[q] = -1;
  __syncthreads();
  if (covered) {
    const int first = __ffsll(static_cast<long long>(same & cov)) - 1;  // the entry's opener
    const int p = __popcll(openers & ((1ull << first) - 1ull));
    s_slot[p * rows + r] = j;
  }
  __syncthreads();
  if (t < n_ids) {
    if (opens) u_eid[__popcll(openers & below)] = id;
    if (t >= n_union) u_eid[t] = -1;
    if (slot_perm != nullptr) slot_perm[t] = covered ? t : -1;
  }
  for (int q = t; q < n_ids * rows; q += 64) u_slot[q] = s_slot[q];
  if (counters != nullptr && t == 0) {
    counters[0] = n_union;
    counters[1] = n_ids - __popcll(cov);
  }
}

// ------------------------------------------------------------------------- union GEMV

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kChunkK = 256;       // k per step
constexpr int kMaxRows = 16;       // routed rows a launch may have: one MFMA tile of B
constexpr int kSlotsPerCu = 3;     // resident blocks per CU (VGPR-limited)
constexpr int kCus = 256;
constexpr int64_t kLdsPerCu = 160 * 1024;
constexpr int kGemvMaxIds = 512;   // rows * top_k: the entries' metadata live in LDS
static_assert(kThreads == 256, "build_code_table_lut: one E4M3 code per thread");

// One lane's data of one step: packed weights of its two tiles (k in [64 kb, 64 kb + 32)
// and [64 kb + 32, 64 kb + 64)), the four block-scale codes of each tile, and its
// activations: loaded directly (kNQ = 0), its token's 64 k in eight 16-byte pieces;
// staged, kNQ 16-byte pieces, each of a pair of tokens' step, on their way to LDS.
template <int kNQ>
struct StepRegs {
  u32x4_t wa[2], wb[2];
  uint32_t sc[2];
  u32x4_t x[kNQ ? kNQ : 8];
};
// Staged activations: a token's 256 k of a step (512 bytes), rows padded to 528 bytes so
// that the 16 lanes of a B read that differ in token start on different banks.
constexpr int kXsRowBytes = kChunkK * 2 + 16;

// A live union entry (its expert present in the table), as the block's waves read it.
struct LiveEntry {
  uint64_t packed, scales;
  float scale2;
  int32_t p;  // union entry
};
// Dynamic LDS per union entry: the entry (if live) and the output row of each of its up
// to 16 tokens (the entry's routed rows in order; -1 past the last).
constexpr int kEntryLdsBytes = static_cast<int>(sizeof(LiveEntry)) + 16 * 2;

// One work item as a wave sees it: the expert's buffers and scale2 (uniform), the rows of
// the wave's two tiles as byte offsets into them (uniform: they ride in the scalar offset
// of the buffer loads; a tile past the last row is off and loads nothing), and the lane's
// activation row and output row (the entry's token r16).
struct Item {
  __amdgpu_buffer_rsrc_t w, s;
  uint32_t w_base[2], s_base[2];
  float scale2;
  bool on[2];
  uint32_t x_voff;  // per lane, kNoLoad if the lane has no token
  int32_t dst_row;  // per lane, -1 if the lane has no token
  uint32_t xq[4];   // staged: offset of this lane's 16 bytes of token 2 q + lane / 32
};

// The work of a launch is (live entry, group of 32 * kGroups weight rows) items, dealt to
// the persistent blocks round-robin. Items are alike (the same rows and K), so a static
// deal is balanced, and a block streams its items back to back: the waves load the next
// item's first step while computing the current item's last one, and each item's decode
// table is built during the item before it (double-buffered), so no item pays a start-up.
template <bool kSwiglu, int kKSplit, int kNQ>
__global__ __launch_bounds__(kThreads, kSlotsPerCu) void gemv_union_kernel(
    const uint16_t *__restrict__ a, int64_t lda, int32_t a_rows, int32_t a_per_slot,
    const uint64_t *__restrict__ packed_ptrs, const uint64_t *__restrict__ scale_ptrs,
    const float *__restrict__ scale2s, const int32_t *__restrict__ u_eid,
    const int32_t *__restrict__ u_slot, int32_t rows, int32_t top_k, int32_t num_experts,
    uint16_t *__restrict__ c, int64_t ldc, int32_t N, int32_t K, float limit) {
  constexpr int kGroups = kWaves / kKSplit;  // 32-row groups per item
  constexpr int kItemRows = kSwiglu ? 16 * kGroups : 32 * kGroups;  // gate rows if fused
  __shared__ __attribute__((aligned(16))) uint8_t lut[2][256 * 16];
  __shared__ __attribute__((aligned(16))) f32x4_t red[2][kWaves][2][64];
  __shared__ __attribute__((aligned(16))) uint8_t xs[kNQ ? kWaves * 2 * kNQ * kXsRowBytes : 16];
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
  __shared__ int32_t n_live_s;
  const int n_ids = rows * top_k;
  LiveEntry *live = reinterpret_cast<LiveEntry *>(dyn_lds);
  int16_t *tok = reinterpret_cast<int16_t *>(dyn_lds + n_ids * sizeof(LiveEntry));  // [n_ids][16]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave % kKSplit, nw = wave / kKSplit;
  const int r16 = lane & 15, kb = lane >> 4;
  const int mi = N / 2;
  const int row_end0 = kSwiglu ? mi : N;
  const int items_per_entry = (row_end0 + kItemRows - 1) / kItemRows;
  const uint32_t row_bytes = static_cast<uint32_t>(K) / 2, srow_bytes = static_cast<uint32_t>(K) / 16;
  const int n_steps = K / kChunkK;
  const int n_mine = n_steps > kw ? (n_steps - kw + kKSplit - 1) / kKSplit : 0;
  // Lane parts of the weight and scale offsets (row r16 of a tile, bytes for k in
  // [64 kb, 64 kb + 64) of a step); the tile's rows and the step go in the scalar offset.
  const uint32_t w_lane = static_cast<uint32_t>(r16) * row_bytes + 32u * kb;
  const uint32_t s_lane = static_cast<uint32_t>(r16) * srow_bytes + 4u * kb;

  // The live entries, compacted in LDS by wave 0: an entry with an expert id in range and
  // a non-null table address.
  if (wave == 0) {
    int n = 0;
    for (int q0 = 0; q0 < n_ids; q0 += 64) {
      const int q = q0 + lane;
      const int e = q < n_ids ? u_eid[q] : -1;
      const bool in = e >= 0 && e < num_experts;
      // the entry's three table values in one round trip
      const uint64_t pk = in ? packed_ptrs[e] : 0;
      const uint64_t sp = in ? scale_ptrs[e] : 0;
      const float s2 = in ? scale2s[e] : 0.0f;
      const bool ok = pk != 0;
      const uint64_t m = __ballot(ok);
      if (ok) {
        LiveEntry le;
        le.packed = pk;
        le.scales = sp;
        le.scale2 = s2;
        le.p = q;
        live[n + __popcll(m & ((1ull << lane) - 1ull))] = le;
      }
      n += __popcll(m);
    }
    if (lane == 0) n_live_s = n;
  }
  __syncthreads();
  const int n_live = n_live_s;
  const int n_items = n_live * items_per_entry;
  if (static_cast<int>(blockIdx.x) >= n_items) return;  // uniform: the whole block
  // readfirstlane works on int: widen through uint32_t, so that a low word with its top
  // bit set is not sign-extended into the high word of an address.
  const auto rfl32 = [](uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
  };
  const auto rfl64 = [&](uint64_t v) {
    return (static_cast<uint64_t>(rfl32(static_cast<uint32_t>(v >> 32))) << 32) |
           static_cast<uint64_t>(rfl32(static_cast<uint32_t>(v)));
  };
  const __amdgpu_buffer_rsrc_t x_rsrc =
      make_rsrc(a, static_cast<uint32_t>(a_rows) * static_cast<uint32_t>(lda) * 2u);
  // Item it without its tokens: its entry's buffers (uniform) and its rows.
  const auto make_item_w = [&](int it) {
    Item m;
    const int li = it / items_per_entry, g = it - li * items_per_entry;
    const LiveEntry &le = live[li];
    m.w = make_rsrc(reinterpret_cast<const void *>(rfl64(le.packed)), static_cast<uint32_t>(N) * row_bytes);
    m.s = make_rsrc(reinterpret_cast<const void *>(rfl64(le.scales)), static_cast<uint32_t>(N) * srow_bytes);
    m.scale2 = __builtin_bit_cast(float, rfl32(__builtin_bit_cast(uint32_t, le.scale2)));
    const int n_t0 = kSwiglu ? (g * kGroups + nw) * 16 : (g * kGroups + nw) * 32;
    const int n_t1 = kSwiglu ? mi + n_t0 : n_t0 + 16;
    m.on[0] = n_t0 < row_end0;
    m.on[1] = n_t1 < N && (!kSwiglu || m.on[0]);
    m.w_base[0] = static_cast<uint32_t>(n_t0) * row_bytes;
    m.w_base[1] = static_cast<uint32_t>(n_t1) * row_bytes;
    m.s_base[0] = static_cast<uint32_t>(n_t0) * srow_bytes;
    m.s_base[1] = static_cast<uint32_t>(n_t1) * srow_bytes;
    return m;
  };
  // This lane's token of item it (the entry's token r16: output row and input row).
  const auto set_tokens = [&](Item &m, int it) {
    const int li = it / items_per_entry;
    m.dst_row = tok[li * 16 + r16];
    const int src = m.dst_row < 0 ? -1 : (a_per_slot ? m.dst_row : m.dst_row / top_k);
    m.x_voff = (src >= 0 && src < a_rows)
                   ? (static_cast<uint32_t>(src) * static_cast<uint32_t>(lda) + 64u * kb) * 2u
                   : kNoLoad;
    if (kNQ) {
      // Staged: the lane loads bytes [16 (lane % 32), + 16) of each step of token
      // 2 q + lane / 32 (zeros past the entry's tokens).
#pragma unroll
      for (int q = 0; q < kNQ; ++q) {
        const int tq = tok[li * 16 + 2 * q + (lane >> 5)];
        const int sq = tq < 0 ? -1 : (a_per_slot ? tq : tq / top_k);
        uint32_t row_off = static_cast<uint32_t>(sq) * static_cast<uint32_t>(lda);
        asm volatile("" : "+v"(row_off));
        m.xq[q] = (sq >= 0 && sq < a_rows) ? row_off * 2u + 16u * (lane & 31) : kNoLoad;
      }
    }
  };
  // The whole Item of it: its entry's buffers (uniform), its rows, this lane's token.
  const auto make_item = [&](int it) {
    Item m = make_item_w(it);
    set_tokens(m, it);
    return m;
  };
  // Step i of this wave's share of an item (steps kw, kw + kKSplit, ...); live = false
  // loads nothing, so every load stays unconditional.
  const auto load_w = [&](StepRegs<kNQ> &st, const Item &m, int i, bool live_step) {
    const int step = kw + i * kKSplit;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bool on = live_step && m.on[t];
      const uint32_t v = on ? w_lane : kNoLoad;
      const uint32_t soff = m.w_base[t] + static_cast<uint32_t>(step) * (kChunkK / 2);
      st.wa[t] = load16(m.w, v, soff);
      st.wb[t] = load16(m.w, v + 16, soff);
      st.sc[t] = __builtin_amdgcn_raw_buffer_load_b32(
          m.s, static_cast<int>(on ? s_lane : kNoLoad),
          static_cast<int>(m.s_base[t] + static_cast<uint32_t>(step) * 16u), 0);
    }
  };
  const auto load_x = [&](StepRegs<kNQ> &st, const Item &m, int i, bool live_step) {
    const int step = kw + i * kKSplit;
    const uint32_t xsoff = static_cast<uint32_t>(step) * (kChunkK * 2);
    if (kNQ) {
#pragma unroll
      for (int q = 0; q < kNQ; ++q) st.x[q] = load16(x_rsrc, live_step ? m.xq[q] : kNoLoad, xsoff);
    } else {
      const uint32_t xv = live_step ? m.x_voff : kNoLoad;
#pragma unroll
      for (int q = 0; q < 8; ++q) st.x[q] = load16(x_rsrc, xv + 16u * q, xsoff);
    }
  };
  const auto load_step = [&](StepRegs<kNQ> &st, const Item &m, int i, bool live_step) {
    load_w(st, m, i, live_step);
    load_x(st, m, i, live_step);
  };

  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  // The tables of blocks 2h, 2h + 1 (bytes of sc) are read per half, which keeps half of
  // them out of the registers at a time.
  const auto tables_of = [&](uint32_t sc, int h, const uint8_t *tab, moe::Fp4Table *blk) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const u32x4_t t = *reinterpret_cast<const u32x4_t *>(
          tab + (((sc >> (8 * (2 * h + g))) & 0xFFu) << 4));
      blk[g].lo03 = t[0];
      blk[g].lo47 = t[1];
      blk[g].hi03 = t[2];
      blk[g].hi47 = t[3];
    }
  };
  // Staged form: this wave's piece of LDS holds the step's 2 kNQ tokens, each group of 8 k
  // already in the decoder's order. Lane l writes its 16 bytes of token 2 q + l / 32 and
  // reads its B operand from token r16; a lane past the staged tokens (r16 >= 2 kNQ >=
  // rows) has no token and reads token r16 mod 2 kNQ, a column that is never stored.
  // Writes of a step follow the reads of the step before in the wave's program order, so
  // one piece per wave suffices.
  uint8_t *xs_w = xs + wave * (2 * (kNQ ? kNQ : 1) * kXsRowBytes);
  const int xs_tok = kNQ ? r16 % (2 * (kNQ ? kNQ : 1)) : 0;
  const auto run_step = [&](const StepRegs<kNQ> &st, const uint8_t *tab, bool t1_on) {
    if (kNQ) {
#pragma unroll
      for (int q = 0; q < kNQ; ++q)
        *reinterpret_cast<u32x4_t *>(xs_w + (2 * q + (lane >> 5)) * kXsRowBytes + 16 * (lane & 31)) =
            moe::permute_k8(st.x[q]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      moe::Fp4Table blk0[2], blk1[2];
      tables_of(st.sc[0], h, tab, blk0);
      tables_of(st.sc[1], h, tab, blk1);
      bf16x8_t B[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4_t xv = kNQ ? *reinterpret_cast<const u32x4_t *>(
                                     xs_w + xs_tok * kXsRowBytes + 128 * kb + 16 * (4 * h + q))
                               : moe::permute_k8(st.x[(4 * h + q) % (kNQ ? kNQ : 8)]);
        B[q] = __builtin_bit_cast(bf16x8_t, xv);
      }
      const u32x4_t &x0 = h ? st.wb[0] : st.wa[0];
      const uint32_t w0w[4] = {x0[0], x0[1], x0[2], x0[3]};
      moe::mfma4(w0w, blk0[0], blk0[1], B, acc[0]);
      if (t1_on) {
        const u32x4_t &x1 = h ? st.wb[1] : st.wa[1];
        const uint32_t w1w[4] = {x1[0], x1[1], x1[2], x1[3]};
        moe::mfma4(w1w, blk1[0], blk1[1], B, acc[1]);
      }
    }
  };

  // The first item's weights go out before the token maps are built (they need only its
  // entry), its activations after.
  int item = blockIdx.x;
  Item cur = make_item_w(item);
  StepRegs<kNQ> sA, sB;
  load_w(sA, cur, 0, true);

  // Each live entry's tokens: its routed rows (u_slot[p, r] >= 0) in order of r, as
  // output rows r * top_k + slot. A wave reads the u_slot rows of 64 / rows entries at
  // once, one lane per (entry, row); a present row's token index is its rank in its
  // entry's lanes.
  for (int q = tid; q < n_live * 16; q += kThreads) tok[q] = -1;
  __syncthreads();
  {
    const int epw = 64 / rows;  // entries per wave and pass (rows >= 1 here)
    const int le_lane = lane / rows, r = lane - le_lane * rows;
    const int seg0 = le_lane * rows;
    for (int base = wave * epw; base < n_live; base += kWaves * epw) {
      const int li = base + le_lane;
      const bool mine = le_lane < epw && li < n_live;
      const int slot = mine ? u_slot[static_cast<int64_t>(live[li].p) * rows + r] : -1;
      const uint64_t m = __ballot(slot >= 0);
      if (slot >= 0) {
        const uint64_t below = (1ull << lane) - 1ull, seg_below = (1ull << seg0) - 1ull;
        const int rank = __popcll(m & below & ~seg_below);
        tok[li * 16 + rank] = static_cast<int16_t>(r * top_k + slot);
      }
    }
  }
  __syncthreads();

  const int G = gridDim.x;
  set_tokens(cur, item);
  load_x(sA, cur, 0, true);
  moe::build_code_table_lut(lut[0], tid, cur.scale2);
  __syncthreads();  // table 0 is complete

  for (int j = 0;; ++j) {
    const bool has_next = item + G < n_items;
    const Item nxt = make_item(has_next ? item + G : item);
    if (has_next) moe::build_code_table_lut(lut[(j + 1) & 1], tid, nxt.scale2);
    const uint8_t *tab = lut[j & 1];

    // This item's steps in pairs: slot A holds step i, slot B takes step i + 1; after an
    // odd share, the pair's second step is empty. The step after this item's last is the
    // next item's first, into slot A. The last pair is peeled out of the loop, so the
    // pairs before it load from this item with no per-pair selects between the two items
    // (down GEMV at 8 rows 60.5-62.3 -> 59.6-60.0 us, gate_up level, same bits).
    int i = 0;
    for (; i + 2 < n_mine; i += 2) {
      load_step(sB, cur, i + 1, true);
      if (cur.on[0]) run_step(sA, tab, cur.on[1]);
      load_step(sA, cur, i + 2, true);
      if (cur.on[0]) run_step(sB, tab, cur.on[1]);
    }
    if (i < n_mine) {  // uniform
      load_step(sB, cur, i + 1, i + 1 < n_mine);
      if (cur.on[0]) run_step(sA, tab, cur.on[1]);
      load_step(sA, nxt, 0, has_next);
      if (i + 1 < n_mine && cur.on[0]) run_step(sB, tab, cur.on[1]);
    }

    // Sum the kKSplit partial tiles of each 32-row group in wave order, store.
    if (kKSplit > 1 && kw > 0) {
      red[j & 1][wave][0][lane] = acc[0];
      red[j & 1][wave][1][lane] = acc[1];
    }
    __syncthreads();  // the partials and the next table are complete
    if (kw == 0) {
#pragma unroll
      for (int q = 1; q < kKSplit; ++q) {
        acc[0] += red[j & 1][wave + q][0][lane];
        acc[1] += red[j & 1][wave + q][1][lane];
      }
      // acc[t][i] = result for weight row n_t + 4 kb + i and the entry's token r16.
      if (cur.dst_row >= 0 && cur.on[0]) {
        const int i0 = item / items_per_entry, g = item - i0 * items_per_entry;
        const int n_t0 = kSwiglu ? (g * kGroups + nw) * 16 : (g * kGroups + nw) * 32;
        const int n_t1 = kSwiglu ? mi + n_t0 : n_t0 + 16;
        uint16_t *crow = c + static_cast<size_t>(cur.dst_row) * ldc;
        if (kSwiglu) {
          float o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t gu = moe::pack_bf16x2(acc[0][i], acc[1][i]);
            o[i] = moe::swiglu_clamp1(__uint_as_float(gu << 16),
                                      __uint_as_float(gu & 0xFFFF0000u), limit);
          }
          uint2 v;
          v.x = moe::pack_bf16x2(o[0], o[1]);
          v.y = moe::pack_bf16x2(o[2], o[3]);
          *reinterpret_cast<uint2 *>(crow + n_t0 + 4 * kb) = v;
        } else {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if (t == 0 || cur.on[1]) {
              uint2 v;
              v.x = moe::pack_bf16x2(acc[t][0], acc[t][1]);
              v.y = moe::pack_bf16x2(acc[t][2], acc[t][3]);
              *reinterpret_cast<uint2 *>(crow + (t == 0 ? n_t0 : n_t1) + 4 * kb) = v;
            }
          }
        }
      }
    }
    acc[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (!has_next) break;  // uniform
    item += G;
    cur = nxt;
  }
}

// K split across the waves of a 32-row group: each wave keeps at least a few steps.
int k_split(int32_t k) {
  const int n_steps = k / kChunkK;
  return n_steps >= 16 ? 4 : (n_steps >= 8 ? 2 : 1);
}

template <bool kSwiglu, int kNQ>
int launch_gemv_union_nq(const char *name, int split, int32_t item_rows, void *stream,
                      const uint16_t *a, int64_t lda, int32_t a_rows, int32_t a_per_slot,
                      const uint64_t *packed_ptrs, const uint64_t *scale_ptrs,
                      const float *scale2, const int32_t *u_eid, const int32_t *u_slot,
                      int32_t rows, int32_t top_k, int32_t num_experts, uint16_t *c,
                      int64_t ldc, int32_t n, int32_t k, float limit) {
  // At most every union entry is live: one block per item up to a full chip of resident
  // blocks. Three fit a CU unless the entries' metadata make the LDS the limit (with the
  // most ids a launch takes, 512, the staged forms fit two).
  const int64_t items =
      static_cast<int64_t>(rows) * top_k * (((kSwiglu ? n / 2 : n) + item_rows - 1) / item_rows);
  constexpr int64_t kStaticLds = 2 * 256 * 16 + 2 * kWaves * 2 * 64 * 16 +
                                 (kNQ ? kWaves * 2 * kNQ * kXsRowBytes : 16) + 64;
  const int64_t lds = kStaticLds + static_cast<int64_t>(rows) * top_k * kEntryLdsBytes;
  const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(kSlotsPerCu, kLdsPerCu / lds));
  const dim3 grid(static_cast<unsigned>(std::min<int64_t>(items, per_cu * kCus)));
  const auto go = [&](auto kern) {
    return moe::launch(name, kern, grid, dim3(kThreads),
                       static_cast<size_t>(rows) * top_k * kEntryLdsBytes, stream, a, lda, a_rows,
                       a_per_slot,
                       packed_ptrs, scale_ptrs, scale2, u_eid, u_slot, rows, top_k, num_experts,
                       c, ldc, n, k, limit);
  };
  if (split == 4) return go(gemv_union_kernel<kSwiglu, 4, kNQ>);
  if (split == 2) return go(gemv_union_kernel<kSwiglu, 2, kNQ>);
  return go(gemv_union_kernel<kSwiglu, 1, kNQ>);
}

// Activations staged through LDS per wave when a launch has at most 8 rows, loaded
// straight into the B layout above that.
template <bool kSwiglu>
int launch_gemv_union(const char *name, int split, int32_t item_rows, void *stream,
                      const uint16_t *a, int64_t lda, int32_t a_rows, int32_t a_per_slot,
                      const uint64_t *packed_ptrs, const uint64_t *scale_ptrs,
                      const float *scale2, const int32_t *u_eid, const int32_t *u_slot,
                      int32_t rows, int32_t top_k, int32_t num_experts, uint16_t *c,
                      int64_t ldc, int32_t n, int32_t k, float limit) {
  const auto go = [&](auto nq) {
    return launch_gemv_union_nq<kSwiglu, decltype(nq)::value>(
        name, split, item_rows, stream, a, lda, a_rows, a_per_slot, packed_ptrs, scale_ptrs,
        scale2, u_eid, u_slot, rows, top_k, num_experts, c, ldc, n, k, limit);
  };
  if (rows <= 2) return go(std::integral_constant<int, 1>{});
  if (rows <= 4) return go(std::integral_constant<int, 2>{});
  if (rows <= 8) return go(std::integral_constant<int, 4>{});
  return go(std::integral_constant<int, 0>{});
}

int check_union_gemv_args(const char *name, const uint16_t *a, int64_t lda, int32_t a_rows,
                          const uint64_t *packed_ptrs, const uint64_t *scale_ptrs,
                          const float *scale2, const int32_t *u_eid, const int32_t *u_slot,
                          int32_t rows, int32_t top_k, int32_t num_experts, const uint16_t *c,
                          int64_t ldc, int32_t n, int32_t n_out, int32_t k) {
  MOE_REQUIRE(rows >= 0 && rows <= kMaxRows, "%s: rows must be in [0, %d] (got %d)", name,
              kMaxRows, rows);
  MOE_REQUIRE(top_k >= 1 && static_cast<int64_t>(rows) * top_k <= kGemvMaxIds,
              "%s: need top_k >= 1 and rows * top_k <= %d", name, kGemvMaxIds);
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
  // Buffer offsets are 32-bit and a skipped load uses offset 2^31: one expert's packed
  // weights stay below 2 GiB.
  MOE_REQUIRE(static_cast<uint64_t>(n) * k / 2 < (1ull << 31),
              "%s: one expert's packed weights must be smaller than 2 GiB", name);
  return MOE_OK;
}

}  // namespace

extern "C" int moe_row_union(const int32_t *topk_ids, int32_t rows, int32_t top_k,
                             int32_t num_experts, const uint64_t *present, int32_t *u_eid,
                             int32_t *u_slot, int32_t *slot_perm, int32_t *counters,
                             void *stream) {
  moe::clear_error();
  MOE_REQUIRE(rows >= 0 && top_k >= 1 && num_experts >= 1,
              "row_union: need rows >= 0, top_k >= 1, num_experts >= 1");
  MOE_REQUIRE(static_cast<int64_t>(rows) * top_k <= kUnionMaxIds,
              "row_union: rows * top_k must be <= %d (got %lld)", kUnionMaxIds,
              static_cast<long long>(rows) * top_k);
  if (rows == 0) return MOE_OK;
  MOE_REQUIRE(topk_ids && u_eid && u_slot, "row_union: a required pointer is NULL");
  const int n_ids = rows * top_k;
  if (n_ids <= 64)
    return moe::launch("moe_row_union", row_union_wave_kernel, dim3(1), dim3(64), 0, stream,
                       topk_ids, rows, top_k, num_experts, present, u_eid, u_slot, slot_perm,
                       counters);
  const int threads = (n_ids + 63) / 64 * 64;
  if (num_experts <= kUnionMapExperts)
    return moe::launch("moe_row_union", row_union_map_kernel, dim3(1), dim3(threads), 0,
                       stream, topk_ids, rows, top_k, num_experts, present, u_eid, u_slot,
                       slot_perm, counters);
  return moe::launch("moe_row_union", row_union_kernel, dim3(1), dim3(threads), 0, stream,
                     topk_ids, rows, top_k, num_experts, present, u_eid, u_slot, slot_perm,
                     counters);
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
  return launch_gemv_union<false>("moe_w4a16_gemv_union", split, 32 * (kWaves / split), stream,
                                  a, lda, a_rows, a_per_slot != 0, packed_ptrs, scale_ptrs,
                                  scale2, u_eid, u_slot, rows, top_k, num_experts, c, ldc, n, k,
                                  0.0f);
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
  return launch_gemv_union<true>("moe_w4a16_gemv_union_swiglu", split, 16 * (kWaves / split),
                                 stream, a, lda, a_rows, a_per_slot != 0, packed_ptrs, scale_ptrs,
                                 scale2, u_eid, u_slot, rows, top_k, num_experts, act, ld_act,
                                 2 * mi, k, limit);
}
