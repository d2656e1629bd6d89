// moe_w4a16_grouped_gemm (and its SwiGLU-fused form): one launch over all experts of a
// routed MoE layer.
//
// What it computes follows "Module forward_prefill_gemm": the expert-sorted rows of
// each expert (expert_offsets prefix sum, rows gathered in-kernel through
// sorted_token_ids) are multiplied by that expert's NVFP4 weight, N-major [N, K/2] with
// the even k in the low nibble, E4M3 block scale per 16 k, FP32 scale2 per expert, each
// weight rounded to a BF16 operand, FP32 accumulation; a null table entry is skipped so
// the caller's zeros stand (layout table; "What is NOT bit-identical", item 2). The point
// of the grouped form ("What this replaces") is that each expert's weights are read from
// HBM once per launch.
//
// gfx950 design (the pages' mma.sync/shared-memory tiling is not used):
//   - grid = (N / 128 weight-row tiles, experts + overflow chunks); a block of 4 wave64s
//     owns 128 weight rows of one expert over the whole K, and loops over up to 64 of
//     that expert's sorted rows 16 at a time (one MFMA tile), so its weight bytes are
//     streamed once per 16 rows (once per launch for an expert with at most 16 routed
//     rows). An expert with more than 64 rows is cut into 64-row chunks, each chunk an
//     overflow block of its own, so a hot expert (skewed routing) is spread over several
//     blocks instead of making one block run many passes while the rest of the chip
//     idles. Three blocks share a CU.
//     Workgroups are dealt to the 8 XCDs round-robin by linear id, and the grid runs in
//     its natural order: an expert's weight-row tiles are spread over all eight XCDs, so
//     every XCD gets the same share of the work however skewed the routing.
//   - Each wave owns two MFMA tiles of 16 weight rows: block rows [16w, 16w + 16) and
//     [64 + 16w, 64 + 16w + 16). Both tiles multiply the same activation operands, so a
//     wave reads each staged activation once per 32 weight rows.
//   - The weights are the MFMA A operand (v_mfma_f32_16x16x32_bf16, M = 16 weight rows):
//     each lane reads 2 x 16 bytes of packed nibbles (64 k of one row) per tile and
//     256-k step with raw buffer loads (16 rows x 64 contiguous bytes per wave
//     instruction), one step ahead in a two-slot register ring, and decodes them in
//     registers (nvfp4_decode.h) straight into A; no dequantised weight goes through LDS.
//     The L1 can track only about a step's worth of a CU's weight lines, so a deeper ring
//     only leaves waves stalled at load issue instead of decoding. The decode is one
//     branch-free byte-table path for every scale code (nvfp4_decode.h).
//   - The gathered activation rows are the B operand (16 rows per MFMA tile). They are
//     loaded one step ahead into registers and staged per 256-k step in LDS
//     (double buffered, one barrier per step), shared by the 4 waves, with k permuted
//     inside each group of 8 to match the decoder's order.
//   - Block scales are read a whole 128-byte line (8 steps) per row at a time and staged
//     in LDS 4 steps at a time: the first half goes to LDS at once, the second half waits
//     in registers for its stage (reading half lines lets L2 evict a line between its two
//     halves, which doubles the scale traffic). Each block turns every E4M3 code into its
//     decode table once (a 256-entry LUT of the exact BF16 magnitudes for its scale2).
//   - Output: each lane holds 4 consecutive weight rows of one sorted row per tile, rounded
//     to BF16 (round-to-nearest-even) and put in LDS; the block then stores its output
//     tile 16 bytes per lane, consecutive lanes along an output row (whole 128-byte
//     lines; 8-byte stores from each lane measured 1 % slower on the down launch).
//   - SwiGLU-fused form: the weight is the fused gate_up projection (gate rows [0, mi),
//     up rows [mi, 2 mi)). A block owns gate rows [64 b, 64 b + 64) in its first tiles
//     and the matching up rows in its second tiles, so each lane holds the gate and up
//     sums of the same 4 columns; both are rounded to BF16 (the values the unfused path
//     would store) and the clamped SwiGLU (swiglu.h) is applied in registers. The gate_up
//     output never reaches memory.
#include "buffer_io.h"
#include "common.h"
#include "nvfp4_decode.h"
#include "swiglu.h"
#include "w4a16_mma.h"

namespace {

using moe::bf16x8_t;
using moe::f32x4_t;
using moe::u32x4_t;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTiles = 2;                         // MFMA tiles of 16 weight rows per wave
constexpr int kBlockN = kWaves * 16 * kTiles;     // weight rows per block
constexpr int kHalfN = kBlockN / 2;               // block rows per tile index
constexpr int kChunkK = 256;                      // k per main-loop step
constexpr int kBlockM = 16;                       // sorted rows per pass: one MFMA tile
constexpr int kChunkRows = 64;                    // sorted rows per block at most
constexpr int kFrontChunks = 16;                  // overflow rows dispatched before experts
constexpr int kLdsRowBytes = kChunkK * 2 + 16;    // staged activation row, padded
constexpr int kPiecesPerRow = kChunkK / 8;        // 16-byte pieces per staged row
constexpr int kXPieces = kBlockM * kPiecesPerRow / kThreads;  // per thread per step
constexpr int kXAhead = 1;                        // activation ring: steps in flight
constexpr int kStageSteps = 4;                    // steps per staged block of scales
constexpr int kLineSteps = 2 * kStageSteps;       // steps per 128-byte line of scales
constexpr int kScaleRowBytes = kStageSteps * 16 + 16;  // 4 steps x 16 scale bytes, padded
constexpr int kScaleBufBytes = kBlockN * kScaleRowBytes;
constexpr int kSPieces = kBlockN * kStageSteps / kThreads;  // scale pieces per thread
static_assert(kBlockM * kPiecesPerRow == kXPieces * kThreads, "whole activation pieces");
static_assert(kBlockN * kStageSteps == kSPieces * kThreads, "whole scale pieces");
static_assert(kSPieces == kTiles, "one scale piece per thread and tile half");

using moe::build_code_table_lut;
using moe::kNoLoad;
using moe::load16;
using moe::lut_blocks;
using moe::make_rsrc;
using moe::mfma4;
using moe::permute_k8;
static_assert(kThreads == 256, "build_code_table_lut: one E4M3 code per thread");

// One lane's packed weights of a step: per tile, 64 k of one row as two 16-byte loads;
// the wave reads 16 rows x 64 contiguous bytes per load.
struct WeightRegs {
  u32x4_t a[kTiles];  // k in [32 kb, 32 kb + 32) of the step
  u32x4_t b[kTiles];  // k in [128 + 32 kb, 128 + 32 kb + 32)
};

// Loads of a step past the last one get bit 31 set in their offset (past the end of any
// buffer below 2 GiB: zeros, no traffic), so every load stays unconditional (see the main
// loop) without re-reading data that L2 may already have evicted. The bit is set
// arithmetically: written as a select on the (uniform) step count, the compiler turned it
// into a branch around the loads, and its wait counting then assumed two more loads in
// flight after the join than there are, so each step's first decode also waited for the
// activation loads just issued for the next step (1-2 % of the launch).
__device__ __forceinline__ void load_weights(WeightRegs &w, __amdgpu_buffer_rsrc_t r,
                                             const uint32_t *voff, int step, int n_steps) {
  const uint32_t soff = static_cast<uint32_t>(step) * (kChunkK / 2);
  const uint32_t dead = static_cast<uint32_t>(step >= n_steps) << 31;
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    const uint32_t v = voff[t] | dead;
    w.a[t] = load16(r, v, soff);
    w.b[t] = load16(r, v + 64, soff);
  }
}

// A row's 16 scale bytes of one step -> four dwords, dword kb holding the bytes lane kb
// needs: groups 2kb, 2kb+1 (low half) and 8+2kb, 9+2kb (high half).
__device__ __forceinline__ u32x4_t permute_scales(u32x4_t v) {
  u32x4_t o;
  o[0] = moe::byte_perm(v[2], v[0], 0x05040100u);
  o[1] = moe::byte_perm(v[2], v[0], 0x07060302u);
  o[2] = moe::byte_perm(v[3], v[1], 0x05040100u);
  o[3] = moe::byte_perm(v[3], v[1], 0x07060302u);
  return o;
}

// Rows of expert e the grouped GEMM covers: [max(off[e], 0), min(off[e + 1], max_rows)).
// An expert with more than chunk_rows rows is done wholly by overflow blocks, one per
// chunk_rows-row chunk: overflow(e) = ceil(rows / chunk_rows) chunks, else none. Returns
// (expert, chunk index) of overflow chunk `oc` in expert order, or (-1, 0) when there are
// at most `oc` overflow chunks. Every thread of the block
// calls it (it holds barriers); all get the same answer.
__device__ int2 find_overflow_chunk(const int32_t *__restrict__ offsets, int num_experts,
                                    int chunk_rows, int max_rows, int oc) {
  __shared__ int s_wave_sum[kWaves];
  __shared__ int2 s_found;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_found = make_int2(-1, 0);
  int carry = 0;
  for (int base = 0; base < num_experts && carry <= oc; base += kThreads) {
    const int x = base + tid;
    int n_over = 0;
    if (x < num_experts) {
      const int rows = min(offsets[x + 1], max_rows) - max(offsets[x], 0);
      n_over = rows > chunk_rows ? (rows + chunk_rows - 1) / chunk_rows : 0;
    }
    int incl = n_over;  // inclusive scan over the wave, then over the waves
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d, 64);
      if (lane >= d) incl += t;
    }
    if (lane == 63) s_wave_sum[wave] = incl;
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int ws = s_wave_sum[w];
      if (w < wave) incl += ws;
      total += ws;
    }
    const int excl = carry + incl - n_over;
    if (n_over > 0 && excl <= oc && oc < excl + n_over) s_found = make_int2(x, oc - excl);
    carry += total;
    __syncthreads();  // s_wave_sum is rewritten by the next round; s_found is published
  }
  return s_found;
}

// kSwiglu = false: c[s, n] for the N weight rows.
// kSwiglu = true: N = 2 mi; c[s, j] = swiglu(gate sum of row j, up sum of row mi + j) for
// j < mi (c is the activation buffer, ldc its leading dimension).
//
// kMT: 16-row MFMA tiles of sorted rows per pass (1 or 2). With 2, each decoded weight
// feeds two tiles: half the decode work and weight re-reads for experts with more than
// 16 rows, at two blocks per CU (registers and LDS).
template <bool kSwiglu, int kMT>
__global__ __launch_bounds__(kThreads, kMT == 1 ? 3 : 2) void grouped_gemm_kernel(
    const uint16_t *__restrict__ a, int64_t lda, int32_t a_rows,
    const int32_t *__restrict__ gather, const uint64_t *__restrict__ packed_ptrs,
    const uint64_t *__restrict__ scale_ptrs, const float *__restrict__ scale2s,
    const int32_t *__restrict__ offsets, int32_t num_experts, int32_t chunk_rows,
    const int32_t *__restrict__ active, const int32_t *__restrict__ n_active_p,
    int32_t expert_rows, uint16_t *__restrict__ c, int64_t ldc, int32_t max_rows, int32_t N,
    int32_t K, float limit) {
  constexpr int kPassM = kBlockM * kMT;                      // sorted rows per pass
  constexpr int kXBufBytes = kPassM * kLdsRowBytes;
  constexpr int kXP = kPassM * kPiecesPerRow / kThreads;       // pieces per thread per step
  static_assert(kPassM * kPiecesPerRow == kXP * kThreads, "whole activation pieces");
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][kXBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ss[2][kScaleBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lut[256 * 16];

  // Workgroups go to the 8 XCDs round-robin by linear id, so in grid order the N tiles
  // of one grid row (one expert or overflow chunk) are spread over all eight XCDs and
  // every XCD gets an eighth of every row's work, however the rows are routed. (Giving
  // each XCD whole rows, so that an expert's activation rows are fetched into one L2
  // only, left the XCDs up to 14 % apart in work under Zipf(1.1) routing, where a few
  // experts hold most rows, and made that launch 7 % slower; with uniform routing it
  // measured the same as grid order. The activation rows are small next to the weights
  // and come from the last-level cache.)
  //
  // Grid rows [0, num_experts) are the experts with at most chunk_rows rows; rows past
  // them are overflow chunks (the chunk_rows-row pieces of the more heavily routed
  // experts, in expert order), so that no block runs more than chunk_rows / 16 passes
  // over its weights and a hot expert's rows spread over several blocks. The first
  // kFrontChunks overflow rows are dispatched first (the longest blocks start first, the
  // chunks of one expert next to each other, reading the same weights at about the same
  // time), then the experts in order (a contiguous range of absent ones, an
  // expert-parallel rank's share, exits at the tail), then the remaining overflow rows.
  // The room for overflow chunks is a worst-case bound; the rows past the actual chunks
  // exit after one scan of the offsets, and dispatching only a few of them first keeps
  // that cost off the start of a launch whose experts are all light.
  // With `active` (the sort's list of experts that have rows, and its count), the
  // expert_rows (< num_experts) expert rows of the grid take the listed experts in turn:
  // a launch with fewer rows than experts then dispatches no block for an expert without
  // rows (at 8 decode rows and 256 experts, 2,048 blocks instead of 8,192).
  const int tile = blockIdx.x;
  const int y = blockIdx.y;
  const int front = min(static_cast<int>(gridDim.y) - expert_rows, kFrontChunks);
  int e = y - front, chunk = 0;
  const bool over = y < front || y >= front + expert_rows;
  if (over) {
    const int oc = y < front ? y : y - expert_rows;
    const int2 found = find_overflow_chunk(offsets, num_experts, chunk_rows, max_rows, oc);
    if (found.x < 0) return;  // fewer overflow chunks than grid rows
    e = found.x;
    chunk = found.y;
  } else if (active != nullptr) {  // uniform
    if (e >= *n_active_p) return;  // fewer experts with rows than expert rows in the grid
    e = active[e];
    if (e < 0 || e >= num_experts) return;
  }
  // All of the expert's metadata in one memory round trip: the empty asm needs every
  // value before the early exits, so the five loads are issued together instead of one
  // exit test at a time.
  const uint64_t packed_u = packed_ptrs[e], scales_u = scale_ptrs[e];
  const float scale2 = scale2s[e];
  const int off_lo = offsets[e], off_hi = offsets[e + 1];
  asm volatile("" ::"s"(packed_u), "s"(scales_u), "s"(scale2), "s"(off_lo), "s"(off_hi));
  const uint8_t *packed = reinterpret_cast<const uint8_t *>(packed_u);
  if (packed == nullptr) return;  // expert not present: its rows keep the caller's values
  const int end = min(off_hi, max_rows);
  if (!over && end - max(off_lo, 0) > chunk_rows) return;  // left to overflow blocks
  const int lo = max(off_lo, 0) + chunk * chunk_rows;
  const int hi = end - lo > chunk_rows ? lo + chunk_rows : end;  // no overflow at INT32_MAX
  if (hi <= lo) return;
  const uint8_t *scales = reinterpret_cast<const uint8_t *>(scales_u);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int r16 = lane & 15, kb = lane >> 4;
  // Weight rows of block row j: base[j / kHalfN] + j % kHalfN. Plain: the block's 128
  // consecutive rows. Fused: 64 gate rows, then the matching 64 up rows.
  const int mi = N / 2;
  const int row_base0 = tile * (kSwiglu ? kHalfN : kBlockN);
  const int row_base1 = row_base0 + (kSwiglu ? mi : kHalfN);
  const int row_end0 = kSwiglu ? mi : N;  // rows past it are out (N, mi multiples of 16)
  // This wave's tiles: block rows 16 w + [0, 16) and kHalfN + 16 w + [0, 16).
  const int n_tile0 = row_base0 + 16 * wave, n_tile1 = row_base1 + 16 * wave;
  const bool tile0_on = n_tile0 < row_end0;
  const bool tile1_on = n_tile1 < N && (!kSwiglu || tile0_on);
  const uint32_t row_bytes = static_cast<uint32_t>(K) / 2, srow_bytes = static_cast<uint32_t>(K) / 16;
  const int n_steps = K / kChunkK;
  const int n_groups = (n_steps + kLineSteps - 1) / kLineSteps;

  const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(packed, static_cast<uint32_t>(N) * row_bytes);
  const __amdgpu_buffer_rsrc_t s_rsrc = make_rsrc(scales, static_cast<uint32_t>(N) * srow_bytes);
  const __amdgpu_buffer_rsrc_t x_rsrc =
      make_rsrc(a, static_cast<uint32_t>(a_rows) * static_cast<uint32_t>(lda) * 2u);

  // This lane's weight rows; rows past N lie past the buffer end and read zeros. A fused
  // block's gate rows past mi would read real up rows: those tiles are off (no output),
  // their loads are harmless.
  const uint32_t w_voff[kTiles] = {
      static_cast<uint32_t>(n_tile0 + r16) * row_bytes + 16u * kb,
      static_cast<uint32_t>(n_tile1 + r16) * row_bytes + 16u * kb};
  // Scale staging: thread -> block rows tid / 4 (tile-0 half) and kHalfN + tid / 4
  // (tile-1 half), step tid % 4 of each half line; four threads read a row's 128-byte
  // line of 8 steps as two 16-byte pieces each.
  const int s_sub = tid & (kStageSteps - 1);
  const int s_row = tid / kStageSteps;
  const uint32_t s_voff[kSPieces] = {
      static_cast<uint32_t>(row_base0 + s_row) * srow_bytes,
      static_cast<uint32_t>(row_base1 + s_row) * srow_bytes};
  const int s_lds = s_row * kScaleRowBytes + s_sub * 16;
  constexpr int kScaleHalfLds = kHalfN * kScaleRowBytes;
  // Vector offset of step (8 g + 4 h + s_sub) of piece p's scale row; kNoLoad past the
  // row's last step.
  const auto scale_voff = [&](int p, int g, int h) {
    const int st = g * kLineSteps + h * kStageSteps + s_sub;
    return st < n_steps ? s_voff[p] + static_cast<uint32_t>(st) * 16u : kNoLoad;
  };
  // This lane's scale dword of tile 0 within a staged block (tile 1: + kScaleHalfLds).
  const int s_read = (16 * wave + r16) * kScaleRowBytes + 4 * kb;

  for (int m0 = lo; m0 < hi; m0 += kPassM) {
    const int m_cnt = min(kPassM, hi - m0);
    // Activation staging: thread -> (row of the pass, 16-byte piece of a step) for rows
    // tid / 32 and 8 + tid / 32. Rows past the pass and out-of-range gather indices read
    // zeros (offset past the end). The gather indices are loaded first, the step's
    // weights and scales next, so that only the gather is waited for before the
    // activation loads can be addressed.
    int g_row[kXP], piece_col[kXP], lds_off[kXP];
#pragma unroll
    for (int p = 0; p < kXP; ++p) {
      const int piece = tid + p * kThreads;
      const int piece_row = piece / kPiecesPerRow;
      piece_col[p] = piece % kPiecesPerRow;
      lds_off[p] = piece_row * kLdsRowBytes + piece_col[p] * 16;
      int g = -1;
      if (piece_row < m_cnt) {
        const int srow = m0 + piece_row;
        g = gather != nullptr ? gather[srow] : srow;
      }
      g_row[p] = g;
    }

    f32x4_t acc[kTiles][kMT];
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) acc[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    WeightRegs w0, w1;
    load_weights(w0, w_rsrc, w_voff, 0, n_steps);
    // Scales of steps 0-3 to LDS now; steps 4-7 wait in sc_keep.
    u32x4_t sc_keep[kSPieces], sc_next[kSPieces];
#pragma unroll
    for (int p = 0; p < kSPieces; ++p) {
      sc_next[p] = load16(s_rsrc, scale_voff(p, 0, 0), 0);
      sc_keep[p] = load16(s_rsrc, scale_voff(p, 0, 1), 0);
    }
    // The decode tables, built while the first loads are in flight and published by the
    // barrier below. Later passes write the same values again (every read of the previous
    // pass is behind its last barrier), which costs less than a branch around it.
    build_code_table_lut(lut, tid, scale2);
    uint32_t x_voff[kXP];
#pragma unroll
    for (int p = 0; p < kXP; ++p) {
      const int g = g_row[p];
      x_voff[p] = (g >= 0 && g < a_rows)
                      ? (static_cast<uint32_t>(g) * static_cast<uint32_t>(lda) + piece_col[p] * 8u) * 2u
                      : kNoLoad;
    }
#pragma unroll
    for (int p = 0; p < kSPieces; ++p)
      *reinterpret_cast<u32x4_t *>(ss[0] + s_lds + p * kScaleHalfLds) = permute_scales(sc_next[p]);
#pragma unroll
    for (int p = 0; p < kXP; ++p)
      *reinterpret_cast<u32x4_t *>(xs[0] + lds_off[p]) = permute_k8(load16(x_rsrc, x_voff[p], 0));
    u32x4_t xr[kXAhead][kXP];
#pragma unroll
    for (int d = 1; d < kXAhead; ++d)
#pragma unroll
      for (int p = 0; p < kXP; ++p)
        xr[d][p] = load16(x_rsrc, d < n_steps ? x_voff[p] : kNoLoad,
                          static_cast<uint32_t>(d) * (kChunkK * 2));
    __syncthreads();

    // Steps of one 8-step group of scales (LDS stage i / 4), weights prefetched one step
    // ahead in a two-slot ring. Every load here is unconditional (past the end it reads
    // nothing): a load behind a branch leaves the wait counters unknown at the join, and
    // the compiler then drains all of them.
    auto run_step = [&](int g, int i, WeightRegs &cur, WeightRegs &ahead) {
      const int step = g * kLineSteps + i;
      if (i == 4) {  // the next group's line, both halves in one go (sc_keep is free now)
#pragma unroll
        for (int p = 0; p < kSPieces; ++p) {
          sc_next[p] = load16(s_rsrc, scale_voff(p, g + 1, 0), 0);
          sc_keep[p] = load16(s_rsrc, scale_voff(p, g + 1, 1), 0);
        }
      }
#pragma unroll
      for (int p = 0; p < kXP; ++p)
        xr[i % kXAhead][p] = load16(x_rsrc, step + kXAhead < n_steps ? x_voff[p] : kNoLoad,
                                    static_cast<uint32_t>(step + kXAhead) * (kChunkK * 2));
      load_weights(ahead, w_rsrc, w_voff, step + 1, n_steps);
      if (tile0_on) {
        const uint8_t *srow = ss[i / kStageSteps] + s_read + 16 * (i % kStageSteps);
        const uint32_t sc0 = *reinterpret_cast<const uint32_t *>(srow);
        const uint32_t sc1 = *reinterpret_cast<const uint32_t *>(srow + kScaleHalfLds);
        const uint8_t *brow = xs[step & 1] + r16 * kLdsRowBytes + 64 * kb;
        moe::Fp4Table blk0[4], blk1[4];
        lut_blocks(sc0, lut, blk0);
        lut_blocks(sc1, lut, blk1);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8_t B[kMT][4];
#pragma unroll
          for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              B[mt][j] = *reinterpret_cast<const bf16x8_t *>(
                  brow + 16 * mt * kLdsRowBytes + 256 * h + 16 * j);
          const u32x4_t &x0 = h ? cur.b[0] : cur.a[0];
          const uint32_t w0w[4] = {x0[0], x0[1], x0[2], x0[3]};
          moe::mfma4_tiles<kMT>(w0w, blk0[2 * h], blk0[2 * h + 1], B, acc[0]);
          if (tile1_on) {
            const u32x4_t &x1 = h ? cur.b[1] : cur.a[1];
            const uint32_t w1w[4] = {x1[0], x1[1], x1[2], x1[3]};
            moe::mfma4_tiles<kMT>(w1w, blk1[2 * h], blk1[2 * h + 1], B, acc[1]);
          }
        }
      }
#pragma unroll
      for (int p = 0; p < kXP; ++p)
        *reinterpret_cast<u32x4_t *>(xs[(step + 1) & 1] + lds_off[p]) =
            permute_k8(xr[(i + 1) % kXAhead][p]);
      // Each stage buffer is filled mid-way through the other stage (its last reads are
      // a barrier behind): steps 4-7 of this group at step 2, steps 0-3 of the next
      // group at step 6.
      if (i == 2) {
#pragma unroll
        for (int p = 0; p < kSPieces; ++p)
          *reinterpret_cast<u32x4_t *>(ss[1] + s_lds + p * kScaleHalfLds) =
              permute_scales(sc_keep[p]);
      }
      if (i == 6) {
#pragma unroll
        for (int p = 0; p < kSPieces; ++p)
          *reinterpret_cast<u32x4_t *>(ss[0] + s_lds + p * kScaleHalfLds) =
              permute_scales(sc_next[p]);
      }
      __syncthreads();
    };
    for (int g = 0; g < n_groups; ++g) {
      const int s0 = g * kLineSteps;
      run_step(g, 0, w0, w1);
      if (s0 + 1 < n_steps) run_step(g, 1, w1, w0);
      if (s0 + 2 < n_steps) run_step(g, 2, w0, w1);
      if (s0 + 3 < n_steps) run_step(g, 3, w1, w0);
      if (s0 + 4 < n_steps) run_step(g, 4, w0, w1);
      if (s0 + 5 < n_steps) run_step(g, 5, w1, w0);
      if (s0 + 6 < n_steps) run_step(g, 6, w0, w1);
      if (s0 + 7 < n_steps) run_step(g, 7, w1, w0);
    }

    // acc[t][mt][i] = result for weight row n_tile_t + 4 kb + i and sorted row
    // m0 + 16 mt + r16. The block's output tile goes through LDS (the second activation
    // buffer, free after the last step's barrier) so that the global stores are 16 bytes
    // per lane with consecutive lanes covering whole 128-byte lines of an output row.
    {
      constexpr int kOutCols = kSwiglu ? kHalfN : kBlockN;     // output columns per block
      constexpr int kOutRowBytes = kOutCols * 2 + 16;           // padded staged row
      static_assert(kPassM * kOutRowBytes <= kXBufBytes, "output tile fits one buffer");
      uint8_t *ot = xs[1];
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        uint8_t *orow = ot + (16 * mt + r16) * kOutRowBytes;
        if (kSwiglu) {
          float o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // the BF16 values the unfused path stores, then its SwiGLU
            const uint32_t gu = moe::pack_bf16x2(acc[0][mt][i], acc[1][mt][i]);
            o[i] = moe::swiglu_clamp1(__uint_as_float(gu << 16),
                                      __uint_as_float(gu & 0xFFFF0000u), limit);
          }
          uint2 v;
          v.x = moe::pack_bf16x2(o[0], o[1]);
          v.y = moe::pack_bf16x2(o[2], o[3]);
          *reinterpret_cast<uint2 *>(orow + (16 * wave + 4 * kb) * 2) = v;
        } else {
#pragma unroll
          for (int tt = 0; tt < kTiles; ++tt) {
            uint2 v;
            v.x = moe::pack_bf16x2(acc[tt][mt][0], acc[tt][mt][1]);
            v.y = moe::pack_bf16x2(acc[tt][mt][2], acc[tt][mt][3]);
            *reinterpret_cast<uint2 *>(orow + (tt * kHalfN + 16 * wave + 4 * kb) * 2) = v;
          }
        }
      }
      __syncthreads();
      constexpr int kChunksPerRow = kOutCols * 2 / 16;
      const int col_end = min(row_end0 - row_base0, kOutCols);  // valid columns of the tile
      for (int q = tid; q < kPassM * kChunksPerRow; q += kThreads) {
        const int r = q / kChunksPerRow, ch = q - r * kChunksPerRow;
        if (r >= m_cnt || ch * 8 >= col_end) continue;
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(ot + r * kOutRowBytes + ch * 16);
        *reinterpret_cast<u32x4_t *>(c + static_cast<size_t>(m0 + r) * ldc + row_base0 + ch * 8) = v;
      }
    }
  }
}

// Diagnostic: the BF16 weight operand in natural k order. One thread per 32 k of a row.
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ packed,
                                                      const uint8_t *__restrict__ scales,
                                                      float scale2, uint16_t *__restrict__ out,
                                                      int32_t N, int32_t K) {
  const int per_row = K / 32;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(N) * per_row) return;
  const int n = static_cast<int>(idx / per_row), q = static_cast<int>(idx % per_row);
  const uint4 v = *reinterpret_cast<const uint4 *>(packed + static_cast<size_t>(n) * (K / 2) +
                                                   q * 16);
  const uint32_t sc = *reinterpret_cast<const uint16_t *>(scales +
                                                          static_cast<size_t>(n) * (K / 16) +
                                                          2 * q);
  float d0, d1;
  moe::e4m3x2_to_f32(sc, d0, d1);
  const moe::Fp4Table b0 = moe::make_table(d0, scale2), b1 = moe::make_table(d1, scale2);
  const uint32_t words[4] = {v.x, v.y, v.z, v.w};
  uint4 *dst = reinterpret_cast<uint4 *>(out + static_cast<size_t>(n) * K + q * 32);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t wd[4];
    moe::decode8(words[j], j < 2 ? b0 : b1, wd);
    // (k0,k2) (k4,k6) (k1,k3) (k5,k7) -> (k0,k1) (k2,k3) (k4,k5) (k6,k7)
    uint4 o;
    o.x = moe::byte_perm(wd[2], wd[0], 0x05040100u);
    o.y = moe::byte_perm(wd[2], wd[0], 0x07060302u);
    o.z = moe::byte_perm(wd[3], wd[1], 0x05040100u);
    o.w = moe::byte_perm(wd[3], wd[1], 0x07060302u);
    dst[j] = o;
  }
}

// Shared argument checks of the two GEMM entry points (n = weight rows, n_out = columns
// of c). Returns MOE_OK or MOE_EINVAL with the error recorded.
int check_gemm_args(const char *name, const uint16_t *a, int64_t lda, int32_t a_rows,
                    const uint64_t *packed_ptrs, const uint64_t *scale_ptrs,
                    const float *scale2, const int32_t *expert_offsets, int32_t num_experts,
                    const uint16_t *c, int64_t ldc, int32_t max_rows, int32_t n,
                    int32_t n_out, int32_t k) {
  MOE_REQUIRE(k > 0 && k % kChunkK == 0, "%s: k must be a positive multiple of %d (got %d)",
              name, kChunkK, k);
  MOE_REQUIRE(lda >= k && lda % 8 == 0, "%s: lda must be >= k and a multiple of 8", name);
  MOE_REQUIRE(ldc >= n_out && ldc % 8 == 0, "%s: ldc must be >= %d and a multiple of 8", name,
              n_out);
  MOE_REQUIRE(num_experts >= 1 && num_experts <= 65535,
              "%s: num_experts must be in [1, 65535] (got %d)", name, num_experts);
  MOE_REQUIRE(max_rows >= 0 && a_rows >= 0, "%s: max_rows and a_rows must be >= 0", name);
  MOE_REQUIRE(a && packed_ptrs && scale_ptrs && scale2 && expert_offsets && c,
              "%s: a required pointer is NULL", name);
  MOE_REQUIRE(moe::aligned16(a) && moe::aligned16(c), "%s: a and c must be 16-byte aligned",
              name);
  if (max_rows == 0) return MOE_OK;
  MOE_REQUIRE(a_rows >= 1, "%s: a_rows must be >= 1 when max_rows > 0", name);
  // Buffer offsets are 32-bit and a skipped load uses offset 2^31, past any buffer below
  // 2 GiB: activations and one expert's packed weights stay below 2 GiB.
  MOE_REQUIRE(static_cast<uint64_t>(a_rows) * lda * 2 < (1ull << 31),
              "%s: the activation buffer must be smaller than 2 GiB", name);
  MOE_REQUIRE(static_cast<uint64_t>(n) * k / 2 < (1ull << 31),
              "%s: one expert's packed weights must be smaller than 2 GiB", name);
  return MOE_OK;
}

// Grid rows of a GEMM launch: the experts, then room for every overflow chunk. An expert
// with r > C = kChunkRows rows has ceil(r / C) <= 2 r / (C + 1) chunks (the left side steps
// to k + 1 at r = k C + 1, where 2 (k C + 1) >= (k + 1)(C + 1) because (k - 1)(C - 1) >= 0),
// so all experts together (at most max_rows rows) have at most 2 max_rows / (C + 1), and
// none when max_rows <= C. Where that would pass the grid's row limit, blocks take all of
// their expert's rows (no overflow chunks).
int grid_rows(int32_t expert_rows, int32_t max_rows, int *chunk_rows) {
  const int64_t chunks =
      max_rows > kChunkRows ? 2 * static_cast<int64_t>(max_rows) / (kChunkRows + 1) : 0;
  const int64_t rows = expert_rows + chunks;
  if (rows <= 65535) {
    *chunk_rows = kChunkRows;
    return static_cast<int>(rows);
  }
  *chunk_rows = INT32_MAX;
  return expert_rows;
}

// Grid rows for the experts: one per expert, or, given the sort's active-expert list and
// count, one per slot when there are fewer slots than experts (at most that many experts
// have rows). The list costs each block one more dependent load, so it is used only
// where it removes blocks.
int expert_grid_rows(int32_t num_experts, int32_t max_rows, const int32_t *active,
                     const int32_t *counters) {
  return active != nullptr && counters != nullptr && max_rows < num_experts ? max_rows
                                                                            : num_experts;
}

// Two 16-row tiles per pass when the experts average at least 24 rows: passes over 32
// rows then halve the decode work and the weight re-reads. (The average comes from the
// sizes alone; a few hot experts among light ones, as under skewed routing, keep one
// tile per pass and three blocks per CU.)
bool two_row_tiles(int32_t num_experts, int32_t max_rows) {
  return static_cast<int64_t>(max_rows) >= 24LL * num_experts;
}

}  // namespace

extern "C" int moe_w4a16_grouped_gemm(const uint16_t *a, int64_t lda, int32_t a_rows,
                                      const int32_t *a_gather, const uint64_t *packed_ptrs,
                                      const uint64_t *scale_ptrs, const float *scale2,
                                      const int32_t *expert_offsets, int32_t num_experts,
                                      const int32_t *active_experts, const int32_t *counters,
                                      uint16_t *c, int64_t ldc, int32_t max_rows, int32_t n,
                                      int32_t k, void *stream) {
  moe::clear_error();
  MOE_REQUIRE(n > 0 && n % 16 == 0, "grouped_gemm: n must be a positive multiple of 16 (got %d)",
              n);
  const int rc = check_gemm_args("grouped_gemm", a, lda, a_rows, packed_ptrs, scale_ptrs, scale2,
                                 expert_offsets, num_experts, c, ldc, max_rows, n, n, k);
  if (rc != MOE_OK || max_rows == 0) return rc;
  int chunk_rows = 0;
  const int x_rows = expert_grid_rows(num_experts, max_rows, active_experts, counters);
  const bool listed = x_rows < num_experts;
  const dim3 grid((n + kBlockN - 1) / kBlockN, grid_rows(x_rows, max_rows, &chunk_rows));
  return moe::launch("moe_w4a16_grouped_gemm",
                     two_row_tiles(num_experts, max_rows) ? grouped_gemm_kernel<false, 2>
                                                          : grouped_gemm_kernel<false, 1>,
                     grid, dim3(kThreads), 0, stream, a, lda, a_rows, a_gather, packed_ptrs,
                     scale_ptrs, scale2, expert_offsets, num_experts, chunk_rows,
                     listed ? active_experts : nullptr, listed ? counters : nullptr, x_rows, c,
                     ldc, max_rows, n, k, 0.0f);
}

extern "C" int moe_w4a16_grouped_gemm_swiglu(const uint16_t *a, int64_t lda, int32_t a_rows,
                                             const int32_t *a_gather,
                                             const uint64_t *packed_ptrs,
                                             const uint64_t *scale_ptrs, const float *scale2,
                                             const int32_t *expert_offsets, int32_t num_experts,
                                             const int32_t *active_experts,
                                             const int32_t *counters, uint16_t *act,
                                             int64_t ld_act, int32_t max_rows, int32_t mi,
                                             int32_t k, float limit, void *stream) {
  moe::clear_error();
  MOE_REQUIRE(mi > 0 && mi % 16 == 0,
              "grouped_gemm_swiglu: mi must be a positive multiple of 16 (got %d)", mi);
  MOE_REQUIRE(mi <= (1 << 29), "grouped_gemm_swiglu: mi too large (got %d)", mi);
  MOE_REQUIRE(limit > 0.0f, "grouped_gemm_swiglu: limit must be > 0");
  const int rc = check_gemm_args("grouped_gemm_swiglu", a, lda, a_rows, packed_ptrs, scale_ptrs,
                                 scale2, expert_offsets, num_experts, act, ld_act, max_rows,
                                 2 * mi, mi, k);
  if (rc != MOE_OK || max_rows == 0) return rc;
  int chunk_rows = 0;
  const int x_rows = expert_grid_rows(num_experts, max_rows, active_experts, counters);
  const bool listed = x_rows < num_experts;
  const dim3 grid((mi + kHalfN - 1) / kHalfN, grid_rows(x_rows, max_rows, &chunk_rows));
  return moe::launch("moe_w4a16_grouped_gemm_swiglu",
                     two_row_tiles(num_experts, max_rows) ? grouped_gemm_kernel<true, 2>
                                                          : grouped_gemm_kernel<true, 1>,
                     grid, dim3(kThreads), 0, stream, a, lda, a_rows, a_gather, packed_ptrs,
                     scale_ptrs, scale2, expert_offsets, num_experts, chunk_rows,
                     listed ? active_experts : nullptr, listed ? counters : nullptr, x_rows,
                     act, ld_act, max_rows, 2 * mi, k, limit);
}

extern "C" int moe_w4a16_dequant_bf16(const uint8_t *packed, const uint8_t *scales,
                                      float scale2, uint16_t *out, int32_t n, int32_t k,
                                      void *stream) {
  moe::clear_error();
  MOE_REQUIRE(n > 0 && k > 0 && k % 32 == 0,
              "dequant_bf16: need n > 0 and k a positive multiple of 32");
  MOE_REQUIRE(packed && scales && out, "dequant_bf16: a required pointer is NULL");
  MOE_REQUIRE(moe::aligned16(packed) && moe::aligned16(scales) && moe::aligned16(out),
              "dequant_bf16: pointers must be 16-byte aligned");
  const int64_t threads = static_cast<int64_t>(n) * (k / 32);
  MOE_REQUIRE(threads / 256 < INT32_MAX, "dequant_bf16: matrix too large");
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  return moe::launch("moe_w4a16_dequant_bf16", dequant_kernel, grid, dim3(256), 0, stream,
                     packed, scales, scale2, out, n, k);
}
