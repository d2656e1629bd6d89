// moe_dense_gemm_bf16 and moe_dense_gate_up_swiglu_bf16: the shared expert's BF16 GEMMs.
//
// What they compute follows forward_dense and the gemm helper above it (both
// glm5next_mlp forward.rs pages): C[M, N] = A[M, K] B[N, K]^T with BF16 operands and
// output and FP32 accumulation, for the gate, up and down projections of the shared
// expert, a BF16 SwiGLU MLP run once over all rows. The gate/up form applies the clamped
// SwiGLU (swiglu.h) to the BF16-rounded gate and up sums in its epilogue, so its output
// has the bits of the two GEMMs followed by swiglu_clamp.
//
// gfx950 design:
//   - A block of 4 wave64s owns a tile of 16 kMT rows of A by 16 kNT rows of B (output
//     columns) over the whole K. The waves split K, not the tile: wave w takes the 64-k
//     chunks w, w + 4, w + 8, ..., so no operand is shared between waves and the main
//     loop needs neither LDS nor barriers. Each lane loads its MFMA operands straight
//     from memory with raw buffer loads (16 rows x 64 contiguous bytes per instruction),
//     kRing chunks ahead in a register ring; the four waves together read 512
//     contiguous bytes of every row at a time.
//   - v_mfma_f32_16x16x32_bf16 with the B rows (weights) as the MFMA A operand and the A
//     rows (tokens) as the MFMA B operand: a lane then holds 4 consecutive output
//     columns of one row.
//   - The four FP32 partial tiles are summed through LDS in wave order (the same order
//     for every tile shape, so the gate/up form reproduces the plain GEMM's sums bit for
//     bit) and written as BF16, 16 lanes per 128 bytes of an output row.
//   - Rows of A past M and rows of B past N lie outside their buffer resource and read
//     zeros; their outputs are not stored.
//   - Block order: workgroups are dealt to the 8 XCDs round-robin by linear id. When the
//     column tiles divide by 8, the blocks that share B rows (one column tile, all row
//     tiles) are dealt to one XCD back to back, so each weight line is fetched into one
//     L2 and hits there for the other row tiles.
#include <mutex>

#include "buffer_io.h"
#include "common.h"
#include "nvfp4_decode.h"  // moe::pack_bf16x2
#include "swiglu.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
using moe::kNoLoad;
using moe::load16;
using moe::make_rsrc;
using moe::u32x4_t;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kChunkK = 64;            // k per chunk: two MFMA k-steps of 32
constexpr int kChunkBytes = kChunkK * 2;
constexpr int kPad = 4;                // floats of padding per partial-tile row in LDS

// One lane's operands of one chunk: per 16-row tile, 2 x 8 BF16 (k 8 kb + [0, 8) of each
// 32-k half).
template <int kMT, int kNT>
struct Chunk {
  u32x4_t w[kNT][2];  // B rows (weights)
  u32x4_t x[kMT][2];  // A rows (tokens)
};

// Loads the wave's j-th chunk (k chunk `c`); past the wave's last chunk (`live` false)
// every offset is kNoLoad: zeros, no traffic. B tiles [0, kSplit) read through `w_lo`,
// the others through `w_hi` (the gate and up weights of the gate/up form).
template <int kMT, int kNT, int kSplit>
__device__ __forceinline__ void load_chunk(Chunk<kMT, kNT> &ch, __amdgpu_buffer_rsrc_t w_lo,
                                           __amdgpu_buffer_rsrc_t w_hi, const uint32_t *w_voff,
                                           __amdgpu_buffer_rsrc_t xr, const uint32_t *x_voff,
                                           int c, bool live) {
  const uint32_t soff = live ? static_cast<uint32_t>(c) * kChunkBytes : 0u;
  // Offsets stay below 2^30, so setting bit 31 moves them past the end (no branch).
  const uint32_t dead = live ? 0u : kNoLoad;
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    const uint32_t v = w_voff[t] | dead;
    ch.w[t][0] = load16(t < kSplit ? w_lo : w_hi, v, soff);
    ch.w[t][1] = load16(t < kSplit ? w_lo : w_hi, v + 64, soff);
  }
#pragma unroll
  for (int t = 0; t < kMT; ++t) {
    const uint32_t v = x_voff[t] | dead;
    ch.x[t][0] = load16(xr, v, soff);
    ch.x[t][1] = load16(xr, v + 64, soff);
  }
}

template <int kMT, int kNT>
__device__ __forceinline__ void mma_chunk(const Chunk<kMT, kNT> &ch, f32x4_t (&acc)[kMT][kNT]) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, ch.w[nt][h]), __builtin_bit_cast(bf16x8_t, ch.x[mt][h]),
            acc[mt][nt], 0, 0, 0);
}

// kSwiglu = false: c[m, n] = sum_k a[m, k] b0[n, k] for n < N.
// kSwiglu = true: N = inter; the block's first 8 kNT tile rows are gate rows of b0, the
// other 8 kNT the same rows of b1 (up), and c[m, j] = swiglu(gate sum, up sum) of row j.
template <int kMT, int kNT, int kRing, bool kSwiglu>
__global__ __launch_bounds__(kThreads, 2) void dense_gemm_kernel(
    const uint16_t *__restrict__ a, int64_t lda, int32_t M, const uint16_t *__restrict__ b0,
    const uint16_t *__restrict__ b1, int64_t ldb, uint16_t *__restrict__ c, int64_t ldc,
    int32_t N, int32_t K, float limit) {
  constexpr int BM = 16 * kMT, BN = 16 * kNT;
  constexpr int kRowF = BN + kPad;
  static_assert(!kSwiglu || kNT % 2 == 0, "gate and up halves");
  __shared__ __attribute__((aligned(16))) float red[kWaves][BM][kRowF];

  // Block -> (row tile, column tile). Column tiles of one XCD: xcd, xcd + 8, ...
  const int MT = gridDim.y, NT = gridDim.x;
  int mt_blk, nt_blk;
  {
    const int lin = blockIdx.y * NT + blockIdx.x;
    if ((NT & 7) == 0) {
      const int xcd = lin & 7, seq = lin >> 3;
      mt_blk = seq % MT;
      nt_blk = (seq / MT) * 8 + xcd;
    } else {
      mt_blk = lin % MT;
      nt_blk = lin / MT;
    }
  }
  const int m0 = mt_blk * BM;
  // First B row of the block (kSwiglu: in b0 and b1 each).
  const int n0 = nt_blk * (kSwiglu ? BN / 2 : BN);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, kb = lane >> 4;
  const uint32_t xrow_bytes = static_cast<uint32_t>(lda) * 2u;
  const uint32_t wrow_bytes = static_cast<uint32_t>(ldb) * 2u;

  // Resources start at the tile's first row and end after its last valid row.
  const int m_valid = min(BM, M - m0);
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(a + static_cast<int64_t>(m0) * lda, static_cast<uint32_t>(m_valid) * xrow_bytes);
  __amdgpu_buffer_rsrc_t wr, wr_up;
  uint32_t w_voff[kNT];
  {
    const int rows_b = kSwiglu ? BN / 2 : BN;
    const int n_valid = min(rows_b, N - n0);
    wr = make_rsrc(b0 + static_cast<int64_t>(n0) * ldb, static_cast<uint32_t>(n_valid) * wrow_bytes);
    wr_up = kSwiglu ? make_rsrc(b1 + static_cast<int64_t>(n0) * ldb,
                                static_cast<uint32_t>(n_valid) * wrow_bytes)
                    : wr;
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      const int row = kSwiglu ? (t % (kNT / 2)) * 16 + r16 : t * 16 + r16;
      w_voff[t] = static_cast<uint32_t>(row) * wrow_bytes + 16u * kb;
    }
  }
  uint32_t x_voff[kMT];
#pragma unroll
  for (int t = 0; t < kMT; ++t) x_voff[t] = static_cast<uint32_t>(t * 16 + r16) * xrow_bytes + 16u * kb;

  f32x4_t acc[kMT][kNT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // This wave's chunks: k chunk wave + 4 j for j < n_w.
  const int n_chunks = K / kChunkK;
  const int n_w = wave < n_chunks ? (n_chunks - wave + kWaves - 1) / kWaves : 0;
  constexpr int kSplit = kSwiglu ? kNT / 2 : kNT;

  Chunk<kMT, kNT> ring[kRing];
#pragma unroll
  for (int r = 0; r < kRing; ++r)
    load_chunk<kMT, kNT, kSplit>(ring[r], wr, wr_up, w_voff, xr, x_voff, wave + kWaves * r,
                                 r < n_w);
  int j = 0;
  // Every load in the loop is unconditional (past the wave's last chunk it reads
  // nothing): a load behind a branch leaves the wait counters unknown at the join and
  // the compiler then drains them all.
  for (; j + kRing <= n_w; j += kRing) {
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
      mma_chunk<kMT, kNT>(ring[r], acc);
      const int jn = j + r + kRing;
      load_chunk<kMT, kNT, kSplit>(ring[r], wr, wr_up, w_voff, xr, x_voff, wave + kWaves * jn,
                                   jn < n_w);
      // Keep the refill here: scheduled after the next slot's products, it would make
      // them wait for every load in flight.
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // The last n_w - j < kRing chunks are already in ring[0 .. n_w - j).
#pragma unroll
  for (int r = 0; r < kRing - 1; ++r)
    if (j + r < n_w) mma_chunk<kMT, kNT>(ring[r], acc);

  // acc[mt][nt][i]: row m0 + 16 mt + r16, B row (tile column) 16 nt + 4 kb + i.
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
      *reinterpret_cast<f32x4_t *>(&red[wave][16 * mt + r16][16 * nt + 4 * kb]) = acc[mt][nt];
  __syncthreads();

  // Sum the partials in wave order; one unit = 4 consecutive output columns of one row.
  constexpr int kOutCols = kSwiglu ? BN / 2 : BN;
  constexpr int kUnitsPerRow = kOutCols / 4;
  for (int u = tid; u < BM * kUnitsPerRow; u += kThreads) {
    const int m = u / kUnitsPerRow, q = u % kUnitsPerRow;
    const int row = m0 + m, col = n0 + 4 * q;
    if (row >= M || col >= N) continue;
    f32x4_t s = *reinterpret_cast<const f32x4_t *>(&red[0][m][4 * q]);
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += *reinterpret_cast<const f32x4_t *>(&red[w][m][4 * q]);
    uint2 v;
    if (kSwiglu) {
      f32x4_t su = *reinterpret_cast<const f32x4_t *>(&red[0][m][BN / 2 + 4 * q]);
#pragma unroll
      for (int w = 1; w < kWaves; ++w)
        su += *reinterpret_cast<const f32x4_t *>(&red[w][m][BN / 2 + 4 * q]);
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // the BF16 values the two plain GEMMs store, then the SwiGLU
        const uint32_t gu = moe::pack_bf16x2(s[i], su[i]);
        o[i] = moe::swiglu_clamp1(__uint_as_float(gu << 16), __uint_as_float(gu & 0xFFFF0000u),
                                  limit);
      }
      v.x = moe::pack_bf16x2(o[0], o[1]);
      v.y = moe::pack_bf16x2(o[2], o[3]);
    } else {
      v.x = moe::pack_bf16x2(s[0], s[1]);
      v.y = moe::pack_bf16x2(s[2], s[3]);
    }
    *reinterpret_cast<uint2 *>(c + static_cast<int64_t>(row) * ldc + col) = v;
  }
}

// ------------------------------------------------------------------ split-K form
//
// With a workspace the GEMMs run split over K with larger tiles, in two launches. The
// single-pass kernel above streams a 64-row tile of A and of B per block, so A is read
// once per 64 output columns and B once per 64 rows; what bounds it is the bytes each CU
// pulls through its L1 (misses in flight per CU, not HBM): about 400 MB for the shared
// expert's gate/up at 256 rows. Tiles of 128 x 128 halve those bytes, and splitting K
// S ways restores the block count (one to two blocks per CU at the shared expert's
// shapes).
//   1. Partial GEMM. 4 waves as 2 x 2, each owning 64 A rows x 64 B rows (16 MFMA tiles,
//      64 accumulator VGPRs). A and B tiles of 64 k are staged in LDS, one barrier per
//      step: when the grid fits one block per CU, loaded straight into LDS, three stages
//      in flight; else double buffered through registers, the global loads three steps
//      ahead (two blocks per CU). LDS rows are 128 bytes with the 16-byte pieces
//      XOR-swizzled by the row (piece c of row r at c ^ (r & 7)), so the 16 rows x 4
//      pieces an MFMA operand read touches fall in distinct banks. Each block writes its
//      FP32 partial tile to the workspace in fragment order (1 KB contiguous per wave and
//      MFMA tile), or row-major for a reduction inside the combine.
//   2. Reduction. One thread per output fragment (4 columns of one row) sums the S
//      partials in split order (deterministic), rounds to BF16 and, in the gate/up form,
//      applies the SwiGLU to the BF16 gate and up sums; the whole chip reads the
//      partials in parallel.
//   The gate/up form puts 64 gate rows and the same 64 up rows in one B tile, so the gate
//   and up sums of an output column sit in fragments f and f + 2048 of a tile. S depends
//   on K only, so its G and U have the bits of the plain split-K GEMM's.
constexpr int kLT = 128;                        // rows of A and of B per tile
constexpr int kLK = 64;                         // k per LDS stage
constexpr int kLRowBytes = kLK * 2;             // 128: staged rows are not padded
constexpr int kLOperand = kLT * kLRowBytes;     // 16 KB: one operand's stage
constexpr int kLStage = 2 * kLOperand;          // A and B
constexpr int kLLds = 2 * kLStage;              // double buffered: 64 KB
constexpr int kLDmaStages = 3;                   // LDS-direct stages (96 KB, one block per CU)
constexpr int kLPieces = kLT * (kLRowBytes / 16) / kThreads;  // 16-byte pieces per thread
constexpr int kLFrags = kWaves * 16 * 64;       // f32x4 fragments per tile partial
constexpr int kLMaxWays = 4;
static_assert(kLPieces == 4, "four pieces of each operand per thread and step");

// Split count for K: the largest power of two up to 4, and up to 8 / (row tiles), that
// divides the 64-k steps evenly and leaves each split at least 8 steps per row tile.
// Every split adds M x N FP32 partials that are written at the block's end and read back
// by the reduction, and at the shared expert's shapes those bytes cost about as much as
// the weights (the writes run at ~2.5 TB/s, all blocks at once after their last step).
// With more row tiles there are more blocks per split, so fewer splits fill the chip: at
// 256 rows the gate/up GEMM (K = 6144) splits 4 ways (256 blocks) and the down GEMM
// (K = 2048) 2 ways (192 blocks; 4 ways filled the chip but doubled the partials and was
// 2.7 us slower); at 128 rows the down GEMM keeps 4 ways. 8 ways at the gate/up gave two
// blocks per CU but twice the partial bytes: no faster. It depends on m and k, not n, so
// the gate/up form and the plain GEMM of the same rows split alike.
int splitk_ways(int32_t m, int32_t k) {
  const int steps = k / kLK;
  const int row_tiles = (m + kLT - 1) / kLT;
  for (int s = kLMaxWays; s > 1; s /= 2)
    if (s * row_tiles <= 8 && steps % s == 0 && steps / s >= 8 * row_tiles) return s;
  return 1;
}

struct SplitKShape {
  int tiles_m, tiles_n, ways;
  int64_t tiles, bytes;
};

SplitKShape splitk_shape(int32_t m, int32_t n, int32_t k, bool swiglu) {
  SplitKShape sh;
  sh.tiles_m = (m + kLT - 1) / kLT;
  sh.tiles_n = (n + (swiglu ? kLT / 2 : kLT) - 1) / (swiglu ? kLT / 2 : kLT);
  sh.ways = splitk_ways(m, k);
  sh.tiles = static_cast<int64_t>(sh.tiles_m) * sh.tiles_n;
  sh.bytes = sh.tiles * sh.ways * kLFrags * 16;
  return sh;
}

// Phase 1: the partial tile of (row tile, column tile, split) for rows A and B rows over
// the split's K range. Fused: B tile rows [0, 64) are gate rows n0 + r of b0 and [64, 128)
// the same rows of b1 (up). kRowMajor (plain form only): the partials go to an FP32
// [split][M][N] array instead, for a consumer that reads whole rows (the combine).
// kStages = 0: staged through registers, double-buffered LDS (64 KB: two blocks per CU);
// kStages > 0: loaded straight into LDS, kStages stages (one block per CU).
template <bool kSwiglu, bool kRowMajor, int kStages>
__global__ __launch_bounds__(kThreads, 2) void dense_partial_kernel(
    const uint16_t *__restrict__ a, int64_t lda, int32_t M, const uint16_t *__restrict__ b0,
    const uint16_t *__restrict__ b1, int64_t ldb, int32_t N, int32_t K,
    f32x4_t *__restrict__ partials) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int TN = gridDim.x, TM = gridDim.y, S = gridDim.z;

  // Block -> (row tile, column tile, split). Blocks that read the same B rows (one column
  // tile and split, every row tile) go to one XCD back to back.
  int tm, tn, ks;
  {
    const int lin = (blockIdx.z * TM + blockIdx.y) * TN + blockIdx.x;
    if (((TN * S) & 7) == 0) {
      const int xcd = lin & 7, seq = lin >> 3;
      tm = seq % TM;
      const int g = (seq / TM) * 8 + xcd;
      tn = g % TN;
      ks = g / TN;
    } else {
      tn = blockIdx.x;
      tm = blockIdx.y;
      ks = blockIdx.z;
    }
  }
  const int m0 = tm * kLT;
  const int n0 = tn * (kSwiglu ? kLT / 2 : kLT);  // first B row (in b0 and b1 if fused)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int r16 = lane & 15, kb = lane >> 4;
  const uint32_t arow = static_cast<uint32_t>(lda) * 2u, brow = static_cast<uint32_t>(ldb) * 2u;

  // Resources from the tile's first row to its last valid row: rows past them read 0.
  const __amdgpu_buffer_rsrc_t ar =
      make_rsrc(a + static_cast<int64_t>(m0) * lda, static_cast<uint32_t>(min(kLT, M - m0)) * arow);
  const int b_rows = kSwiglu ? kLT / 2 : kLT;
  const uint32_t b_valid = static_cast<uint32_t>(min(b_rows, N - n0)) * brow;
  const __amdgpu_buffer_rsrc_t br0 = make_rsrc(b0 + static_cast<int64_t>(n0) * ldb, b_valid);
  const __amdgpu_buffer_rsrc_t br1 =
      kSwiglu ? make_rsrc(b1 + static_cast<int64_t>(n0) * ldb, b_valid) : br0;

  // This thread's staging pieces: piece p = tid + 256 i is row p / 8, 16-byte column p % 8,
  // so pieces i < 2 are rows [0, 64) and pieces i >= 2 rows [64, 128): in the gate/up form
  // the up rows. That split is fixed per i, which keeps each load's buffer resource uniform
  // across the wave (a per-lane choice would make the compiler loop over the distinct
  // resources for every load).
  static_assert(kThreads / 8 * (kLPieces / 2) == kLT / 2, "the up rows are pieces i >= 2");
  uint32_t a_voff[kLPieces], b_voff[kLPieces], st_off[kLPieces];
#pragma unroll
  for (int i = 0; i < kLPieces; ++i) {
    const int p = tid + kThreads * i, row = p >> 3, col = p & 7;
    a_voff[i] = static_cast<uint32_t>(row) * arow + 16u * col;
    const int brow_i = kSwiglu ? (row & (kLT / 2 - 1)) : row;
    b_voff[i] = static_cast<uint32_t>(brow_i) * brow + 16u * col;
    st_off[i] = static_cast<uint32_t>(row) * kLRowBytes + 16u * (col ^ (row & 7));
  }

  const int steps = K / kLK / S;
  const int k_first = ks * steps;
  struct Regs {
    u32x4_t a[kLPieces], b[kLPieces];
  };
  // One operand of step j (A rows, or B rows when b_half); j >= steps loads nothing.
  const auto load_half = [&](Regs &r, int j, bool b_half) {
    const uint32_t dead = j < steps ? 0u : kNoLoad;
    const uint32_t soff = j < steps ? static_cast<uint32_t>(k_first + j) * kLRowBytes : 0u;
#pragma unroll
    for (int i = 0; i < kLPieces; ++i) {
      if (!b_half) r.a[i] = load16(ar, a_voff[i] | dead, soff);
      else r.b[i] = load16(kSwiglu && i >= kLPieces / 2 ? br1 : br0, b_voff[i] | dead, soff);
    }
  };
  const auto load_step = [&](Regs &r, int j) {
    load_half(r, j, false);
    load_half(r, j, true);
  };
  const auto stage_step = [&](const Regs &r, int buf) {
    uint8_t *sa = lds + buf * kLStage, *sb = sa + kLOperand;
#pragma unroll
    for (int i = 0; i < kLPieces; ++i) {
      *reinterpret_cast<u32x4_t *>(sa + st_off[i]) = r.a[i];
      *reinterpret_cast<u32x4_t *>(sb + st_off[i]) = r.b[i];
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // The products of one 32-k half h of the step in LDS buffer buf.
  const auto compute_half = [&](int buf, int h) {
    const uint8_t *sa = lds + buf * kLStage, *sb = sa + kLOperand;
    const int piece = 4 * h + kb;
    bf16x8_t wf[4], xf[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int rw = 64 * wn + 16 * t + r16, rx = 64 * wm + 16 * t + r16;
      wf[t] = *reinterpret_cast<const bf16x8_t *>(sb + rw * kLRowBytes + 16 * (piece ^ (rw & 7)));
      xf[t] = *reinterpret_cast<const bf16x8_t *>(sa + rx * kLRowBytes + 16 * (piece ^ (rx & 7)));
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[nt], xf[mt], acc[mt][nt], 0, 0, 0);
  };

  if constexpr (kStages == 0) {
    // Step s reads LDS buffer s & 1. The global loads run kDepth steps ahead in kDepth
    // register sets: set s % kDepth holds step s from its load until it is staged (at the
    // end of step s - 1), then takes step s + kDepth during step s, so staging step s + 1
    // waits only for loads issued two steps earlier. The refill is split over the step, the
    // A rows before the first 32-k half of the products and the B rows before the second
    // (one burst of all eight loads at the top measured 1-2 us slower at the shared
    // expert's gate/up, and two or four register sets slower than three), and pinned there
    // with scheduling barriers. The stages are unconditional (past the last step the loads
    // read nothing and the stage writes zeros to a buffer no step reads): a stage behind a
    // branch lets the compiler sink the loads into it, next to their wait.
    constexpr int kDepth = 3, kUnroll = 6;  // kUnroll: a multiple of kDepth and of 2
    Regs r[kDepth];
  #pragma unroll
    for (int i = 0; i < kDepth; ++i) load_step(r[i], i);
    stage_step(r[0], 0);
    __syncthreads();
    for (int j = 0; j < steps; j += kUnroll) {
  #pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int s = j + u;  // u % kDepth == s % kDepth, u & 1 == s & 1
        if (s >= steps) break;
        load_half(r[u % kDepth], s + kDepth, false);
        __builtin_amdgcn_sched_barrier(0);
        compute_half(u & 1, 0);
        load_half(r[u % kDepth], s + kDepth, true);
        __builtin_amdgcn_sched_barrier(0);
        compute_half(u & 1, 1);
        stage_step(r[(u + 1) % kDepth], (u + 1) & 1);
        __syncthreads();
      }
    }
  } else {
    // Straight into LDS (buffer_load ... lds): a wave instruction fills 8 rows x 128 bytes
    // of a stage, lane l writing row 8 w + 32 i + l / 8 at physical piece l % 8, so it
    // loads logical piece (l % 8) ^ (l / 8) of that row (the swizzle of the register
    // path). Stage s goes to buffer s % kStages; stages run kStages - 1 steps ahead. The
    // waits are explicit (the wave's own loads of stage s, then a barrier for the other
    // waves'); a plain s_barrier, not __syncthreads, so that the compiler does not add a
    // full vmcnt(0) wait for the loads still in flight. With the registers free of
    // staging, a block needs ~100 VGPRs.
    uint32_t a_dma[kLPieces], b_dma[kLPieces];
#pragma unroll
    for (int i = 0; i < kLPieces; ++i) {
      const int row = 8 * wave + 32 * i + (lane >> 3);
      const int col = (lane & 7) ^ (lane >> 3);
      a_dma[i] = static_cast<uint32_t>(row) * arow + 16u * col;
      const int brow_i = kSwiglu ? (row & (kLT / 2 - 1)) : row;
      b_dma[i] = static_cast<uint32_t>(brow_i) * brow + 16u * col;
    }
    const auto dma_step = [&](int j) {
      const uint32_t dead = j < steps ? 0u : kNoLoad;
      const int soff = j < steps ? (k_first + j) * kLRowBytes : 0;
      uint8_t *sa = lds + (j % kStages) * kLStage, *sb = sa + kLOperand;
#pragma unroll
      for (int i = 0; i < kLPieces; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ar, (__attribute__((address_space(3))) void *)(sa + 1024 * wave + 4096 * i), 16,
            static_cast<int>(a_dma[i] | dead), soff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            kSwiglu && i >= kLPieces / 2 ? br1 : br0,
            (__attribute__((address_space(3))) void *)(sb + 1024 * wave + 4096 * i), 16,
            static_cast<int>(b_dma[i] | dead), soff, 0, 0);
      }
    };
    // s_waitcnt immediate for vmcnt(N), no expcnt or lgkmcnt wait: N = the loads of the
    // kStages - 2 stages issued after stage s.
    constexpr int kWaitN = 2 * kLPieces * (kStages - 2);
    static_assert(kStages >= 2 && kWaitN < 64, "vmcnt holds 6 bits");
    constexpr int kWaitImm = (kWaitN & 15) | ((kWaitN >> 4) << 14) | (7 << 4) | (15 << 8);
#pragma unroll
    for (int j = 0; j < kStages - 1; ++j) dma_step(j);
    for (int s = 0; s < steps; ++s) {
      __builtin_amdgcn_s_waitcnt(kWaitImm);  // this wave's loads of stage s are in LDS
      __builtin_amdgcn_s_barrier();           // every wave's; and stage s - 1 is read
      dma_step(s + kStages - 1);              // into stage s - 1's buffer
      compute_half(s % kStages, 0);
      compute_half(s % kStages, 1);
    }
    // The past-the-end stages' loads write LDS (zeros) too: they finish before the block.
    __builtin_amdgcn_s_waitcnt(0);
  }

  if constexpr (kRowMajor && kStages >= 3) {
    static_assert(!kSwiglu, "row-major partials: plain form only");
    // The tile goes through LDS (free after the last step; 128 rows of 132 floats, the
    // padding spreading a fragment's 16 rows over the banks), so that each store
    // instruction writes two 512-byte row pieces instead of 16 rows x 64 bytes.
    constexpr int kTS = kLT + 4;
    static_assert(kLT * kTS * 4 <= kStages * kLStage, "the tile fits the stages");
    float *t = reinterpret_cast<float *>(lds);
    __builtin_amdgcn_s_barrier();  // every wave's operand reads are done (waited above)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        *reinterpret_cast<f32x4_t *>(t + (64 * wm + 16 * mt + r16) * kTS + 64 * wn + 16 * nt +
                                     4 * kb) = acc[mt][nt];
    __syncthreads();
    float *mine = reinterpret_cast<float *>(partials) + static_cast<int64_t>(ks) * M * N;
#pragma unroll
    for (int i = 0; i < kLT * kLT / 4 / kThreads; ++i) {
      const int q = tid + kThreads * i, r = q / (kLT / 4), c = 4 * (q % (kLT / 4));
      const int row = m0 + r, col = n0 + c;
      if (row < M && col < N)
        *reinterpret_cast<f32x4_t *>(mine + static_cast<int64_t>(row) * N + col) =
            *reinterpret_cast<const f32x4_t *>(t + r * kTS + c);
    }
  } else if constexpr (kRowMajor) {
    static_assert(!kSwiglu, "row-major partials: plain form only");
    // acc[mt][nt][i]: row m0 + 64 wm + 16 mt + r16, column n0 + 64 wn + 16 nt + 4 kb + i
    // (N is a multiple of 16, so a fragment's four columns are all in range or all out).
    float *mine = reinterpret_cast<float *>(partials) + static_cast<int64_t>(ks) * M * N;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int row = m0 + 64 * wm + 16 * mt + r16;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int col = n0 + 64 * wn + 16 * nt + 4 * kb;
        if (row < M && col < N)
          *reinterpret_cast<f32x4_t *>(mine + static_cast<int64_t>(row) * N + col) = acc[mt][nt];
      }
    }
  } else {
    // The partial tile in fragment order: [split][tile][wave][mt * 4 + nt][lane].
    f32x4_t *mine = partials + (static_cast<int64_t>(ks) * TM * TN + tm * TN + tn) * kLFrags +
                    wave * 1024;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) mine[(mt * 4 + nt) * 64 + lane] = acc[mt][nt];
  }
}

// Phase 2: output fragment g of the tile grid (fragment f = g % kOutFrags of tile
// g / kOutFrags). Fragment f: wave f / 1024, MFMA tile (f / 64) % 16, lane f % 64; its
// element i is A row 64 (w & 1) + 16 mt + (lane & 15) and B row
// 64 (w >> 1) + 16 nt + 4 (lane >> 4) + i.
template <bool kSwiglu>
__global__ __launch_bounds__(kThreads) void dense_reduce_kernel(
    const f32x4_t *__restrict__ partials, int32_t tiles_n, int64_t n_tiles, int32_t ways,
    uint16_t *__restrict__ c, int64_t ldc, int32_t M, int32_t N, float limit) {
  constexpr int kOutFrags = kSwiglu ? kLFrags / 2 : kLFrags;  // fused: the gate fragments
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (g >= n_tiles * kOutFrags) return;
  const int64_t tile = g / kOutFrags;
  const int f = static_cast<int>(g - tile * kOutFrags);
  const int tm = static_cast<int>(tile / tiles_n), tn = static_cast<int>(tile - static_cast<int64_t>(tm) * tiles_n);
  const int w = f >> 10, q = (f >> 6) & 15, l = f & 63;
  const int row = tm * kLT + 64 * (w & 1) + 16 * (q >> 2) + (l & 15);
  const int col = tn * (kSwiglu ? kLT / 2 : kLT) + 64 * (w >> 1) + 16 * (q & 3) + 4 * (l >> 4);
  if (row >= M || col >= N) return;
  const int64_t stride = n_tiles * kLFrags;
  const f32x4_t *p = partials + tile * kLFrags + f;
  f32x4_t s = p[0];
  for (int k = 1; k < ways; ++k) s += p[k * stride];
  uint2 v;
  if (kSwiglu) {
    const f32x4_t *pu = p + kLFrags / 2;  // the up rows: waves 2, 3
    f32x4_t su = pu[0];
    for (int k = 1; k < ways; ++k) su += pu[k * stride];
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t gu = moe::pack_bf16x2(s[i], su[i]);
      o[i] = moe::swiglu_clamp1(__uint_as_float(gu << 16), __uint_as_float(gu & 0xFFFF0000u),
                                limit);
    }
    v.x = moe::pack_bf16x2(o[0], o[1]);
    v.y = moe::pack_bf16x2(o[2], o[3]);
  } else {
    v.x = moe::pack_bf16x2(s[0], s[1]);
    v.y = moe::pack_bf16x2(s[2], s[3]);
  }
  *reinterpret_cast<uint2 *>(c + static_cast<int64_t>(row) * ldc + col) = v;
}

int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return cus > 0 ? cus : 256;
}

// Phase 1 of the split-K form: the LDS-direct kernel when the grid fits one block per CU
// (its 96 KB of LDS allow no second), else the register-staged one at two per CU.
// Measured at the shared expert's shapes (H 6144, width 2048): 256 rows, 256 and 192
// blocks, gate/up 31.4 -> 30.8 us and down 23.3 -> 22.0 us from cold caches; 1024 rows,
// gate/up (256 blocks) 77.8 -> 73.8 us, but down (384 blocks) 52.4 -> 59.0 us, so the
// larger grids keep the register-staged kernel.
template <bool kSwiglu, bool kRowMajor>
int launch_partial(const char *name, const SplitKShape &sh, const uint16_t *a, int64_t lda,
                   int32_t m, const uint16_t *b0, const uint16_t *b1, int64_t ldb, int32_t n,
                   int32_t k, f32x4_t *partials, void *stream) {
  MOE_REQUIRE(sh.tiles_n <= 65535 && sh.tiles_m <= 65535,
              "%s: too many tiles for the split-K form", name);
  const dim3 grid(static_cast<unsigned>(sh.tiles_n), static_cast<unsigned>(sh.tiles_m),
                  static_cast<unsigned>(sh.ways));
  const bool direct = sh.tiles * sh.ways <= device_cus();
  const auto kern = direct ? dense_partial_kernel<kSwiglu, kRowMajor, kLDmaStages>
                           : dense_partial_kernel<kSwiglu, kRowMajor, 0>;
  const int lds = direct ? kLDmaStages * kLStage : kLLds;
  static const hipError_t attr_err[2] = {
      hipFuncSetAttribute(reinterpret_cast<const void *>(dense_partial_kernel<kSwiglu, kRowMajor, 0>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLLds),
      hipFuncSetAttribute(
          reinterpret_cast<const void *>(dense_partial_kernel<kSwiglu, kRowMajor, kLDmaStages>),
          hipFuncAttributeMaxDynamicSharedMemorySize, kLDmaStages * kLStage)};
  if (attr_err[direct ? 1 : 0] != hipSuccess) {
    moe::set_error("%s: cannot raise the LDS limit: %s", name,
                   hipGetErrorString(attr_err[direct ? 1 : 0]));
    return MOE_ELAUNCH;
  }
  return moe::launch(name, kern, grid, dim3(kThreads), lds, stream, a, lda, m, b0, b1, ldb, n,
                     k, partials);
}

template <bool kSwiglu>
int launch_splitk(const uint16_t *a, int64_t lda, int32_t m, const uint16_t *b0,
                  const uint16_t *b1, int64_t ldb, uint16_t *c, int64_t ldc, int32_t n,
                  int32_t k, float limit, void *workspace, int64_t workspace_bytes,
                  void *stream) {
  const char *name = kSwiglu ? "moe_dense_gate_up_swiglu_bf16" : "moe_dense_gemm_bf16";
  const SplitKShape sh = splitk_shape(m, n, k, kSwiglu);
  MOE_REQUIRE_CODE(workspace_bytes >= sh.bytes, MOE_ECAPACITY,
                   "%s: the workspace holds %lld bytes, the split-K form needs %lld", name,
                   static_cast<long long>(workspace_bytes), static_cast<long long>(sh.bytes));
  MOE_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0,
              "%s: the workspace must be 256-byte aligned", name);
  f32x4_t *partials = static_cast<f32x4_t *>(workspace);
  const int rc = launch_partial<kSwiglu, false>(name, sh, a, lda, m, b0, b1, ldb, n, k,
                                                partials, stream);
  if (rc != MOE_OK) return rc;
  const int64_t frags = sh.tiles * (kSwiglu ? kLFrags / 2 : kLFrags);
  return moe::launch(name, dense_reduce_kernel<kSwiglu>,
                     dim3(static_cast<unsigned>((frags + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, partials, sh.tiles_n, sh.tiles, sh.ways, c, ldc,
                     m, n, limit);
}

// Phase 1 alone with row-major partials: ways x m x n FP32 (ways = splitk_ways(m, k)).
int launch_partials_row_major(const uint16_t *a, int64_t lda, int32_t m, const uint16_t *b,
                              int64_t ldb, int32_t n, int32_t k, float *partials,
                              void *stream) {
  return launch_partial<false, true>("moe_dense_gemm_bf16_partials", splitk_shape(m, n, k, false),
                                     a, lda, m, b, b, ldb, n, k,
                                     reinterpret_cast<f32x4_t *>(partials), stream);
}

struct Tile {
  int mt, nt;
};

// Tile shape for an M x N problem. Each CU streams its blocks' operands through its L1
// at a roughly fixed rate (limited by the misses it can keep in flight), so the time goes
// with the rows of A and B one CU loads: (blocks per CU, rounded up) x (16 kMT + 16 kNT)
// rows of K. The shape with the fewest such rows wins; ties go to the larger tile.
Tile pick_tile(int M, int N, bool swiglu, int cus) {
  static const Tile kTiles[] = {{4, 4}, {4, 2}, {2, 4}, {2, 2}, {1, 4}, {1, 2}};
  Tile best = kTiles[0];
  long long best_cost = -1;
  for (const Tile &t : kTiles) {
    if (t.mt > 1 && M <= 16 * (t.mt / 2)) continue;  // a row tile mostly empty
    const int out_cols = (swiglu ? 8 : 16) * t.nt;
    const long long blocks = static_cast<long long>((M + 16 * t.mt - 1) / (16 * t.mt)) *
                             ((N + out_cols - 1) / out_cols);
    const long long cost = (blocks + cus - 1) / cus * (16 * t.mt + 16 * t.nt);
    if (best_cost < 0 || cost < best_cost) {
      best = t;
      best_cost = cost;
    }
  }
  return best;
}

template <int kMT, int kNT, bool kSwiglu>
int launch_tile(const uint16_t *a, int64_t lda, int32_t m, const uint16_t *b0, const uint16_t *b1,
                int64_t ldb, uint16_t *c, int64_t ldc, int32_t n, int32_t k, float limit,
                void *stream) {
  const int bm = 16 * kMT, bn = (kSwiglu ? 8 : 16) * kNT;
  const dim3 grid(static_cast<unsigned>((n + bn - 1) / bn), static_cast<unsigned>((m + bm - 1) / bm));
  return moe::launch(kSwiglu ? "moe_dense_gate_up_swiglu_bf16" : "moe_dense_gemm_bf16",
                     dense_gemm_kernel<kMT, kNT, 2, kSwiglu>, grid, dim3(kThreads), 0, stream, a,
                     lda, m, b0, b1, ldb, c, ldc, n, k, limit);
}

template <bool kSwiglu>
int dispatch(const uint16_t *a, int64_t lda, int32_t m, const uint16_t *b0, const uint16_t *b1,
             int64_t ldb, uint16_t *c, int64_t ldc, int32_t n, int32_t k, float limit,
             void *stream) {
  const Tile t = pick_tile(m, n, kSwiglu, device_cus());
#define MOE_DENSE_TILE(MT_, NT_)                                                        \
  if (t.mt == MT_ && t.nt == NT_)                                                       \
    return launch_tile<MT_, NT_, kSwiglu>(a, lda, m, b0, b1, ldb, c, ldc, n, k, limit, \
                                          stream);
  MOE_DENSE_TILE(4, 4)
  MOE_DENSE_TILE(4, 2)
  MOE_DENSE_TILE(2, 4)
  MOE_DENSE_TILE(2, 2)
  MOE_DENSE_TILE(1, 4)
  MOE_DENSE_TILE(1, 2)
#undef MOE_DENSE_TILE
  moe::set_error("dense gemm: no kernel for tile %dx%d", t.mt, t.nt);
  return MOE_EINVAL;
}

// Shared argument checks: sizes, strides, alignment and the 32-bit buffer ranges.
int check_dense_args(const char *name, const void *a, int64_t lda, const void *b0,
                     const void *b1, int64_t ldb, const void *c, int64_t ldc, int32_t m,
                     int32_t n, int32_t k) {
  MOE_REQUIRE(m >= 0 && n >= 0 && k >= 0, "%s: negative size", name);
  MOE_REQUIRE(n % 16 == 0, "%s: the output width must be a multiple of 16 (got %d)", name, n);
  MOE_REQUIRE(k % kChunkK == 0, "%s: K must be a multiple of %d (got %d)", name, kChunkK, k);
  MOE_REQUIRE(lda >= k && ldb >= k && ldc >= n, "%s: a leading dimension is below its width",
              name);
  MOE_REQUIRE(lda % 8 == 0 && ldb % 8 == 0 && ldc % 4 == 0,
              "%s: lda and ldb must be multiples of 8, ldc of 4", name);
  // A block's resource spans at most 64 rows of A or B.
  MOE_REQUIRE(lda <= (1LL << 23) && ldb <= (1LL << 23),
              "%s: lda and ldb must be at most 2^23 elements", name);
  if (m == 0 || n == 0) return MOE_OK;
  MOE_REQUIRE(c != nullptr, "%s: c is NULL", name);
  if (k == 0) return MOE_OK;  // the empty sum: a and b are not read
  MOE_REQUIRE(a && b0 && b1, "%s: a required pointer is NULL", name);
  MOE_REQUIRE(moe::aligned16(a) && moe::aligned16(b0) && moe::aligned16(b1),
              "%s: a and b must be 16-byte aligned", name);
  MOE_REQUIRE((reinterpret_cast<uintptr_t>(c) & 7u) == 0, "%s: c must be 8-byte aligned", name);
  return MOE_OK;
}

}  // namespace

// ------------------------------------------------------------ no-allocation variant
//
// moe_dense_gemm_bf16_noalloc runs the split-K form with its FP32 partial tiles in the
// library's own device array instead of a caller workspace. Each GPU the library runs on
// holds one copy of the array (module-scope device memory, until the process ends); every
// call on that GPU shares it and it keeps the last call's contents. The split-K partial
// kernel writes every partial tile before the reduction reads it, so nothing needs to
// start at zero.
static __device__ __align__(256) uint8_t scratch[MOE_DENSE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per device (in
// host code the array's name is only a stand-in, never a device address). Returns
// MOE_OK and sets *ptr, or an error status with the message recorded.
int scratch_on_current_device(void **ptr) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) {
    moe::set_error("moe_dense_gemm_bf16_noalloc: hipGetDevice failed: %s", hipGetErrorString(err));
    return MOE_ELAUNCH;
  }
  MOE_REQUIRE_CODE(dev >= 0 && dev < kMaxDevices, MOE_ELAUNCH,
                   "moe_dense_gemm_bf16_noalloc: device %d beyond the %d the library tracks", dev,
                   kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || p == nullptr) {
      moe::set_error("moe_dense_gemm_bf16_noalloc: hipGetSymbolAddress(scratch) failed: %s",
                     hipGetErrorString(err));
      return MOE_ELAUNCH;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_dense_gemm_bf16_noalloc(const uint16_t *a, int64_t lda, const uint16_t *b,
                                           int64_t ldb, uint16_t *c, int64_t ldc, int32_t m,
                                           int32_t n, int32_t k, void *stream) {
  moe::clear_error();
  const char *name = "moe_dense_gemm_bf16_noalloc";
  const int rc = check_dense_args(name, a, lda, b, b, ldb, c, ldc, m, n, k);
  if (rc != MOE_OK || m == 0 || n == 0) return rc;
  const int64_t need = splitk_shape(m, n, k, false).bytes;
  MOE_REQUIRE_CODE(need <= MOE_DENSE_NOALLOC_SCRATCH_BYTES, MOE_ECAPACITY,
                   "%s: m %d, n %d, k %d need %lld bytes of split-K partials; the library's "
                   "scratch holds %lld (use moe_dense_gemm_bf16 with a workspace)",
                   name, m, n, k, static_cast<long long>(need),
                   static_cast<long long>(MOE_DENSE_NOALLOC_SCRATCH_BYTES));
  void *ws = nullptr;
  const int src = scratch_on_current_device(&ws);
  if (src != MOE_OK) return src;
  return launch_splitk<false>(a, lda, m, b, b, ldb, c, ldc, n, k, 0.f, ws,
                              MOE_DENSE_NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" int64_t moe_dense_workspace_bytes(int32_t m, int32_t n, int32_t k, int32_t swiglu) {
  if (m <= 0 || n <= 0 || k < 0) return 0;
  return splitk_shape(m, n, k, swiglu != 0).bytes;
}

extern "C" int moe_dense_gemm_bf16(const uint16_t *a, int64_t lda, const uint16_t *b,
                                   int64_t ldb, uint16_t *c, int64_t ldc, int32_t m, int32_t n,
                                   int32_t k, void *workspace, int64_t workspace_bytes,
                                   void *stream) {
  moe::clear_error();
  const int rc = check_dense_args("moe_dense_gemm_bf16", a, lda, b, b, ldb, c, ldc, m, n, k);
  if (rc != MOE_OK || m == 0 || n == 0) return rc;
  if (workspace != nullptr)
    return launch_splitk<false>(a, lda, m, b, b, ldb, c, ldc, n, k, 0.f, workspace,
                                workspace_bytes, stream);
  return dispatch<false>(a, lda, m, b, b, ldb, c, ldc, n, k, 0.f, stream);
}

extern "C" int moe_dense_gate_up_swiglu_bf16(const uint16_t *a, int64_t lda,
                                             const uint16_t *gate_w, const uint16_t *up_w,
                                             int64_t ldw, uint16_t *act, int64_t ld_act,
                                             int32_t m, int32_t inter, int32_t k, float limit,
                                             void *workspace, int64_t workspace_bytes,
                                             void *stream) {
  moe::clear_error();
  const int rc = check_dense_args("moe_dense_gate_up_swiglu_bf16", a, lda, gate_w, up_w, ldw, act,
                                  ld_act, m, inter, k);
  if (rc != MOE_OK) return rc;
  MOE_REQUIRE(limit == limit && limit > 0.f,
              "moe_dense_gate_up_swiglu_bf16: limit must be positive (got %g)",
              static_cast<double>(limit));
  if (m == 0 || inter == 0) return MOE_OK;
  if (workspace != nullptr)
    return launch_splitk<true>(a, lda, m, gate_w, up_w, ldw, act, ld_act, inter, k, limit,
                               workspace, workspace_bytes, stream);
  return dispatch<true>(a, lda, m, gate_w, up_w, ldw, act, ld_act, inter, k, limit, stream);
}

extern "C" int32_t moe_dense_splitk_ways(int32_t m, int32_t k) {
  if (m <= 0 || k <= 0 || k % kLK != 0) return 1;
  return splitk_ways(m, k);
}

extern "C" int moe_dense_gemm_bf16_partials(const uint16_t *a, int64_t lda, const uint16_t *b,
                                            int64_t ldb, float *partials, int32_t m, int32_t n,
                                            int32_t k, int64_t partials_bytes, void *stream) {
  moe::clear_error();
  const char *name = "moe_dense_gemm_bf16_partials";
  // c is not written: the partials stand in for it in the shared checks.
  const int rc = check_dense_args(name, a, lda, b, b, ldb, partials, n, m, n, k);
  if (rc != MOE_OK || m == 0 || n == 0) return rc;
  const int64_t need = static_cast<int64_t>(splitk_ways(m, k)) * m * n * 4;
  MOE_REQUIRE_CODE(partials_bytes >= need, MOE_ECAPACITY,
                   "%s: the partials buffer holds %lld bytes, m %d, n %d, k %d need %lld", name,
                   static_cast<long long>(partials_bytes), m, n, k,
                   static_cast<long long>(need));
  MOE_REQUIRE(moe::aligned16(partials), "%s: partials must be 16-byte aligned", name);
  return launch_partials_row_major(a, lda, m, b, ldb, n, k, partials, stream);
}
