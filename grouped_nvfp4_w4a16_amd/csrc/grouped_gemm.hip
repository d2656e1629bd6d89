// moe_w4a16_grouped_gemm: one launch over all experts of a routed MoE layer.
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
//   - grid = (N / 128 weight-row tiles, experts); a block of 8 wave64s owns 128 weight
//     rows of one expert (16 per wave) over the whole K, and loops over that expert's
//     sorted rows 32 at a time, so its weight bytes are streamed once per 32 rows.
//   - The weights are the MFMA A operand (v_mfma_f32_16x16x32_bf16, M = 16 weight rows):
//     each lane loads 2 x 16 bytes of packed nibbles (64 k of one row) plus the row's 16
//     scale bytes per 256-k step with 128-bit loads, and decodes them in registers
//     (nvfp4_decode.h) straight into A; no dequantised weight goes through LDS.
//   - The gathered activation rows are the B operand (16 rows per MFMA tile). They are
//     staged per 256-k step in LDS (double buffered, one barrier per step), shared by the
//     8 waves, with k permuted inside each group of 8 to match the decoder's order.
//   - Output: each lane holds 4 consecutive weight rows of one sorted row -> one 8-byte
//     store of BF16 (round-to-nearest-even).
#include "common.h"
#include "nvfp4_decode.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 16;
constexpr int kBlockN = kWaves * kRowsPerWave;    // weight rows per block
constexpr int kChunkK = 256;                      // k per main-loop step
constexpr int kTokTiles = 2;                      // 16-row MFMA tiles per pass
constexpr int kBlockM = 16 * kTokTiles;           // sorted rows per pass
constexpr int kLdsRowBytes = kChunkK * 2 + 16;    // staged activation row, padded
constexpr int kLdsBufBytes = kBlockM * kLdsRowBytes;
constexpr int kPiecesPerRow = kChunkK / 8;        // 16-byte pieces per staged row
constexpr int kPiecesPerThread = kBlockM * kPiecesPerRow / kThreads;
static_assert(kPiecesPerThread * kThreads == kBlockM * kPiecesPerRow, "staging split");

struct WeightRegs {
  uint4 a;  // packed bytes for k in [32 kb, 32 kb + 32) of the step
  uint4 b;  // packed bytes for k in [128 + 32 kb, 128 + 32 kb + 32)
  uint4 s;  // the row's 16 block-scale bytes of the step
};

__device__ __forceinline__ WeightRegs load_weights(const uint8_t *wrow, const uint8_t *srow,
                                                   int step, int kb) {
  WeightRegs r;
  const uint8_t *p = wrow + static_cast<size_t>(step) * (kChunkK / 2);
  r.a = *reinterpret_cast<const uint4 *>(p + 16 * kb);
  r.b = *reinterpret_cast<const uint4 *>(p + 64 + 16 * kb);
  r.s = *reinterpret_cast<const uint4 *>(srow + static_cast<size_t>(step) * (kChunkK / 16));
  return r;
}

// 8 BF16 (k0..k7) -> order (k0,k2) (k4,k6) (k1,k3) (k5,k7), the decoder's order.
__device__ __forceinline__ uint4 permute_k8(uint4 v) {
  uint4 o;
  o.x = moe::byte_perm(v.y, v.x, 0x05040100u);
  o.y = moe::byte_perm(v.w, v.z, 0x05040100u);
  o.z = moe::byte_perm(v.y, v.x, 0x07060302u);
  o.w = moe::byte_perm(v.w, v.z, 0x07060302u);
  return o;
}

__device__ __forceinline__ void stage_load(uint4 (&v)[kPiecesPerThread],
                                           const uint16_t *const (&src)[kPiecesPerThread],
                                           const int (&kofs)[kPiecesPerThread], int step) {
#pragma unroll
  for (int i = 0; i < kPiecesPerThread; ++i) {
    v[i] = src[i] != nullptr
               ? *reinterpret_cast<const uint4 *>(src[i] + step * kChunkK + kofs[i])
               : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void stage_store(uint8_t *buf, const uint4 (&v)[kPiecesPerThread],
                                            const int (&lds_off)[kPiecesPerThread]) {
#pragma unroll
  for (int i = 0; i < kPiecesPerThread; ++i)
    *reinterpret_cast<uint4 *>(buf + lds_off[i]) = permute_k8(v[i]);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint32_t (&w)[4]) {
  uint4 u = make_uint4(w[0], w[1], w[2], w[3]);
  return __builtin_bit_cast(bf16x8_t, u);
}

__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(
    const uint16_t *__restrict__ a, int64_t lda, int32_t a_rows,
    const int32_t *__restrict__ gather, const uint64_t *__restrict__ packed_ptrs,
    const uint64_t *__restrict__ scale_ptrs, const float *__restrict__ scale2s,
    const int32_t *__restrict__ offsets, uint16_t *__restrict__ c, int64_t ldc,
    int32_t max_rows, int32_t N, int32_t K) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][kLdsBufBytes];

  const int e = blockIdx.y;
  const uint8_t *packed = reinterpret_cast<const uint8_t *>(packed_ptrs[e]);
  if (packed == nullptr) return;  // expert not present: its rows keep the caller's values
  const int lo = max(offsets[e], 0);
  const int hi = min(offsets[e + 1], max_rows);
  if (hi <= lo) return;
  const uint8_t *scales = reinterpret_cast<const uint8_t *>(scale_ptrs[e]);
  const float scale2 = scale2s[e];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, kb = lane >> 4;
  const int n_wave0 = blockIdx.x * kBlockN + wave * kRowsPerWave;
  const bool wave_on = n_wave0 < N;  // N % 16 == 0: a wave's 16 rows are all in or all out
  const int n_row = wave_on ? n_wave0 + r16 : 0;
  const uint8_t *wrow = packed + static_cast<size_t>(n_row) * (K / 2);
  const uint8_t *srow = scales + static_cast<size_t>(n_row) * (K / 16);
  const int n_steps = K / kChunkK;

  // This lane's scale bytes within a step: groups 2kb, 2kb+1 (first 32 k) and
  // 8+2kb, 9+2kb (second 32 k).
  const int s_shift = (kb & 1) * 16;

  for (int m0 = lo; m0 < hi; m0 += kBlockM) {
    const int m_cnt = min(kBlockM, hi - m0);

    const uint16_t *src[kPiecesPerThread];
    int kofs[kPiecesPerThread], lds_off[kPiecesPerThread];
#pragma unroll
    for (int i = 0; i < kPiecesPerThread; ++i) {
      const int piece = tid + i * kThreads;
      const int row = piece / kPiecesPerRow, col = piece % kPiecesPerRow;
      kofs[i] = col * 8;
      lds_off[i] = row * kLdsRowBytes + col * 16;
      src[i] = nullptr;
      if (row < m_cnt) {
        const int s = m0 + row;
        const int g = gather != nullptr ? gather[s] : s;
        if (g >= 0 && g < a_rows) src[i] = a + static_cast<size_t>(g) * lda;
      }
    }

    f32x4_t acc[kTokTiles];
#pragma unroll
    for (int t = 0; t < kTokTiles; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    WeightRegs w{};
    if (wave_on) w = load_weights(wrow, srow, 0, kb);
    uint4 xv[kPiecesPerThread];
    stage_load(xv, src, kofs, 0);
    stage_store(xs[0], xv, lds_off);
    __syncthreads();

    for (int step = 0; step < n_steps; ++step) {
      const bool more = step + 1 < n_steps;
      WeightRegs wn{};
      if (more) {
        if (wave_on) wn = load_weights(wrow, srow, step + 1, kb);
        stage_load(xv, src, kofs, step + 1);
      }
      if (wave_on) {
        const uint8_t *xb = xs[step & 1];
        const uint32_t s_lo = ((kb & 2) ? w.s.y : w.s.x) >> s_shift;
        const uint32_t s_hi = ((kb & 2) ? w.s.w : w.s.z) >> s_shift;
        float d0, d1, d2, d3;
        moe::e4m3x2_to_f32(s_lo, d0, d1);
        moe::e4m3x2_to_f32(s_hi, d2, d3);
        const moe::Fp4Block blk[4] = {moe::make_block(d0, scale2), moe::make_block(d1, scale2),
                                      moe::make_block(d2, scale2), moe::make_block(d3, scale2)};
        const uint32_t words[8] = {w.a.x, w.a.y, w.a.z, w.a.w, w.b.x, w.b.y, w.b.z, w.b.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint32_t wd[4];
          moe::decode8(words[j], blk[j >> 1], scale2, wd);
          const bf16x8_t A = as_bf16x8(wd);
          const int kx = (j < 4 ? 32 * kb + 8 * j : 128 + 32 * kb + 8 * (j - 4)) * 2;
#pragma unroll
          for (int t = 0; t < kTokTiles; ++t) {
            if (t * 16 < m_cnt) {
              const bf16x8_t B =
                  *reinterpret_cast<const bf16x8_t *>(xb + (t * 16 + r16) * kLdsRowBytes + kx);
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[t], 0, 0, 0);
            }
          }
        }
      }
      if (more) stage_store(xs[(step + 1) & 1], xv, lds_off);
      __syncthreads();
      w = wn;
    }

    // acc[t][i] = result for weight row n_wave0 + 4 kb + i and sorted row m0 + 16 t + r16.
    if (wave_on) {
#pragma unroll
      for (int t = 0; t < kTokTiles; ++t) {
        const int tok = t * 16 + r16;
        if (tok < m_cnt) {
          uint2 o;
          o.x = moe::pack_bf16x2(acc[t][0], acc[t][1]);
          o.y = moe::pack_bf16x2(acc[t][2], acc[t][3]);
          *reinterpret_cast<uint2 *>(c + static_cast<size_t>(m0 + tok) * ldc + n_wave0 + 4 * kb) =
              o;
        }
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
  const moe::Fp4Block b0 = moe::make_block(d0, scale2), b1 = moe::make_block(d1, scale2);
  const uint32_t words[4] = {v.x, v.y, v.z, v.w};
  uint4 *dst = reinterpret_cast<uint4 *>(out + static_cast<size_t>(n) * K + q * 32);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t wd[4];
    moe::decode8(words[j], j < 2 ? b0 : b1, scale2, wd);
    // (k0,k2) (k4,k6) (k1,k3) (k5,k7) -> (k0,k1) (k2,k3) (k4,k5) (k6,k7)
    uint4 o;
    o.x = moe::byte_perm(wd[2], wd[0], 0x05040100u);
    o.y = moe::byte_perm(wd[2], wd[0], 0x07060302u);
    o.z = moe::byte_perm(wd[3], wd[1], 0x05040100u);
    o.w = moe::byte_perm(wd[3], wd[1], 0x07060302u);
    dst[j] = o;
  }
}

}  // namespace

extern "C" int moe_w4a16_grouped_gemm(const uint16_t *a, int64_t lda, int32_t a_rows,
                                      const int32_t *a_gather, const uint64_t *packed_ptrs,
                                      const uint64_t *scale_ptrs, const float *scale2,
                                      const int32_t *expert_offsets, int32_t num_experts,
                                      uint16_t *c, int64_t ldc, int32_t max_rows, int32_t n,
                                      int32_t k, void *stream) {
  moe::clear_error();
  MOE_REQUIRE(n > 0 && n % 16 == 0, "grouped_gemm: n must be a positive multiple of 16 (got %d)",
              n);
  MOE_REQUIRE(k > 0 && k % kChunkK == 0,
              "grouped_gemm: k must be a positive multiple of %d (got %d)", kChunkK, k);
  MOE_REQUIRE(lda >= k && lda % 8 == 0, "grouped_gemm: lda must be >= k and a multiple of 8");
  MOE_REQUIRE(ldc >= n && ldc % 8 == 0, "grouped_gemm: ldc must be >= n and a multiple of 8");
  MOE_REQUIRE(num_experts >= 1 && num_experts <= 65535,
              "grouped_gemm: num_experts must be in [1, 65535] (got %d)", num_experts);
  MOE_REQUIRE(max_rows >= 0 && a_rows >= 0, "grouped_gemm: max_rows and a_rows must be >= 0");
  MOE_REQUIRE(a && packed_ptrs && scale_ptrs && scale2 && expert_offsets && c,
              "grouped_gemm: a required pointer is NULL");
  MOE_REQUIRE(moe::aligned16(a) && moe::aligned16(c),
              "grouped_gemm: a and c must be 16-byte aligned");
  if (max_rows == 0) return MOE_OK;
  const dim3 grid((n + kBlockN - 1) / kBlockN, num_experts);
  return moe::launch("moe_w4a16_grouped_gemm", grouped_gemm_kernel, grid, dim3(kThreads), 0,
                     stream, a, lda, a_rows, a_gather, packed_ptrs, scale_ptrs, scale2,
                     expert_offsets, c, ldc, max_rows, n, k);
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
