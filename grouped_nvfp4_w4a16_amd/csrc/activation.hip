// swiglu_clamp, moe_combine and moe_zero_rows: the bandwidth-bound steps around the
// grouped GEMMs.
//
// swiglu_clamp follows swiglu_rows on the 2026-09-25 glm5next_mlp forward.rs page:
// out = silu(min(gate, limit)) * clamp(up, -limit, limit). moe_combine follows that
// page's forward_moe: one launch for all rows, each slot's expert-sorted row found
// through token_to_perm, weighted by its top-k weight, plus the shared-expert output.
// moe_zero_rows is that forward_moe's zero-first step on expert_out, so that the rows of
// remote experts (never written by the down GEMM) add zero in the combine.
//
// Both kernels move 16 bytes (8 BF16) per thread per operand with 128-bit loads and
// stores and compute in FP32; a block of 256 threads covers 2048 columns of one row.
#include "buffer_io.h"
#include "common.h"
#include "nvfp4_decode.h"  // moe::pack_bf16x2: the rounding the dense GEMM's output uses
#include "swiglu.h"

namespace {

constexpr int kThreads = 256;
constexpr int kColsPerBlock = kThreads * 8;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const __bf16 a = static_cast<__bf16>(lo), b = static_cast<__bf16>(hi);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ void unpack8(uint4 v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
}

// The shared term of 8 columns: BF16 values of `shared`, or, with `sp` (FP32 split-K
// partials [ways][rows][hidden] of the shared expert's down projection), their sum in split
// order rounded to BF16 as the dense GEMM rounds its output, so both give the same bits.
__device__ __forceinline__ void add_shared(float (&acc)[8], const uint16_t *__restrict__ shared,
                                           int64_t ld_s, const float *__restrict__ sp,
                                           int32_t sp_ways, int64_t sp_stride, int row, int col,
                                           int32_t hidden) {
  if (sp != nullptr) {  // uniform
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    const f32x4_t *q =
        reinterpret_cast<const f32x4_t *>(sp + static_cast<int64_t>(row) * hidden + col);
    f32x4_t s0 = q[0], s1 = q[1];
    for (int w = 1; w < sp_ways; ++w) {
      const f32x4_t *qw = reinterpret_cast<const f32x4_t *>(
          sp + w * sp_stride + static_cast<int64_t>(row) * hidden + col);
      s0 += qw[0];
      s1 += qw[1];
    }
    const uint4 v = make_uint4(moe::pack_bf16x2(s0[0], s0[1]), moe::pack_bf16x2(s0[2], s0[3]),
                               moe::pack_bf16x2(s1[0], s1[1]), moe::pack_bf16x2(s1[2], s1[3]));
    float sh[8];
    unpack8(v, sh);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += sh[i];
  } else if (shared != nullptr) {
    float sh[8];
    unpack8(*reinterpret_cast<const uint4 *>(shared + static_cast<size_t>(row) * ld_s + col), sh);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += sh[i];
  }
}

__global__ __launch_bounds__(kThreads) void swiglu_clamp_kernel(
    const uint16_t *__restrict__ gate, const uint16_t *__restrict__ up, int64_t ld_in,
    uint16_t *__restrict__ out, int64_t ld_out, int32_t n, float limit) {
  const int row = blockIdx.y;
  const int col = (blockIdx.x * kThreads + threadIdx.x) * 8;
  if (col >= n) return;
  const size_t in_off = static_cast<size_t>(row) * ld_in + col;
  float g[8], u[8], o[8];
  unpack8(*reinterpret_cast<const uint4 *>(gate + in_off), g);
  unpack8(*reinterpret_cast<const uint4 *>(up + in_off), u);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = moe::swiglu_clamp1(g[i], u[i], limit);
  *reinterpret_cast<uint4 *>(out + static_cast<size_t>(row) * ld_out + col) = pack8(o);
}

__global__ __launch_bounds__(kThreads) void moe_combine_kernel(
    const uint16_t *__restrict__ expert_out, int64_t ld_e, int32_t expert_rows,
    const int32_t *__restrict__ token_to_perm, const float *__restrict__ weights,
    const uint16_t *__restrict__ shared, int64_t ld_s, const float *__restrict__ sp,
    int32_t sp_ways, int64_t sp_stride, uint16_t *__restrict__ out, int64_t ld_out,
    int32_t hidden, int32_t top_k) {
  const int row = blockIdx.y;
  const int col = (blockIdx.x * kThreads + threadIdx.x) * 8;
  if (col >= hidden) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < top_k; ++j) {
    const int p = token_to_perm[static_cast<size_t>(row) * top_k + j];
    if (p < 0 || p >= expert_rows) continue;  // excluded slot: adds zero
    const float w = weights[static_cast<size_t>(row) * top_k + j];
    float v[8];
    unpack8(*reinterpret_cast<const uint4 *>(expert_out + static_cast<size_t>(p) * ld_e + col), v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += w * v[i];
  }
  add_shared(acc, shared, ld_s, sp, sp_ways, sp_stride, row, col, hidden);
  *reinterpret_cast<uint4 *>(out + static_cast<size_t>(row) * ld_out + col) = pack8(acc);
}

// Zeroes rows x cols of a BF16 matrix: one 16-byte store per thread.
__global__ __launch_bounds__(kThreads) void zero_rows_kernel(uint16_t *__restrict__ c,
                                                             int64_t ldc, int64_t units_per_row,
                                                             int64_t units) {
  const int64_t u = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (u >= units) return;
  const int64_t row = u / units_per_row, col8 = u - row * units_per_row;
  *reinterpret_cast<uint4 *>(c + row * ldc + col8 * 8) = make_uint4(0u, 0u, 0u, 0u);
}

// The same combine for top_k == 8 with the expert rows read through a buffer resource:
// the eight slot indices and weights are loaded first, then the eight rows together (an
// excluded slot's offset is past the end and reads zeros without a memory access), so a
// thread waits on two memory round trips instead of two per slot. The sum is still taken
// in slot order and skips excluded slots, so the result has the generic kernel's bits.
__global__ __launch_bounds__(kThreads) void moe_combine8_kernel(
    const uint16_t *__restrict__ expert_out, int64_t ld_e, int32_t expert_rows,
    const int32_t *__restrict__ token_to_perm, const float *__restrict__ weights,
    const uint16_t *__restrict__ shared, int64_t ld_s, const float *__restrict__ sp,
    int32_t sp_ways, int64_t sp_stride, uint16_t *__restrict__ out, int64_t ld_out,
    int32_t hidden) {
  constexpr int kK = 8;
  const int row = blockIdx.y;
  const int col = (blockIdx.x * kThreads + threadIdx.x) * 8;
  if (col >= hidden) return;
  const __amdgpu_buffer_rsrc_t er = moe::make_rsrc(
      expert_out, static_cast<uint32_t>(static_cast<uint64_t>(expert_rows) * ld_e * 2));
  int p[kK];
  float w[kK];
#pragma unroll
  for (int j = 0; j < kK; ++j) {
    p[j] = token_to_perm[static_cast<size_t>(row) * kK + j];
    w[j] = weights[static_cast<size_t>(row) * kK + j];
  }
  moe::u32x4_t v[kK];
#pragma unroll
  for (int j = 0; j < kK; ++j) {
    const bool ok = p[j] >= 0 && p[j] < expert_rows;
    const uint32_t off = ok ? (static_cast<uint32_t>(p[j]) * static_cast<uint32_t>(ld_e) +
                               static_cast<uint32_t>(col)) * 2u
                            : moe::kNoLoad;
    v[j] = moe::load16(er, off, 0);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kK; ++j) {
    if (p[j] < 0 || p[j] >= expert_rows) continue;  // excluded slot: adds nothing
    float f[8];
    unpack8(make_uint4(v[j][0], v[j][1], v[j][2], v[j][3]), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += w[j] * f[i];
  }
  add_shared(acc, shared, ld_s, sp, sp_ways, sp_stride, row, col, hidden);
  *reinterpret_cast<uint4 *>(out + static_cast<size_t>(row) * ld_out + col) = pack8(acc);
}

}  // namespace

extern "C" int moe_zero_rows(uint16_t *c, int64_t ldc, int32_t rows, int32_t cols,
                             void *stream) {
  moe::clear_error();
  MOE_REQUIRE(rows >= 0 && cols >= 0 && cols % 8 == 0,
              "zero_rows: need rows >= 0 and cols >= 0 a multiple of 8 (rows=%d cols=%d)", rows,
              cols);
  MOE_REQUIRE(ldc >= cols && ldc % 8 == 0,
              "zero_rows: ldc must be >= cols and a multiple of 8");
  if (rows == 0 || cols == 0) return MOE_OK;
  MOE_REQUIRE(c != nullptr && moe::aligned16(c), "zero_rows: c must be non-NULL and 16-byte aligned");
  const int64_t per_row = cols / 8, units = per_row * rows;
  MOE_REQUIRE((units + kThreads - 1) / kThreads <= INT32_MAX, "zero_rows: matrix too large");
  return moe::launch("moe_zero_rows", zero_rows_kernel,
                     dim3(static_cast<unsigned>((units + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, c, ldc, per_row, units);
}

extern "C" int swiglu_clamp(const uint16_t *gate, const uint16_t *up, int64_t ld_in,
                            uint16_t *out, int64_t ld_out, int32_t rows, int32_t n, float limit,
                            void *stream) {
  moe::clear_error();
  MOE_REQUIRE(rows >= 0 && n >= 0 && n % 8 == 0,
              "swiglu_clamp: need rows >= 0 and n >= 0 a multiple of 8 (rows=%d n=%d)", rows, n);
  MOE_REQUIRE(limit > 0.0f, "swiglu_clamp: limit must be > 0");
  MOE_REQUIRE(ld_in >= n && ld_in % 8 == 0 && ld_out >= n && ld_out % 8 == 0,
              "swiglu_clamp: leading dimensions must be >= n and multiples of 8");
  MOE_REQUIRE(rows <= 65535, "swiglu_clamp: rows must be <= 65535 (got %d)", rows);
  if (rows == 0 || n == 0) return MOE_OK;
  MOE_REQUIRE(gate && up && out, "swiglu_clamp: a required pointer is NULL");
  MOE_REQUIRE(moe::aligned16(gate) && moe::aligned16(up) && moe::aligned16(out),
              "swiglu_clamp: pointers must be 16-byte aligned");
  const dim3 grid((n + kColsPerBlock - 1) / kColsPerBlock, rows);
  return moe::launch("swiglu_clamp", swiglu_clamp_kernel, grid, dim3(kThreads), 0, stream, gate,
                     up, ld_in, out, ld_out, n, limit);
}

namespace {

int combine_launch(const char *name, const uint16_t *expert_out, int64_t ld_e,
                   int32_t expert_rows, const int32_t *token_to_perm,
                   const float *topk_weights, const uint16_t *shared, int64_t ld_s,
                   const float *sp, int32_t sp_ways, uint16_t *out, int64_t ld_out, int32_t rows,
                   int32_t hidden, int32_t top_k, void *stream) {
  MOE_REQUIRE(rows >= 0 && hidden >= 0 && hidden % 8 == 0,
              "%s: need rows >= 0 and hidden >= 0 a multiple of 8", name);
  MOE_REQUIRE(top_k >= 1 && expert_rows >= 0, "%s: need top_k >= 1, expert_rows >= 0", name);
  MOE_REQUIRE(ld_e >= hidden && ld_e % 8 == 0 && ld_out >= hidden && ld_out % 8 == 0,
              "%s: leading dimensions must be >= hidden and multiples of 8", name);
  MOE_REQUIRE(shared == nullptr || (ld_s >= hidden && ld_s % 8 == 0),
              "%s: ld_s must be >= hidden and a multiple of 8", name);
  MOE_REQUIRE(rows <= 65535, "%s: rows must be <= 65535 (got %d)", name, rows);
  if (rows == 0 || hidden == 0) return MOE_OK;
  MOE_REQUIRE(expert_out && token_to_perm && topk_weights && out,
              "%s: a required pointer is NULL", name);
  MOE_REQUIRE(moe::aligned16(expert_out) && moe::aligned16(out) &&
                  (shared == nullptr || moe::aligned16(shared)) &&
                  (sp == nullptr || moe::aligned16(sp)),
              "%s: BF16 and FP32 pointers must be 16-byte aligned", name);
  const int64_t sp_stride = static_cast<int64_t>(rows) * hidden;
  const dim3 grid((hidden + kColsPerBlock - 1) / kColsPerBlock, rows);
  // top_k 8 with expert rows below 2 GiB (buffer offsets are 32-bit; an excluded slot's
  // offset 2^31 must lie past the end): all slot rows in flight at once.
  if (top_k == 8 && static_cast<uint64_t>(expert_rows) * ld_e * 2 < (1ull << 31))
    return moe::launch(name, moe_combine8_kernel, grid, dim3(kThreads), 0, stream, expert_out,
                       ld_e, expert_rows, token_to_perm, topk_weights, shared, ld_s, sp, sp_ways,
                       sp_stride, out, ld_out, hidden);
  return moe::launch(name, moe_combine_kernel, grid, dim3(kThreads), 0, stream, expert_out,
                     ld_e, expert_rows, token_to_perm, topk_weights, shared, ld_s, sp, sp_ways,
                     sp_stride, out, ld_out, hidden, top_k);
}

}  // namespace

extern "C" int moe_combine(const uint16_t *expert_out, int64_t ld_e, int32_t expert_rows,
                           const int32_t *token_to_perm, const float *topk_weights,
                           const uint16_t *shared, int64_t ld_s, uint16_t *out, int64_t ld_out,
                           int32_t rows, int32_t hidden, int32_t top_k, void *stream) {
  moe::clear_error();
  return combine_launch("moe_combine", expert_out, ld_e, expert_rows, token_to_perm,
                        topk_weights, shared, ld_s, nullptr, 0, out, ld_out, rows, hidden, top_k,
                        stream);
}

extern "C" int moe_combine_partials(const uint16_t *expert_out, int64_t ld_e,
                                    int32_t expert_rows, const int32_t *token_to_perm,
                                    const float *topk_weights, const float *shared_partials,
                                    int32_t ways, int64_t partials_bytes, uint16_t *out,
                                    int64_t ld_out, int32_t rows, int32_t hidden, int32_t top_k,
                                    void *stream) {
  moe::clear_error();
  MOE_REQUIRE(ways >= 1 && ways <= 64, "moe_combine_partials: ways must be in [1, 64] (got %d)",
              ways);
  if (rows > 0 && hidden > 0) {
    MOE_REQUIRE(shared_partials != nullptr, "moe_combine_partials: shared_partials is NULL");
    const int64_t need = static_cast<int64_t>(ways) * rows * hidden * 4;
    MOE_REQUIRE_CODE(partials_bytes >= need, MOE_ECAPACITY,
                     "moe_combine_partials: %lld bytes of partials, %d x %d x %d need %lld",
                     static_cast<long long>(partials_bytes), ways, rows, hidden,
                     static_cast<long long>(need));
  }
  return combine_launch("moe_combine_partials", expert_out, ld_e, expert_rows, token_to_perm,
                        topk_weights, nullptr, 0, shared_partials, ways, out, ld_out, rows,
                        hidden, top_k, stream);
}
