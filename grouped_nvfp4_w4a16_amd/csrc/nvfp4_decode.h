// NVFP4 -> BF16 weight decode for gfx950, bit-exact to
//   w = bf16_rne( fp32( fp32(e2m1(q) * e4m3(d)) * scale2 ) )
// the operand the grouped GEMM stages for its BF16 matrix multiply ("Module
// forward_prefill_gemm", section "What is NOT bit-identical", item 2; codebook, block
// scale and per-tensor scale rows of its layout table).
//
// Why not one multiply per element: at HBM speed the chip has only about three VALU
// operations per weight element to spend, so the decode works on bit patterns.
//
// For a 16-k block with scale d (and the expert's scale2) every E2M1 magnitude is
// m * 2^j with m in {1, 1.5}: {0, .5, 1, 1.5, 2, 3, 4, 6}. The first product v * d is
// exact in FP32, and scaling by 2^j commutes with both roundings while the values stay
// normal, so with
//   P = bf16(fp32(d * scale2)),   Q = bf16(fp32(fp32(1.5 * d) * scale2))
// the eight BF16 results are {0, P - 0x80, P, Q, P + 0x80, Q + 0x80, P + 0x100, Q + 0x100}
// as bit patterns (0x80 is one step of the BF16 exponent). Their low and high bytes form
// two 8-entry byte tables, and v_perm_b32 looks up four elements per instruction; the
// nibble's sign bit is ORed into the high byte. About 1.75 VALU operations per element
// plus about 12 per 16-element block for the tables.
//
// The identity needs P's exponent field >= 3 (so P - 0x80 and the FP32 value halved stay
// normal) and Q + 0x100 finite; a zero, negative, subnormal-range, huge or NaN scale fails
// that check and the block takes the exact per-element path instead.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

__device__ __forceinline__ uint32_t byte_perm(uint32_t hi4, uint32_t lo4, uint32_t sel) {
  // Result byte i = byte sel[i] of the 8-byte pool {hi4 (bytes 4-7) : lo4 (bytes 0-3)};
  // selector 12 gives 0x00.
  return __builtin_amdgcn_perm(hi4, lo4, sel);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // Round-to-nearest-even, one v_cvt_pk_bf16_f32.
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Two E4M3 (OCP FN) codes in the low 16 bits of `codes` -> FP32 (exact).
__device__ __forceinline__ void e4m3x2_to_f32(uint32_t codes, float &d0, float &d1) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes), false);
  d0 = v[0];
  d1 = v[1];
}

// Two E4M3 codes in the high 16 bits of `codes` -> FP32 (exact).
__device__ __forceinline__ void e4m3x2_to_f32_hi(uint32_t codes, float &d0, float &d1) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes), true);
  d0 = v[0];
  d1 = v[1];
}

struct Fp4Block {
  uint32_t lo03, lo47;  // low bytes of the 8 BF16 magnitudes (codes 0-3, 4-7)
  uint32_t hi03, hi47;  // high bytes
  uint32_t pq;          // P in bits 0-15, Q in bits 16-31
  float d;              // block scale value, for the exact path
};

// The bit-pattern identity holds for a block with these P (low half) and Q (high half).
__device__ __forceinline__ bool fast_pq(uint32_t pq) {
  return (pq & 0xFFFFu) >= 0x0180u && (pq >> 16) < 0x7E80u;
}

// Whether it holds for all four blocks: the smallest P and the largest Q decide
// (packed 16-bit min/max).
__device__ __forceinline__ bool fast_pq4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  const u16x2 x = __builtin_bit_cast(u16x2, a), y = __builtin_bit_cast(u16x2, b);
  const u16x2 z = __builtin_bit_cast(u16x2, c), w = __builtin_bit_cast(u16x2, d);
  const u16x2 mn = __builtin_elementwise_min(__builtin_elementwise_min(x, y),
                                             __builtin_elementwise_min(z, w));
  const u16x2 mx = __builtin_elementwise_max(__builtin_elementwise_max(x, y),
                                             __builtin_elementwise_max(z, w));
  return mn[0] >= 0x0180u && mx[1] < 0x7E80u;
}

__device__ __forceinline__ Fp4Block make_block(float d, float scale2) {
  Fp4Block b;
  const float p = d * scale2;
  const float q = (d * 1.5f) * scale2;  // 1.5 * d is exact: d has at most 4 significant bits
  const uint32_t pq = pack_bf16x2(p, q);  // P in bits 0-15, Q in bits 16-31
  b.pq = pq;
  const uint32_t r0 = pq - 0x80u;         // P - 0x80 in the low half
  const uint32_t r2 = pq + 0x00800080u;   // P + 0x80, Q + 0x80
  const uint32_t r3 = pq + 0x01000100u;   // P + 0x100, Q + 0x100
  // codes 0..3: {0, P - 0x80, P, Q};  codes 4..7: {P + 0x80, Q + 0x80, P + 0x100, Q + 0x100}
  b.lo03 = byte_perm(pq, r0, 0x0604000Cu);
  b.hi03 = byte_perm(pq, r0, 0x0705010Cu);
  b.lo47 = byte_perm(r3, r2, 0x06040200u);
  b.hi47 = byte_perm(r3, r2, 0x07050301u);
  b.d = d;
  return b;
}

// Exact per-element path: the formula itself, one FP32 product at a time.
__device__ __forceinline__ uint32_t decode_one_exact(uint32_t nib, float d, float scale2) {
  const uint32_t c = nib & 7u;
  const float m = (c & 1u) ? 1.5f : 1.0f;
  float mag = c == 0 ? 0.0f : (c == 1 ? 0.5f : ldexpf(m, static_cast<int>(c >> 1) - 1));
  const float v = (nib & 8u) ? -mag : mag;
  const float w = (v * d) * scale2;
  return pack_bf16x2(w, 0.0f) & 0xFFFFu;
}

// Fast path of decode8 (fast_pq must hold for the block): 14 VALU operations.
__device__ __forceinline__ void decode8_fast(uint32_t x, const Fp4Block &b, uint32_t out[4]) {
  const uint32_t se = x & 0x07070707u;          // magnitude codes of k0, k2, k4, k6
  const uint32_t so = (x >> 4) & 0x07070707u;   // magnitude codes of k1, k3, k5, k7
  const uint32_t le = byte_perm(b.lo47, b.lo03, se);
  const uint32_t he = byte_perm(b.hi47, b.hi03, se) | ((x << 4) & 0x80808080u);
  const uint32_t lo = byte_perm(b.lo47, b.lo03, so);
  const uint32_t ho = byte_perm(b.hi47, b.hi03, so) | (x & 0x80808080u);
  out[0] = byte_perm(he, le, 0x05010400u);
  out[1] = byte_perm(he, le, 0x07030602u);
  out[2] = byte_perm(ho, lo, 0x05010400u);
  out[3] = byte_perm(ho, lo, 0x07030602u);
}

// Exact path of decode8: the formula one element at a time.
__device__ __forceinline__ void decode8_exact(uint32_t x, float d, float scale2, uint32_t out[4]) {
  const auto e = [&](int i) { return decode_one_exact((x >> (4 * i)) & 15u, d, scale2); };
  out[0] = e(0) | (e(2) << 16);
  out[1] = e(4) | (e(6) << 16);
  out[2] = e(1) | (e(3) << 16);
  out[3] = e(5) | (e(7) << 16);
}

// Decodes the 8 nibbles of x (k = 0..7, even k in the low nibble of each byte) into four
// BF16 pairs in the order (k0,k2) (k4,k6) (k1,k3) (k5,k7). The matrix-core operand uses
// this k order; the activations are staged in the same order.
__device__ __forceinline__ void decode8(uint32_t x, const Fp4Block &b, float scale2,
                                        uint32_t out[4]) {
  if (fast_pq(b.pq)) {
    decode8_fast(x, b, out);
  } else {
    decode8_exact(x, b.d, scale2, out);
  }
}

}  // namespace moe
