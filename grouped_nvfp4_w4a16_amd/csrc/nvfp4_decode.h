// NVFP4 -> BF16 weight decode for gfx950, bit-exact to
//   w = bf16_rne( fp32( fp32(e2m1(q) * e4m3(d)) * scale2 ) )
// the operand the grouped GEMM stages for its BF16 matrix multiply ("Module
// forward_prefill_gemm", section "What is NOT bit-identical", item 2; codebook, block
// scale and per-tensor scale rows of its layout table).
//
// Why not one multiply per element: at HBM speed the chip has only about three VALU
// operations per weight element to spend, so the decode works on bit patterns.
//
// Within one 16-k block every weight takes one of 16 values: the 8 E2M1 magnitudes
// {0, .5, 1, 1.5, 2, 3, 4, 6} through the formula, each with either sign. IEEE
// multiplication and round-to-nearest-even are symmetric in the sign of an operand, so
// the BF16 value of nibble q is the value of its magnitude code (q & 7) with bit 15
// flipped when q has its sign bit (bit 3) set. That holds for every block scale and
// scale2, zero, negative, subnormal and NaN included, so one path serves every block.
//
// The 8 BF16 magnitudes of a block, each computed by the formula itself, form a table
// (Fp4Table). Its low and high bytes are two 8-entry byte tables; v_perm_b32 looks up
// four elements per instruction, the nibble's sign is XORed into the high byte and the
// bytes are interleaved into BF16 pairs: 14 VALU operations per 8 elements. The table
// depends only on the scale code and scale2, so a caller that decodes many blocks builds
// it once per code.
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

// The BF16 values of the 8 E2M1 magnitude codes of one block, split into byte tables.
struct Fp4Table {
  uint32_t lo03, lo47;  // low bytes of the BF16 values of codes 0-3 and 4-7
  uint32_t hi03, hi47;  // high bytes
};

// The table of a block with scale d, each entry by the formula: the first product is
// exact in FP32 (a magnitude has at most 2 significant bits, d at most 4), the second is
// rounded to FP32, then to BF16 by round-to-nearest-even.
__device__ __forceinline__ Fp4Table make_table(float d, float scale2) {
  const auto w = [&](float m) { return (m * d) * scale2; };
  const uint32_t p01 = pack_bf16x2(w(0.0f), w(0.5f)), p23 = pack_bf16x2(w(1.0f), w(1.5f));
  const uint32_t p45 = pack_bf16x2(w(2.0f), w(3.0f)), p67 = pack_bf16x2(w(4.0f), w(6.0f));
  Fp4Table t;
  t.lo03 = byte_perm(p23, p01, 0x06040200u);
  t.hi03 = byte_perm(p23, p01, 0x07050301u);
  t.lo47 = byte_perm(p67, p45, 0x06040200u);
  t.hi47 = byte_perm(p67, p45, 0x07050301u);
  return t;
}

// Decodes the 8 nibbles of x (k = 0..7, even k in the low nibble of each byte) into four
// BF16 pairs in the order (k0,k2) (k4,k6) (k1,k3) (k5,k7). The matrix-core operand uses
// this k order; the activations are staged in the same order. 14 VALU operations.
__device__ __forceinline__ void decode8(uint32_t x, const Fp4Table &t, uint32_t out[4]) {
  const uint32_t se = x & 0x07070707u;          // magnitude codes of k0, k2, k4, k6
  const uint32_t so = (x >> 4) & 0x07070707u;   // magnitude codes of k1, k3, k5, k7
  const uint32_t le = byte_perm(t.lo47, t.lo03, se);
  const uint32_t he = byte_perm(t.hi47, t.hi03, se) ^ ((x << 4) & 0x80808080u);
  const uint32_t lo = byte_perm(t.lo47, t.lo03, so);
  const uint32_t ho = byte_perm(t.hi47, t.hi03, so) ^ (x & 0x80808080u);
  out[0] = byte_perm(he, le, 0x05010400u);
  out[1] = byte_perm(he, le, 0x07030602u);
  out[2] = byte_perm(ho, lo, 0x05010400u);
  out[3] = byte_perm(ho, lo, 0x07030602u);
}

}  // namespace moe
