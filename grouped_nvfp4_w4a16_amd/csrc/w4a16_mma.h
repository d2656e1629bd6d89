// Device helpers shared by the W4A16 kernels (grouped GEMM, union GEMV): the decoded
// weight tile as the A operand of v_mfma_f32_16x16x32_bf16, the activation operand in the
// decoder's k order, and the per-block table of decode tables (one entry per E4M3 code).
//
// Operand layout: lane (r16 = lane % 16, kb = lane / 16) holds, for one MFMA, 8 k of
// weight row r16 (A) and 8 k of activation row r16 (B). A lane's 16 bytes of packed
// nibbles (32 k) feed four MFMAs, one packed dword (8 k) each, so the decoder's order of
// those 8 k, (k0,k2) (k4,k6) (k1,k3) (k5,k7), is the order the activations are put in.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "buffer_io.h"
#include "nvfp4_decode.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 8 BF16 (k0..k7) -> order (k0,k2) (k4,k6) (k1,k3) (k5,k7), the decoder's order.
__device__ __forceinline__ u32x4_t permute_k8(u32x4_t v) {
  u32x4_t o;
  o[0] = byte_perm(v[1], v[0], 0x05040100u);
  o[1] = byte_perm(v[3], v[2], 0x05040100u);
  o[2] = byte_perm(v[1], v[0], 0x07060302u);
  o[3] = byte_perm(v[3], v[2], 0x07060302u);
  return o;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint32_t (&w)[4]) {
  const u32x4_t u = {w[0], w[1], w[2], w[3]};
  return __builtin_bit_cast(bf16x8_t, u);
}

// Multiply four packed dwords (32 k of one weight row per lane), decoded with the tables
// of their two 16-k blocks, into acc against four B operands.
__device__ __forceinline__ void mfma4(const uint32_t *words, const Fp4Table &b0,
                                      const Fp4Table &b1, const bf16x8_t *B, f32x4_t &acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t wd[4];
    decode8(words[j], j < 2 ? b0 : b1, wd);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wd), B[j], acc, 0, 0, 0);
  }
}

// As mfma4 for kMT B tiles (kMT x 16 activation rows): each packed dword is decoded once
// and multiplied into every tile's accumulator.
template <int kMT>
__device__ __forceinline__ void mfma4_tiles(const uint32_t *words, const Fp4Table &b0,
                                            const Fp4Table &b1, const bf16x8_t (*B)[4],
                                            f32x4_t *acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t wd[4];
    decode8(words[j], j < 2 ? b0 : b1, wd);
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wd), B[mt][j], acc[mt], 0, 0, 0);
  }
}

// The decode tables of four blocks whose E4M3 codes are the bytes of `sc`, from the LUT.
__device__ __forceinline__ void lut_blocks(uint32_t sc, const uint8_t *lut, Fp4Table *blk) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const u32x4_t t =
        *reinterpret_cast<const u32x4_t *>(lut + (((sc >> (8 * g)) & 0xFFu) << 4));
    blk[g].lo03 = t[0];
    blk[g].lo47 = t[1];
    blk[g].hi03 = t[2];
    blk[g].hi47 = t[3];
  }
}

// The decode table of every E4M3 scale code for an expert's scale2, one 16-byte entry per
// code {lo03, lo47, hi03, hi47} (4 KB of LDS). Thread `tid` of a 256-thread block writes
// code tid; no loop, so that it is scheduled behind the loads that precede it.
__device__ __forceinline__ void build_code_table_lut(uint8_t *lut, int tid, float scale2) {
  float d, unused;
  e4m3x2_to_f32(static_cast<uint32_t>(tid), d, unused);
  const Fp4Table b = make_table(d, scale2);
  const u32x4_t t = {b.lo03, b.lo47, b.hi03, b.hi47};
  *reinterpret_cast<u32x4_t *>(lut + tid * 16) = t;
}

}  // namespace moe
