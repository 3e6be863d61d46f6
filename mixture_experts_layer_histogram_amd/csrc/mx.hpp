// MXFP8 codec on gfx950: E4M3 elements sharing one E8M0 scale per 32 values along K.
//
// The MoK article (kucoin.com/es "Cursor's MoK logra un aumento del 2.37x ...", section
// 02) fuses MXFP8 quantisation into the dispatch, grouped-GEMM and SwiGLU data paths
// without giving the rule; the rule used is OCP Microscaling v1.0:
//   scale exponent e = floor(log2 amax) - 8 clamped to [-127, 127]  (code e + 127),
//   element = E4M3(v * 2^-e), nearest-even, saturated to +-448,
//   an all-zero block has scale code 0 and zero elements.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kMxBlock = 32;
constexpr int kMxTileK = 128;     // K values of one scale word (four blocks)

// Scale layout shared by every MXFP8 operand: for a matrix of `rows` rows, the scale code of
// block b of row r sits at byte 4 * (rows * (b / 4) + r) + b % 4 -- one 32-bit word per
// (128-value K tile, row), K tiles outermost.  A wave reading the words of 64 consecutive
// rows for one K tile then touches 256 contiguous bytes instead of 64 scattered lines.
__device__ __forceinline__ int64_t mx_scale_index(int64_t rows, int64_t r, int b) {
  return 4 * (rows * (b >> 2) + r) + (b & 3);
}

// Rows per workgroup chunk of the quantising gather, which keeps the chunk's scale words in
// LDS ([rows][d / 128 + 1] words) and writes each K-tile plane's words as one run.  Up to 32
// rows, within 32 KiB.
inline int mx_chunk_rows(int d) {
  const int per_row = 4 * ((d >> 7) + 1);
  int cr = 32;
  while (cr > 4 && cr * per_row > 32768) cr >>= 1;
  return cr;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Unbiased exponent of the block scale, from the fp32 bit pattern of the block's largest
// magnitude (> 0).  The exponent field is floor(log2 amax) + 127 for a normal amax; a
// subnormal amax has field 0 and lands on the lower clamp, as its true exponent would.
__device__ __forceinline__ int mx_block_exp(uint32_t amax_bits) {
  const int e = int(amax_bits >> 23) - 127 - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^-e as an fp32 (for finite amax, e <= 119, so 127 - e lies in [8, 254]: a normal float)
__device__ __forceinline__ float mx_inv_scale(int e) { return __uint_as_float(uint32_t(127 - e) << 23); }

__device__ __forceinline__ float mx_clamp(float y) { return fminf(fmaxf(y, -448.0f), 448.0f); }

// Four values times 2^-e, saturated and rounded to E4M3, packed little-endian.
// v_cvt_pk_fp8_f32 rounds to nearest even (checked against the rule on every bf16 value)
// but turns magnitudes from 464 up into NaN, hence the clamp to +-448 first.
__device__ __forceinline__ uint32_t mx_pack4(float a, float b, float c, float d, float inv) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(mx_clamp(a * inv), mx_clamp(b * inv), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(mx_clamp(c * inv), mx_clamp(d * inv), r, true);
  return uint32_t(r);
}

// Max over the 4 lanes of an aligned lane quad (the 4 lanes holding one 32-value block).
// Two DPP quad permutations (lanes 1,0,3,2 then 2,3,0,1), no LDS round trip.
__device__ __forceinline__ uint32_t quad_max(uint32_t m) {
  m = max(m, uint32_t(__builtin_amdgcn_update_dpp(int(m), int(m), 0xB1, 0xF, 0xF, false)));
  return max(m, uint32_t(__builtin_amdgcn_update_dpp(int(m), int(m), 0x4E, 0xF, 0xF, false)));
}

// The 4 block scales of one K-tile plane, held by lanes 16c, +4, +8, +12 of a 16-lane DPP
// row, as the little-endian 32-bit word the scale layout stores (valid in lanes 16c; row_shl
// 4, 8 and 12 read lane l + 4, 8, 12 of the same row).
__device__ __forceinline__ uint32_t mx_scale_word(uint32_t sc) {
  const uint32_t s1 = uint32_t(__builtin_amdgcn_update_dpp(0, int(sc), 0x104, 0xF, 0xF, false));
  const uint32_t s2 = uint32_t(__builtin_amdgcn_update_dpp(0, int(sc), 0x108, 0xF, 0xF, false));
  const uint32_t s3 = uint32_t(__builtin_amdgcn_update_dpp(0, int(sc), 0x10C, 0xF, 0xF, false));
  return (sc & 0xFFu) | ((s1 & 0xFFu) << 8) | ((s2 & 0xFFu) << 16) | ((s3 & 0xFFu) << 24);
}

// Quantise 8 consecutive bf16 values (one 16-byte vector) that form a quarter of a block
// held by an aligned lane quad.  Returns the 8 codes; *scale receives the block's scale
// code.  Every lane of the wave must call it (quad shuffles); lanes without data pass 0.
__device__ __forceinline__ uint2 mx_quant8_bf16(const u32x4 v, uint32_t* scale) {
  uint32_t m = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) m = max(m, max(v[w] & 0x7FFFu, (v[w] >> 16) & 0x7FFFu));
  m = quad_max(m << 16);
  if (m == 0) {
    *scale = 0;
    return make_uint2(0, 0);
  }
  const int e = mx_block_exp(m);
  const float inv = mx_inv_scale(e);
  *scale = uint32_t(e + 127);
  uint2 q;
  q.x = mx_pack4(__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u),
                 __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xFFFF0000u), inv);
  q.y = mx_pack4(__uint_as_float(v[2] << 16), __uint_as_float(v[2] & 0xFFFF0000u),
                 __uint_as_float(v[3] << 16), __uint_as_float(v[3] & 0xFFFF0000u), inv);
  return q;
}

// Same for 8 consecutive fp32 values.
__device__ __forceinline__ uint2 mx_quant8_f32(const f32x4 a, const f32x4 b, uint32_t* scale) {
  uint32_t m = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    m = max(m, max(__float_as_uint(a[w]) & 0x7FFFFFFFu, __float_as_uint(b[w]) & 0x7FFFFFFFu));
  m = quad_max(m);
  if (m == 0) {
    *scale = 0;
    return make_uint2(0, 0);
  }
  const int e = mx_block_exp(m);
  const float inv = mx_inv_scale(e);
  *scale = uint32_t(e + 127);
  return make_uint2(mx_pack4(a[0], a[1], a[2], a[3], inv), mx_pack4(b[0], b[1], b[2], b[3], inv));
}

}  // namespace moe
