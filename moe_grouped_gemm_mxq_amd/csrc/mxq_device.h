// Device-side helpers shared by the libmxq kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

constexpr int kBlock = 32;  // elements per MX block

typedef short v2i16 __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- lane exchange
// DPP quad permutations: lane i reads lane i^1 / i^2 of its quad; row half
// mirror: lane i of each 8-lane group reads lane 7-i (the other quad).
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_half_mirror(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);
}
// max over the 4 lanes of a quad (unsigned)
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  v = max(v, dpp_xor1(v));
  v = max(v, dpp_xor2(v));
  return v;
}

// ---------------------------------------------------------------- bf16 helpers
// max of the two bf16 magnitudes held in a dword, as an unsigned 16-bit value
__device__ __forceinline__ uint32_t absmax_bf16x2(uint32_t a, uint32_t b) {
  v2u16 x = __builtin_bit_cast(v2u16, a & 0x7FFF7FFFu);
  v2u16 y = __builtin_bit_cast(v2u16, b & 0x7FFF7FFFu);
  v2u16 m = __builtin_elementwise_max(x, y);
  return __builtin_bit_cast(uint32_t, m);
}
// per-half maximum of two packed unsigned 16-bit pairs (a plain 32-bit max would
// compare the high halves first and could drop a larger low half)
__device__ __forceinline__ uint32_t pkmax_u16(uint32_t a, uint32_t b) {
  v2u16 m = __builtin_elementwise_max(__builtin_bit_cast(v2u16, a), __builtin_bit_cast(v2u16, b));
  return __builtin_bit_cast(uint32_t, m);
}
__device__ __forceinline__ uint32_t hmax_u16x2(uint32_t v) { return max(v & 0xFFFFu, v >> 16); }

// ---------------------------------------------------------------- MXFP8 (E4M3)
// E8M0 scale byte of a block from its largest bf16 magnitude (sign cleared):
// shared = floor(log2 amax) - 8 clamped at -127, i.e. byte = max(Efield - 8, 0);
// zero and subnormal maxima give byte 0.
__device__ __forceinline__ uint32_t mxfp8_scale_byte(uint32_t amax16) {
  uint32_t e = amax16 >> 7;
  return e > 8u ? e - 8u : 0u;
}

// The scaled conversion divides by the power of two held in the exponent field of
// its fp32 scale operand (only that field is used), then rounds to nearest-even;
// it does not saturate, so magnitudes from 464*scale up come out as the NaN code.
// Four packed codes: turn S.1111.111 into S.1111.110 (448), the saturated value.
__device__ __forceinline__ uint32_t e4m3_saturate4(uint32_t c) {
  uint32_t m = ((c & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
  return c - (m >> 7);
}

// Four bf16 values (two dwords, element order lo..hi) -> four E4M3 codes.
__device__ __forceinline__ uint32_t e4m3_encode4(uint32_t lo, uint32_t hi, float scale) {
  v2i16 r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf16, lo), scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf16, hi), scale, true);
  return e4m3_saturate4(__builtin_bit_cast(uint32_t, r));
}

__device__ __forceinline__ float e8m0_as_scale(uint32_t byte) { return __uint_as_float(byte << 23); }

// Byte offset of the scale of row r, block b in a GEMM operand's scale array
// (nblk blocks per row): 128-row groups, then blocks, then r % 32, then
// (r / 32) % 4.  The four bytes of a dword are the scales of rows r, r+32,
// r+64, r+96 of one group for one block -- the four MFMA row blocks a GEMM
// lane multiplies -- so a GEMM stage fetches a 128-row group's scales for
// two K-blocks with one 64-lane dword load (256 consecutive bytes).  Array
// size ceil128(rows) * nblk bytes; bytes of rows past the last are padding.
__device__ __forceinline__ int64_t scale_offset(int64_t r, int64_t b, int64_t nblk) {
  return (((r >> 7) * nblk + b) * 32 + (r & 31)) * 4 + ((r >> 5) & 3);
}

// ---------------------------------------------------------------- MXFP4 (E2M1)
// Exact round(log2(amax/6)) clamped at -30 from the fp32 bits of amax: with
// amax = m * 2^E (m in [1,2)), log2(amax/6) rounds up to E-2 iff m >= 3/(2*sqrt 2),
// i.e. iff the mantissa field is >= 0x7C3B7, else to E-3.  Subnormal or zero
// maxima lie far below 6*2^-30.5, so they take the clamp.
// Exponent rule of an MXFP4 block for an fp32 scale factor sf:
// round(log2(amax / sf)), taken exactly.  Write sf * sqrt(2) = (1 + t) * 2^F
// and amax = (1 + a) * 2^E; then round(log2(amax / sf)) =
// floor(log2(amax / (sf sqrt 2))) + 1 = E - F + [a >= t].  t is irrational,
// so with T = ceil(t * 2^23) the test is an integer compare of amax's
// mantissa field (T = 2^23 never matches).  sf = 6 gives F = 3, T = 0x7C3B7.
struct Fp4Scale {
  int F;
  uint32_t T;
};

// raw scale clamped at 2^-30: e >= -30; subnormal amax (and 0) lands on the
// clamp for every sf >= 2^-64 (amax / sf < 2^-62).
__device__ __forceinline__ int mxfp4_scale_exp(uint32_t amax_bits, Fp4Scale p) {
  int ef = (int)(amax_bits >> 23);
  if (ef == 0) return -30;
  int e = ef - 127 - p.F + ((amax_bits & 0x7FFFFFu) >= p.T ? 1 : 0);
  return e < -30 ? -30 : e;
}

// codebook index (0..7 for 0,0.5,1,1.5,2,3,4,6) of |x| / 2^e: the number of
// midpoints (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) that yabs = |x| * 2^-e
// (exact) reaches, so ties go up.  Every midpoint starts a quarter of its
// binade, so the index depends only on the exponent and the top two mantissa
// bits: bits >> 21, clamped to the 21 values from [0.21875, 0.25) (index 0,
// like everything below) to [7, 8) (index 7, like everything above), picks a
// 3-bit entry of kFp4IndexTable.  Checked against the midpoint count for every
// finite non-negative fp32 value.
constexpr uint64_t kFp4IndexTable = 0x7ff6b646d2449248ull;  // entries 0,1,1,1,1,1,1,2,2,2,3,3,4,4,5,5,6,6,7,7,7
__device__ __forceinline__ uint32_t mxfp4_index(float yabs) {
  const uint32_t k = min(max(__float_as_uint(yabs) >> 21, 499u), 519u) - 499u;
  return (uint32_t)(kFp4IndexTable >> (3 * k)) & 7u;
}

// fp32 bits of codebook[idx] * 2^e with the sign bit `sign` (0 or 0x80000000).
// codebook[idx] for idx >= 2 has exponent field 126 + idx/2 and top mantissa bit
// idx&1, so its bits are (126 << 23) + (idx << 22); 0.5 is 126 << 23.  Adding
// e << 23 multiplies by 2^e exactly (results stay normal: e >= -30, value >= 0.5).
__device__ __forceinline__ uint32_t mxfp4_value_bits(uint32_t idx, int e, uint32_t sign) {
  uint32_t b = idx >= 2u ? (126u << 23) + (idx << 22) : (idx ? (126u << 23) : 0u);
  if (idx) b += (uint32_t)e << 23;
  return b | sign;
}

}  // namespace mxq
