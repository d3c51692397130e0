// MXFP4 quantise-dequantise for gfx950 (AMCT FakeQuant article, section 2
// "MXFP4 数值模型" and section 3.3): blocks of 32 along the last dim, each row
// padded on its own; scale 2^round(log2(max|x|/6)) with the raw scale clamped
// at 2^-30 (round taken exactly); element -> nearest E2M1 codebook value with
// ties to the larger magnitude (the page's midpoint cascade); output
// sign(x) * code * scale.  One fused pass: read fp32 once, write fp32 once
// (plus optional packed nibbles and scale bytes).
#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

namespace {

constexpr int kThreads = 256;

// Four elements of one lane -> output bits, nibbles (packed into 16 bits).
struct Qdq4 {
  uint32_t out[4];
  uint32_t nibbles;
};

__device__ __forceinline__ Qdq4 qdq4(const uint32_t (&xb)[4], int e) {
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, e in [-30, 125]
  Qdq4 r;
  r.nibbles = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint32_t sign = xb[j] & 0x80000000u;
    const float yabs = __uint_as_float(xb[j] & 0x7FFFFFFFu) * inv;  // exact
    const uint32_t idx = mxfp4_index(yabs);
    r.out[j] = mxfp4_value_bits(idx, e, sign);
    r.nibbles |= ((sign >> 28) | idx) << (4 * j);
  }
  return r;
}

__device__ __forceinline__ uint32_t absmax4(const uint32_t (&xb)[4]) {
  return max(max(xb[0] & 0x7FFFFFFFu, xb[1] & 0x7FFFFFFFu), max(xb[2] & 0x7FFFFFFFu, xb[3] & 0x7FFFFFFFu));
}

// eight lanes (aligned) hold one block: reduce their maxima
__device__ __forceinline__ uint32_t oct_max(uint32_t v) {
  v = quad_max_u32(v);
  return max(v, dpp_half_mirror(v));
}

// L % 32 == 0 and 16-byte aligned x / y: the tensor is a flat run of blocks.
__global__ __launch_bounds__(kThreads) void qdq_flat_kernel(const float* __restrict__ x,
                                                           float* __restrict__ y, int64_t n_chunks,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_chunks;
       i += (int64_t)gridDim.x * kThreads) {
    const uint4 v = reinterpret_cast<const uint4*>(x)[i];
    const uint32_t xb[4] = {v.x, v.y, v.z, v.w};
    const uint32_t amax = oct_max(absmax4(xb));
    const int e = mxfp4_scale_exp(amax);
    const Qdq4 r = qdq4(xb, e);
    reinterpret_cast<uint4*>(y)[i] = make_uint4(r.out[0], r.out[1], r.out[2], r.out[3]);
    if (codes) reinterpret_cast<uint16_t*>(codes)[i] = (uint16_t)r.nibbles;
    if (scales && (i & 7) == 0) scales[i >> 3] = (uint8_t)(e + 127);
  }
}

// General L: eight lanes per (row, block), four guarded scalar elements each.
__global__ __launch_bounds__(kThreads) void qdq_rows_kernel(const float* __restrict__ x,
                                                           float* __restrict__ y, int64_t rows,
                                                           int64_t L, uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  const int64_t nbr = (L + 31) / 32;  // blocks per row
  const int64_t n_chunks = rows * nbr * 8;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_chunks;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t blk = i >> 3;
    const int64_t row = blk / nbr;
    const int64_t col = (blk - row * nbr) * 32 + (i & 7) * 4;
    uint32_t xb[4];
#pragma unroll
    for (int j = 0; j < 4; j++) xb[j] = col + j < L ? __float_as_uint(x[row * L + col + j]) : 0u;
    const uint32_t amax = oct_max(absmax4(xb));
    const int e = mxfp4_scale_exp(amax);
    const Qdq4 r = qdq4(xb, e);
#pragma unroll
    for (int j = 0; j < 4; j++)
      if (col + j < L) y[row * L + col + j] = __uint_as_float(r.out[j]);
    if (codes) *reinterpret_cast<uint16_t*>(codes + row * (nbr * 16) + col / 2) = (uint16_t)r.nibbles;
    if (scales && (i & 7) == 0) scales[blk] = (uint8_t)(e + 127);
  }
}

}  // namespace

hipError_t launch_qdq_fp4(const float* x, float* y, int64_t rows, int64_t L, uint8_t* codes,
                          uint8_t* scales, hipStream_t st) {
  // One chunk per thread and one workgroup per 256 chunks (4 KB of fp32),
  // capped only by the grid-size limit: measured on MI355X, many short
  // workgroups over contiguous chunks stream HBM faster (a plain copy:
  // 6.1 TB/s) than a grid-stride loop over a CU-sized grid (5.1-5.4 TB/s).
  const int cap = 0x7FFFFFFF / kThreads;
  const bool flat = L % 32 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)y % 16 == 0;
  const int64_t n_chunks = flat ? rows * L / 4 : rows * ((L + 31) / 32) * 8;
  const int64_t want = (n_chunks + kThreads - 1) / kThreads;
  const int grid = (int)(want < cap ? want : cap);
  if (flat)
    qdq_flat_kernel<<<grid, kThreads, 0, st>>>(x, y, n_chunks, codes, scales);
  else
    qdq_rows_kernel<<<grid, kThreads, 0, st>>>(x, y, rows, L, codes, scales);
  return hipGetLastError();
}

}  // namespace mxq
