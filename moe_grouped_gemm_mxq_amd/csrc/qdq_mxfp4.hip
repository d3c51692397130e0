// MXFP4 quantise-dequantise for gfx950 (AMCT FakeQuant article, section 2
// "MXFP4 数值模型" and section 3.3): blocks of 32 along the last dim, each row
// padded on its own; scale 2^round(log2(max|x| / scale_factor)) with the raw
// scale clamped at 2^-30 (round taken exactly; scale_factor 6 by default);
// element -> nearest E2M1 codebook value with ties to the larger magnitude
// (the page's midpoint cascade); output sign(x) * code * scale.  One fused
// pass: read fp32 once, write fp32 once, plus optional packed nibbles, scale
// bytes and the clipped-STE saturation mask (section 4.1): one bit per
// element, set where |x| > 6 * scale, i.e. where the quantiser clipped.
// The STE backward reads that mask and passes the gradient where it is clear.
#include <string.h>

#include "mxq_device.h"
#include "mxq_groups.h"
#include "mxq_internal.h"

namespace mxq {

namespace {

constexpr int kThreads = 256;

// Four elements of one lane -> output bits, nibbles (packed into 16 bits) and
// saturation bits (low 4 bits).
struct Qdq4 {
  uint32_t out[4];
  uint32_t nibbles;
  uint32_t sat;
};

__device__ __forceinline__ Qdq4 qdq4(const uint32_t (&xb)[4], int e) {
  Qdq4 r;
  r.nibbles = 0;
  r.sat = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint32_t sign = xb[j] & 0x80000000u;
    // |x| * 2^-e: exact wherever the result is normal; a subnormal result is
    // below 2^-126 and maps to code 0 however it rounds.
    const float yabs = __builtin_amdgcn_ldexpf(__uint_as_float(xb[j] & 0x7FFFFFFFu), -e);
    const uint32_t idx = mxfp4_index(yabs);
    r.out[j] = mxfp4_value_bits(idx, e, sign);
    r.nibbles |= ((sign >> 28) | idx) << (4 * j);
    r.sat |= (uint32_t)(yabs > 6.0f) << j;
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

// OR over the eight lanes of a block (each lane contributes disjoint bits)
__device__ __forceinline__ uint32_t oct_or(uint32_t v) {
  v |= dpp_xor1(v);
  v |= dpp_xor2(v);
  return v | dpp_half_mirror(v);
}

// L % 32 == 0 and 16-byte aligned x / y: the tensor is a flat run of blocks,
// chunk i = elements 4i..4i+3, block i / 8.
// y null: quantise only.  nbr > 0: scales in the GEMM operand layout
// (scale_offset) for rows of nbr blocks; 0: row-major.
__global__ __launch_bounds__(kThreads) void qdq_flat_kernel(const float* __restrict__ x,
                                                           float* __restrict__ y, int64_t n_chunks,
                                                           Fp4Scale p, uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales,
                                                           uint32_t* __restrict__ sat_mask, int64_t nbr) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_chunks;
       i += (int64_t)gridDim.x * kThreads) {
    const uint4 v = reinterpret_cast<const uint4*>(x)[i];
    const uint32_t xb[4] = {v.x, v.y, v.z, v.w};
    const uint32_t amax = oct_max(absmax4(xb));
    const int e = mxfp4_scale_exp(amax, p);
    const Qdq4 r = qdq4(xb, e);
    if (y) reinterpret_cast<uint4*>(y)[i] = make_uint4(r.out[0], r.out[1], r.out[2], r.out[3]);
    if (codes) reinterpret_cast<uint16_t*>(codes)[i] = (uint16_t)r.nibbles;
    if (scales && (i & 7) == 0) {
      const int64_t blk = i >> 3;
      const int64_t row = nbr > 0 ? blk / nbr : 0;
      scales[nbr > 0 ? scale_offset(row, blk - row * nbr, nbr) : blk] = (uint8_t)(e + 127);
    }
    if (sat_mask) {
      const uint32_t word = oct_or(r.sat << (4 * (i & 7)));
      if ((i & 7) == 0) sat_mask[i >> 3] = word;
    }
  }
}

// General L: eight lanes per (row, block), four guarded scalar elements each.
__global__ __launch_bounds__(kThreads) void qdq_rows_kernel(const float* __restrict__ x,
                                                           float* __restrict__ y, int64_t rows,
                                                           int64_t L, Fp4Scale p,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales,
                                                           uint32_t* __restrict__ sat_mask, bool operand_layout) {
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
    const int e = mxfp4_scale_exp(amax, p);
    const Qdq4 r = qdq4(xb, e);
    if (y) {
#pragma unroll
      for (int j = 0; j < 4; j++)
        if (col + j < L) y[row * L + col + j] = __uint_as_float(r.out[j]);
    }
    if (codes) *reinterpret_cast<uint16_t*>(codes + row * (nbr * 16) + col / 2) = (uint16_t)r.nibbles;
    if (scales && (i & 7) == 0)
      scales[operand_layout ? scale_offset(row, blk - row * nbr, nbr) : blk] = (uint8_t)(e + 127);
    if (sat_mask) {
      // padding elements are 0 and never saturate, so their bits stay clear
      const uint32_t word = oct_or(r.sat << (4 * (i & 7)));
      if ((i & 7) == 0) sat_mask[blk] = word;  // row stride Lp/8 bytes = nbr words
    }
  }
}

// GEMM operand copy (codes and packed scales, no dequantised output) of rows
// whose length is a multiple of 1024: a unit is 1024 elements (32 blocks) of
// one row, 256 lanes of four elements, so the row and its first block are
// uniform per unit and a lane's scale offset needs no division.  A workgroup
// takes kOpUnits consecutive units and issues all their loads before any
// arithmetic.  (Dealing each 128-row group's workgroups to one XCD, so that
// its L2 completes the group's scale lines, measured 3.5% slower here: the
// scale bytes are 1/128 of the input.)
constexpr int kOpUnits = 2;

__global__ __launch_bounds__(kThreads) void quant_fp4_rows_kernel(const float* __restrict__ x, int64_t rows,
                                                                 int64_t L, Fp4Scale p,
                                                                 uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales) {
  const int64_t upr = L / 1024;      // units per row
  const int64_t nbr = L / 32;        // blocks per row
  const int64_t n_units = rows * upr;
  const int64_t w = blockIdx.x;
  const int t = threadIdx.x;
  uint4 v[kOpUnits];
#pragma unroll
  for (int k = 0; k < kOpUnits; k++) {
    const int64_t u = w * kOpUnits + k;
    // units are whole rows' 1024-element pieces, so unit u starts at element 1024 u
    if (u < n_units) v[k] = reinterpret_cast<const uint4*>(x)[u * 256 + t];
  }
  // row and piece of the first unit (uniform); the next unit is the next piece
  int64_t row = w * kOpUnits / upr;
  int64_t seg = w * kOpUnits - row * upr;
#pragma unroll
  for (int k = 0; k < kOpUnits; k++) {
    const int64_t u = w * kOpUnits + k;
    if (u < n_units) {
      const uint32_t xb[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
      const int e = mxfp4_scale_exp(oct_max(absmax4(xb)), p);
      uint32_t nib = 0;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const uint32_t sign = xb[j] & 0x80000000u;
        const float yabs = __builtin_amdgcn_ldexpf(__uint_as_float(xb[j] & 0x7FFFFFFFu), -e);
        nib |= ((sign >> 28) | mxfp4_index(yabs)) << (4 * j);
      }
      reinterpret_cast<uint16_t*>(codes)[u * 256 + t] = (uint16_t)nib;
      if ((t & 7) == 0) scales[scale_offset(row, seg * 32 + (t >> 3), nbr)] = (uint8_t)(e + 127);
    }
    if (++seg == upr) {
      seg = 0;
      row++;
    }
  }
}

// Clipped STE backward, flat layout: grad_x = bit ? 0 : grad_y.
// grad_x may alias grad_y (each element is read, then written, by one lane).
__global__ __launch_bounds__(kThreads) void ste_flat_kernel(const float* gy, const uint32_t* __restrict__ sat_mask,
                                                           float* gx, int64_t n_chunks) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_chunks;
       i += (int64_t)gridDim.x * kThreads) {
    const uint4 g = reinterpret_cast<const uint4*>(gy)[i];
    const uint32_t m = sat_mask[i >> 3] >> (4 * (i & 7));
    reinterpret_cast<uint4*>(gx)[i] = make_uint4(m & 1u ? 0u : g.x, m & 2u ? 0u : g.y,
                                                 m & 4u ? 0u : g.z, m & 8u ? 0u : g.w);
  }
}

__global__ __launch_bounds__(kThreads) void ste_rows_kernel(const float* gy, const uint32_t* __restrict__ sat_mask,
                                                           float* gx, int64_t rows, int64_t L) {
  const int64_t nbr = (L + 31) / 32;
  const int64_t n_chunks = rows * nbr * 8;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_chunks;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t blk = i >> 3;
    const int64_t row = blk / nbr;
    const int64_t col = (blk - row * nbr) * 32 + (i & 7) * 4;
    const uint32_t m = sat_mask[blk] >> (4 * (i & 7));
#pragma unroll
    for (int j = 0; j < 4; j++)
      if (col + j < L) {
        const int64_t o = row * L + col + j;
        const float g = gy[o];
        gx[o] = (m >> j) & 1u ? 0.0f : g;
      }
  }
}

// ------------------------------------------------------------------ grouped token axis
// MXFP4 GEMM operands of the expert weight gradient: blocks of 32 run down
// the token axis of x [T][C] within each group (the same block rule and
// element rounding as the QDQ above), group g's tokens at padded positions
// [P_g, P_g + ceil32(m_g)) of output row c = column c of x.  A workgroup
// takes 256 padded positions (8 blocks) x 32 columns: it loads the 256 fp32
// rows' 128-byte pieces into LDS, then each thread quantises one column over
// one block (32 values down the column) and stores its 16 code bytes; the
// eight blocks of a column make one 128-byte code line.  Tile rows are
// stored with one spare row per 32 (row r at r + r/32), so the two blocks a
// wave reads at once sit in opposite halves of the LDS banks.
constexpr int kTokTile = 256, kColTile = 32;
constexpr int kTokRows = kTokTile + kTokTile / 32;
constexpr int kGrpColTiles = 4;  // column tiles per workgroup

// the eight 16-byte pieces of one thread: rows (t / 8) + 32 i, columns col4 ..
template <bool VEC>
__device__ __forceinline__ void load_fp4_tile_pieces(const float* const (&xr)[8], uint32_t row_ok, int64_t col4,
                                                     int64_t C, float4 (&w)[8]) {
#pragma unroll
  for (int i = 0; i < 8; i++) {
    w[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row_ok >> i & 1u) {
      if (VEC && col4 + 4 <= C) {
        w[i] = *reinterpret_cast<const float4*>(xr[i] + col4);
      } else {
        if (col4 < C) w[i].x = xr[i][col4];
        if (col4 + 1 < C) w[i].y = xr[i][col4 + 1];
        if (col4 + 2 < C) w[i].z = xr[i][col4 + 2];
        if (col4 + 3 < C) w[i].w = xr[i][col4 + 3];
      }
    }
  }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void quant_fp4_grouped_kernel(
    const float* __restrict__ x, int64_t T, int64_t C, int64_t ldx, const int32_t* __restrict__ group_end,
    int32_t G, int64_t ldq, int n_col_tiles, int n_col_groups, Fp4Scale p, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales) {
  __shared__ __attribute__((aligned(16))) float tile[kTokRows * kColTile];
  __shared__ int32_t bstart[kMaxGroups + 1];
  __shared__ int64_t rb_src[kTokTile / 32];   // first source row of each block of the tile
  __shared__ int32_t rb_valid[kTokTile / 32]; // its valid rows (0: no output block)
  static_assert(kThreads * sizeof(int64_t) <= sizeof(tile), "the group scan's scratch reuses the tile");
  const int t = threadIdx.x;
  const int rt = blockIdx.x / n_col_groups;
  const int ct_begin = (blockIdx.x - rt * n_col_groups) * kGrpColTiles;
  const int ct_end = min(ct_begin + kGrpColTiles, n_col_tiles);
  const int64_t p0 = (int64_t)rt * kTokTile;  // first padded position of the tile
  build_block_starts<kThreads>(group_end, G, T, 32, nullptr, nullptr, bstart, reinterpret_cast<int64_t*>(tile));
  if (t < kTokTile / 32) {
    const int64_t pb = p0 / 32 + t;
    int64_t src = 0;
    int32_t valid = 0;
    if (pb < bstart[G] && (pb + 1) * 32 <= ldq) {
      const int g = find_block_group(bstart, G, (int32_t)pb);
      int32_t gstart, gsize;
      group_span(group_end, g, T, gstart, gsize);
      // (bstart is non-decreasing and bstart[g] <= pb < bstart[g] + ceil32(gsize) / 32)
      const int64_t off = (pb - bstart[g]) * 32;
      src = (int64_t)gstart + off;
      valid = (int32_t)min<int64_t>(32, gsize - off);
    }
    rb_src[t] = src;
    rb_valid[t] = valid;
  }
  __syncthreads();
  if (rb_valid[0] <= 0) return;  // the tile lies past the last block (uniform)

  // source rows of this thread's eight pieces, the same for every column tile
  const int cq = t & 7;
  const float* xr[8];
  uint32_t row_ok = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int lr = (t >> 3) + 32 * i;
    const int rb = lr >> 5;
    const bool ok = (lr & 31) < rb_valid[rb];
    row_ok |= (uint32_t)ok << i;
    xr[i] = x + (ok ? rb_src[rb] + (lr & 31) : 0) * ldx;
  }
  const int blk = t >> 5, col = t & 31;
  const bool blk_ok = rb_valid[blk] > 0;
  const int64_t pos = p0 + 32 * blk;  // padded position of this thread's block

  // The workgroup walks its column tiles with the next tile's loads in flight
  // while the current one is quantised from LDS.
  float4 w[8];
  load_fp4_tile_pieces<VEC>(xr, row_ok, (int64_t)ct_begin * kColTile + 4 * cq, C, w);
  for (int ct = ct_begin; ct < ct_end; ct++) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int lr = (t >> 3) + 32 * i;
      *reinterpret_cast<float4*>(tile + (lr + (lr >> 5)) * kColTile + 4 * cq) = w[i];
    }
    __syncthreads();
    if (ct + 1 < ct_end) load_fp4_tile_pieces<VEC>(xr, row_ok, (int64_t)(ct + 1) * kColTile + 4 * cq, C, w);

    // ---- one column over one block per thread
    uint32_t v[32];
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 32; i++) {
      const int lr = blk * 32 + i;
      v[i] = __float_as_uint(tile[(lr + blk) * kColTile + col]);
      amax = max(amax, v[i] & 0x7FFFFFFFu);
    }
    const int e = mxfp4_scale_exp(amax, p);
    uint32_t nib[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; i++) {
      const uint32_t sign = v[i] & 0x80000000u;
      const float yabs = __builtin_amdgcn_ldexpf(__uint_as_float(v[i] & 0x7FFFFFFFu), -e);
      nib[i >> 3] |= ((sign >> 28) | mxfp4_index(yabs)) << (4 * (i & 7));
    }
    const int64_t cg = (int64_t)ct * kColTile + col;
    if (blk_ok && cg < C) {
      *reinterpret_cast<uint4*>(codes + cg * (ldq / 2) + pos / 2) = make_uint4(nib[0], nib[1], nib[2], nib[3]);
      scales[scale_offset(cg, pos / 32, ldq / 32)] = (uint8_t)(e + 127);
    }
    __syncthreads();  // every wave has read the tile before the next one is written
  }
}

// One chunk per thread and one workgroup per 256 chunks (4 KB of fp32),
// capped only by the grid-size limit: measured on MI355X, many short
// workgroups over contiguous chunks stream HBM faster (a plain copy:
// 6.1 TB/s) than a grid-stride loop over a CU-sized grid (5.1-5.4 TB/s).
int grid_for(int64_t n_chunks) {
  const int cap = 0x7FFFFFFF / kThreads;
  const int64_t want = (n_chunks + kThreads - 1) / kThreads;
  return (int)(want < cap ? want : cap);
}

}  // namespace

bool fp4_scale_params(float scale_factor, int* F, uint32_t* T) {
  uint32_t b;
  memcpy(&b, &scale_factor, 4);
  const int ef = (int)(b >> 23);  // sign bit included: negatives fail the range test
  if (ef < 127 - 64 || ef > 127 + 63) return false;  // sf in [2^-64, 2^64), normal, positive
  const uint64_t ms = (1u << 23) | (b & 0x7FFFFFu);    // sf = ms * 2^(ef - 150)
  // (1 + f) * sqrt(2) >= 2 exactly when ms^2 >= 2^47: then F is one above sf's exponent
  const int d = ms * ms >= (1ull << 47) ? 1 : 0;
  *F = ef - 127 + d;
  // smallest M = 2^23 + T with M / 2^23 >= (1 + t) = ms * sqrt(2) / 2^(23 + d):
  // M^2 >= 2 ms^2 (d = 0) or 2 M^2 >= ms^2 (d = 1), compared in integers
  auto ok = [&](uint64_t M) { return d ? 2 * M * M >= ms * ms : M * M >= 2 * ms * ms; };
  uint64_t M = (uint64_t)(d ? (double)ms * 0.70710678118654752 : (double)ms * 1.4142135623730951);
  while (M < (1ull << 23)) M++;
  while (!ok(M)) M++;
  while (M > (1ull << 23) && ok(M - 1)) M--;
  *T = (uint32_t)(M - (1ull << 23));
  return true;
}

hipError_t launch_qdq_fp4(const float* x, float* y, int64_t rows, int64_t L, int F, uint32_t T,
                          uint8_t* codes, uint8_t* scales, uint8_t* sat_mask, hipStream_t st, bool operand_layout) {
  const Fp4Scale p{F, T};
  if (operand_layout && !y && !sat_mask && L % 1024 == 0 && (uintptr_t)x % 16 == 0) {
    const int64_t n_wg = (rows * (L / 1024) + kOpUnits - 1) / kOpUnits;
    if (n_wg <= 0x7FFFFFFF) {
      quant_fp4_rows_kernel<<<(unsigned)n_wg, kThreads, 0, st>>>(x, rows, L, p, codes, scales);
      return hipGetLastError();
    }
  }
  const bool flat = L % 32 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)y % 16 == 0;
  const int64_t n_chunks = flat ? rows * L / 4 : rows * ((L + 31) / 32) * 8;
  uint32_t* mask = reinterpret_cast<uint32_t*>(sat_mask);
  if (flat)
    qdq_flat_kernel<<<grid_for(n_chunks), kThreads, 0, st>>>(x, y, n_chunks, p, codes, scales, mask,
                                                             operand_layout ? L / 32 : 0);
  else
    qdq_rows_kernel<<<grid_for(n_chunks), kThreads, 0, st>>>(x, y, rows, L, p, codes, scales, mask, operand_layout);
  return hipGetLastError();
}

hipError_t launch_quant_fp4_grouped(const float* x, int64_t T, int64_t C, int64_t ldx, const int32_t* group_end,
                                    int32_t G, int64_t ldq, int F, uint32_t Tth, uint8_t* codes, uint8_t* scales,
                                    hipStream_t st) {
  const Fp4Scale p{F, Tth};
  const int64_t n_row_tiles = (T + 31 * (int64_t)G + kTokTile - 1) / kTokTile;
  const int n_col_tiles = (int)((C + kColTile - 1) / kColTile);
  const int n_col_groups = (n_col_tiles + kGrpColTiles - 1) / kGrpColTiles;
  const int64_t grid = n_row_tiles * n_col_groups;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const bool vec = ldx % 4 == 0 && (uintptr_t)x % 16 == 0;
  if (vec)
    quant_fp4_grouped_kernel<true><<<(unsigned)grid, kThreads, 0, st>>>(x, T, C, ldx, group_end, G, ldq, n_col_tiles,
                                                                         n_col_groups, p, codes, scales);
  else
    quant_fp4_grouped_kernel<false><<<(unsigned)grid, kThreads, 0, st>>>(x, T, C, ldx, group_end, G, ldq,
                                                                          n_col_tiles, n_col_groups, p, codes, scales);
  return hipGetLastError();
}

hipError_t launch_ste_backward_fp4(const float* grad_y, const uint8_t* sat_mask, float* grad_x,
                                   int64_t rows, int64_t L, hipStream_t st) {
  const bool flat = L % 32 == 0 && (uintptr_t)grad_y % 16 == 0 && (uintptr_t)grad_x % 16 == 0;
  const int64_t n_chunks = flat ? rows * L / 4 : rows * ((L + 31) / 32) * 8;
  const uint32_t* mask = reinterpret_cast<const uint32_t*>(sat_mask);
  if (flat)
    ste_flat_kernel<<<grid_for(n_chunks), kThreads, 0, st>>>(grad_y, mask, grad_x, n_chunks);
  else
    ste_rows_kernel<<<grid_for(n_chunks), kThreads, 0, st>>>(grad_y, mask, grad_x, rows, L);
  return hipGetLastError();
}

}  // namespace mxq
