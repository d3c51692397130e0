// MXFP8 quantisers for gfx950: row copy, column copy (quantised transpose),
// dual-axis (both from one read) and grouped token-axis column copy.
//
// Per block of 32 values along the quantised axis (torchtitan-npu guide,
// "线性层低精度" / "MoE 专家层低精度"): scale byte = max(exponent field of the
// largest bf16 magnitude - 8, 0) (OCP MX shared exponent floor(log2 amax) - 8),
// element = E4M3 round-to-nearest-even of v / 2^(byte-127), saturated at 448.
// The element conversion is the hardware scaled conversion plus a saturation
// fix-up (see mxq_device.h); it was checked exhaustively over every bf16 value
// and every scale byte against the CPU oracle.  Scales are written in the
// GEMM operand layout of scale_offset().
#include "mxq_device.h"
#include "mxq_groups.h"
#include "mxq_internal.h"

namespace mxq {

namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------------ row copy
// A row is Cp/8 chunks of 8 bf16 (16 bytes); four consecutive lanes hold one
// block.  `tpr` (threads per row, a power of two in [8, 256]) lanes share a
// row.  A lane takes up to kRowUnroll chunks of its row at once and issues all
// their loads before any arithmetic, so enough bytes are in flight to cover
// the HBM latency.
//
// The scale bytes of one block of rows r, r+32, r+64, r+96 of a 128-row group
// share a dword, and the dwords of consecutive r%32 are adjacent, so a byte
// store per row and block touches one cache line each, which costs as much as
// the row's loads.  A workgroup therefore takes four 256-thread sub-groups,
// sub-group j on rows 32j + q .. 32j + q + rps - 1 of a group (rps = 256/tpr),
// gathers their scale bytes in LDS and writes them as dwords: one line per
// block for 4 * rps rows.  The workgroups of one 128-row group run on
// one XCD (see the unit mapping in the kernel).
constexpr int kRowUnroll = 4;
constexpr int kRowSub = 256, kRowThreads = 4 * kRowSub;

// one 16-byte load, non-temporal (streamed past the caches' retention) or ordinary
__device__ __forceinline__ uint4 load16(const uint16_t* p, bool nt) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  if (nt) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  }
  return *reinterpret_cast<const uint4*>(p);
}

template <bool VEC>
__device__ __forceinline__ void load_chunk(const uint16_t* xr, int64_t col, int64_t C, uint32_t (&w)[4]) {
  if (VEC && col + 8 <= C) {
    const uint4 v = *reinterpret_cast<const uint4*>(xr + col);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint32_t lo = col + 2 * j < C ? xr[col + 2 * j] : 0u;
      const uint32_t hi = col + 2 * j + 1 < C ? xr[col + 2 * j + 1] : 0u;
      w[j] = lo | (hi << 16);
    }
  }
}

template <bool VEC>
__global__ __launch_bounds__(kRowThreads) void quant_row_kernel(const uint16_t* __restrict__ x, int64_t R,
                                                               int64_t C, int64_t ldx, int tpr_log2,
                                                               uint8_t* __restrict__ q,
                                                               uint8_t* __restrict__ s, BatchStrides bs) {
  // matrix blockIdx.y of a batch
  x += blockIdx.y * bs.x;
  q += blockIdx.y * bs.q_row;
  s += blockIdx.y * bs.s_row;
  // scale dwords of one column step, double-buffered across steps
  __shared__ uint32_t sc_lds[2][kRowSub];
  const int64_t Cp = (C + 31) / 32 * 32;
  const int64_t nblk = Cp / 32;
  const int cpr = (int)(Cp / 8);  // chunks per row (a multiple of 4)
  const int tpr = 1 << tpr_log2;
  const int rps_log2 = 8 - tpr_log2;  // rows per sub-group, <= 32
  const int t = threadIdx.x;
  const int j = t >> 8;                       // sub-group: 32-row block of the group
  const int i = (t & (kRowSub - 1)) >> tpr_log2;  // row within the sub-group's run
  const int lc = t & (tpr - 1);               // lane within the row
  const int per_group = 32 >> rps_log2;       // workgroups per 128-row group
  const int64_t n_units = (R + 127) / 128 * per_group;
  const int n_steps = (cpr + kRowUnroll * tpr - 1) / (kRowUnroll * tpr);  // uniform
  int parity = 0;
  // A 128-row group's scale lines are completed by its per_group workgroups
  // (each writes its rows' dwords).  Workgroups are dealt to the 8 XCDs round
  // robin, so within each run of 8 groups workgroup b takes a unit that puts
  // all of a group's workgroups on one XCD, whose L2 merges their pieces of
  // each line before it is written back (spread over the XCDs, the pieces
  // went out as partial lines: 1.075 of the algorithmic bytes written for
  // 131072 x 7168).
  const int64_t span = 8 * (int64_t)per_group;
  const int64_t full = n_units / span * span;
  for (int64_t b = blockIdx.x; b < n_units; b += gridDim.x) {
    int64_t unit = b;
    if (b < full) {
      const int64_t r = b % span;
      unit = b - r + (r & 7) * per_group + (r >> 3);
    }
    const int64_t g = unit / per_group;
    const int qb = (int)(unit - g * per_group) << rps_log2;
    const int64_t row = g * 128 + 32 * j + qb + i;
    const bool row_ok = row < R;  // uniform per quad
    const uint16_t* xr = x + (row_ok ? row : 0) * ldx;
    for (int step = 0; step < n_steps; step++, parity ^= 1) {
      uint8_t* lds_bytes = reinterpret_cast<uint8_t*>(sc_lds[parity]);
      const int c0 = step * kRowUnroll * tpr + lc;
      uint32_t w[kRowUnroll][4];
      if (VEC && C % 8 == 0) {
        // unconditional 16-byte loads from clamped columns (chunks past C are
        // zeroed), so the loads issue back to back with no wait between them
#pragma unroll
        for (int u = 0; u < kRowUnroll; u++) {
          const int64_t col = (int64_t)(c0 + u * tpr) * 8;
          const uint4 v = *reinterpret_cast<const uint4*>(xr + min(col, C - 8));
          const bool ok = col < C;
          w[u][0] = ok ? v.x : 0u;
          w[u][1] = ok ? v.y : 0u;
          w[u][2] = ok ? v.z : 0u;
          w[u][3] = ok ? v.w : 0u;
        }
      } else {
#pragma unroll
        for (int u = 0; u < kRowUnroll; u++) {
          const int c8 = c0 + u * tpr;
          if (c8 < cpr) load_chunk<VEC>(xr, (int64_t)c8 * 8, C, w[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < kRowUnroll; u++) {
        const int c8 = c0 + u * tpr;
        if (c8 >= cpr) break;  // (uniform per quad: cpr and tpr are multiples of 4)
        const int64_t col = (int64_t)c8 * 8;
        uint32_t m = hmax_u16x2(pkmax_u16(absmax_bf16x2(w[u][0], w[u][1]), absmax_bf16x2(w[u][2], w[u][3])));
        m = quad_max_u32(m);
        const uint32_t byte = mxfp8_scale_byte(m);
        const float sc = e8m0_as_scale(byte);
        uint2 codes;
        codes.x = e4m3_encode4(w[u][0], w[u][1], sc);
        codes.y = e4m3_encode4(w[u][2], w[u][3], sc);
        if (row_ok) *reinterpret_cast<uint2*>(q + row * Cp + col) = codes;
        if ((c8 & 3) == 0) {
          const int bl = (c8 >> 2) - step * tpr;  // block within the step, < tpr
          lds_bytes[((bl << rps_log2) + i) * 4 + j] = row_ok ? (uint8_t)byte : (uint8_t)0;
        }
      }
      __syncthreads();
      // one dword per (block, row of the run): bytes of rows +0, +32, +64, +96;
      // the next step fills the other buffer, and the one after that waits at
      // the next step's barrier, which these reads precede
      if (t < kRowSub) {
        const int bl = t >> rps_log2, ii = t & ((1 << rps_log2) - 1);
        const int64_t blk = (int64_t)step * tpr + bl;
        if (blk < nblk) {
          uint8_t* dst = s + ((g * nblk + blk) * 32 + qb + ii) * 4;
          const uint32_t v = sc_lds[parity][t];
          const int64_t r0 = g * 128 + qb + ii;
          if (r0 + 96 < R) {
            *reinterpret_cast<uint32_t*>(dst) = v;
          } else {  // last, partial group: bytes of rows past R stay untouched
#pragma unroll
            for (int jj = 0; jj < 4; jj++)
              if (r0 + 32 * jj < R) dst[jj] = (uint8_t)(v >> (8 * jj));
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ tile kernel
// A 128 x 128 bf16 tile (128 rows of padded position space = 4 blocks, 128
// columns) is read once with coalesced 16-byte loads, optionally quantised
// along its rows (four lanes per block), staged in LDS, and quantised down its
// columns: each thread takes a column pair and one block of 32 rows.  The
// column codes go back through LDS as a [column][row] code tile, so that eight
// lanes store one column's 128 codes together: stored straight from the
// column-pair lanes, every 16-byte store would touch its own cache line.
constexpr int kTR = 128, kTC = 128, kLdsStride = kTC * 2 + 16;
constexpr int kCodePitch = kTR + 16;  // code tile row pitch: 16-byte aligned, 4-pass b128 reads
static_assert(kTC * kCodePitch <= kTR * kLdsStride, "the code tile reuses the bf16 tile's LDS");
static_assert(kThreads * sizeof(int64_t) <= kTR * kLdsStride, "the group scan's scratch reuses the tile's LDS");

// Phase 2 of a tile, once it is staged in LDS (and a barrier has published
// it): the column copy.  Each thread takes a column pair and one block of 32
// rows; the codes go back through LDS as a [column][row] code tile, so that
// eight lanes store one column's 128 codes together.  Every thread reaches the
// two barriers inside; it returns after the code stores, whose LDS reads must
// precede any new write to the tile.
__device__ __forceinline__ void column_phase(uint8_t* tile, const int32_t* rb_valid, int t, int64_t c0,
                                             int64_t p0, int64_t C, int64_t ldq, uint8_t* __restrict__ q_colT,
                                             uint8_t* __restrict__ s_colT) {
  const int pr = t & 63;  // column pair
  const int rb = t >> 6;  // block of 32 tile rows
  const int64_t col = c0 + 2 * pr;
  const bool blk_ok = rb_valid[rb] > 0 && col < C;  // (every thread reaches both barriers below)
  const int64_t pb = p0 / 32 + rb;  // padded block = output block column
  uint32_t clo[8], chi[8];
  {
    uint32_t d[32];
#pragma unroll
    for (int i = 0; i < 32; i++)
      d[i] = *reinterpret_cast<const uint32_t*>(tile + (rb * 32 + i) * kLdsStride + 4 * pr);
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 32; i += 2) m = pkmax_u16(m, absmax_bf16x2(d[i], d[i + 1]));
    // absmax_bf16x2 keeps per-half maxima: low half = column col, high half = col + 1
    const uint32_t byte_lo = mxfp8_scale_byte(m & 0xFFFFu);
    const uint32_t byte_hi = mxfp8_scale_byte(m >> 16);
    const float sc_lo = e8m0_as_scale(byte_lo), sc_hi = e8m0_as_scale(byte_hi);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const uint32_t a0 = __builtin_amdgcn_perm(d[4 * i + 1], d[4 * i], 0x05040100u);
      const uint32_t a1 = __builtin_amdgcn_perm(d[4 * i + 3], d[4 * i + 2], 0x05040100u);
      const uint32_t b0 = __builtin_amdgcn_perm(d[4 * i + 1], d[4 * i], 0x07060302u);
      const uint32_t b1 = __builtin_amdgcn_perm(d[4 * i + 3], d[4 * i + 2], 0x07060302u);
      clo[i] = e4m3_encode4(a0, a1, sc_lo);
      chi[i] = e4m3_encode4(b0, b1, sc_hi);
    }
    if (blk_ok) {
      // one byte per column and block: the 128 columns of a wave share one line
      const int64_t nsb = ldq / 32;
      s_colT[scale_offset(col, pb, nsb)] = (uint8_t)byte_lo;
      if (col + 1 < C) s_colT[scale_offset(col + 1, pb, nsb)] = (uint8_t)byte_hi;
    }
  }
  __syncthreads();  // every thread has read its column pair: the tile's LDS now holds codes
  {
    uint8_t* cl = tile + (2 * pr) * kCodePitch + rb * 32;
    reinterpret_cast<uint4*>(cl)[0] = make_uint4(clo[0], clo[1], clo[2], clo[3]);
    reinterpret_cast<uint4*>(cl)[1] = make_uint4(clo[4], clo[5], clo[6], clo[7]);
    cl += kCodePitch;
    reinterpret_cast<uint4*>(cl)[0] = make_uint4(chi[0], chi[1], chi[2], chi[3]);
    reinterpret_cast<uint4*>(cl)[1] = make_uint4(chi[4], chi[5], chi[6], chi[7]);
  }
  __syncthreads();
  // lane l of wave w stores 16 codes (rows 16 (l % 8) ..) of tile column
  // 8 (4 i + w) + l / 8: eight lanes cover one output row's 128 bytes
  const int k = t & 7;
  const int rbk = k >> 1;  // block of those rows
  if (rb_valid[rbk] > 0) {
#pragma unroll
    for (int i = 0; i < kTC / 32; i++) {
      const int cc = 8 * (4 * i + (t >> 6)) + ((t & 63) >> 3);
      const int64_t cg = c0 + cc;
      if (cg < C)
        *reinterpret_cast<uint4*>(q_colT + cg * ldq + p0 + 16 * k) =
            *reinterpret_cast<const uint4*>(tile + cc * kCodePitch + 16 * k);
    }
  }
}

template <bool ROW, bool VEC>
__global__ __launch_bounds__(kThreads) void quant_tile_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t C, int64_t ldx, int64_t ldq, int n_col_tiles,
    uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row, uint8_t* __restrict__ q_colT,
    uint8_t* __restrict__ s_colT, BatchStrides bs) {
  // matrix blockIdx.y of a batch
  x += blockIdx.y * bs.x;
  if constexpr (ROW) {
    q_row += blockIdx.y * bs.q_row;
    s_row += blockIdx.y * bs.s_row;
  }
  q_colT += blockIdx.y * bs.q_colT;
  s_colT += blockIdx.y * bs.s_colT;
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTR * kLdsStride];
  __shared__ int64_t rb_src[kTR / 32];   // first source row of each block of the tile
  __shared__ int32_t rb_valid[kTR / 32]; // valid rows in that block (0: no output block)
  const int t = threadIdx.x;
  // Workgroups go to the 8 XCDs round robin; within each run of 64,
  // workgroup b takes tile b - r + 8 (r % 8) + r / 8 (r = b % 64), so an XCD
  // runs eight consecutive tiles of a row of tiles (2 KB of each input row)
  // rather than every eighth (measured 3-5% faster).
  int bt = blockIdx.x;
  {
    const int full = (int)(gridDim.x / 64 * 64);
    if (bt < full) {
      const int r = bt & 63;
      bt = bt - r + (r & 7) * 8 + (r >> 3);
    }
  }
  const int rt = bt / n_col_tiles;
  const int ct = bt - rt * n_col_tiles;
  const int64_t p0 = (int64_t)rt * kTR;  // first padded position of the tile
  const int64_t c0 = (int64_t)ct * kTC;

  if (t < kTR / 32) {
    const int64_t r0 = p0 + 32 * t;
    rb_src[t] = r0;
    rb_valid[t] = r0 < R ? (int32_t)min<int64_t>(32, R - r0) : 0;
  }
  __syncthreads();
  if (rb_valid[0] <= 0) return;  // tile lies past the last block (uniform)

  const int64_t Cp = (C + 31) / 32 * 32;
  // ---- phase 1: load (+ row copy), stage in LDS.  All eight loads of a
  // thread are issued before any arithmetic, so they are in flight together.
  const int c16 = t & 15;
  const int64_t col1 = c0 + c16 * 8;
  uint32_t w[8][4];
  if (VEC && c0 + kTC <= C) {
    // no column tail in this tile: unconditional 16-byte loads (rows past the
    // valid range read the tile's first row, always valid, and are zeroed),
    // so the eight loads issue back to back with no wait between them.  A
    // single matrix is read with non-temporal loads (its bf16 input is read
    // once): in the bench step the dense dual copies of X and W took 0.140
    // instead of 0.154 ms and that of dY 0.107 instead of 0.110 ms; a batch
    // (the expert weights) measured 1-4% slower with them and keeps ordinary
    // loads.
    const bool nt = gridDim.y == 1;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int lr = (t >> 4) + 16 * i;  // tile row
      const int rb = lr >> 5;
      const bool row_ok = (lr & 31) < rb_valid[rb];
      const int64_t src = row_ok ? rb_src[rb] + (lr & 31) : rb_src[0];
      const uint4 v = load16(x + src * ldx + col1, nt);
      w[i][0] = row_ok ? v.x : 0u;
      w[i][1] = row_ok ? v.y : 0u;
      w[i][2] = row_ok ? v.z : 0u;
      w[i][3] = row_ok ? v.w : 0u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int lr = (t >> 4) + 16 * i;
      const int rb = lr >> 5;
      const bool row_ok = (lr & 31) < rb_valid[rb];
      const int64_t src = rb_src[rb] + (lr & 31);
      w[i][0] = w[i][1] = w[i][2] = w[i][3] = 0u;
      if (row_ok) load_chunk<VEC>(x + src * ldx, col1, C, w[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int lr = (t >> 4) + 16 * i;
    if constexpr (ROW) {
      const int rb = lr >> 5;
      const bool row_ok = (lr & 31) < rb_valid[rb];
      const int64_t src = rb_src[rb] + (lr & 31);
      uint32_t m = hmax_u16x2(pkmax_u16(absmax_bf16x2(w[i][0], w[i][1]), absmax_bf16x2(w[i][2], w[i][3])));
      m = quad_max_u32(m);
      const uint32_t byte = mxfp8_scale_byte(m);
      const float sc = e8m0_as_scale(byte);
      uint2 codes;
      codes.x = e4m3_encode4(w[i][0], w[i][1], sc);
      codes.y = e4m3_encode4(w[i][2], w[i][3], sc);
      if (row_ok && col1 < Cp) {
        *reinterpret_cast<uint2*>(q_row + src * Cp + col1) = codes;
        if ((c16 & 3) == 0) s_row[scale_offset(src, col1 / 32, Cp / 32)] = (uint8_t)byte;
      }
    }
    *reinterpret_cast<uint4*>(tile + lr * kLdsStride + c16 * 16) = make_uint4(w[i][0], w[i][1], w[i][2], w[i][3]);
  }
  __syncthreads();

  column_phase(tile, rb_valid, t, c0, p0, C, ldq, q_colT, s_colT);
}


// The grouped token-axis copy (rows = routed tokens in expert order, output
// padded per group to whole 32-row blocks): tiles of 128 padded positions.  A
// workgroup builds the group table once and walks kGrpWalk column tiles of
// one row tile, the next tile's loads in flight while the current one is
// quantised.  Measured on 131072 x 7168 against one tile per workgroup: the
// token-axis copy 0.593 -> 0.569 ms, with the row copy (x 4096) 0.446 ->
// 0.441 ms; two or eight tiles per workgroup, or re-reading the source rows
// from LDS per tile (126 instead of 156 VGPRs, four workgroups per CU instead
// of three), no better.  Consecutive
// workgroups take consecutive column groups of a row tile: dealing them to
// the XCDs like the ungrouped tiles measured 35% slower with one tile per
// workgroup and 1-2% slower with the walk.
constexpr int kGrpWalk = 4;

template <bool ROW, bool VEC>
__global__ __launch_bounds__(kThreads) void quant_tile_grouped_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t C, int64_t ldx, const int32_t* __restrict__ group_end,
    int32_t G, int64_t ldq, int n_col_tiles, int n_col_groups, uint8_t* __restrict__ q_row,
    uint8_t* __restrict__ s_row, uint8_t* __restrict__ q_colT, uint8_t* __restrict__ s_colT) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTR * kLdsStride];
  __shared__ int64_t rb_src[kTR / 32];   // first source row of each block of the tile
  __shared__ int32_t rb_valid[kTR / 32]; // valid rows in that block (0: no output block)
  const int t = threadIdx.x;
  const int rt = blockIdx.x / n_col_groups;
  const int ct_begin = (blockIdx.x - rt * n_col_groups) * kGrpWalk;
  const int ct_end = min(ct_begin + kGrpWalk, n_col_tiles);
  const int64_t p0 = (int64_t)rt * kTR;  // first padded position of the tile

  // block starts only (the tile's few groups re-read their spans from
  // group_end), keeping LDS small enough for four workgroups per CU;
  // the scan's scratch is the tile buffer, not yet in use
  __shared__ int32_t bstart[kMaxGroups + 1];
  build_block_starts<kThreads>(group_end, G, R, 32, nullptr, nullptr, bstart,
                               reinterpret_cast<int64_t*>(tile));
  if (t < kTR / 32) {
    const int64_t pb = p0 / 32 + t;
    int64_t src = 0;
    int32_t valid = 0;
    if (pb < bstart[G] && (pb + 1) * 32 <= ldq) {
      const int g = find_block_group(bstart, G, (int32_t)pb);
      int32_t gstart, gsize;
      group_span(group_end, g, R, gstart, gsize);
      // (bstart is non-decreasing and bstart[g] <= pb < bstart[g] + ceil32(gsize) / 32)
      const int64_t off = (pb - bstart[g]) * 32;
      src = (int64_t)gstart + off;
      valid = (int32_t)min<int64_t>(32, gsize - off);
      if (valid <= 0) valid = -1;  // cannot happen for consistent tables
    }
    rb_src[t] = src;
    rb_valid[t] = valid;
  }
  __syncthreads();
  if (rb_valid[0] <= 0) return;  // tile lies past the last block (uniform)

  const int64_t Cp = (C + 31) / 32 * 32;
  // source rows of this thread's eight chunks (rows (t / 16) + 16 i of the
  // tile), the same for every column tile; rows past a block's valid range
  // read the tile's first row, always valid, and are zeroed where used
  const int c16 = t & 15;
  int64_t srow[8];
  uint32_t row_ok = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int lr = (t >> 4) + 16 * i;
    const int rb = lr >> 5;
    const bool ok = (lr & 31) < rb_valid[rb];
    row_ok |= (uint32_t)ok << i;
    srow[i] = ok ? rb_src[rb] + (lr & 31) : rb_src[0];
  }
  // All eight loads of a thread are issued back to back, before any use, so
  // they are in flight together; the loaded words are used only after the
  // next barrier, so the loads of the next column tile stay in flight while
  // the current one is quantised from LDS.
  auto load_tile = [&](int64_t c0, uint32_t (&w)[8][4]) {
    const int64_t col1 = c0 + c16 * 8;
    if (VEC && c0 + kTC <= C) {  // no column tail in this tile
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint4 v = *reinterpret_cast<const uint4*>(x + srow[i] * ldx + col1);
        w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++) {
        w[i][0] = w[i][1] = w[i][2] = w[i][3] = 0u;
        if (row_ok >> i & 1u) load_chunk<VEC>(x + srow[i] * ldx, col1, C, w[i]);
      }
    }
  };
  uint32_t w[8][4];
  load_tile((int64_t)ct_begin * kTC, w);
#pragma unroll 1
  for (int ct = ct_begin; ct < ct_end; ct++) {
    const int64_t c0 = (int64_t)ct * kTC;
    const int64_t col1 = c0 + c16 * 8;
    // ---- phase 1: (row copy,) stage the tile in LDS
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int lr = (t >> 4) + 16 * i;
      const bool ok = row_ok >> i & 1u;
      const uint32_t u0 = ok ? w[i][0] : 0u, u1 = ok ? w[i][1] : 0u;
      const uint32_t u2 = ok ? w[i][2] : 0u, u3 = ok ? w[i][3] : 0u;
      if constexpr (ROW) {
        uint32_t m = hmax_u16x2(pkmax_u16(absmax_bf16x2(u0, u1), absmax_bf16x2(u2, u3)));
        m = quad_max_u32(m);
        const uint32_t byte = mxfp8_scale_byte(m);
        const float sc = e8m0_as_scale(byte);
        uint2 codes;
        codes.x = e4m3_encode4(u0, u1, sc);
        codes.y = e4m3_encode4(u2, u3, sc);
        if (ok && col1 < Cp) {
          *reinterpret_cast<uint2*>(q_row + srow[i] * Cp + col1) = codes;
          if ((c16 & 3) == 0) s_row[scale_offset(srow[i], col1 / 32, Cp / 32)] = (uint8_t)byte;
        }
      }
      *reinterpret_cast<uint4*>(tile + lr * kLdsStride + c16 * 16) = make_uint4(u0, u1, u2, u3);
    }
    __syncthreads();
    if (ct + 1 < ct_end) load_tile(c0 + kTC, w);

    column_phase(tile, rb_valid, t, c0, p0, C, ldq, q_colT, s_colT);
    if (ct + 1 < ct_end) __syncthreads();  // the code tile is read before the next tile is staged (uniform)
  }
}

}  // namespace

hipError_t launch_quant_row(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, uint8_t* q,
                            uint8_t* s, hipStream_t st, int batch, BatchStrides bs) {
  const int64_t cpr = (C + 31) / 32 * 4;
  int tpr_log2 = 3;  // at most 32 rows per sub-group
  while ((1 << tpr_log2) < cpr && tpr_log2 < 8) tpr_log2++;
  const int64_t per_group = 32 >> (8 - tpr_log2);
  const int64_t want = (R + 127) / 128 * per_group;
  // one workgroup per unit of rows (many short workgroups stream HBM faster
  // than a grid-stride loop over a CU-sized grid); capped by the grid limit
  const int64_t cap = 0x7FFFFFFF;
  const int grid = (int)(want < cap ? want : cap);
  const bool vec = (ldx % 8 == 0) && ((uintptr_t)x % 16 == 0) && (batch == 1 || bs.x % 8 == 0);
  const dim3 g((unsigned)grid, (unsigned)batch);
  if (vec)
    quant_row_kernel<true><<<g, kRowThreads, 0, st>>>(x, R, C, ldx, tpr_log2, q, s, bs);
  else
    quant_row_kernel<false><<<g, kRowThreads, 0, st>>>(x, R, C, ldx, tpr_log2, q, s, bs);
  return hipGetLastError();
}

hipError_t launch_quant_tile(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                             const int32_t* group_end, int32_t G, int64_t ldq, uint8_t* q_row,
                             uint8_t* s_row, uint8_t* q_colT, uint8_t* s_colT, hipStream_t st, int batch,
                             BatchStrides bs) {
  const bool grouped = group_end != nullptr;
  const bool row = q_row != nullptr;
  const bool vec = (ldx % 8 == 0) && ((uintptr_t)x % 16 == 0) && (batch == 1 || bs.x % 8 == 0);
  const int64_t padded = grouped ? (R + 31 * (int64_t)G) : R;
  const int64_t n_row_tiles = (padded + kTR - 1) / kTR;
  const int n_col_tiles = (int)((C + kTC - 1) / kTC);
  if (grouped) {
    const int n_col_groups = (n_col_tiles + kGrpWalk - 1) / kGrpWalk;
    const int64_t grid = n_row_tiles * n_col_groups;
    if (grid > 0x7FFFFFFF || batch != 1) return hipErrorInvalidValue;
#define MXQ_TILE_LAUNCH(ROWv, VECv)                                                             \
  quant_tile_grouped_kernel<ROWv, VECv><<<(unsigned)grid, kThreads, 0, st>>>(                   \
      x, R, C, ldx, group_end, G, ldq, n_col_tiles, n_col_groups, q_row, s_row, q_colT, s_colT)
    if (row) { if (vec) MXQ_TILE_LAUNCH(true, true); else MXQ_TILE_LAUNCH(true, false); }
    else { if (vec) MXQ_TILE_LAUNCH(false, true); else MXQ_TILE_LAUNCH(false, false); }
#undef MXQ_TILE_LAUNCH
    return hipGetLastError();
  }
  const int64_t grid = n_row_tiles * n_col_tiles;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
#define MXQ_TILE_LAUNCH(ROWv, VECv)                                                                  \
  quant_tile_kernel<ROWv, VECv><<<dim3((unsigned)grid, (unsigned)batch), kThreads, 0, st>>>(         \
      x, R, C, ldx, ldq, n_col_tiles, q_row, s_row, q_colT, s_colT, bs)
  if (row) { if (vec) MXQ_TILE_LAUNCH(true, true); else MXQ_TILE_LAUNCH(true, false); }
  else { if (vec) MXQ_TILE_LAUNCH(false, true); else MXQ_TILE_LAUNCH(false, false); }
#undef MXQ_TILE_LAUNCH
  return hipGetLastError();
}

}  // namespace mxq
