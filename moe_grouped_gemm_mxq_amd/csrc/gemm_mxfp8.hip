// Block-scaled MXFP8 GEMMs for gfx950: C[m][n] = sum_k deq(A)[m][k] deq(B)[n][k]
// with E4M3 codes, one E8M0 scale per 32 values along K, fp32 accumulation and
// fp32 output (the FP8 linear and expert GEMMs of the torchtitan-npu guide,
// "线性层低精度" and "MoE 专家层低精度").
//
// One main loop serves three problem shapes:
//   dense    -- one A [M][K], one B [N][K];
//   ragged M -- rows of A split into expert groups, group g multiplies B[g]
//               (expert forward and input gradient);
//   ragged K -- the reduction axis split into groups, one output per group
//               (expert weight gradient over each group's padded tokens).
//
// Tiling: 256 x 256 output tile per workgroup of 4 waves (2 x 2), each wave a
// 128 x 128 sub-tile of 8 x 8 MFMA blocks of 16 x 16; K advances 128 codes per
// step.  Operand tiles go from global memory straight into LDS
// (global_load_lds_dwordx4, no register staging), double-buffered: the loads
// of step k+1 are in flight while step k is multiplied.
//
// Operand layout of v_mfma_scale_f32_16x16x128_f8f6f4 for FP8 (found by
// probing): lane l holds row l%16; its bytes 0-15 are K = 16g..16g+15 and
// bytes 16-31 are K = 64+16g..64+16g+15 with g = l/16; its scale byte (chosen
// by op_sel) scales row l%16 over K-block g (K = 32g..32g+31).  Accumulator
// element i of lane l is C[4*(l/16) + i][l%16].
#include "mxq_device.h"
#include "mxq_groups.h"
#include "mxq_internal.h"

namespace mxq {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 256, BK = 128;  // BK in codes (bytes) per step
constexpr int WM = 128, WN = 128;             // wave tile
constexpr int TM = WM / 16, TN = WN / 16;     // MFMA blocks per wave
constexpr int kTileBytes = BM * BK;           // one operand tile per stage (32 KB)
constexpr int kScaleBytes = 4 * BM;           // scale bytes of one operand tile per stage
constexpr int kStageBytes = 2 * kTileBytes + 2 * kScaleBytes;
constexpr int kXcds = 8;                      // XCDs per MI355X; workgroups are dealt round robin
constexpr int kGroupM = 8;                    // m-tiles per raster group

enum Mode { kDense = 0, kRaggedM = 1, kRaggedK = 2 };

// op_sel must be an immediate: dispatch the 16 combinations (folded away once
// the calling loops are unrolled).
template <int OA, int OB>
__device__ __forceinline__ v4f mfma_os(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, OA, sa, OB, sb);
}
__device__ __forceinline__ v4f mfma_scaled(int oa, int ob, const v8i& a, const v8i& b, const v4f& c,
                                           int sa, int sb) {
  switch (oa * 4 + ob) {
    case 0: return mfma_os<0, 0>(a, b, c, sa, sb);
    case 1: return mfma_os<0, 1>(a, b, c, sa, sb);
    case 2: return mfma_os<0, 2>(a, b, c, sa, sb);
    case 3: return mfma_os<0, 3>(a, b, c, sa, sb);
    case 4: return mfma_os<1, 0>(a, b, c, sa, sb);
    case 5: return mfma_os<1, 1>(a, b, c, sa, sb);
    case 6: return mfma_os<1, 2>(a, b, c, sa, sb);
    case 7: return mfma_os<1, 3>(a, b, c, sa, sb);
    case 8: return mfma_os<2, 0>(a, b, c, sa, sb);
    case 9: return mfma_os<2, 1>(a, b, c, sa, sb);
    case 10: return mfma_os<2, 2>(a, b, c, sa, sb);
    case 11: return mfma_os<2, 3>(a, b, c, sa, sb);
    case 12: return mfma_os<3, 0>(a, b, c, sa, sb);
    case 13: return mfma_os<3, 1>(a, b, c, sa, sb);
    case 14: return mfma_os<3, 2>(a, b, c, sa, sb);
    default: return mfma_os<3, 3>(a, b, c, sa, sb);
  }
}

// LDS position of 16-byte chunk c (0..7) of tile row r: XOR swizzle so that the
// 16 rows one MFMA fragment read touches fall in distinct bank groups.
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ ((r >> 1) & 7)) << 4); }

// LDS position of the scale byte of tile row r, K-block g: each lane later
// reads the 8 bytes of its 8 MFMA row blocks (rows wave*128 + i*16 + l%16,
// i = 0..7) with one 64-bit load; byte i%4 of dword i/4 is op_sel'ed.
__device__ __forceinline__ int sidx(int r, int g) {
  return ((g * 2 + (r >> 7)) * 16 + (r & 15)) * 8 + ((r & 127) >> 4);
}

// One operand of one workgroup tile: tile rows [0, rows_valid) of a matrix
// whose row r starts at base + r*ld (codes) and sbase + r*(ld/32) (scales).
// Rows at or past rows_valid are loaded from row rows_valid-1 (their results
// are never stored).
struct Operand {
  const uint8_t* base;
  const uint8_t* sbase;
  int64_t ld;
  int rows_valid;
};

// Direct loads of one operand tile: wave w issues 8 dwordx4 loads; load j
// fills LDS bytes [(8w + j) * 1024, +1024), i.e. tile rows 8(8w+j) .. +8, lane l
// writing 16-byte slot l%8 of row 8(8w+j) + l/8, which holds global chunk
// slot ^ swizzle(row).  swizzle(row) = (row >> 1) & 7 = (4*(j&1) + l/16) & 7, so
// the chunk a lane moves depends only on the parity of j.
__device__ __forceinline__ int load_chunk(int lane, int j) { return (lane & 7) ^ ((4 * (j & 1) + (lane >> 4)) & 7); }

// Issue the 8 direct loads of one operand tile for the K step at k.  In the
// tail step chunks past the last valid one (last_chunk) are fetched from the
// last valid chunk instead (always in bounds) and zeroed by zero_tail() once
// they have landed.  Addresses are formed on the fly (no held offsets).
__device__ __forceinline__ void issue_loads(const Operand& op, uint8_t* lds_tile, int wave, int lane,
                                            int64_t k, int last_chunk) {
  int r0 = wave * 64 + (lane >> 3);
  // opaque to the optimiser: keeps the 16 load addresses from being hoisted out
  // of the K loop (holding them would cost 32+ registers and spill)
  asm volatile("" : "+v"(r0));
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int c = load_chunk(lane, j);
    const int cc = c <= last_chunk ? c : last_chunk;
    const int r = min(r0 + 8 * j, op.rows_valid - 1);
    __builtin_amdgcn_global_load_lds(op.base + (int64_t)r * op.ld + k + cc * 16,
                                     (lds_ptr)(lds_tile + (wave * 8 + j) * 1024), 16, 0, 0);
  }
}

// After the tail step's loads have landed: zero the chunks past the end of K.
__device__ __forceinline__ void zero_tail(uint8_t* lds_tile, int wave, int lane, int last_chunk) {
#pragma unroll
  for (int j = 0; j < 8; j++)
    if (load_chunk(lane, j) > last_chunk)
      *reinterpret_cast<uint4*>(lds_tile + (wave * 8 + j) * 1024 + lane * 16) = make_uint4(0u, 0u, 0u, 0u);
}

// Scale bytes: thread t needs the 4 bytes of tile row t for K-blocks
// k/32 .. k/32+3 (row length ld/32 bytes, so rows need not be dword aligned).
// Two aligned dword loads cover them: the dwords holding the first byte and
// the last valid byte (both inside the allocation).  The raw dwords are
// combined only after the MFMAs (combine_scales), so the loads are waited for
// once per step, not one by one.
struct ScaleRaw {
  uint32_t lo, hi;
  int shift;  // byte offset of the first byte within `lo`
};

__device__ __forceinline__ ScaleRaw load_scales(const Operand& op, int64_t k, int last_block) {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  const int r = t < op.rows_valid ? t : op.rows_valid - 1;
  const uint8_t* p = op.sbase + (int64_t)r * (op.ld / 32) + k / 32;
  const uintptr_t a0 = (uintptr_t)p, a1 = (uintptr_t)(p + last_block);
  ScaleRaw s;
  s.lo = *reinterpret_cast<const uint32_t*>(a0 & ~(uintptr_t)3);
  s.hi = *reinterpret_cast<const uint32_t*>(a1 & ~(uintptr_t)3);
  s.shift = (int)(a0 & 3);
  return s;
}

// the 4 scale bytes in K order; blocks past last_block become 127 (their codes
// are zero, any finite scale will do)
__device__ __forceinline__ uint32_t combine_scales(const ScaleRaw& s, int last_block) {
  // bytes lo[shift..3] followed by hi[0..]: when the 4 bytes sit in one dword, hi == lo
  // and the shift is 0, so the funnel shift returns lo itself
  uint32_t v = __builtin_amdgcn_alignbyte(s.hi, s.lo, (uint32_t)s.shift);
  if (last_block < 3) {
    const uint32_t keep = 0xFFFFFFFFu >> (8 * (3 - last_block));
    v = (v & keep) | (0x7F7F7F7Fu & ~keep);
  }
  return v;
}

__device__ __forceinline__ void store_scales(uint8_t* lds_scales, uint32_t sc) {
  const int t = threadIdx.x;
#pragma unroll
  for (int g = 0; g < 4; g++) lds_scales[sidx(t, g)] = (uint8_t)(sc >> (8 * g));
}

// fragment of the MFMA row block starting at tile row r0 for this lane
__device__ __forceinline__ v8i load_frag(const uint8_t* lds_codes, int r0, int lane) {
  const int r = r0 + (lane & 15);
  const int g = lane >> 4;
  const uint4 lo = *reinterpret_cast<const uint4*>(lds_codes + swz(r, g));
  const uint4 hi = *reinterpret_cast<const uint4*>(lds_codes + swz(r, 4 + g));
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

// Logical tile order: workgroups are dealt to the XCDs round robin, so remap
// blockIdx so that each XCD walks a contiguous run of the logical order (tiles
// that share operand panels then share that XCD's L2).
// (Used where every tile carries the same work; bid < n.)
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int per = n / kXcds;
  const int x = bid % kXcds, i = bid / kXcds;
  if (i >= per) return bid;  // the last partial round stays in place
  return x * per + i;
}

// grouped raster: kGroupM m-tiles at a time, m fastest
__device__ __forceinline__ void raster(int t, int tiles_m, int tiles_n, int& mt, int& nt) {
  const int span = kGroupM * tiles_n;
  const int grp = t / span;
  const int first = grp * kGroupM;
  const int gm = min(kGroupM, tiles_m - first);
  const int r = t - grp * span;
  mt = first + r % gm;
  nt = r / gm;
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_mxfp8_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ sB, float* __restrict__ C, int64_t M, int64_t N, int64_t K,
    int64_t ldc, const int32_t* __restrict__ group_end, int32_t G, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kStageBytes];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int bid = blockIdx.x;

  // ---- which output tile, and the operands behind it
  int64_t m0, n0 = 0, k_begin = 0, k_end = K;
  int rows_a;
  const uint8_t *b_base = B, *sb_base = sB;
  float* c_base = C;
  const int64_t lda = K;
  if constexpr (MODE == kDense) {
    int mt, nt;
    raster(xcd_remap(bid, gridDim.x), tiles_m, tiles_n, mt, nt);
    m0 = (int64_t)mt * BM;
    n0 = (int64_t)nt * BN;
    rows_a = (int)min<int64_t>(BM, M - m0);
  } else {
    __shared__ GroupTable gt;
    __shared__ int32_t scan_tmp[kThreads];
    if constexpr (MODE == kRaggedM) {
      build_group_table<kThreads>(group_end, G, M, BM, gt, scan_tmp);
      // the grid covers an upper bound of m-tiles; the real ones are bstart[G]
      const int real_m = gt.bstart[G];
      const int n_real = real_m * tiles_n;
      if (bid >= n_real) return;  // uniform
      int mt, nt;
      raster(xcd_remap(bid, n_real), real_m, tiles_n, mt, nt);
      const int g = find_group(gt, G, mt);
      const int local = mt - gt.bstart[g];
      m0 = (int64_t)gt.start[g] + (int64_t)local * BM;
      n0 = (int64_t)nt * BN;
      rows_a = min(BM, gt.size[g] - local * BM);
      b_base = B + (int64_t)g * N * K;
      sb_base = sB + (int64_t)g * N * (K / 32);
    } else {
      build_group_table<kThreads>(group_end, G, (int64_t)1 << 40, 32, gt, scan_tmp);
      // largest groups first (their tiles carry the longest K loops)
      __shared__ int32_t order[kMaxGroups];
      for (int g = t; g < G; g += kThreads) {
        const int32_t sz = gt.size[g];
        int rank = 0;
        for (int h = 0; h < G; h++) {
          const int32_t sh = gt.size[h];
          rank += (sh > sz) || (sh == sz && h < g);
        }
        order[rank] = g;
      }
      __syncthreads();
      // groups are taken largest first; inside a group's run of workgroups the
      // XCD remap gives every XCD an equal, contiguous share of that group's
      // tiles (balanced across XCDs, and each XCD's concurrent tiles share
      // operand panels in its L2)
      const int per_g = tiles_m * tiles_n;
      const int gi = bid / per_g;
      const int g = order[gi];
      int mt, nt;
      raster(xcd_remap(bid - gi * per_g, per_g), tiles_m, tiles_n, mt, nt);
      m0 = (int64_t)mt * BM;
      n0 = (int64_t)nt * BN;
      rows_a = (int)min<int64_t>(BM, M - m0);
      k_begin = (int64_t)gt.bstart[g] * 32;
      k_end = min<int64_t>((int64_t)gt.bstart[g + 1] * 32, K);  // never past the row length
      if (k_end < k_begin) k_end = k_begin;
      c_base = C + (int64_t)g * M * N;
    }
  }
  const int rows_b = (int)min<int64_t>(BN, N - n0);

  const Operand opa{A + m0 * lda, sA + m0 * (lda / 32), lda, rows_a};
  const Operand opb{b_base + n0 * lda, sb_base + n0 * (lda / 32), lda, rows_b};

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nk = (int)((k_end - k_begin + BK - 1) / BK);
  // chunks / blocks of the last step that lie before k_end (7 / 3 when K steps evenly)
  const int tail_chunks = (int)((k_end - k_begin) - (int64_t)(nk - 1) * BK) / 16;  // 2..8
  const int tail_blocks = tail_chunks / 2;                                            // 1..4

  // Per step: (1) scale bytes of step s+1 to registers, (2) all fragments and
  // scales of step s from LDS to registers, (3) direct loads of step s+1 into
  // the other stage, (4) the 64 MFMAs.  Issuing the direct loads only after the
  // LDS reads keeps the compiler from waiting on them before those reads, so
  // they stream in while the MFMAs run.
  auto last_block = [&](int s) { return s == nk - 1 ? tail_blocks - 1 : 3; };
  auto load_step_scales = [&](int s, ScaleRaw& nsa, ScaleRaw& nsb) {
    const int64_t k = k_begin + (int64_t)s * BK;
    nsa = load_scales(opa, k, last_block(s));
    nsb = load_scales(opb, k, last_block(s));
  };
  auto load_step_codes = [&](uint8_t* dst, int s) {
    const int64_t k = k_begin + (int64_t)s * BK;
    const int lc = s == nk - 1 ? tail_chunks - 1 : 7;
    issue_loads(opa, dst, wave, lane, k, lc);
    issue_loads(opb, dst + kTileBytes, wave, lane, k, lc);
  };
  // after the loads of step s have landed in stage `dst`
  auto settle = [&](uint8_t* dst, int s, const ScaleRaw& nsa, const ScaleRaw& nsb) {
    store_scales(dst + 2 * kTileBytes, combine_scales(nsa, last_block(s)));
    store_scales(dst + 2 * kTileBytes + kScaleBytes, combine_scales(nsb, last_block(s)));
    const int lc = s == nk - 1 ? tail_chunks - 1 : 7;  // 7: nothing to zero
    zero_tail(dst, wave, lane, lc);
    zero_tail(dst + kTileBytes, wave, lane, lc);
  };

  ScaleRaw nsa{0u, 0u, 0}, nsb{0u, 0u, 0};
  if (nk > 0) {
    load_step_scales(0, nsa, nsb);
    load_step_codes(lds, 0);
    __builtin_amdgcn_s_waitcnt(0);
    settle(lds, 0, nsa, nsb);
  }
  __syncthreads();
  // The body is branch-free (one basic block) so the scheduling barrier below
  // can keep the MFMAs ahead of the wait: the last step re-fetches itself into
  // the idle stage instead of skipping the prefetch.
  for (int kt = 0; kt < nk; kt++) {
    uint8_t* cur = lds + (kt & 1) * kStageBytes;
    uint8_t* nxt = lds + ((kt + 1) & 1) * kStageBytes;
    const int sn = min(kt + 1, nk - 1);
    load_step_scales(sn, nsa, nsb);
    // fragments of step kt
    const uint2 sa = *reinterpret_cast<const uint2*>(cur + 2 * kTileBytes + sidx(wm * 128 + (lane & 15), lane >> 4));
    const uint2 sb = *reinterpret_cast<const uint2*>(cur + 2 * kTileBytes + kScaleBytes +
                                                     sidx(wn * 128 + (lane & 15), lane >> 4));
    v8i fa[TM], fb[TN];
#pragma unroll
    for (int i = 0; i < TM; i++) fa[i] = load_frag(cur, wm * WM + i * 16, lane);
#pragma unroll
    for (int j = 0; j < TN; j++) fb[j] = load_frag(cur + kTileBytes, wn * WN + j * 16, lane);
    load_step_codes(nxt, sn);
#pragma unroll
    for (int j = 0; j < TN; j++) {
      const int sbj = (int)(j < 4 ? sb.x : sb.y);
#pragma unroll
      for (int i = 0; i < TM; i++) {
        const int sai = (int)(i < 4 ? sa.x : sa.y);
        acc[i][j] = mfma_scaled(i & 3, j & 3, fa[i], fb[j], acc[i][j], sai, sbj);
      }
    }
    // Keep the MFMAs ahead of the wait: they only touch registers, so the
    // compiler would otherwise sink them below it (even into the next
    // iteration) and serialise the loads and the math.  An empty volatile asm
    // reading each accumulator pins every MFMA before the wait.
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int j = 0; j < TN; j++) asm volatile("" : "+a"(acc[i][j]));
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    settle(nxt, sn, nsa, nsb);
    __syncthreads();
  }

  // ---- epilogue: fp32 stores, rows/cols past the tile's valid range skipped
  const int64_t ldo = MODE == kRaggedK ? N : ldc;
#pragma unroll
  for (int i = 0; i < TM; i++) {
#pragma unroll
    for (int j = 0; j < TN; j++) {
      const int col = wn * WN + j * 16 + (lane & 15);
      if (col >= rows_b) continue;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int row = wm * WM + i * 16 + 4 * (lane >> 4) + e;
        if (row < rows_a) c_base[(m0 + row) * ldo + n0 + col] = acc[i][j][e];
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(int mode, const uint8_t* A, const uint8_t* sA, const uint8_t* B,
                       const uint8_t* sB, float* C, int64_t M, int64_t N, int64_t K, int64_t ldc,
                       const int32_t* group_end, int32_t G, hipStream_t st) {
  const int tiles_n = (int)((N + BN - 1) / BN);
  if (mode == kDense) {
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int64_t grid = (int64_t)tiles_m * tiles_n;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    gemm_mxfp8_kernel<kDense><<<(unsigned)grid, kThreads, 0, st>>>(A, sA, B, sB, C, M, N, K, ldc,
                                                                    nullptr, 1, tiles_m, tiles_n);
  } else if (mode == kRaggedM) {
    // every group adds at most one partial tile
    const int tiles_m = (int)((M + BM - 1) / BM + G);
    const int64_t grid = (int64_t)tiles_m * tiles_n;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    gemm_mxfp8_kernel<kRaggedM><<<(unsigned)grid, kThreads, 0, st>>>(A, sA, B, sB, C, M, N, K, ldc,
                                                                      group_end, G, tiles_m, tiles_n);
  } else {
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int64_t grid = (int64_t)G * tiles_m * tiles_n;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    gemm_mxfp8_kernel<kRaggedK><<<(unsigned)grid, kThreads, 0, st>>>(A, sA, B, sB, C, M, N, K, N,
                                                                      group_end, G, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

}  // namespace mxq
