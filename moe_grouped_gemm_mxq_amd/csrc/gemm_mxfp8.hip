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
// 128 x 128 sub-tile of 4 x 4 MFMA blocks of 32 x 32; K advances 64 codes per
// step (one v_mfma_scale_f32_32x32x64_f8f6f4 per block and step).
//
// Pipeline: codes (global_load_lds_dwordx4) and scale bytes
// (global_load_lds_ubyte) go from global memory straight into LDS, into a
// ring of four stages; step k's loads are issued four steps ahead, into the
// stage that step k-4 used.  Each wave keeps two register sets of MFMA
// fragments: while the MFMAs of step k run on one, the LDS reads of step k+1
// fill the other, so the matrix cores never wait on LDS.  One s_barrier per
// step (raw, with explicit vmcnt / lgkmcnt waits: a full __syncthreads would
// drain the loads in flight) publishes stage k+1 and retires stage k.  The four
// stages are separate LDS arrays and the loop is unrolled by four, so the
// compiler can tell the stage being read from the stages being filled and
// never waits on the latter.
//
// Operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 for FP8 (found by
// probing): lane l holds row l%32; its bytes 0-15 are K = 16g..16g+15 and
// bytes 16-31 are K = 32+16g..32+16g+15 with g = l/32; its scale byte (chosen
// by op_sel) scales row l%32 over K-block g.  Accumulator element e of lane l
// is C[8*(e/4) + 4*(l/32) + e%4][l%32].
#include "mxq_device.h"
#include "mxq_groups.h"
#include "mxq_internal.h"

namespace mxq {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 256, BK = 64;   // BK in codes (bytes) per step
constexpr int WM = 128, WN = 128;             // wave tile
constexpr int TM = WM / 32, TN = WN / 32;     // MFMA blocks per wave
constexpr int kTileBytes = BM * BK;           // codes of one operand tile per stage (16 KB)
constexpr int kScaleRegion = 4 * 2 * BM;      // one dword per (tile row, K-block) of one operand
constexpr int kStageBytes = 2 * kTileBytes + 2 * kScaleRegion;  // A, B codes, A, B scales (36 KB)
constexpr int kVmemPerStep = 12;              // per wave and step: 4 + 4 code loads, 2 + 2 scale loads
constexpr int kXcds = 8;                      // XCDs per MI355X; workgroups are dealt round robin
constexpr int kGroupM = 8;                    // m-tiles per raster group

enum Mode { kDense = 0, kRaggedM = 1, kRaggedK = 2 };

__device__ __forceinline__ v16f mfma_scaled(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// LDS position of 16-byte chunk c (0..3) of tile row r (64 bytes): XOR swizzle
// so that the 16 rows a fragment read touches at once fall in distinct banks.
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ ((r >> 2) & 3)) << 4); }

// One operand of one workgroup tile: tile rows [0, rows_valid), which are rows
// row0 .. row0 + rows_valid - 1 of a matrix with codes at base + (r - row0)*ld
// and scales at sbase + scale_offset(r, block, ld/32) (the 32-row interleaved
// layout the quantisers write).  Rows at or past rows_valid are read from row
// rows_valid-1 (their results are never stored).
struct Operand {
  const uint8_t* base;   // codes of tile row 0
  const uint8_t* sbase;  // scale array of the whole matrix
  int64_t row0;
  int64_t ld;
  int rows_valid;
};

// Direct loads of one operand's codes (16 KB) for the step at k: wave w issues
// 4 dwordx4 loads; load j fills LDS bytes [(4w + j) * 1024, +1024) = tile rows
// 16(4w+j) .. +16, lane l writing 16-byte slot l%4 of row 16(4w+j) + l/4, which
// holds global chunk slot ^ swizzle(row) = (l%4) ^ ((l/16)%4).  Chunks past
// the end of K (the tail step) are fetched from the last valid chunk (always
// in bounds) and zeroed by zero_codes() once they have landed.
__device__ __forceinline__ int dma_chunk(int lane) { return (lane & 3) ^ ((lane >> 4) & 3); }

__device__ __forceinline__ void issue_codes(const Operand& op, uint8_t* tile, int wave, int lane, int64_t k,
                                            int valid_chunks) {
  int l = lane;
  asm volatile("" : "+v"(l));  // keep the addresses from being hoisted out of the K loop
  const int c = dma_chunk(l);
  const int cc = c < valid_chunks ? c : valid_chunks - 1;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int r = min((wave * 4 + j) * 16 + (l >> 2), op.rows_valid - 1);
    __builtin_amdgcn_global_load_lds(op.base + (int64_t)r * op.ld + k + cc * 16,
                                     (lds_ptr)(tile + (wave * 4 + j) * 1024), 16, 0, 0);
  }
}

// Zero the code chunks at or past valid_chunks (0 zeroes the whole step) in
// the bytes this wave's own loads wrote; called after those loads landed.
__device__ __forceinline__ void zero_codes(uint8_t* tile, int wave, int lane, int valid_chunks) {
  if (dma_chunk(lane) >= valid_chunks)
#pragma unroll
    for (int j = 0; j < 4; j++)
      *reinterpret_cast<uint4*>(tile + (wave * 4 + j) * 1024 + lane * 16) = make_uint4(0u, 0u, 0u, 0u);
}

// Scale slot d (0..511) of one operand and step, one dword each (the scale in
// its low byte): d = ((h*2 + g)*32 + r)*4 + i holds the scale of tile row
// h*128 + i*32 + r over K-block g of the step.  A lane of wave half h reading
// the 16 bytes at slot ((h*2 + l/32)*32 + l%32)*4 gets its four MFMA row
// blocks' scales.  Wave w fills slots [128w, 128w+128) with two ubyte loads;
// in the interleaved scale layout the 64 lanes of one load read 4 runs of 16
// consecutive bytes.  A K-block past the end of K re-reads block 0 (its codes
// are zeroed).
__device__ __forceinline__ void issue_scales(const Operand& op, uint8_t* region, int wave, int lane, int64_t k,
                                             int valid_blocks) {
  int l = lane;
  asm volatile("" : "+v"(l));
  const int64_t nblk = op.ld / 32;
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int d = (wave * 2 + j) * 64 + l;
    const int i = d & 3, r = (d >> 2) & 31, g = (d >> 7) & 1, h = d >> 8;
    const int row = min(h * 128 + i * 32 + r, op.rows_valid - 1);
    const int gg = min(g, valid_blocks - 1);
    __builtin_amdgcn_global_load_lds(op.sbase + scale_offset(op.row0 + row, k / 32 + gg, nblk),
                                     (lds_ptr)(region + (wave * 2 + j) * 256), 1, 0, 0);
  }
}

// MFMA operands of one step for one wave: 4 row blocks of A, 4 of B (32 bytes
// per lane each), and the lane's 4 + 4 block scales.
struct Frags {
  v8i a[TM], b[TN];
  uint4 sa, sb;
};

__device__ __forceinline__ v8i load_frag(const uint8_t* codes, int r0, int lane) {
  const int r = r0 + (lane & 31);
  const int g = lane >> 5;
  const uint4 lo = *reinterpret_cast<const uint4*>(codes + swz(r, g));
  const uint4 hi = *reinterpret_cast<const uint4*>(codes + swz(r, 2 + g));
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

__device__ __forceinline__ void read_frags(const uint8_t* st, int wm, int wn, int lane, Frags& f) {
  const int so = (((lane >> 5) * 32 + (lane & 31)) * 4) * 4;
  f.sa = *reinterpret_cast<const uint4*>(st + 2 * kTileBytes + wm * 1024 + so);
  f.sb = *reinterpret_cast<const uint4*>(st + 2 * kTileBytes + kScaleRegion + wn * 1024 + so);
#pragma unroll
  for (int i = 0; i < TM; i++) f.a[i] = load_frag(st, wm * WM + i * 32, lane);
#pragma unroll
  for (int j = 0; j < TN; j++) f.b[j] = load_frag(st + kTileBytes, wn * WN + j * 32, lane);
}

__device__ __forceinline__ int u4_get(const uint4& v, int i) {
  return (int)(i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w);
}

__device__ __forceinline__ void mfma_step(v16f (&acc)[TM][TN], const Frags& f) {
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++) acc[i][j] = mfma_scaled(f.a[i], f.b[j], acc[i][j], u4_get(f.sa, i), u4_get(f.sb, j));
}

// s_waitcnt with vmcnt(n) only (expcnt / lgkmcnt left at their maximum), gfx9 encoding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (0x7 << 4)); }

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

// group bookkeeping of the grouped modes, placed in the last stage (used
// only before that stage's first load is issued)
struct GroupScratch {
  GroupTable gt;
  int32_t scan_tmp[kThreads];
  int32_t order[kMaxGroups];
};
static_assert(sizeof(GroupScratch) <= kStageBytes, "group scratch must fit in one stage");

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_mxfp8_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ sB, float* __restrict__ C, int64_t M, int64_t N, int64_t K,
    int64_t ldc, const int32_t* __restrict__ group_end, int32_t G, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage3[kStageBytes];
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
    GroupScratch& gs = *reinterpret_cast<GroupScratch*>(stage3);
    GroupTable& gt = gs.gt;
    int32_t* const scan_tmp = gs.scan_tmp;
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
      sb_base = sB + (int64_t)g * ((N + 31) / 32 * 32) * (K / 32);  // expert scale arrays hold ceil32(N) rows
    } else {
      build_group_table<kThreads>(group_end, G, (int64_t)1 << 40, 32, gt, scan_tmp);
      // largest groups first (their tiles carry the longest K loops)
      int32_t* const order = gs.order;
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
  if constexpr (MODE != kDense) __syncthreads();  // group scratch read; stage 3 may now be loaded

  const Operand opa{A + m0 * lda, sA, m0, lda, rows_a};
  const Operand opb{b_base + n0 * lda, sb_base, n0, lda, rows_b};

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.f;

  const int nk = (int)((k_end - k_begin + BK - 1) / BK);
  const int last = nk - 1;
  const int tail_chunks = nk > 0 ? (int)((k_end - k_begin) - (int64_t)last * BK) / 16 : 4;  // 2 or 4
  uint8_t* const stages[4] = {stage0, stage1, stage2, stage3};

  // issue step s into stage `slot`; steps past the last re-load the last step
  // (every step issues the same loads, so the vmcnt arithmetic is fixed)
  auto issue = [&](int slot, int s) {
    const int sc = min(s, last);
    const int64_t k = k_begin + (int64_t)sc * BK;
    const int vc = sc == last ? tail_chunks : 4;
    uint8_t* st = stages[slot];
    issue_codes(opa, st, wave, lane, k, vc);
    issue_codes(opb, st + kTileBytes, wave, lane, k, vc);
    issue_scales(opa, st + 2 * kTileBytes, wave, lane, k, vc / 2);
    issue_scales(opb, st + 2 * kTileBytes + kScaleRegion, wave, lane, k, vc / 2);
  };
  // once step s has landed in `slot` (this wave's part): zero the chunks past
  // the end of K, or the whole step if it only pads the loop to a multiple of four
  auto fix = [&](int slot, int s) {
    const int vc = s > last ? 0 : s == last ? tail_chunks : 4;
    if (vc < 4) {
      zero_codes(stages[slot], wave, lane, vc);
      zero_codes(stages[slot] + kTileBytes, wave, lane, vc);
    }
  };

  if (nk > 0) {
    const int nsteps = (nk + 3) & ~3;
    issue(0, 0);
    issue(1, 1);
    issue(2, 2);
    issue(3, 3);
    wait_vmcnt<3 * kVmemPerStep>();  // step 0 landed
    fix(0, 0);
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    Frags f0, f1;
    read_frags(stage0, wm, wn, lane, f0);
    wait_lgkmcnt0();
    // step k: publish stage k+1, refill stage k with step k+4, read step k+1's
    // fragments while the MFMAs of step k run
    auto step = [&](int cur, int s, Frags& fc, Frags& fn) {
      wait_vmcnt<2 * kVmemPerStep>();  // this wave's loads of step s+1 landed
      fix((cur + 1) & 3, s + 1);
      wait_lgkmcnt0();
      __builtin_amdgcn_s_barrier();  // step s+1 complete; every wave done with stage `cur`
      __builtin_amdgcn_sched_barrier(0);
      // LDS reads first (the scheduler would otherwise sink them under the
      // MFMAs, leaving their latency exposed at the end of the step)
      read_frags(stages[(cur + 1) & 3], wm, wn, lane, fn);
      __builtin_amdgcn_sched_barrier(0);
      issue(cur, s + 4);
      mfma_step(acc, fc);
      wait_lgkmcnt0();
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) asm volatile("" : "+a"(acc[i][j]));
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int kt = 0; kt < nsteps; kt += 4) {
      step(0, kt + 0, f0, f1);
      step(1, kt + 1, f1, f0);
      step(2, kt + 2, f0, f1);
      step(3, kt + 3, f1, f0);
    }
    wait_vmcnt<0>();  // the loads still in flight land before the LDS goes away
  }

  // ---- epilogue: fp32 stores (32 consecutive floats per half-wave), rows/cols
  // past the tile's valid range skipped
  const int64_t ldo = MODE == kRaggedK ? N : ldc;
#pragma unroll
  for (int i = 0; i < TM; i++) {
#pragma unroll
    for (int j = 0; j < TN; j++) {
      const int col = wn * WN + j * 32 + (lane & 31);
      if (col >= rows_b) continue;
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int row = wm * WM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
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
