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
// step through double-buffered LDS (one v_mfma_scale_f32_16x16x128_f8f6f4 per
// 16 x 16 block and step).  Operand layout of that instruction for FP8 (found
// by probing): lane l holds row l%16; its bytes 0-15 are K = 16g..16g+15 and
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

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 256, BK = 128;  // BK in codes (bytes) per step
constexpr int WM = 128, WN = 128;             // wave tile
constexpr int TM = WM / 16, TN = WN / 16;     // MFMA blocks per wave
constexpr int kTileBytes = BM * BK;           // one operand tile per stage (32 KB)
constexpr int kScaleBytes = 4 * BM;           // scale bytes of one operand tile per stage

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

// One operand of one workgroup tile: rows [0, rows_valid) of a matrix whose row
// r starts at base + r*ld (codes) and sbase + r*(ld/32) (scales); K range
// [k_begin, k_end), k_end - k_begin a multiple of 32.
struct Operand {
  const uint8_t* base;
  const uint8_t* sbase;
  int64_t ld;
  int rows_valid;
};

struct Prefetch {
  uint4 chunk[8];
  uint32_t sc;  // 4 scale bytes of this thread's row
};

// thread t loads chunks t + 256*i: row (t >> 3) + 32*i, chunk t & 7; and the 4
// scale bytes of row t.
__device__ __forceinline__ void load_tile(const Operand& op, int64_t k, int64_t k_end, Prefetch& p) {
  const int t = threadIdx.x;
  const int c = t & 7;
  const bool kc_ok = k + (c + 1) * 16 <= k_end;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int r = (t >> 3) + 32 * i;
    if (kc_ok && r < op.rows_valid)
      p.chunk[i] = *reinterpret_cast<const uint4*>(op.base + r * op.ld + k + c * 16);
    else
      p.chunk[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  uint32_t sc = 0;
  const int64_t kb = k / 32;
  const int64_t nsb = op.ld / 32;
#pragma unroll
  for (int g = 0; g < 4; g++) {
    uint32_t b = 127u;  // any finite scale for padding (its codes are zero)
    if (t < op.rows_valid && k + (g + 1) * 32 <= k_end) b = op.sbase[t * nsb + kb + g];
    sc |= b << (8 * g);
  }
  p.sc = sc;
}

__device__ __forceinline__ void store_tile(uint8_t* lds_codes, uint8_t* lds_scales, const Prefetch& p) {
  const int t = threadIdx.x;
  const int c = t & 7;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int r = (t >> 3) + 32 * i;
    *reinterpret_cast<uint4*>(lds_codes + swz(r, c)) = p.chunk[i];
  }
#pragma unroll
  for (int g = 0; g < 4; g++) lds_scales[sidx(t, g)] = (uint8_t)(p.sc >> (8 * g));
}

// fragment of MFMA row block starting at tile row r0 for this lane
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

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_mxfp8_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ sB, float* __restrict__ C, int64_t M, int64_t N, int64_t K,
    int64_t ldc, const int32_t* __restrict__ group_end, int32_t G, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (2 * kTileBytes + 2 * kScaleBytes)];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- which output tile, and the operands behind it
  int64_t m0, n0 = 0, k_begin = 0, k_end = K;
  int rows_a, rows_b;
  const uint8_t *a_base = A, *sa_base = sA, *b_base = B, *sb_base = sB;
  float* c_base = C;
  int64_t lda = K;
  if constexpr (MODE == kDense) {
    const int mt = blockIdx.x % tiles_m;
    const int nt = blockIdx.x / tiles_m;
    m0 = (int64_t)mt * BM;
    n0 = (int64_t)nt * BN;
    rows_a = (int)min<int64_t>(BM, M - m0);
  } else {
    __shared__ GroupTable gt;
    __shared__ int32_t scan_tmp[kThreads];
    if constexpr (MODE == kRaggedM) {
      build_group_table<kThreads>(group_end, G, M, BM, gt, scan_tmp);
      const int mt = blockIdx.x % tiles_m;  // tiles_m = upper bound of m-tiles over all groups
      const int nt = blockIdx.x / tiles_m;
      if (mt >= gt.bstart[G]) return;  // uniform
      const int g = find_group(gt, G, mt);
      const int local = mt - gt.bstart[g];
      m0 = (int64_t)gt.start[g] + (int64_t)local * BM;
      n0 = (int64_t)nt * BN;
      rows_a = min(BM, gt.size[g] - local * BM);
      b_base = B + (int64_t)g * N * K;
      sb_base = sB + (int64_t)g * N * (K / 32);
    } else {
      build_group_table<kThreads>(group_end, G, (int64_t)1 << 40, 32, gt, scan_tmp);
      const int per_g = tiles_m * tiles_n;
      const int g = blockIdx.x / per_g;
      const int rem = blockIdx.x - g * per_g;
      const int mt = rem % tiles_m;
      const int nt = rem / tiles_m;
      m0 = (int64_t)mt * BM;
      n0 = (int64_t)nt * BN;
      rows_a = (int)min<int64_t>(BM, M - m0);
      k_begin = (int64_t)gt.bstart[g] * 32;
      k_end = min<int64_t>((int64_t)gt.bstart[g + 1] * 32, K);  // never past the row length
      if (k_end < k_begin) k_end = k_begin;
      c_base = C + (int64_t)g * M * N;
    }
  }
  rows_b = (int)min<int64_t>(BN, N - n0);

  Operand opa{a_base + m0 * lda, sa_base + m0 * (lda / 32), lda, rows_a};
  Operand opb{b_base + n0 * lda, sb_base + n0 * (lda / 32), lda, rows_b};

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nk = (int)((k_end - k_begin + BK - 1) / BK);
  auto stage_codes_a = [&](int s) { return lds + s * (2 * kTileBytes + 2 * kScaleBytes); };
  auto stage_codes_b = [&](int s) { return stage_codes_a(s) + kTileBytes; };
  auto stage_scales_a = [&](int s) { return stage_codes_a(s) + 2 * kTileBytes; };
  auto stage_scales_b = [&](int s) { return stage_scales_a(s) + kScaleBytes; };

  Prefetch pa, pb;
  if (nk > 0) {
    load_tile(opa, k_begin, k_end, pa);
    load_tile(opb, k_begin, k_end, pb);
    store_tile(stage_codes_a(0), stage_scales_a(0), pa);
    store_tile(stage_codes_b(0), stage_scales_b(0), pb);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; kt++) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int64_t k = k_begin + (int64_t)(kt + 1) * BK;
      load_tile(opa, k, k_end, pa);
      load_tile(opb, k, k_end, pb);
    }
    const uint8_t* ca = stage_codes_a(cur);
    const uint8_t* cb = stage_codes_b(cur);
    const uint2 sa = *reinterpret_cast<const uint2*>(stage_scales_a(cur) + sidx(wm * 128 + (lane & 15), lane >> 4));
    const uint2 sb = *reinterpret_cast<const uint2*>(stage_scales_b(cur) + sidx(wn * 128 + (lane & 15), lane >> 4));
    v8i fa[TM];
#pragma unroll
    for (int i = 0; i < TM; i++) fa[i] = load_frag(ca, wm * WM + i * 16, lane);
#pragma unroll
    for (int j = 0; j < TN; j++) {
      const v8i fb = load_frag(cb, wn * WN + j * 16, lane);
      const int sbj = (int)(j < 4 ? sb.x : sb.y);
#pragma unroll
      for (int i = 0; i < TM; i++) {
        const int sai = (int)(i < 4 ? sa.x : sa.y);
        acc[i][j] = mfma_scaled(i & 3, j & 3, fa[i], fb, acc[i][j], sai, sbj);
      }
    }
    if (more) {
      store_tile(stage_codes_a(cur ^ 1), stage_scales_a(cur ^ 1), pa);
      store_tile(stage_codes_b(cur ^ 1), stage_scales_b(cur ^ 1), pb);
    }
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
