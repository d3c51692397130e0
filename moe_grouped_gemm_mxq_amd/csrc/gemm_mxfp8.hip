// Block-scaled MX GEMMs for gfx950: C[m][n] = sum_k deq(A)[m][k] deq(B)[n][k]
// with E4M3 codes (or E2M1 codes, two per byte), one E8M0 scale per 32 values
// along K, fp32 accumulation and fp32 output (the FP8 linear and expert GEMMs
// of the torchtitan-npu guide, "线性层低精度" and "MoE 专家层低精度"; the
// optional MXFP4 of routed experts in the torchao_npu RFC's recipes).
//
// One main loop serves three problem shapes:
//   dense    -- one A [M][K], one B [N][K];
//   ragged M -- rows of A split into expert groups, group g multiplies B[g]
//               (expert forward and input gradient);
//   ragged K -- the reduction axis split into groups, one output per group
//               (expert weight gradient over each group's padded tokens).
//
// Tiling: 256 x 256 output tile per workgroup of 8 waves (2 x 4, two per
// SIMD), each wave a 128 x 64 sub-tile of 4 x 2 MFMA blocks of 32 x 32; K
// advances 64 codes per step (one v_mfma_scale_f32_32x32x64_f8f6f4 per block
// and step).  Two waves per SIMD let one wave's MFMAs run while the other
// waits on its LDS reads, and keep enough LDS requests in flight for the LDS
// to serve both the fragment reads and the direct loads writing into it.
//
// Element formats (Fmt): an E4M3 or E2M1 stage holds 128 code bytes per tile
// row (128 or 256 elements, 2 or 4 MFMA steps).
//
// Pipeline: codes (global_load_lds_dwordx4) and scale dwords
// (global_load_lds_dword) go from global memory straight into LDS.  LDS holds
// two stages (with 128 code bytes per tile row every 16-byte lane load belongs
// to a fully used 128-byte line); the loads of a stage are issued one stage
// before its first use.  One s_barrier per stage (raw, with explicit vmcnt /
// lgkmcnt waits: a full __syncthreads would drain the loads in flight)
// publishes the next stage and retires the current one.  The two stages are
// separate LDS arrays and the loop is unrolled over both, so the compiler can
// tell the stage being read from the stage being filled and never waits on
// the latter.
//
// Exact groups for short reductions: the FP8 MFMA adds each group of 8
// consecutive-K products keeping only about 13 bits below the group's
// largest product, an error that long reductions average out but short ones
// do not.  A reduction of at most kIlvMaxK elements (dense and ragged M: K;
// ragged K: an expert's token count) therefore runs "interleaved": each MFMA
// step takes 8 real K values and places value j alone in product group j (the
// other 7 positions of the group hold zero codes), so every group sum is one
// exact product and only the fp32 accumulation rounds.  It costs 8 MFMA steps
// where the plain loop takes one.  E2M1 products are summed exactly by the
// hardware and always take the plain loop.
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

constexpr int kThreads = 512;
constexpr int BM = 256, BN = 256, BK = 64;   // BK: codes (bytes) per MFMA step
constexpr int WM = 128, WN = 64;              // wave tile
constexpr int TM = WM / 32, TN = WN / 32;     // MFMA blocks per wave

// Layout of one LDS stage per operand kind: 128 code bytes per tile row, so
// every load reads whole 128-byte lines.  E4M3 codes take a byte, E2M1 codes
// (two per byte, element 2j in the low nibble) half of one.
//   kE4M3:  128 elements (2 MFMA steps) per tile row, a 66 KB stage;
//   kE2M1:  256 elements (4 steps) with twice the scales, a 68 KB stage that
//           carries twice the MFMA work for the same code bytes.
enum Kind { kE4M3 = 0, kE2M1 = 1 };
template <int KIND>
struct Fmt {
  static constexpr bool kFp4 = KIND != kE4M3;
  static constexpr int kSteps = kFp4 ? 4 : 2;                            // MFMA steps per stage
  static constexpr int kStageElems = kSteps * BK;                        // elements per tile row and stage
  static constexpr int kRowBytes = 128;                                  // code bytes per tile row
  static constexpr int kChunks = kRowBytes / 16;                         // 16-byte chunks per row
  static constexpr int kElemsPerChunk = kStageElems / kChunks;           // 16 / 32
  static constexpr int kTileBytes = BM * kRowBytes;                      // per operand (32 KB)
  static constexpr int kBlocks = 2 * kSteps;                             // K-blocks per stage
  static constexpr int kScaleRegion = 2 * kBlocks * 32 * 4;              // one dword per (half, block, row % 32)
  static constexpr int kStageBytes = 2 * kTileBytes + 2 * kScaleRegion;  // A, B codes, A, B scales
  static constexpr int kLoads = kTileBytes / (kThreads / 64) / 1024;     // dwordx4 loads per wave and operand
  static constexpr int kLanesPerRow = kRowBytes / 16;                    // lanes of one load on one row
  static constexpr int kScaleLoads = kScaleRegion / 256 / 4;             // dword loads per wave (4 waves an operand)
};
constexpr int kXcds = 8;                      // XCDs per MI355X; workgroups are dealt round robin
constexpr int kIlvSteps = 16;                 // interleaved steps per E4M3 stage (8 K values each)
constexpr int kGroupM = 8;                    // m-tiles per raster group

enum Mode { kDense = 0, kRaggedM = 1, kRaggedK = 2 };

// format codes of the f8f6f4 MFMA operands: 0 = E4M3, 4 = E2M1; op_sel
// picks byte I of the A scale dword and byte J of the B one
template <int KIND, int I, int J>
__device__ __forceinline__ v16f mfma_scaled(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  constexpr int f = KIND == kE4M3 ? 0 : 4;
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, f, f, I, sa, J, sb);
}

// LDS position of 16-byte chunk c of tile row r (8 chunks, 128 bytes per
// row).  A fragment read has its lanes on consecutive rows at one chunk; the
// XOR swizzle f(r) = (r & 7) ^ ((r >> 3) & 1) makes any 8 aligned consecutive
// rows land on 8 distinct 16-byte bank groups of a 128-byte bank row (32
// banks) and any 16 on 16 distinct groups of a 256-byte one (64 banks), so
// the read is conflict-free.
__device__ __forceinline__ int swz(int r, int c) {
  return r * 128 + ((c ^ ((r & 7) ^ ((r >> 3) & 1))) << 4);
}

// One operand of one workgroup tile: tile rows [0, rows_valid), which are rows
// row0 .. row0 + rows_valid - 1 of a matrix with codes at base + (r - row0)*ld
// and scales at sbase + scale_offset(r, block, nblk) (the layout the
// quantisers write).  row0 is a multiple of 128, so the tile's two halves are
// whole 128-row groups of the scale array.  Code rows at or past rows_valid
// are read from row rows_valid-1, and a half with no valid row reads the
// scales of the first half (their results are never stored).
struct Operand {
  const uint8_t* base;   // codes of tile row 0
  const uint8_t* sbase;  // scale array of the whole matrix
  int64_t row0;
  int64_t ld;    // code row pitch (bytes)
  int64_t nblk;  // scale blocks per row (K / 32)
  int rows_valid;
};

// Per-lane load addresses of one operand, computed once per tile: the loads
// of a stage then only add the stage's K offset (uniform) to a per-lane
// 32-bit offset, so the K loop spends almost no VALU on addressing.
//
// Codes (32 KB per operand and stage): wave w issues 4 dwordx4 loads; load j
// fills LDS bytes [q * 1024, +1024), q = 4w + j, = tile rows 8q .. 8q+7, lane
// l writing 16-byte slot l%8 of row 8q + l/8, which holds global chunk
// c = slot ^ f(row) = (l%8) ^ (l/8) ^ (j%2).  One load thus reads eight whole
// 128-byte lines.  Chunks at or past the valid ones (the tail of K) are
// fetched from the last valid chunk (always in bounds) and zeroed by
// zero_codes() once they have landed.
//
// Scales: dword d = (h * NB + b) * 32 + r of one operand and stage (NB
// K-blocks per stage) holds the scales of tile rows h*128 + i*32 + r, i =
// 0..3 (byte i), over K-block b: exactly the dword of the global layout for
// that 128-row group, block and r, so one 64-lane dword load moves two
// blocks of a half (256 consecutive bytes) into place.  The waves of one
// operand (0-3 for A, 4-7 for B) share its NB loads.  A lane reads the dword
// of its row r and K-block of the step, and the MFMA's op_sel picks the row
// block.  A K-block past the end of K re-reads the last valid one (its codes
// are zeroed).
struct OperandAddr {
  const uint8_t* cbase;  // codes of tile row 0
  const uint8_t* sbase;  // scale bytes of the tile's first 128-row group, block 0
  uint32_t coff[4];      // per load: row offset of the lane's row
  uint32_t sgroup;       // scale bytes per 128-row group (128 * blocks per row)
  int halves;            // 128-row halves of the tile with a valid row (1 or 2)
};

// Load j of wave w covers tile rows 8q .. 8q+7 (q = 4w + j), 8 lanes a row.
// Lane l fills slot l % 8 of its row, which holds chunk slot ^ f(row).
__device__ __forceinline__ int dma_chunk(int j, int lane) {
  return (lane & 7) ^ (lane >> 3) ^ (j & 1);
}

// per-lane code row offsets and the tile's scale base of one operand
template <int KIND>
__device__ __forceinline__ OperandAddr make_addr(const Operand& op, int wave, int lane) {
  using F = Fmt<KIND>;
  OperandAddr ad;
  const int64_t nblk = op.nblk;
  ad.cbase = op.base;
  ad.sbase = op.sbase + (op.row0 >> 7) * nblk * 128;
  ad.sgroup = (uint32_t)(nblk * 128);
  ad.halves = op.rows_valid > 128 ? 2 : 1;
#pragma unroll
  for (int j = 0; j < F::kLoads; j++) {
    const int row = min((wave * F::kLoads + j) * (64 / F::kLanesPerRow) + lane / F::kLanesPerRow, op.rows_valid - 1);
    ad.coff[j] = (uint32_t)((int64_t)row * op.ld);
  }
  return ad;
}

// kb: byte offset of the stage along the row
template <int KIND>
__device__ __forceinline__ void issue_codes(const OperandAddr& ad, uint8_t* tile, int wave, int lane, int64_t kb,
                                            int valid_chunks) {
  using F = Fmt<KIND>;
  const uint8_t* base = ad.cbase + kb;
  const uint32_t c0 = (uint32_t)min(dma_chunk(0, lane), valid_chunks - 1) * 16;
  const uint32_t c1 = (uint32_t)min(dma_chunk(1, lane), valid_chunks - 1) * 16;
#pragma unroll
  for (int j = 0; j < F::kLoads; j++)
    __builtin_amdgcn_global_load_lds(base + (ad.coff[j] + ((j & 1) ? c1 : c0)),
                                     (lds_ptr)(tile + (wave * F::kLoads + j) * 1024), 16, 0, 0);
}

// Zero the code chunks at or past valid_chunks (0 zeroes the whole stage) in
// the bytes this wave's own loads wrote; called after those loads landed.
template <int KIND>
__device__ __forceinline__ void zero_codes(uint8_t* tile, int wave, int lane, int valid_chunks) {
  using F = Fmt<KIND>;
#pragma unroll
  for (int j = 0; j < F::kLoads; j++)
    if (dma_chunk(j, lane) >= valid_chunks)
      *reinterpret_cast<uint4*>(tile + (wave * F::kLoads + j) * 1024 + lane * 16) = make_uint4(0u, 0u, 0u, 0u);
}

// the same for the chunks before `head_chunks` (ragged K: tokens of earlier
// experts at the start of an expert's first stage)
template <int KIND>
__device__ __forceinline__ void zero_head_codes(uint8_t* tile, int wave, int lane, int head_chunks) {
  using F = Fmt<KIND>;
#pragma unroll
  for (int j = 0; j < F::kLoads; j++)
    if (dma_chunk(j, lane) < head_chunks)
      *reinterpret_cast<uint4*>(tile + (wave * F::kLoads + j) * 1024 + lane * 16) = make_uint4(0u, 0u, 0u, 0u);
}

// this wave's share of one operand's scale loads for the stage at element k
// (waves 0-3 load A's, 4-7 B's; unit u covers half u / (NB/2), blocks
// 2 (u % (NB/2)) and one more)
template <int KIND>
__device__ __forceinline__ void issue_scales(const OperandAddr& ad, uint8_t* region, int wave, int lane, int64_t k,
                                             int valid_blocks) {
  using F = Fmt<KIND>;
  constexpr int UPH = F::kBlocks / 2;  // loads per half
#pragma unroll
  for (int j = 0; j < F::kScaleLoads; j++) {
    const int u = (wave & 3) * F::kScaleLoads + j;  // (uniform)
    const int h = u / UPH, bp = u % UPH;
    const int blk = min(2 * bp + (lane >> 5), valid_blocks - 1);
    const int hs = h < ad.halves ? h : 0;  // a half without valid rows reads the first half's scales
    __builtin_amdgcn_global_load_lds(ad.sbase + (hs * ad.sgroup + ((k >> 5) + blk) * 128 + (lane & 31) * 4),
                                     (lds_ptr)(region + (h * F::kBlocks + 2 * bp) * 128), 4, 0, 0);
  }
}

// MFMA operands of one step for one wave: 4 row blocks of A, 2 of B (32 bytes
// per lane each), and the lane's 4 + 2 block scales.
struct Frags {
  v8i a[TM], b[TN];
  uint32_t sa, sb;  // byte i: row block i of A / B column block (bytes 0, 1 used)
};

// fragment of the MFMA row block starting at tile row r0, step s of the
// stage.  E4M3: bytes 0-15 of lane l are K 16g .. 16g+15 of the step, bytes
// 16-31 K 32+16g .. (g = l/32).  E2M1: bytes 0-15 are the 32 nibbles of K
// 32g .. 32g+31, the upper half is not read by the MFMA.
template <int KIND>
__device__ __forceinline__ v8i load_frag(const uint8_t* codes, int r0, int s, int lane) {
  const int r = r0 + (lane & 31);
  const int g = lane >> 5;
  v8i f;
  if constexpr (KIND != kE4M3) {
    const uint4 lo = *reinterpret_cast<const uint4*>(codes + swz(r, 2 * s + g));
    f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
    f[4] = 0; f[5] = 0; f[6] = 0; f[7] = 0;
  } else {
    const uint4 lo = *reinterpret_cast<const uint4*>(codes + swz(r, 4 * s + g));
    const uint4 hi = *reinterpret_cast<const uint4*>(codes + swz(r, 4 * s + 2 + g));
    f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
    f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  }
  return f;
}

// A lane's scale registers for step s: A's dword of its row r = lane % 32 in
// the wave's half wm, whose byte i scales row block i; B's dword of half wn/2,
// whose bytes 2*(wn%2) and 2*(wn%2)+1 scale the wave's two column blocks
// (B rows wn*64 .. wn*64+63), shifted down to bytes 0 and 1 for op_sel.
template <int KIND>
__device__ __forceinline__ void read_frags(const uint8_t* st, int s, int wm, int wn, int lane, Frags& f) {
  using F = Fmt<KIND>;
  constexpr int kTileBytes = F::kTileBytes, kScaleRegion = F::kScaleRegion;
  const int so = (2 * s * 32 + lane) * 4;  // block 2s + lane/32, row lane % 32
  f.sa = *reinterpret_cast<const uint32_t*>(st + 2 * kTileBytes + wm * (F::kBlocks * 128) + so);
  // B: the wave's column blocks are row blocks 2 (wn % 2) and 2 (wn % 2) + 1 of half wn / 2
  f.sb = *reinterpret_cast<const uint32_t*>(st + 2 * kTileBytes + kScaleRegion + (wn >> 1) * (F::kBlocks * 128) +
                                            so) >> (16 * (wn & 1));
#pragma unroll
  for (int i = 0; i < TM; i++) f.a[i] = load_frag<KIND>(st, wm * WM + i * 32, s, lane);
#pragma unroll
  for (int j = 0; j < TN; j++) f.b[j] = load_frag<KIND>(st + kTileBytes, wn * WN + j * 32, s, lane);
}

// Interleaved fragment of the MFMA row block at tile row r0 for interleaved
// step s (K values 8s .. 8s+7 of the E4M3 stage): product group j of the
// MFMA's 64 K positions (bytes 0-7 / 8-15 of lane half j/2 for j < 4, bytes
// 16-23 / 24-31 of lane half (j-4)/2 for j >= 4) holds K value 8s + j in its
// first byte and zero codes in the other seven.  Lane half g thus needs values
// 8s + {2g, 2g+1, 4+2g, 5+2g}: bytes of one 8-byte read, placed in the low
// bytes of dwords 0, 2, 4, 6.
__device__ __forceinline__ v8i load_frag_ilv(const uint8_t* codes, int r0, int s, int lane) {
  const int r = r0 + (lane & 31);
  const int sh = 16 * (lane >> 5);
  const int k0 = 8 * s;
  const uint2 v = *reinterpret_cast<const uint2*>(codes + swz(r, k0 >> 4) + (k0 & 15));
  v8i f;
  f[0] = (int)((v.x >> sh) & 0xFFu);
  f[1] = 0;
  f[2] = (int)((v.x >> (sh + 8)) & 0xFFu);
  f[3] = 0;
  f[4] = (int)((v.y >> sh) & 0xFFu);
  f[5] = 0;
  f[6] = (int)((v.y >> (sh + 8)) & 0xFFu);
  f[7] = 0;
  return f;
}

// Fragments and scales of interleaved step s: all eight K values come from
// K-block s / 4 of the stage, so both lane halves pass that block's scales.
__device__ __forceinline__ void read_frags_ilv(const uint8_t* st, int s, int wm, int wn, int lane, Frags& f) {
  using F = Fmt<kE4M3>;
  constexpr int kTileBytes = F::kTileBytes, kScaleRegion = F::kScaleRegion;
  const int so = ((s >> 2) * 32 + (lane & 31)) * 4;
  f.sa = *reinterpret_cast<const uint32_t*>(st + 2 * kTileBytes + wm * (F::kBlocks * 128) + so);
  f.sb = *reinterpret_cast<const uint32_t*>(st + 2 * kTileBytes + kScaleRegion + (wn >> 1) * (F::kBlocks * 128) +
                                            so) >> (16 * (wn & 1));
#pragma unroll
  for (int i = 0; i < TM; i++) f.a[i] = load_frag_ilv(st, wm * WM + i * 32, s, lane);
#pragma unroll
  for (int j = 0; j < TN; j++) f.b[j] = load_frag_ilv(st + kTileBytes, wn * WN + j * 32, s, lane);
}

template <int KIND, bool PRIO = false>
__device__ __forceinline__ void mfma_step(v16f (&acc)[TM][TN], const Frags& f) {
  static_assert(TM == 4 && TN == 2, "the op_sel byte of each block is spelled out");
  const int sa = (int)f.sa, sb = (int)f.sb;
  // PRIO (E2M1 ragged K): the wave issuing its MFMAs takes precedence over the
  // other wave of the SIMD (1.3% faster there; E4M3 kernels measured slower)
  if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
  acc[0][0] = mfma_scaled<KIND, 0, 0>(f.a[0], f.b[0], acc[0][0], sa, sb);
  acc[0][1] = mfma_scaled<KIND, 0, 1>(f.a[0], f.b[1], acc[0][1], sa, sb);
  acc[1][0] = mfma_scaled<KIND, 1, 0>(f.a[1], f.b[0], acc[1][0], sa, sb);
  acc[1][1] = mfma_scaled<KIND, 1, 1>(f.a[1], f.b[1], acc[1][1], sa, sb);
  acc[2][0] = mfma_scaled<KIND, 2, 0>(f.a[2], f.b[0], acc[2][0], sa, sb);
  acc[2][1] = mfma_scaled<KIND, 2, 1>(f.a[2], f.b[1], acc[2][1], sa, sb);
  acc[3][0] = mfma_scaled<KIND, 3, 0>(f.a[3], f.b[0], acc[3][0], sa, sb);
  acc[3][1] = mfma_scaled<KIND, 3, 1>(f.a[3], f.b[1], acc[3][1], sa, sb);
  if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
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

// group bookkeeping of the grouped modes, placed in stage 1 (used only
// before the first load is issued)
struct GroupScratch {
  GroupTable gt;
  int64_t scan_tmp[kThreads];
  int32_t order[kMaxGroups];
};
static_assert(sizeof(GroupScratch) <= Fmt<kE4M3>::kStageBytes && sizeof(GroupScratch) <= Fmt<kE2M1>::kStageBytes,
              "group scratch must fit in one stage");

// One output tile: where its operands and output live and which K range it
// reduces over.  All fields are workgroup-uniform.
struct Tile {
  int64_t m0, n0;          // first output row / column (multiples of 128)
  int rows_a, rows_b;      // output rows / columns of the tile end here (<= 256)
  int row_lo;              // ... and its output rows start here (ragged M: group start - m0)
  int rows_load;           // A rows of the tile that exist in the matrix (>= rows_a)
  int64_t k_begin, klen;   // reduction range; klen == 0: an empty expert (zeros)
  const uint8_t* b_base;   // B codes of the tile's expert (ragged M) or B
  const uint8_t* sb_base;  // B scales of the tile's expert
  float* c_base;           // output matrix of the tile (ragged K: the expert's)
  int nst;                 // K stages, rounded up to even (0 if klen == 0)
  int last, tail_chunks;   // last real stage and its valid 16-byte chunks per row
  int head_chunks;         // ragged K: 16-byte chunks of real stage 0 before the expert's first token
  int lag;                 // 1: the tile walks K one stage behind (real stages last, 0, 1, .., last-1)
  int rot;                 // E2M1 ragged K: the walk starts at real stage rot and wraps (rot = XCD eighths)
};

// fp32 stores of one tile's accumulators (32 consecutive floats per half
// wave); rows / columns past the tile's valid range are skipped.  The row
// pointer advances one row at a time (a 64-bit add), so the stores need no
// per-element address arithmetic and few registers.  The stores are
// non-temporal: the output is never read back by the GEMM, and streaming it
// past the caches keeps the operand panels resident in the memory-side cache
// (and leaves no dirty output lines for the next kernel to write back).
__device__ __forceinline__ void store_tile(const v16f (&acc)[TM][TN], const Tile& tl, int64_t ldo, int wm,
                                           int wn, int lane) {
  const int col0 = wn * WN + (lane & 31);
  const int row0 = wm * WM + 4 * (lane >> 5);
  float* p = tl.c_base + (tl.m0 + row0) * ldo + tl.n0 + col0;
  const bool c_ok0 = col0 < tl.rows_b, c_ok1 = col0 + 32 < tl.rows_b;
#pragma unroll
  for (int i = 0; i < TM; i++) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int row = row0 + i * 32 + 8 * q + r;
        if (row >= tl.row_lo && row < tl.rows_a) {
          if (c_ok0) __builtin_nontemporal_store(acc[i][0][q * 4 + r], p);
          if (c_ok1) __builtin_nontemporal_store(acc[i][1][q * 4 + r], p + 32);
        }
        // next row of this lane: +1 within a run of 4, else +5 (27 -> 32 too)
        p += (r < 3 ? 1 : 5) * ldo;
        asm volatile("" : "+v"(p));
      }
    }
  }
}

// The grouped modes run persistent: one workgroup per CU walks its tiles (see
// tile_id), and a tile's last stage loads the next tile's first, so the
// pipeline does not drain between tiles and the output stores of one tile
// drain while the next one computes.  Dense is launched with one workgroup
// per tile (measured faster).
//
// ILV: interleaved steps (exact product groups, E4M3 only).  Ragged K splits
// the experts between two launches of the same walk: the plain kernel takes
// the experts with more than kIlvMaxK tokens, the interleaved one the rest
// (empty experts included).
template <int MODE, int KIND, bool ILV>
__global__ __launch_bounds__(kThreads, 1) void gemm_mx_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ sB, float* __restrict__ C, int64_t M, int64_t N, int64_t K,
    int64_t ldc, const int32_t* __restrict__ group_end, int32_t G, int tiles_m, int tiles_n) {
  using F = Fmt<KIND>;
  constexpr bool FP4 = F::kFp4;
  static_assert(!ILV || KIND == kE4M3, "E2M1 products need no interleaving");
  constexpr int kTileBytes = F::kTileBytes, kScaleRegion = F::kScaleRegion, BKS = F::kStageElems;
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[F::kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[F::kStageBytes];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int bid = blockIdx.x;
  const int64_t lda = FP4 ? K / 2 : K;  // code bytes per row of A and B
  const int64_t ldo = MODE == kRaggedK ? N : ldc;

  // ---- the tile list
  int n_tiles;
  const GroupTable* gtp = nullptr;  // ragged M: group starts, sizes, m-tile starts
  const int32_t* kbp = nullptr;     // ragged K: padded 32-token block starts per group (G + 1)
  const int32_t* orderp = nullptr;  // ragged K: groups, largest first
  int first_g = 0;                  // ragged K: position in `order` of this launch's first expert
  if constexpr (MODE == kDense) {
    n_tiles = tiles_m * tiles_n;
  } else if constexpr (MODE == kRaggedM) {
    __shared__ GroupTable gt;  // read by every tile of the workgroup
    build_group_table<kThreads>(group_end, G, M, BM, gt, reinterpret_cast<GroupScratch*>(stage1)->scan_tmp, 128);
    // real m-tiles x n-tiles; a valid table has at most tiles_m + 2G m-tiles
    // (the launcher's bound), a malformed one is cut there
    n_tiles = min(gt.bstart[G], tiles_m + 2 * G) * tiles_n;
    gtp = &gt;
  } else {
    // the table is built in stage 1 (free until the first load); the tile
    // walk keeps only the block starts and the order
    __shared__ int32_t kb[kMaxGroups + 1];
    __shared__ int32_t order[kMaxGroups];
    GroupScratch& gs = *reinterpret_cast<GroupScratch*>(stage1);
    GroupTable& gt = gs.gt;
    // group ends clamped into [0, K]: a valid array (ends <= T <= K) is unchanged
    build_group_table<kThreads>(group_end, G, K, 32, gt, gs.scan_tmp);
    for (int g = t; g <= G; g += kThreads) kb[g] = gt.bstart[g];
    // largest groups first (their tiles carry the longest K loops)
    for (int g = t; g < G; g += kThreads) {
      const int32_t sz = gt.size[g];
      int rank = 0;
      for (int h = 0; h < G; h++) {
        const int32_t sh = gt.size[h];
        rank += (sh > sz) || (sh == sz && h < g);
      }
      order[rank] = g;
    }
    // experts with more than kIlvMaxK tokens come first in `order` (E2M1:
    // every expert takes the plain loop)
    static_assert(2 * kThreads >= kMaxGroups, "two groups per thread");
    const int n_long = KIND != kE4M3 ? G
                                     : __syncthreads_count(t < G && gt.size[t] > kIlvMaxK) +
                                           __syncthreads_count(t + kThreads < G && gt.size[t + kThreads] > kIlvMaxK);
    kbp = kb;
    orderp = order;
    first_g = ILV ? n_long : 0;
    n_tiles = (ILV ? G - n_long : n_long) * tiles_m * tiles_n;
  }

  const int P = gridDim.x;
  // Logical tile of round r for this workgroup, or -1.  Workgroups are dealt
  // to the XCDs round robin (XCD = bid % 8).
  //  - dense is launched with one workgroup per tile (round 0 only) and gives
  //    XCD x the contiguous range [x * per, (x + 1) * per) of the raster, so
  //    the tiles an XCD runs at once share operand panels in its L2;
  //  - the grouped modes run persistent with all XCDs in lockstep: round r
  //    covers the tiles [r * P, (r + 1) * P), XCD x its slice
  //    [x * P/8, (x + 1) * P/8), so every XCD works on the same experts at
  //    once and their panels are shared in the Infinity Cache.  Ragged-K
  //    tiles come largest group first, so the round-robin walk gives every
  //    workgroup a similar share of long and short tiles.
  auto tile_id = [&](int r) -> int {
    if constexpr (MODE == kDense) {
      return r == 0 ? xcd_remap(bid, n_tiles) : -1;
    } else {
      const int base = r * P;
      if (base >= n_tiles) return -1;
      const int id = base + P <= n_tiles ? base + xcd_remap(bid, P) : base + bid;
      return id < n_tiles ? id : -1;
    }
  };
  auto make_tile = [&](int id) {
    Tile tl;
    tl.lag = 0;
    tl.rot = 0;
    tl.head_chunks = 0;
    tl.row_lo = 0;
    tl.k_begin = 0;
    tl.klen = K;
    tl.b_base = B;
    tl.sb_base = sB;
    tl.c_base = C;
    int mt, nt;
    if constexpr (MODE == kDense) {
      raster(id, tiles_m, tiles_n, mt, nt);
      tl.m0 = (int64_t)mt * BM;
      tl.rows_a = (int)min<int64_t>(BM, M - tl.m0);
      tl.rows_load = tl.rows_a;
      // Neighbouring tiles share operand panels and run at once.  On a
      // checkerboard, half of them walk K one stage behind the others, so
      // they find each stage's panel lines already in L2 (fetched by their
      // neighbours a stage earlier) instead of all waiting on the same miss.
      tl.lag = (mt + nt) & 1;
    } else if constexpr (MODE == kRaggedM) {
      // A group's tiles start at the multiple of 128 at or below its first
      // row (the scale array's 128-row groups); rows of the tile outside the
      // group are computed with this expert but not stored.
      raster(id, n_tiles / tiles_n, tiles_n, mt, nt);
      tl.lag = (mt + nt) & 1;  // (as for dense)
      const int g = __builtin_amdgcn_readfirstlane(find_group(*gtp, G, mt));
      const int local = mt - __builtin_amdgcn_readfirstlane(gtp->bstart[g]);
      const int start = __builtin_amdgcn_readfirstlane(gtp->start[g]);
      const int64_t m_al = start & ~127;
      tl.m0 = m_al + (int64_t)local * BM;
      tl.row_lo = local == 0 ? start - (int)m_al : 0;
      tl.rows_a = (int)min<int64_t>(BM, start + __builtin_amdgcn_readfirstlane(gtp->size[g]) - tl.m0);
      tl.rows_load = (int)min<int64_t>(BM, M - tl.m0);
      tl.b_base = B + (int64_t)g * N * lda;
      tl.sb_base = sB + (int64_t)g * ((N + 127) / 128 * 128) * (K / 32);  // expert scale arrays hold ceil128(N) rows
    } else {
      const int per_g = tiles_m * tiles_n;
      const int gi = id / per_g;
      const int g = __builtin_amdgcn_readfirstlane(orderp[first_g + gi]);
      raster(id - gi * per_g, tiles_m, tiles_n, mt, nt);
      // (no lag: the tiles' operands come from HBM, not L2, and a lagged
      // checkerboard measured 0.25% slower here)
      tl.m0 = (int64_t)mt * BM;
      tl.rows_a = (int)min<int64_t>(BM, M - tl.m0);
      tl.rows_load = tl.rows_a;
      // [k_begin, k_end) inside [0, K] (kb is non-decreasing and >= 0)
      tl.k_begin = min<int64_t>((int64_t)__builtin_amdgcn_readfirstlane(kbp[g]) * 32, K);
      const int64_t k_end = min<int64_t>((int64_t)__builtin_amdgcn_readfirstlane(kbp[g + 1]) * 32, K);
      tl.klen = k_end > tl.k_begin ? k_end - tl.k_begin : 0;
      if constexpr (!ILV) {
        // Start the reduction at the 128-byte code line at or below the
        // expert's first token block, so that every stage's row loads are
        // whole lines when the row pitch is a multiple of 128 bytes (the
        // groups start at multiples of 32 tokens, and a row load straddling
        // two lines costs a second request: 4.2 -> 3.7 ms measured with
        // aligned starts).  The head's codes belong to earlier experts and
        // are zeroed in LDS once they land (fix below).
        if (tl.klen > 0) {
          const int64_t al = tl.k_begin / BKS * BKS;
          tl.head_chunks = (int)((tl.k_begin - al) / F::kElemsPerChunk);
          tl.klen += tl.k_begin - al;
          tl.k_begin = al;
        }
      }
      tl.c_base = C + (int64_t)g * M * N;
    }
    tl.n0 = (int64_t)nt * BN;
    tl.rows_b = (int)min<int64_t>(BN, N - tl.n0);
    const int ns = (int)((tl.klen + BKS - 1) / BKS);
    tl.nst = (ns + 1) & ~1;
    tl.last = ns - 1;
    tl.tail_chunks = ns > 0 ? (int)(tl.klen - (int64_t)tl.last * BKS) / F::kElemsPerChunk : F::kChunks;
    // E2M1 ragged K: each XCD's tiles start their K walk at a different eighth,
    // so the XCDs that share a token panel do not all wait on its HBM misses at
    // once (2.5% faster there; E4M3 measured 1% slower with it)
    if constexpr (MODE == kRaggedK && FP4) tl.rot = (int)((int64_t)(bid & 7) * ns / 8);
    return tl;
  };
  OperandAddr ada, adb;
  auto addr_of = [&](const Tile& tl) {
    const Operand opa{A + tl.m0 * lda, sA, tl.m0, lda, K / 32, tl.rows_load};
    const Operand opb{tl.b_base + tl.n0 * lda, tl.sb_base, tl.n0, lda, K / 32, tl.rows_b};
    ada = make_addr<KIND>(opa, wave, lane);
    adb = make_addr<KIND>(opb, wave, lane);
  };
  const int id0 = tile_id(0);
  auto tile_of = [&](int id) { return make_tile(id); };
  if constexpr (MODE != kDense) __syncthreads();  // group tables ready; stage 1 may now be loaded

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.f;

  uint8_t* const stages[2] = {stage0, stage1};
  // issue stage s of tile `tl` into LDS stage `slot`; stages past its last
  // re-load the last one (every stage issues the same loads)
  // real stage of loop stage s (stages past the last re-load the last)
  auto real_stage = [](const Tile& tl, int s) {
    if (s > tl.last) return tl.last;
    if constexpr (MODE == kRaggedK && FP4) {
      const int r = s + tl.rot;
      return r > tl.last ? r - tl.last - 1 : r;
    }
    return tl.lag ? (s == 0 ? tl.last : s - 1) : s;
  };
  auto issue = [&](int slot, const Tile& tl, int s) {
    const int sc = real_stage(tl, s);
    const int64_t k = tl.k_begin + (int64_t)sc * BKS;  // elements
    const int64_t kb = FP4 ? k / 2 : k;                // code bytes
    const int vc = sc == tl.last ? tl.tail_chunks : F::kChunks;
    const int vb = (int)((unsigned)vc * F::kElemsPerChunk / 32u);  // valid scale blocks
    uint8_t* st = stages[slot];
    issue_codes<KIND>(ada, st, wave, lane, kb, vc);
    issue_codes<KIND>(adb, st + kTileBytes, wave, lane, kb, vc);
    if (wave < 4)  // (uniform) waves 0-3 load A's scales, 4-7 B's
      issue_scales<KIND>(ada, st + 2 * kTileBytes, wave, lane, k, vb);
    else
      issue_scales<KIND>(adb, st + 2 * kTileBytes + kScaleRegion, wave, lane, k, vb);
  };
  // once stage s of `tl` has landed in `slot` (this wave's part): zero the
  // chunks past the end of K, or all of it if it only pads the loop
  auto fix = [&](int slot, const Tile& tl, int s) {
    const int vc = s > tl.last ? 0 : real_stage(tl, s) == tl.last ? tl.tail_chunks : F::kChunks;
    if (vc < F::kChunks) {
      zero_codes<KIND>(stages[slot], wave, lane, vc);
      zero_codes<KIND>(stages[slot] + kTileBytes, wave, lane, vc);
    }
    if constexpr (MODE == kRaggedK && !ILV) {
      if (tl.head_chunks > 0 && s <= tl.last && real_stage(tl, s) == 0) {
        zero_head_codes<KIND>(stages[slot], wave, lane, tl.head_chunks);
        zero_head_codes<KIND>(stages[slot] + kTileBytes, wave, lane, tl.head_chunks);
      }
    }
  };
  auto pin = [&]() {
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int j = 0; j < TN; j++) asm volatile("" : "+a"(acc[i][j]));
  };
  Frags f;
  // The MFMA steps of a stage in LDS stage `cur` (published by the last
  // barrier).  Each wave reads a step's fragments and runs its 8 MFMAs as
  // soon as they arrive (the compiler waits per fragment); the other wave on
  // the SIMD keeps the matrix pipe busy meanwhile.  The loads of the stage
  // that follows (tile nt, stage ns) go out at step 0 (around its fragment
  // reads), into the other LDS stage (every wave finished reading it before
  // the last barrier), and have the stage's steps to land.
  // ILV: `vs` is the number of interleaved steps with real K values in the
  // stage (0 for a stage that only pads the loop).
  auto stage_steps = [&](int cur, const Tile& nt, int ns, int vs) {
    if constexpr (ILV) {
      if (vs > 0) read_frags_ilv(stages[cur], 0, wm, wn, lane, f);
      issue(cur ^ 1, nt, ns);
      if (vs > 0) {
        mfma_step<KIND>(acc, f);
        pin();
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
      for (int st = 1; st < vs; st++) {
        read_frags_ilv(stages[cur], st, wm, wn, lane, f);
        mfma_step<KIND>(acc, f);
        pin();
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // step 0
      // (E4M3: the loads go out before step 0's fragment reads, 0.4-1% faster
      // per GEMM; E2M1 keeps them after, which measured faster for it)
      if constexpr (KIND == kE4M3) {
        issue(cur ^ 1, nt, ns);
        read_frags<KIND>(stages[cur], 0, wm, wn, lane, f);
      } else {
        read_frags<KIND>(stages[cur], 0, wm, wn, lane, f);
        issue(cur ^ 1, nt, ns);
      }
      mfma_step<KIND, MODE == kRaggedK && FP4>(acc, f);
      pin();
      __builtin_amdgcn_sched_barrier(0);
      // steps 1 ..
#pragma unroll
      for (int st = 1; st < F::kSteps; st++) {
        read_frags<KIND>(stages[cur], st, wm, wn, lane, f);
        mfma_step<KIND, MODE == kRaggedK && FP4>(acc, f);
        pin();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // publish the following stage; after the barrier every wave is done reading `cur`
    wait_vmcnt<0>();  // this wave's loads of the following stage landed
    fix(cur ^ 1, nt, ns);
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  int r = 0;
  int id = id0;
  bool ready = false;  // the current tile's stage 0 is loaded and published
  while (id >= 0) {
    const int nid = MODE != kDense ? tile_id(r + 1) : -1;  // (dense: one tile per workgroup)
    bool nxt_ok = false;
    {
      const Tile cur = tile_of(id);
      if (cur.nst > 0) {  // (an empty expert's tile only stores zeros)
        if (!ready) {
          wait_vmcnt<0>();  // loads of an earlier pass into the stages have landed
          __builtin_amdgcn_s_barrier();
          addr_of(cur);
          issue(0, cur, 0);
          wait_vmcnt<0>();  // stage 0 landed
          fix(0, cur, 0);
          wait_lgkmcnt0();
          __builtin_amdgcn_s_barrier();
        }
        // interleaved steps with real K values in loop stage s (8 K values each)
        auto vsteps = [&](int s) {
          if (s > cur.last) return 0;
          return real_stage(cur, s) == cur.last ? cur.tail_chunks * (F::kElemsPerChunk / 8) : kIlvSteps;
        };
        for (int s = 0; s < cur.nst - 2; s += 2) {
          stage_steps(0, cur, s + 1, ILV ? vsteps(s) : 0);
          stage_steps(1, cur, s + 2, ILV ? vsteps(s + 1) : 0);
        }
        stage_steps(0, cur, cur.nst - 1, ILV ? vsteps(cur.nst - 2) : 0);
        // the last stage loads the next tile's first (or, with no next tile,
        // re-loads this tile's last stage, which nobody reads)
        Tile nxt = cur;
        int ns = cur.nst;
        if (nid >= 0) {
          const Tile t2 = tile_of(nid);
          if (t2.nst > 0) {
            nxt = t2;
            ns = 0;
            nxt_ok = true;
            addr_of(nxt);
          }
        }
        stage_steps(1, nxt, ns, ILV ? vsteps(cur.nst - 1) : 0);
      }
    }
    {
      const Tile cur = tile_of(id);  // (recomputed: keeps it out of registers during the K loop)
      store_tile(acc, cur, ldo, wm, wn, lane);
    }
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int j = 0; j < TN; j++)
#pragma unroll
        for (int e = 0; e < 16; e++) acc[i][j][e] = 0.f;
    ready = nxt_ok;
    id = nid;
    r++;
  }
  wait_vmcnt<0>();  // the loads still in flight land before the LDS goes away
}

}  // namespace

// plain or interleaved kernel of one mode (dense and ragged M: interleaved
// iff K <= kIlvMaxK; E2M1 always plain)
template <int MODE, int KIND>
void launch_mode(bool ilv, unsigned grid, hipStream_t st, const uint8_t* A, const uint8_t* sA, const uint8_t* B,
                 const uint8_t* sB, float* C, int64_t M, int64_t N, int64_t K, int64_t ldc, const int32_t* group_end,
                 int32_t G, int tiles_m, int tiles_n) {
  if constexpr (KIND == kE4M3) {
    if (ilv) {
      gemm_mx_kernel<MODE, KIND, true><<<grid, kThreads, 0, st>>>(A, sA, B, sB, C, M, N, K, ldc, group_end, G,
                                                                  tiles_m, tiles_n);
      return;
    }
  }
  gemm_mx_kernel<MODE, KIND, false><<<grid, kThreads, 0, st>>>(A, sA, B, sB, C, M, N, K, ldc, group_end, G,
                                                               tiles_m, tiles_n);
}

template <int KIND>
hipError_t launch_gemm_kind(int mode, const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                            float* C, int64_t M, int64_t N, int64_t K, int64_t ldc, const int32_t* group_end,
                            int32_t G, hipStream_t st) {
  // 32-bit per-lane load offsets: 256 rows of codes of one tile
  if ((int64_t)BM * (KIND != kE4M3 ? K / 2 : K) >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t tiles_m = (M + BM - 1) / BM;
  const int64_t cus = device_cu_count();
  if (mode == kDense) {
    const int64_t total = tiles_m * tiles_n;  // one workgroup per tile
    if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int64_t grid = total;
    launch_mode<kDense, KIND>(K <= kIlvMaxK, (unsigned)grid, st, A, sA, B, sB, C, M, N, K, ldc, nullptr, 1,
                              (int)tiles_m, (int)tiles_n);
  } else if (mode == kRaggedM) {
    // a group's tiles start up to 127 rows before it and it may end in a
    // partial tile: at most two extra m-tiles per group
    const int64_t total = (tiles_m + 2 * (int64_t)G) * tiles_n;
    if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int64_t grid = total < cus ? total : cus;
    launch_mode<kRaggedM, KIND>(K <= kIlvMaxK, (unsigned)grid, st, A, sA, B, sB, C, M, N, K, ldc, group_end, G,
                                (int)tiles_m, (int)tiles_n);
  } else {
    const int64_t total = (int64_t)G * tiles_m * tiles_n;
    if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int64_t grid = total < cus ? total : cus;
    // E4M3: experts with more than kIlvMaxK tokens, then the others (each
    // launch finds its experts from group_end on the device); E2M1: one
    // launch for all experts
    launch_mode<kRaggedK, KIND>(false, (unsigned)grid, st, A, sA, B, sB, C, M, N, K, N, group_end, G,
                                (int)tiles_m, (int)tiles_n);
    if (KIND == kE4M3) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      launch_mode<kRaggedK, KIND>(true, (unsigned)grid, st, A, sA, B, sB, C, M, N, K, N, group_end, G,
                                  (int)tiles_m, (int)tiles_n);
    }
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int mode, bool fp4, const uint8_t* A, const uint8_t* sA, const uint8_t* B,
                       const uint8_t* sB, float* C, int64_t M, int64_t N, int64_t K, int64_t ldc,
                       const int32_t* group_end, int32_t G, hipStream_t st) {
  if (!fp4) return launch_gemm_kind<kE4M3>(mode, A, sA, B, sB, C, M, N, K, ldc, group_end, G, st);
  return launch_gemm_kind<kE2M1>(mode, A, sA, B, sB, C, M, N, K, ldc, group_end, G, st);
}

}  // namespace mxq
