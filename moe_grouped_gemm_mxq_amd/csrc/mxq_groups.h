// Per-workgroup table of ragged groups, built on the device from cumulative
// group ends (used by the grouped quantiser and the grouped GEMM schedulers).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

constexpr int kMaxGroups = 1024;

// start row and size of every group, and the exclusive prefix of
// ceil(size / unit) (bstart[G] = total units).  Group ends are clamped into
// [0, R] (R < 2^31), so a malformed array never sends an access out of
// bounds; a valid (non-decreasing, <= R) array is used unchanged.
struct GroupTable {
  int32_t start[kMaxGroups];
  int32_t size[kMaxGroups];
  int32_t bstart[kMaxGroups + 1];
};

// Clamped start row and size of group g (ends clamped into [0, R]; a group
// ending before it starts is empty).
__device__ __forceinline__ void group_span(const int32_t* __restrict__ group_end, int g, int64_t R,
                                           int32_t& start, int32_t& size) {
  int64_t e = group_end[g];
  int64_t b = g ? (int64_t)group_end[g - 1] : 0;
  e = e < 0 ? 0 : (e > R ? R : e);
  b = b < 0 ? 0 : (b > R ? R : b);
  start = (int32_t)b;
  size = e > b ? (int32_t)(e - b) : 0;
}

// All THREADS threads of the workgroup must call this; G <= 4 * THREADS.
// start / size may be null (only the block starts are written then).  With
// align > 1 a non-empty group's units start at the multiple of `align` at or
// below its first row: it counts ceil((size + start % align) / unit) units.
// The unit counts and their prefix sums are taken in 64 bits and the prefix
// saturates at INT32_MAX, so for any group_end array (even a malformed one)
// bstart is non-decreasing and bstart[g + 1] - bstart[g] never exceeds group
// g's own unit count: a position u in [bstart[g], bstart[g + 1]) always lies
// inside group g's clamped rows.
template <int THREADS>
__device__ void build_block_starts(const int32_t* __restrict__ group_end, int32_t G, int64_t R,
                                   int32_t unit, int32_t* start, int32_t* size, int32_t* bstart /* [G + 1] */,
                                   int64_t* scan_tmp /* [THREADS] */, int32_t align = 1) {
  static_assert(4 * THREADS >= kMaxGroups, "each thread owns at most four groups");
  const int t = threadIdx.x;
  int64_t local = 0;
  int64_t nb[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int g = t * 4 + j;
    nb[j] = 0;
    if (g < G) {
      int32_t b, m;
      group_span(group_end, g, R, b, m);
      if (start) start[g] = b;
      if (size) size[g] = m;
      nb[j] = m > 0 ? ((int64_t)m + b % align + unit - 1) / unit : 0;
      local += nb[j];
    }
  }
  // exclusive scan of `local` over the workgroup (Hillis-Steele in LDS)
  scan_tmp[t] = local;
  __syncthreads();
  for (int off = 1; off < THREADS; off <<= 1) {
    const int64_t v = t >= off ? scan_tmp[t - off] : 0;
    __syncthreads();
    scan_tmp[t] += v;
    __syncthreads();
  }
  constexpr int64_t kSat = 0x7FFFFFFF;
  int64_t run = scan_tmp[t] - local;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int g = t * 4 + j;
    if (g < G) {
      bstart[g] = (int32_t)(run < kSat ? run : kSat);
      run += nb[j];
    }
  }
  if (t == THREADS - 1) bstart[G] = (int32_t)(scan_tmp[t] < kSat ? scan_tmp[t] : kSat);
  __syncthreads();
}

template <int THREADS>
__device__ void build_group_table(const int32_t* __restrict__ group_end, int32_t G, int64_t R,
                                  int32_t unit, GroupTable& gt, int64_t* scan_tmp /* [THREADS] */,
                                  int32_t align = 1) {
  build_block_starts<THREADS>(group_end, G, R, unit, gt.start, gt.size, gt.bstart, scan_tmp, align);
}

// largest g with bstart[g] <= u (u < bstart[G] assumed)
__device__ __forceinline__ int find_block_group(const int32_t* bstart, int G, int32_t u) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (bstart[mid] <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// largest g with bstart[g] <= u (u < bstart[G] assumed)
__device__ __forceinline__ int find_group(const GroupTable& gt, int G, int32_t u) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (gt.bstart[mid] <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace mxq
