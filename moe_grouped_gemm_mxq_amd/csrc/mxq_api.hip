// C ABI of libmxq (declared in include/mxq.h): host-side argument checks, the
// gfx950 device gate, error reporting, and dispatch to the kernel launchers.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/mxq.h"
#include "mxq_internal.h"

namespace mxq {

static_assert(kIlvMaxK == MXQ_EXACT_GROUPS_MAX_K, "the header states the kernels' threshold");

namespace {

thread_local std::string g_last_error;

mxq_status fail(mxq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

mxq_status ok() {
  g_last_error.clear();
  return MXQ_OK;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_cu_count[kMaxDevices];

mxq_status check_device_id(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MXQ_ERR_DEVICE, "HIP device %d out of range", dev);
  int state = g_arch_state[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(MXQ_ERR_DEVICE, "no HIP device %d", dev);
    }
    state = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_state[dev].store(state, std::memory_order_relaxed);
    if (state == 2)
      return fail(MXQ_ERR_DEVICE, "HIP device %d is %s; libmxq runs on gfx950 (MI355X) only", dev,
                  prop.gcnArchName);
  }
  if (state != 1) return fail(MXQ_ERR_DEVICE, "HIP device %d is not gfx950 (MI355X)", dev);
  return MXQ_OK;
}

mxq_status check_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(MXQ_ERR_DEVICE, "no current HIP device");
  }
  return check_device_id(dev);
}

mxq_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MXQ_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace mxq

using namespace mxq;

#define MXQ_REQUIRE(cond, ...) \
  do {                         \
    if (!(cond)) return fail(MXQ_ERR_INVALID_ARGUMENT, __VA_ARGS__); \
  } while (0)

#define MXQ_REQUIRE_DEVICE()                     \
  do {                                           \
    mxq_status _s = check_current_device();      \
    if (_s != MXQ_OK) return _s;                 \
  } while (0)

extern "C" {

int mxq_abi_version(void) { return MXQ_ABI_VERSION; }

const char* mxq_last_error(void) { return g_last_error.c_str(); }

mxq_status mxq_device_check(int device) {
  mxq_status s = check_device_id(device);
  return s == MXQ_OK ? ok() : s;
}

int64_t mxq_grouped_cols_max(int64_t T, int32_t G) {
  if (T < 0 || G < 0) return 0;
  int64_t n = (T + 31 * (int64_t)G + 255) / 256;  // 256-column units
  if (n % 2 == 0) n++;                              // an odd number of them
  return n * 256;
}

mxq_status mxq_operand_sizes(int64_t rows, int64_t K, int fmt, int64_t* code_bytes, int64_t* scale_bytes) {
  MXQ_REQUIRE(code_bytes && scale_bytes, "mxq_operand_sizes: NULL output");
  MXQ_REQUIRE(rows >= 1 && K >= 1, "mxq_operand_sizes: rows and K must be >= 1");
  MXQ_REQUIRE(fmt == MXQ_FMT_E4M3 || fmt == MXQ_FMT_E2M1, "mxq_operand_sizes: unknown format %d", fmt);
  const int64_t Kp = (K + 31) / 32 * 32;
  *code_bytes = fmt == MXQ_FMT_E4M3 ? rows * Kp : rows * (Kp / 2);
  *scale_bytes = (rows + 127) / 128 * 128 * (Kp / 32);
  return MXQ_OK;
}

mxq_status mxq_quantize(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, int axis_mask,
                        uint8_t* q_row, uint8_t* s_row, uint8_t* q_colT, uint8_t* s_colT,
                        hipStream_t st) {
  MXQ_REQUIRE(x != nullptr, "mxq_quantize: x is NULL");
  MXQ_REQUIRE(R >= 1 && C >= 1, "mxq_quantize: R and C must be >= 1 (got %lld x %lld)", (long long)R,
              (long long)C);
  MXQ_REQUIRE(ldx >= C, "mxq_quantize: ldx (%lld) < C (%lld)", (long long)ldx, (long long)C);
  MXQ_REQUIRE(axis_mask >= 1 && axis_mask <= 3, "mxq_quantize: axis_mask must be ROW, COLT or ROW|COLT");
  const bool row = axis_mask & MXQ_AXIS_ROW, col = axis_mask & MXQ_AXIS_COLT;
  MXQ_REQUIRE(!row || (q_row && s_row), "mxq_quantize: row outputs are NULL");
  MXQ_REQUIRE(!col || (q_colT && s_colT), "mxq_quantize: colT outputs are NULL");
  MXQ_REQUIRE((!row || aligned16(q_row)) && (!col || aligned16(q_colT)),
              "mxq_quantize: code outputs must be 16-byte aligned");
  MXQ_REQUIRE(((uintptr_t)x & 1u) == 0, "mxq_quantize: x must be 2-byte aligned");
  MXQ_REQUIRE(!row || ((uintptr_t)s_row & 3u) == 0, "mxq_quantize: s_row must be 4-byte aligned");
  MXQ_REQUIRE_DEVICE();
  if (!col) return launched(launch_quant_row(x, R, C, ldx, q_row, s_row, st), "mxq_quantize(row)");
  const int64_t Rp = (R + 31) / 32 * 32;
  return launched(launch_quant_tile(x, R, C, ldx, nullptr, 1, Rp, row ? q_row : nullptr,
                                    row ? s_row : nullptr, q_colT, s_colT, st),
                  "mxq_quantize(colT)");
}

mxq_status mxq_quantize_batched(const uint16_t* x, int64_t batch, int64_t R, int64_t C, int64_t ldx,
                                int64_t x_stride, int axis_mask, uint8_t* q_row, uint8_t* s_row,
                                uint8_t* q_colT, uint8_t* s_colT, hipStream_t st) {
  MXQ_REQUIRE(x != nullptr, "mxq_quantize_batched: x is NULL");
  MXQ_REQUIRE(batch >= 1 && batch <= 65535, "mxq_quantize_batched: batch must be in [1, 65535] (got %lld)",
              (long long)batch);
  MXQ_REQUIRE(R >= 1 && C >= 1, "mxq_quantize_batched: R and C must be >= 1 (got %lld x %lld)",
              (long long)R, (long long)C);
  MXQ_REQUIRE(ldx >= C, "mxq_quantize_batched: ldx (%lld) < C (%lld)", (long long)ldx, (long long)C);
  MXQ_REQUIRE(batch == 1 || x_stride >= (R - 1) * ldx + C,
              "mxq_quantize_batched: x_stride (%lld) smaller than one matrix", (long long)x_stride);
  MXQ_REQUIRE(axis_mask >= 1 && axis_mask <= 3, "mxq_quantize_batched: axis_mask must be ROW, COLT or ROW|COLT");
  const bool row = axis_mask & MXQ_AXIS_ROW, col = axis_mask & MXQ_AXIS_COLT;
  MXQ_REQUIRE(!row || (q_row && s_row), "mxq_quantize_batched: row outputs are NULL");
  MXQ_REQUIRE(!col || (q_colT && s_colT), "mxq_quantize_batched: colT outputs are NULL");
  MXQ_REQUIRE((!row || aligned16(q_row)) && (!col || aligned16(q_colT)),
              "mxq_quantize_batched: code outputs must be 16-byte aligned");
  MXQ_REQUIRE(((uintptr_t)x & 1u) == 0, "mxq_quantize_batched: x must be 2-byte aligned");
  MXQ_REQUIRE(!row || ((uintptr_t)s_row & 3u) == 0, "mxq_quantize_batched: s_row must be 4-byte aligned");
  MXQ_REQUIRE_DEVICE();
  const int64_t Cp = (C + 31) / 32 * 32, Rp = (R + 31) / 32 * 32;
  // each matrix's outputs exactly as mxq_quantize lays them out, back to back
  // scale arrays hold ceil128(rows) rows (the GEMM operand scale layout)
  const BatchStrides bs{x_stride, R * Cp, (R + 127) / 128 * 128 * (Cp / 32), C * Rp, (C + 127) / 128 * 128 * (Rp / 32)};
  if (!col)
    return launched(launch_quant_row(x, R, C, ldx, q_row, s_row, st, (int)batch, bs), "mxq_quantize_batched(row)");
  return launched(launch_quant_tile(x, R, C, ldx, nullptr, 1, Rp, row ? q_row : nullptr, row ? s_row : nullptr,
                                    q_colT, s_colT, st, (int)batch, bs),
                  "mxq_quantize_batched(colT)");
}

mxq_status mxq_quantize_grouped(const uint16_t* x, int64_t T, int64_t C, int64_t ldx,
                                const int32_t* group_end, int32_t G, int64_t ldq, int axis_mask,
                                uint8_t* q_row, uint8_t* s_row, uint8_t* q_colT, uint8_t* s_colT,
                                hipStream_t st) {
  MXQ_REQUIRE(x != nullptr && group_end != nullptr, "mxq_quantize_grouped: x or group_end is NULL");
  MXQ_REQUIRE(T >= 1 && C >= 1, "mxq_quantize_grouped: T and C must be >= 1");
  MXQ_REQUIRE(T <= INT32_MAX, "mxq_quantize_grouped: T must be < 2^31 (group ends are int32)");
  MXQ_REQUIRE(ldx >= C, "mxq_quantize_grouped: ldx < C");
  MXQ_REQUIRE(G >= 1 && G <= MXQ_MAX_GROUPS, "mxq_quantize_grouped: G must be in [1, %d] (got %d)",
              MXQ_MAX_GROUPS, G);
  MXQ_REQUIRE(axis_mask >= 1 && axis_mask <= 3, "mxq_quantize_grouped: bad axis_mask");
  const bool row = axis_mask & MXQ_AXIS_ROW, col = axis_mask & MXQ_AXIS_COLT;
  MXQ_REQUIRE(!col || (ldq >= 32 && ldq % 32 == 0), "mxq_quantize_grouped: ldq must be a positive multiple of 32");
  MXQ_REQUIRE(!row || (q_row && s_row), "mxq_quantize_grouped: row outputs are NULL");
  MXQ_REQUIRE(!col || (q_colT && s_colT), "mxq_quantize_grouped: colT outputs are NULL");
  MXQ_REQUIRE((!row || aligned16(q_row)) && (!col || aligned16(q_colT)),
              "mxq_quantize_grouped: code outputs must be 16-byte aligned");
  MXQ_REQUIRE(((uintptr_t)x & 1u) == 0, "mxq_quantize_grouped: x must be 2-byte aligned");
  MXQ_REQUIRE(!row || ((uintptr_t)s_row & 3u) == 0, "mxq_quantize_grouped: s_row must be 4-byte aligned");
  MXQ_REQUIRE_DEVICE();
  if (!col) return launched(launch_quant_row(x, T, C, ldx, q_row, s_row, st), "mxq_quantize_grouped(row)");
  return launched(launch_quant_tile(x, T, C, ldx, group_end, G, ldq, row ? q_row : nullptr,
                                    row ? s_row : nullptr, q_colT, s_colT, st),
                  "mxq_quantize_grouped(colT)");
}

mxq_status mxq_qdq_fp4(const float* x, float* y, int64_t rows, int64_t L, uint8_t* codes,
                       uint8_t* scales, hipStream_t st) {
  MXQ_REQUIRE(x != nullptr && y != nullptr, "mxq_qdq_fp4: x or y is NULL");
  MXQ_REQUIRE(rows >= 1 && L >= 1, "mxq_qdq_fp4: rows and L must be >= 1");
  MXQ_REQUIRE(((uintptr_t)x & 3u) == 0 && ((uintptr_t)y & 3u) == 0, "mxq_qdq_fp4: x, y must be 4-byte aligned");
  MXQ_REQUIRE(!codes || aligned16(codes), "mxq_qdq_fp4: codes must be 16-byte aligned");
  int F;
  uint32_t T;
  fp4_scale_params(6.0f, &F, &T);
  MXQ_REQUIRE_DEVICE();
  return launched(launch_qdq_fp4(x, y, rows, L, F, T, codes, scales, nullptr, st), "mxq_qdq_fp4");
}

mxq_status mxq_qdq_fp4_ex(const float* x, float* y, int64_t rows, int64_t L, float scale_factor,
                          uint8_t* codes, uint8_t* scales, uint8_t* sat_mask, hipStream_t st) {
  MXQ_REQUIRE(x != nullptr && y != nullptr, "mxq_qdq_fp4_ex: x or y is NULL");
  MXQ_REQUIRE(rows >= 1 && L >= 1, "mxq_qdq_fp4_ex: rows and L must be >= 1");
  MXQ_REQUIRE(((uintptr_t)x & 3u) == 0 && ((uintptr_t)y & 3u) == 0, "mxq_qdq_fp4_ex: x, y must be 4-byte aligned");
  MXQ_REQUIRE(!codes || aligned16(codes), "mxq_qdq_fp4_ex: codes must be 16-byte aligned");
  MXQ_REQUIRE(!sat_mask || ((uintptr_t)sat_mask & 3u) == 0, "mxq_qdq_fp4_ex: sat_mask must be 4-byte aligned");
  int F;
  uint32_t T;
  MXQ_REQUIRE(fp4_scale_params(scale_factor, &F, &T),
              "mxq_qdq_fp4_ex: scale_factor must be a normal fp32 value in [2^-64, 2^64) (got %g)",
              (double)scale_factor);
  MXQ_REQUIRE_DEVICE();
  return launched(launch_qdq_fp4(x, y, rows, L, F, T, codes, scales, sat_mask, st), "mxq_qdq_fp4_ex");
}

mxq_status mxq_quantize_fp4(const float* x, int64_t rows, int64_t L, float scale_factor, uint8_t* codes,
                            uint8_t* scales, hipStream_t st) {
  MXQ_REQUIRE(x && codes && scales, "mxq_quantize_fp4: NULL operand");
  MXQ_REQUIRE(rows >= 1 && L >= 1, "mxq_quantize_fp4: rows and L must be >= 1");
  MXQ_REQUIRE(((uintptr_t)x & 3u) == 0, "mxq_quantize_fp4: x must be 4-byte aligned");
  MXQ_REQUIRE(aligned16(codes), "mxq_quantize_fp4: codes must be 16-byte aligned");
  int F;
  uint32_t T;
  MXQ_REQUIRE(fp4_scale_params(scale_factor, &F, &T),
              "mxq_quantize_fp4: scale_factor must be a normal fp32 value in [2^-64, 2^64) (got %g)",
              (double)scale_factor);
  MXQ_REQUIRE_DEVICE();
  return launched(launch_qdq_fp4(x, nullptr, rows, L, F, T, codes, scales, nullptr, st, true), "mxq_quantize_fp4");
}

mxq_status mxq_quantize_fp4_grouped(const float* x, int64_t T, int64_t C, int64_t ldx, const int32_t* group_end,
                                    int32_t G, int64_t ldq, float scale_factor, uint8_t* codes, uint8_t* scales,
                                    hipStream_t st) {
  MXQ_REQUIRE(x && group_end && codes && scales, "mxq_quantize_fp4_grouped: NULL pointer");
  MXQ_REQUIRE(T >= 1 && C >= 1, "mxq_quantize_fp4_grouped: T and C must be >= 1");
  MXQ_REQUIRE(T <= INT32_MAX, "mxq_quantize_fp4_grouped: T must be < 2^31 (group ends are int32)");
  MXQ_REQUIRE(ldx >= C, "mxq_quantize_fp4_grouped: ldx < C");
  MXQ_REQUIRE(G >= 1 && G <= MXQ_MAX_GROUPS, "mxq_quantize_fp4_grouped: G must be in [1, %d] (got %d)",
              MXQ_MAX_GROUPS, G);
  MXQ_REQUIRE(ldq >= 32 && ldq % 32 == 0, "mxq_quantize_fp4_grouped: ldq must be a positive multiple of 32");
  MXQ_REQUIRE(((uintptr_t)x & 3u) == 0, "mxq_quantize_fp4_grouped: x must be 4-byte aligned");
  MXQ_REQUIRE(aligned16(codes), "mxq_quantize_fp4_grouped: codes must be 16-byte aligned");
  int F;
  uint32_t Tth;
  MXQ_REQUIRE(fp4_scale_params(scale_factor, &F, &Tth),
              "mxq_quantize_fp4_grouped: scale_factor must be a normal fp32 value in [2^-64, 2^64) (got %g)",
              (double)scale_factor);
  MXQ_REQUIRE_DEVICE();
  return launched(launch_quant_fp4_grouped(x, T, C, ldx, group_end, G, ldq, F, Tth, codes, scales, st),
                  "mxq_quantize_fp4_grouped");
}

mxq_status mxq_ste_backward_fp4(const float* grad_y, const uint8_t* sat_mask, float* grad_x,
                                int64_t rows, int64_t L, hipStream_t st) {
  MXQ_REQUIRE(grad_y && sat_mask && grad_x, "mxq_ste_backward_fp4: NULL operand");
  MXQ_REQUIRE(rows >= 1 && L >= 1, "mxq_ste_backward_fp4: rows and L must be >= 1");
  MXQ_REQUIRE(((uintptr_t)grad_y & 3u) == 0 && ((uintptr_t)grad_x & 3u) == 0 && ((uintptr_t)sat_mask & 3u) == 0,
              "mxq_ste_backward_fp4: grad_y, grad_x and sat_mask must be 4-byte aligned");
  MXQ_REQUIRE(grad_x == grad_y || grad_x + rows * L <= grad_y || grad_y + rows * L <= grad_x,
              "mxq_ste_backward_fp4: grad_x must be grad_y or not overlap it");
  MXQ_REQUIRE_DEVICE();
  return launched(launch_ste_backward_fp4(grad_y, sat_mask, grad_x, rows, L, st), "mxq_ste_backward_fp4");
}

mxq_status mxq_fp4_scale_threshold(float scale_factor, int32_t* F, uint32_t* T) {
  MXQ_REQUIRE(F && T, "mxq_fp4_scale_threshold: NULL output");
  int f;
  MXQ_REQUIRE(fp4_scale_params(scale_factor, &f, T),
              "mxq_fp4_scale_threshold: scale_factor must be a normal fp32 value in [2^-64, 2^64)");
  *F = f;
  return MXQ_OK;
}

mxq_status mxq_gemm(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                    float* C, int64_t M, int64_t N, int64_t K, int64_t ldc, mxq_fmt fmt,
                    hipStream_t st) {
  MXQ_REQUIRE(A && sA && B && sB && C, "mxq_gemm: NULL operand");
  MXQ_REQUIRE(M >= 1 && N >= 1, "mxq_gemm: M and N must be >= 1");
  MXQ_REQUIRE(K >= 32 && K % 32 == 0, "mxq_gemm: K must be a positive multiple of 32 (got %lld)", (long long)K);
  MXQ_REQUIRE(ldc >= N, "mxq_gemm: ldc < N");
  MXQ_REQUIRE(aligned16(A) && aligned16(B) && ((uintptr_t)C & 3u) == 0, "mxq_gemm: A, B must be 16-byte aligned");
  MXQ_REQUIRE((((uintptr_t)sA | (uintptr_t)sB) & 3u) == 0,
              "mxq_gemm: sA, sB must be 4-byte aligned (the kernel reads scale dwords)");
  if (fmt != MXQ_FMT_E4M3 && fmt != MXQ_FMT_E2M1)
    return fail(MXQ_ERR_UNSUPPORTED, "mxq_gemm: unknown operand format %d", (int)fmt);
  MXQ_REQUIRE((fmt == MXQ_FMT_E2M1 ? K / 2 : K) < MXQ_GEMM_MAX_ROW_BYTES,
              "mxq_gemm: K = %lld gives code rows of MXQ_GEMM_MAX_ROW_BYTES or more", (long long)K);
  MXQ_REQUIRE_DEVICE();
  return launched(launch_gemm(0, fmt == MXQ_FMT_E2M1, A, sA, B, sB, C, M, N, K, ldc, nullptr, 1, st), "mxq_gemm");
}

mxq_status mxq_grouped_gemm(mxq_gg_mode mode, const uint8_t* A, const uint8_t* sA,
                            const uint8_t* B, const uint8_t* sB, float* C,
                            int64_t M, int64_t N, int64_t K,
                            const int32_t* group_end, int32_t G, mxq_fmt fmt, hipStream_t st) {
  MXQ_REQUIRE(A && sA && B && sB && C && group_end, "mxq_grouped_gemm: NULL operand");
  MXQ_REQUIRE(mode == MXQ_GG_RAGGED_M || mode == MXQ_GG_RAGGED_K, "mxq_grouped_gemm: bad mode");
  MXQ_REQUIRE(M >= 1 && N >= 1, "mxq_grouped_gemm: M and N must be >= 1");
  MXQ_REQUIRE(K >= 32 && K % 32 == 0, "mxq_grouped_gemm: K must be a positive multiple of 32");
  MXQ_REQUIRE(G >= 1 && G <= MXQ_MAX_GROUPS, "mxq_grouped_gemm: G must be in [1, %d]", MXQ_MAX_GROUPS);
  MXQ_REQUIRE(mode != MXQ_GG_RAGGED_M || M <= INT32_MAX,
              "mxq_grouped_gemm: M must be < 2^31 for MXQ_GG_RAGGED_M (group ends are int32)");
  MXQ_REQUIRE(aligned16(A) && aligned16(B) && ((uintptr_t)C & 3u) == 0, "mxq_grouped_gemm: A, B must be 16-byte aligned");
  MXQ_REQUIRE((((uintptr_t)sA | (uintptr_t)sB) & 3u) == 0,
              "mxq_grouped_gemm: sA, sB must be 4-byte aligned (the kernel reads scale dwords)");
  if (fmt != MXQ_FMT_E4M3 && fmt != MXQ_FMT_E2M1)
    return fail(MXQ_ERR_UNSUPPORTED, "mxq_grouped_gemm: unknown operand format %d", (int)fmt);
  MXQ_REQUIRE((fmt == MXQ_FMT_E2M1 ? K / 2 : K) < MXQ_GEMM_MAX_ROW_BYTES,
              "mxq_grouped_gemm: K = %lld gives code rows of MXQ_GEMM_MAX_ROW_BYTES or more", (long long)K);
  MXQ_REQUIRE_DEVICE();
  return launched(launch_gemm(mode == MXQ_GG_RAGGED_M ? 1 : 2, fmt == MXQ_FMT_E2M1, A, sA, B, sB, C, M, N, K, N,
                              group_end, G, st),
                  "mxq_grouped_gemm");
}

mxq_status mxq_validate_group_end(const int32_t* group_end, int32_t G, int64_t T, int32_t* flag,
                                  hipStream_t st) {
  MXQ_REQUIRE(group_end && flag, "mxq_validate_group_end: NULL pointer");
  MXQ_REQUIRE(G >= 1 && G <= MXQ_MAX_GROUPS, "mxq_validate_group_end: G must be in [1, %d]", MXQ_MAX_GROUPS);
  MXQ_REQUIRE(T >= 0, "mxq_validate_group_end: T must be >= 0");
  MXQ_REQUIRE_DEVICE();
  return launched(launch_validate_group_end(group_end, G, T, flag, st), "mxq_validate_group_end");
}

}  // extern "C"

// ------------------------------------------------------------------ validator kernel
namespace mxq {
namespace {
__global__ __launch_bounds__(1024) void validate_group_end_kernel(const int32_t* __restrict__ ge, int32_t G,
                                                                  int64_t T, int32_t* __restrict__ flag) {
  __shared__ int first_bad;
  const int g = threadIdx.x;
  if (g == 0) first_bad = G;
  __syncthreads();
  if (g < G) {
    const int64_t e = ge[g];
    const int64_t prev = g ? (int64_t)ge[g - 1] : 0;
    if (e < prev || e < 0 || e > T) atomicMin(&first_bad, g);
  }
  __syncthreads();
  if (g == 0) *flag = first_bad == G ? 0 : first_bad + 1;
}
}  // namespace

hipError_t launch_validate_group_end(const int32_t* group_end, int32_t G, int64_t T, int32_t* flag,
                                     hipStream_t st) {
  validate_group_end_kernel<<<1, 1024, 0, st>>>(group_end, G, T, flag);
  return hipGetLastError();
}
}  // namespace mxq
